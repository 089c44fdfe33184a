"""The allocation-free pass 1 (logra_update_sqnorm_noalloc) against the
workspace pass 1 (logra_update_sqnorm) through the C ABI: the same kernels,
so v', rowsq and sqnorm must be bit-identical, on consecutive calls that
reuse the library's device scratch, the second and third with smaller
inputs than the first, and on the fp32 path."""
import pytest
import torch

from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _state(seed, d, r, dev):
    g = inputs.generator("noalloc", seed, d, r)
    S = (torch.randn(d, r, generator=g) * 1e-2).to(dev)
    v = (1e-10 + torch.rand(d, generator=g) * 1e-6).to(dev)
    return S, v


def _both(m, compute, S, v, dev):
    outs = []
    for noalloc in (False, True):
        v_new = torch.full((m.d,), float("nan"), device=dev)
        rowsq = torch.full((m.d,), float("nan"), device=dev)
        sq = torch.full((1,), float("nan"), device=dev)
        if noalloc:
            B.logra_update_sqnorm_noalloc(m, compute, S, v, 0.999, 1e-8, v_new, sq, rowsq)
        else:
            B.logra_update_sqnorm(m, compute, S, v, 0.999, 1e-8, v_new, sq, rowsq)
        torch.cuda.synchronize()
        outs.append((v_new.cpu(), rowsq.cpu(), sq.cpu()))
    return outs


@pytest.mark.parametrize("compute", [B.LOGRA_BF16, B.LOGRA_F32])
def test_noalloc_pass1_equals_workspace_pass1(compute):
    dev = device()
    # the first call fills most of the scratch (at the bf16 path's headline
    # shape), the later ones are smaller and must not see its leftovers
    shapes = [(18944, 3584, 256), (1000, 520, 64), (264, 72, 32)] if compute == B.LOGRA_BF16 else \
             [(40000, 512, 64), (256, 512, 32), (45, 130, 20)]
    for i, (d, k, r) in enumerate(shapes):
        say("noalloc pass 1", "bf16" if compute == B.LOGRA_BF16 else "f32", d, k, r)
        m = B.MatrixDesc(d, k, r, seed=3, step=i, matrix_id=d)
        S, v = _state(100 + i, d, r, dev)
        (va, ra, qa), (vb, rb, qb) = _both(m, compute, S, v, dev)
        assert torch.isfinite(qa).all() and torch.isfinite(va).all()
        assert torch.equal(va, vb) and torch.equal(ra, rb) and torch.equal(qa, qb)


def test_noalloc_pass1_refuses_above_its_limit():
    dev = device()
    d = 6291456 + 16
    m = B.MatrixDesc(d, 64, 256)
    S = torch.empty(16, 256, device=dev)     # never read: the call is refused first
    v = torch.empty(16, device=dev)
    with pytest.raises(B.LograError) as e:
        B.logra_update_sqnorm_noalloc(m, B.LOGRA_BF16, S, v, 0.999, 1e-8, torch.empty(16, device=dev),
                                      torch.empty(1, device=dev))
    assert e.value.status == 3
