"""A whole step of the library's calls (sketch accumulate per microbatch,
pass 1, pass 2) captured in a HIP graph and replayed: every replay must equal
the eager run bit for bit. The kernels zero their own counters and flags
with kernels (no memset nodes), and the caller passes every workspace, so
nothing allocates during capture. Each replay is preceded by eager work and
a synchronisation, and W is reset outside the graph."""
import pytest
import torch

from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def test_step_replays_in_a_hip_graph_equal_eager():
    dev = device()
    d, k, r, T, mbs = 8200, 520, 256, 300, 2     # pair-mode fold, ragged tokens
    m = B.MatrixDesc(d, k, r, seed=3, step=9, matrix_id=4)
    say("graph step", d, k, r, T, mbs)
    Xs, dYs = [], []
    for n in range(mbs):
        X, dY = inputs.random_case(700 + n, T, d, k, dtype=torch.bfloat16, dy_std=1e-2)
        Xs.append(X.to(dev))
        dYs.append(dY.to(dev))
    g = inputs.generator("graph-state", d, k, r)
    v = (1e-10 + torch.rand(d, generator=g) * 1e-6).to(dev)
    W0 = (torch.randn(d, k, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    wq = torch.empty(B.logra_sqnorm_workspace_bytes(m, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    S = torch.empty(d, r, device=dev)
    v_new = torch.empty(d, device=dev)
    sq = torch.empty(1, device=dev)
    W = W0.clone()

    def step():
        for n in range(mbs):
            B.logra_sketch_accumulate(m, Xs[n], dYs[n], S, accumulate=n > 0, ws=ws)
        B.logra_update_sqnorm(m, B.LOGRA_BF16, S, v, 0.999, 1e-8, v_new, sq, ws=wq)
        B.logra_rowadam_apply(m, B.LOGRA_BF16, S, v_new, W, 1e-3, 0.7, 1e-8)

    step()
    torch.cuda.synchronize()
    ref = (S.clone(), v_new.clone(), sq.clone(), W.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        W.copy_(W0)
        step()          # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        W.copy_(W0)
        step()          # the program's own eager work between replays
        torch.cuda.synchronize()
        W.copy_(W0)
        S.zero_(), v_new.zero_(), sq.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((S, v_new, sq, W), ref):
            assert torch.equal(a, b), "replay %d differs from the eager step" % rep
