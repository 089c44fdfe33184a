"""GPU parity of whole optimizer steps run through the package's step
scheduler (rank_gradient_sketching_sketch_amd.step.Step), in the schedule the
benchmark times: the matrices' sketch calls spread over four streams and
their apply passes over three, the lane counts declared to the kernels in the
launch options (64-token projection workgroups and the 128-workgroup pass 2
where they apply), pass 1 batched per apply stream, the v / v' swap, and the
fold's time-out counter. The folds keep the sketch in parts during the
step where the scheduler's policy says so (by default the matrices whose fold
tiles two workgroups share; one test per policy covers every split).

The oracle computes P = X A^T in full for every microbatch (as one fp64
matmul) and everything after it on a seeded sample of rows plus the first and
last; rows of S, Ghat and W are independent once P is known, so the sampled
comparison is exact in what it covers. Inputs come from the seeded generators
of the inputs module, drawn on the GPU (torch's generator) and copied to the
host for the oracle. Metrics and tolerances are those of the other workload
tests (2e-2 for bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from rank_gradient_sketching_sketch_amd import binding as B
from rank_gradient_sketching_sketch_amd import inputs
from rank_gradient_sketching_sketch_amd.step import Matrix, Step
from gpu_util import BF16_TOL, bf16_w_check, device, f32, rel_err, rownorm_err, say, to_f64, w_update_err

pytestmark = pytest.mark.gpu


def _rows(d, n, seed):
    if d <= n + 2:
        return np.arange(d)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, d - 1], rng.choice(d, n, replace=False)]))


def _run_and_check(wl, specs, steps, mbs, nrows=256, sketch_lanes=4, apply_lanes=3, parts="pair"):
    dev = device()
    code = B.LOGRA_BF16
    r, T = wl.r, wl.tokens
    mats, shadows, refs = [], [], []
    for s in specs:
        W_h = inputs.weights(wl, s)
        v_h = inputs.second_moment(wl, s)
        rows = _rows(s.d, nrows, s.matrix_id)
        mats.append(Matrix(s.d, s.k, s.matrix_id, W=W_h.to(dev), v=v_h.to(dev), name=s.name))
        shadows.append(W_h.float().to(dev))
        refs.append({"rows": rows, "W": W_h.double().numpy()[rows], "W32": W_h.double().numpy()[rows],
                     "v": v_h.double().numpy()[rows], "allow": None})
    st = Step(mats, r, T, code, device=dev, sketch_lanes=sketch_lanes, apply_lanes=apply_lanes,
              batch_pass1=True, rowsq=True, parts=parts)
    say("step schedule: %d matrices, %d sketch / %d apply streams, %d batched pass-1 calls, "
        "%d matrices with parts (%s)"
        % (len(mats), st.n_sketch, st.n_apply, sum(1 for b in st.batches if b[2] is not None),
           sum(1 for m in mats if m.parts is not None), parts))
    hp = dict(beta2=f32(wl.beta2), eps=f32(wl.eps), lr=f32(wl.lr))
    for step in range(steps):
        # every input of the step on the GPU before the step starts
        xs, ys = {}, {}
        for mb in range(mbs):
            for s in specs:
                xk = (inputs.INPUT_GROUP[s.name], s.k, mb)
                if xk not in xs:
                    xs[xk] = inputs.activations(wl, s, step, mb, device=dev)
                ys[(s.name, mb)] = inputs.output_grads(wl, s, step, mb, device=dev)
        torch.cuda.synchronize()

        def get(i, mb):
            s = specs[i]
            return xs[(inputs.INPUT_GROUP[s.name], s.k, mb)], ys[(s.name, mb)]

        st.clear_fold_timeouts()
        st.sketch(step, mbs, get)
        st.pass1(wl.beta2, wl.eps)
        sqs = st.sqnorms()
        scales = [inputs.step_scale(wl, s, step) for s in specs]
        v_old = [m.v.clone() for m in mats]
        assert st.pass2(wl.lr, scales, wl.eps) == len(mats)
        # fp32 shadow of every W through the same pass 2 (v' is now m.v)
        for m, W32, sc in zip(mats, shadows, scales):
            B.logra_rowadam_apply(m.desc, code, m.S, m.v, W32, wl.lr, sc, wl.eps)
        torch.cuda.synchronize()
        assert st.fold_timeouts() == 0

        for i, (s, m) in enumerate(zip(specs, mats)):
            ref = refs[i]
            rows = ref["rows"]
            A = oracle.sign_matrix(0, step, s.matrix_id, r, s.k)
            S_ref = None
            for mb in range(mbs):
                X, dY = get(i, mb)
                P = oracle.project_matmul(X.double().cpu().numpy(), A)
                dY_rows = dY[:, torch.from_numpy(rows).to(dev)].double().cpu().numpy()
                S_ref = oracle.sketch_rows(dY_rows, P, S_rows=S_ref, accumulate=mb > 0)
            e_s = rownorm_err(to_f64(m.S)[rows], S_ref)
            sc = f32(scales[i])
            out = oracle.rowadam_rows(S_ref, A, ref["v"], ref["W"], scale=sc, **hp)
            out32 = oracle.rowadam_rows(S_ref, A, ref["v"], ref["W32"], scale=sc, **hp)
            rowsq = to_f64(m.rowsq)
            e_rq = rel_err(rowsq[rows], out["rowsq"])
            e_v = rel_err(to_f64(m.v)[rows], out["v_new"])
            w_ok, w_worst, ref["allow"] = bf16_w_check(to_f64(m.W)[rows], out["W_new"], ref["W"],
                                                       prior=ref["allow"])
            e_w = w_update_err(to_f64(shadows[i])[rows], out32["W_new"], ref["W32"])
            if len(rows) == s.d:
                e_q = abs(sqs[i] / out["sqnorm"] - 1)       # every row sampled: the scalar itself
                kind = "oracle"
            else:
                # over all rows, from the GPU's own rowsq and v (a property of
                # the GPU outputs), the sampled rowsq being checked above
                vh = to_f64(v_old[i])
                vn = hp["beta2"] * vh + (1 - hp["beta2"]) * rowsq / s.k
                e_q = abs(sqs[i] / float((rowsq / (np.sqrt(vn) + hp["eps"]) ** 2).sum()) - 1)
                kind = "identity"
            say("  step %d %-5s %5d x %5d: S %.2e rowsq %.2e v' %.2e dW32 %.2e W-bf16 %.2f sqnorm(%s) %.2e"
                % (step, s.name, s.d, s.k, e_s, e_rq, e_v, e_w, w_worst, kind, e_q))
            assert e_s < BF16_TOL and e_rq < BF16_TOL and e_v < BF16_TOL and e_w < BF16_TOL
            assert w_ok and e_q < BF16_TOL
            ref["W"] = torch.from_numpy(out["W_new"]).to(torch.bfloat16).double().numpy()
            ref["W32"] = out32["W_new"]
            ref["v"] = out["v_new"]
        del xs, ys
        torch.cuda.empty_cache()


def test_step_qwen15b_set_in_full():
    # The 1.5B projection set as the benchmark runs it: 7 matrices x 8
    # microbatches of 2048 tokens, one step.
    wl = inputs.WORKLOADS["qwen1.5b_set"]
    say("step qwen1.5b_set: 7 matrices, 8 x 2048 tokens")
    _run_and_check(wl, wl.matrices, steps=1, mbs=wl.microbatches)


def test_step_qwen7b_one_layer_all_microbatches():
    # One layer of the 28-layer 7B stack (q, k, v, o 3584 / 512, gate, up
    # 18944 x 3584, down 3584 x 18944) with all 8 microbatches of 4096 tokens:
    # the folds' accumulate path at every shape of the stack.
    wl = inputs.WORKLOADS["qwen7b_28layer"]
    say("step qwen7b_28layer layer 0: 8 x 4096 tokens")
    _run_and_check(wl, wl.matrices[:7], steps=1, mbs=wl.microbatches)


def test_step_27b_one_layer_two_carried_steps():
    # One layer of the 64-layer 27B stack, two consecutive steps (A redrawn,
    # W and v carried over), each with all 8 microbatches of 8192 tokens.
    wl = inputs.WORKLOADS["27b_64layer"]
    say("step 27b_64layer layer 0: 2 steps x 8 x 8192 tokens")
    _run_and_check(wl, wl.matrices[:7], steps=2, mbs=wl.microbatches)


def test_step_two_layers_share_lanes_and_batches():
    # Two 7B layers (14 matrices): several matrices per sketch stream and
    # pass-1 batches of several matrices per apply stream, two microbatches,
    # every split fold keeping its sketch in parts.
    wl = inputs.WORKLOADS["qwen7b_28layer"]
    say("step qwen7b_28layer layers 0-1: 2 x 4096 tokens, parts for every split fold")
    _run_and_check(wl, wl.matrices[:14], steps=1, mbs=2, nrows=128, parts="all")


def test_step_qwen15b_set_all_parts_and_none():
    # The 1.5B set with parts for every split fold, and with none (every fold
    # adds into S, the members of a tile exchanging partials in the kernel)
    wl = inputs.WORKLOADS["qwen1.5b_set"]
    for policy in ("all", "none"):
        say("step qwen1.5b_set, parts: %s" % policy)
        _run_and_check(wl, wl.matrices, steps=1, mbs=wl.microbatches, parts=policy)


def test_fence_free_events_time_a_kernel():
    # The step's probe events (created without the system-scope fence) and
    # torch's ordinary events, nested around one spin kernel: the inner,
    # fence-free pair sees the kernel run and holds no more than the outer.
    from rank_gradient_sketching_sketch_amd import hip_timing
    device()
    torch.cuda.synchronize()
    outer = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    inner = (hip_timing.FenceFreeEvent(), hip_timing.FenceFreeEvent())
    outer[0].record()
    inner[0].record()
    torch.cuda._sleep(1_000_000)
    inner[1].record()
    outer[1].record()
    torch.cuda.synchronize()
    t_in, t_out = inner[0].elapsed_time(inner[1]), outer[0].elapsed_time(outer[1])
    say("fence-free pair %.1f us, torch pair %.1f us" % (1e3 * t_in, 1e3 * t_out))
    assert 0 < t_in <= t_out + 1e-3
