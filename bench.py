"""Benchmark of the LoGRA sketch-accumulate + RowAdam-apply path on one GPU.

One step = every microbatch of the step folded into the sketch
(logra_sketch_project + logra_sketch_fold, i.e. logra_sketch_accumulate),
pass 1 (logra_update_sqnorm, v -> v') for every matrix, one device-to-host
read of the sqnorms for the step controller (the library's host controller
runs on them and its decision is reported; the update uses the workload's
drawn scale), pass 2 (logra_rowadam_apply) for every matrix, and the swap of
v and v'. Inputs are synthetic and already resident in HBM; each microbatch of
a step has its own buffers, so the inputs of one step (about 3 GB in the
default workload) stream through the 256 MB last-level cache.

Prints one JSON line. value = sketch-accumulate TFLOP/s (algorithmic
2*T*r*(d+k) per microbatch call, over the HIP-event time of each step's
sketch phase, one event pair per phase); the same line carries the
RowAdam-apply GB/s (passes 1 and 2, the device-to-host read excluded), the
roofline of the dominant kernel (the stage-2 fold, its average launch
duration from a back-to-back run of the step's fold calls after the timed
steps) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "sketch-accum TFLOP/s + RowAdam-apply GB/s at 7B shapes, r=256; % of roofline"
# HBM bytes per fold launch measured with rocprofv3 counters (FETCH_SIZE x 2
# + WRITE_SIZE x 1, the factors a plain device copy gives), per workload; see
# profiles/hbm_traffic_qwen7b_up.md. Only valid for the fold kernel as it was
# when the counters were taken.
FOLD_TRAFFIC_BYTES = {"qwen7b_up": (102539 * 2 + 37940) * 1024}
# Predicted-KL controller run on every step's sqnorms and reported: an
# isotropic Fisher of scale 1 and a budget annealed from 1e-3 to 1e-4 nats
# over 1000 steps (the pages give no values). The update itself uses the
# workload's drawn scale.
KL_PHI = 1.0


def sketch_flop_per_step(wl):
    """Algorithmic FLOPs of one step's sketch: both products, 2 T r (d + k)
    per matrix and microbatch (work the method avoids is not counted)."""
    return sum(2.0 * wl.tokens * wl.r * (s.d + s.k) for s in wl.matrices) * wl.microbatches


def fold_bytes_per_step(wl):
    """Algorithmic bytes of one step's folds: dY and P read, S written, and S
    also read when the fold accumulates (every microbatch but the first)."""
    T, r = wl.tokens, wl.r
    total = 0.0
    for s in wl.matrices:
        for mb in range(wl.microbatches):
            total += 2.0 * T * s.d + 2.0 * T * r + 4.0 * s.d * r * (2 if mb > 0 else 1)
    return total


def apply_bytes_per_step(wl):
    """Algorithmic bytes of one step's apply: W read and written at its
    dtype, S read once, v read, v' written (pass 1) and read (pass 2)."""
    import torch
    wbytes = 2 if wl.w_dtype == torch.bfloat16 else 4
    return sum(2.0 * s.d * s.k * wbytes + 4.0 * s.d * wl.r + 12.0 * s.d for s in wl.matrices)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen7b_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=0,
                    help="streams the matrices' sketch calls are spread over (0: at most 4)")
    ap.add_argument("--apply-streams", type=int, default=0,
                    help="streams the matrices' apply passes are spread over (0: 1 for one matrix, else 3)")
    ap.add_argument("--no-batch", action="store_true",
                    help="pass 1 one matrix per call instead of batches of up to 16 per stream")
    ap.add_argument("--prepare", action="store_true",
                    help="one-matrix workloads: build pass 1's Gram matrix ahead, on a side stream "
                         "during the sketch (logra_sqnorm_prepare), instead of inside pass 1")
    ap.add_argument("--yardstick", action="store_true",
                    help="also time torch.mm (the vendor GEMM) on the fold's contraction and on the "
                         "dense dY^T X it replaces, for context")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (reference for HBM counters)")
    return ap.parse_args()


def calibrate_copy():
    """A plain device-to-device copy of known size: the HBM byte counters of
    a profiler read on it give the factor that converts their readings on
    the library's kernels into bytes."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "launches": 3}), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    from rank_gradient_sketching_sketch_amd import binding as B
    from rank_gradient_sketching_sketch_amd import inputs

    if not os.path.exists(B.LIB_PATH):
        from rank_gradient_sketching_sketch_amd import build_lib
        build_lib.build()
    B.load_library()
    kl_budget = B.KLBudget(1e-3, 1e-4, 1000)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = inputs.WORKLOADS[args.workload]
    code = B.LOGRA_BF16 if wl.act_dtype == torch.bfloat16 else B.LOGRA_F32
    T, r, nmb = wl.tokens, wl.r, wl.microbatches

    # ---- resident state and inputs -------------------------------------
    mats = []
    for spec in wl.matrices:
        mats.append({
            "spec": spec,
            "S": torch.empty(spec.d, r, dtype=torch.float32, device=dev),
            "v": inputs.second_moment(wl, spec, device=dev),
            "W": inputs.weights(wl, spec, device=dev),
            "v_new": torch.empty(spec.d, dtype=torch.float32, device=dev),
            "sq": torch.empty(1, dtype=torch.float32, device=dev),
        })
    ws_bytes = max(B.logra_sketch_workspace_bytes(B.MatrixDesc(s.d, s.k, r), T, code)
                   for s in wl.matrices)
    sq_ws_bytes = max(B.logra_sqnorm_workspace_bytes(B.MatrixDesc(s.d, s.k, r), code)
                      for s in wl.matrices)
    # Independent matrices run on separate streams (matrix i on stream i mod
    # n), each stream with its own workspaces, so small projections (k, v)
    # overlap the large ones instead of leaving most of the GPU idle. Four
    # streams for the sketch phase (HIP gives a process four hardware queues
    # by default; more streams share them and slowed the apply phase that
    # follows), three for the apply phase, whose kernels fill the GPU longer.
    n_sketch = args.streams or min(4, len(mats))
    n_apply = args.apply_streams or (1 if len(mats) == 1 else 3)
    n_sketch = max(1, min(n_sketch, len(mats)))
    n_apply = max(1, min(n_apply, len(mats)))
    # the projections share the chip with the other sketch streams' work
    B.logra_set_sketch_concurrency(n_sketch)
    B.logra_set_apply_concurrency(n_apply)
    n_streams = max(n_sketch, n_apply)
    main = torch.cuda.current_stream()
    lanes = []
    for i in range(n_streams):
        lanes.append({
            "stream": main if i == 0 else torch.cuda.Stream(device=dev),
            "ws": torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev),
            "sq_ws": torch.empty(max(16, sq_ws_bytes), dtype=torch.uint8, device=dev),
        })
    for i, m in enumerate(mats):
        m["lane"] = lanes[i % n_sketch]
        m["alane"] = lanes[i % n_apply]
    # Pass 1 in batches: each apply stream's matrices in as few chunks of at
    # most B.MAX_BATCH as hold them, of equal size (65 matrices: 5 x 13, not
    # 4 x 16 + 1), one call (two launches) per chunk; a chunk of one matrix
    # uses the single-matrix call. Each batched matrix's sqnorm is a view of
    # its chunk's n-float output.
    batches = []
    batch_ws_bytes = 0
    if not args.no_batch:
        for ln in lanes[:n_apply]:
            own = [m for m in mats if m["alane"] is ln]
            n_chunks = -(-len(own) // B.MAX_BATCH)
            bounds = [len(own) * i // max(1, n_chunks) for i in range(n_chunks + 1)]
            for c0, c1 in zip(bounds[:-1], bounds[1:]):
                chunk = own[c0:c1]
                if len(chunk) == 1:
                    batches.append((ln, chunk, None, None))
                    continue
                sq = torch.empty(len(chunk), dtype=torch.float32, device=dev)
                for i, m in enumerate(chunk):
                    m["sq"] = sq[i:i + 1]
                wsb = B.logra_sqnorm_batch_workspace_bytes(
                    [B.MatrixDesc(m["spec"].d, m["spec"].k, r) for m in chunk], code)
                batch_ws_bytes += wsb
                batches.append((ln, chunk, sq, torch.empty(max(16, wsb), dtype=torch.uint8, device=dev)))
    # --prepare: a one-matrix workload builds pass 1's Gram matrix (it
    # depends only on the step's signs) ahead, on a side stream while the
    # sketch runs, into the workspace pass 1 then reads. Off by default: it
    # took about 4 us off pass 1 but cost the sketch about 3 %.
    prep_stream = None
    if len(mats) == 1 and code == B.LOGRA_BF16 and args.prepare and not args.no_batch:
        prep_stream = torch.cuda.Stream(device=dev)

    # Microbatch buffers: every microbatch has its own; layer stacks rotate
    # two sets of per-layer inputs (even and odd layers), which keeps a
    # 28- or 64-layer step within memory while consecutive layers still read
    # different buffers. Projections that read the same activation share X.
    def xkey(spec, mb):
        return (spec.layer % 2, inputs.INPUT_GROUP.get(spec.name, spec.name), spec.k, mb)

    def ykey(spec, mb):
        return (spec.layer % 2, spec.name, spec.d, mb)

    xbuf, ybuf = {}, {}
    for spec in wl.matrices:
        for mb in range(nmb):
            if xkey(spec, mb) not in xbuf:
                xbuf[xkey(spec, mb)] = inputs.activations(wl, spec, 0, mb, device=dev)
            if ykey(spec, mb) not in ybuf:
                ybuf[ykey(spec, mb)] = inputs.output_grads(wl, spec, 0, mb, device=dev)
    torch.cuda.synchronize()
    stream = main

    def fork():
        if n_streams > 1:
            e = torch.cuda.Event()
            e.record(main)
            for ln in lanes[1:]:
                ln["stream"].wait_event(e)

    def join():
        for ln in lanes[1:]:
            e = torch.cuda.Event()
            e.record(ln["stream"])
            main.wait_event(e)

    sketch_flop = sketch_flop_per_step(wl)
    fold_bytes = fold_bytes_per_step(wl)
    apply_bytes = apply_bytes_per_step(wl)

    # Event records cost a few microseconds of GPU time each, so the timed
    # steps record events only at phase boundaries (sketch | pass 1 | pass 2).
    ev_log = []   # (kind, start_event, end_event)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    skipped = [0]

    def sketch_calls(step, m, mb, what):
        spec = m["spec"]
        X = xbuf[xkey(spec, mb)]
        dY = ybuf[ykey(spec, mb)]
        ln = m["lane"]
        if what in ("project", "both"):
            B.logra_sketch_project(m["desc"], X, ln["ws"], ln["stream"])
        if what in ("fold", "both"):
            B.logra_sketch_fold(m["desc"], dY, m["S"], mb > 0, ln["ws"], ln["stream"])

    def one_step(step, timed):
        for m in mats:
            spec = m["spec"]
            m["desc"] = B.MatrixDesc(spec.d, spec.k, r, seed=0, step=step, matrix_id=spec.matrix_id)
        # microbatch-major, as a backward pass produces them: every matrix's
        # sketch takes each microbatch in turn
        e0 = ev() if timed else None
        fork()
        if prep_stream is not None:
            prep_stream.wait_stream(main)
            B.logra_sqnorm_prepare(mats[0]["desc"], code, mats[0]["alane"]["sq_ws"], prep_stream)
        for mb in range(nmb):
            for m in mats:
                sketch_calls(step, m, mb, "both")
        join()
        if prep_stream is not None:
            main.wait_stream(prep_stream)
        e1 = ev() if timed else None
        fork()
        if batches:
            for ln, chunk, sq, bws in batches:
                if sq is None:
                    m = chunk[0]
                    if prep_stream is not None:
                        B.logra_update_sqnorm_prepared(m["desc"], code, m["S"], m["v"], wl.beta2, wl.eps,
                                                       m["v_new"], m["sq"], ln["sq_ws"], None, ln["stream"])
                    else:
                        B.logra_update_sqnorm(m["desc"], code, m["S"], m["v"], wl.beta2, wl.eps, m["v_new"],
                                              m["sq"], None, ln["sq_ws"], ln["stream"])
                else:
                    B.logra_update_sqnorm_batch([m["desc"] for m in chunk], code, [m["S"] for m in chunk],
                                                [m["v"] for m in chunk], wl.beta2, wl.eps,
                                                [m["v_new"] for m in chunk], sq, None, bws, ln["stream"])
        else:
            for m in mats:
                ln = m["alane"]
                B.logra_update_sqnorm(m["desc"], code, m["S"], m["v"], wl.beta2, wl.eps, m["v_new"],
                                      m["sq"], None, ln["sq_ws"], ln["stream"])
        join()
        e2 = ev() if timed else None
        # one device->host read of every sqnorm; the library's host controller
        # predicts the step's KL from them (reported, and timed on the host);
        # the update uses the workload's drawn scale, skipping non-finite ones
        sqs = torch.cat([m["sq"] for m in mats]).cpu().tolist()
        c0 = time.perf_counter()
        gamma, kl_pred, _ = B.logra_kl_step_scale(sqs, wl.lr, KL_PHI, B.logra_kl_budget_at(kl_budget, step))
        ctl_log.append((time.perf_counter() - c0, kl_pred, float(gamma.max()) if len(gamma) else 1.0))
        # the workload's drawn scales (input generation, kept out of the
        # timed pass 2); a matrix with a non-finite sqnorm is skipped
        todo = []
        for m, sq in zip(mats, sqs):
            if not math.isfinite(sq):
                skipped[0] += 1
                continue
            todo.append((m, inputs.step_scale(wl, m["spec"], step)))
        e3 = ev() if timed else None
        fork()
        for m, scale in todo:
            B.logra_rowadam_apply(m["desc"], code, m["S"], m["v_new"], m["W"], wl.lr, scale, wl.eps,
                                  m["alane"]["stream"])
            # the update is applied: v' becomes the next step's v (buffer swap)
            m["v"], m["v_new"] = m["v_new"], m["v"]
        join()
        if timed:
            e4 = ev()
            ev_log.append(("sketch", e0, e1))
            ev_log.append(("sqnorm", e1, e2))
            ev_log.append(("apply", e3, e4))

    ctl_log = []
    for s in range(args.warmup):
        one_step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(args.warmup + s, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Per-kernel averages for the roofline: each half of the sketch launched
    # back to back over the same microbatch buffers, one event pair around
    # the run (the average includes the launch gap between kernels).
    def per_launch_ms(what):
        reps = max(1, 64 // (nmb * len(mats)))
        torch.cuda.synchronize()
        a = ev()
        fork()
        for _ in range(reps):
            for mb in range(nmb):
                for m in mats:
                    sketch_calls(0, m, mb, what)
        join()
        b = ev()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * nmb * len(mats))

    project_ms = per_launch_ms("project")
    fold_ms = per_launch_ms("fold")

    tot = {"sketch": 0.0, "sqnorm": 0.0, "apply": 0.0}
    for kind, a, b in ev_log:
        tot[kind] += a.elapsed_time(b)
    K = args.steps
    sketch_ms = tot["sketch"] / K
    apply_ms = (tot["sqnorm"] + tot["apply"]) / K
    sketch_tflops = sketch_flop / (sketch_ms * 1e-3) / 1e12
    apply_gbps = apply_bytes / (apply_ms * 1e-3) / 1e9
    fold_bytes_avg = fold_bytes / (nmb * len(mats))
    dev_free, dev_total = torch.cuda.mem_get_info(dev)
    fold_gbps = fold_bytes_avg / (fold_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(sketch_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if code == B.LOGRA_BF16 else "f32",
        "data": "synthetic (seeded Gaussian inputs of the workload's shapes; no datasets or weights)",
        "config": {"workload": wl.name, "description": wl.description, "r": r,
                   "microbatches": nmb, "tokens": T, "matrices": len(mats),
                   "shapes": sorted({(s.d, s.k) for s in wl.matrices})},
        "sketch": {"tflops": round(sketch_tflops, 2),
                   "frac_mfma_peak": round(sketch_tflops / PEAK_BF16_TFLOPS, 4),
                   "ms_per_step": round(sketch_ms, 4),
                   "project_ms_per_launch": round(project_ms, 5),
                   "fold_ms_per_launch": round(fold_ms, 5)},
        "apply": {"GBps": round(apply_gbps, 1), "frac_hbm_peak": round(apply_gbps / PEAK_HBM_GBPS, 4),
                  "ms_per_step": round(apply_ms, 4),
                  "sqnorm_ms": round(tot["sqnorm"] / K, 5), "rowadam_ms": round(tot["apply"] / K, 5),
                  "skipped_nonfinite": skipped[0]},
        "roofline": {"kernel": "fold_bf16_kernel (logra_sketch_fold)", "bound": "hbm",
                     "achieved": round(fold_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(fold_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": FOLD_TRAFFIC_BYTES.get(wl.name),
                     "algorithmic_bytes_per_launch": round(fold_bytes_avg)},
        "state_bytes": {"sketch_plus_v": sum(4 * s.d * r + 4 * s.d for s in wl.matrices),
                        "dense_grad_fp32": sum(4 * s.d * s.k for s in wl.matrices)},
        "memory": {"peak_allocated": torch.cuda.max_memory_allocated(dev),
                   "device_in_use": dev_total - dev_free,
                   "weights": sum(m["W"].numel() * m["W"].element_size() for m in mats),
                   "microbatch_inputs": sum(t.numel() * t.element_size()
                                            for t in list(xbuf.values()) + list(ybuf.values())),
                   "workspaces": n_streams * (max(16, ws_bytes) + max(16, sq_ws_bytes)) + batch_ws_bytes},
        "streams": {"sketch": n_sketch, "apply": n_apply, "sketch_concurrency": n_sketch, "apply_concurrency": n_apply,
                    "pass1_batches": sum(1 for b in batches if b[2] is not None),
                    "pass1_prepared": prep_stream is not None},
        "controller": {"fisher_scale": KL_PHI,
                       "budget": [kl_budget.delta_start, kl_budget.delta_end, kl_budget.anneal_steps],
                       "kl_pred_last_step": ctl_log[-1][1], "gamma_last_step": ctl_log[-1][2],
                       "host_us_per_step": round(1e6 * sum(c[0] for c in ctl_log) / len(ctl_log), 2),
                       "applied": False},
    }

    if args.yardstick:
        result["yardstick"] = yardstick(wl, fold_ms if len(mats) == 1 else None)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


def yardstick(wl, fold_ms):
    """Context only, not the product path: the vendor GEMM behind torch.mm on
    the largest matrix's shapes, (a) the fold's contraction dY^T P (d x T x r)
    and (b) the dense gradient dY^T X (d x T x k) that the sketch never forms.
    Operands are contiguous bf16 (dY^T materialised once), rotated over three
    sets so that no launch finds its inputs in the last-level cache."""
    import torch
    spec = max(wl.matrices, key=lambda s: s.d * s.k)
    d, k, T, r = spec.d, spec.k, wl.tokens, wl.r
    g = torch.Generator(device="cuda:0")
    g.manual_seed(1)
    sets = [((torch.randn(d, T, device="cuda:0", generator=g) * 1e-4).bfloat16(),
             torch.randn(T, r, device="cuda:0", generator=g).bfloat16(),
             torch.randn(T, k, device="cuda:0", generator=g).bfloat16()) for _ in range(3)]

    def timed(fn, reps=21):
        for i in range(3):
            fn(i % 3)
        torch.cuda.synchronize()
        times = []
        for i in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn(i % 3)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return sorted(times)[reps // 2]

    t_fold = timed(lambda i: torch.mm(sets[i][0], sets[i][1]))
    t_dense = timed(lambda i: torch.mm(sets[i][0], sets[i][2]))
    out = {"library": "torch.mm (bf16 in, bf16 out)", "shape_dTrk": [d, T, r, k],
           "fold_contraction": {"us": round(t_fold * 1e3, 2),
                                "tflops": round(2.0 * d * T * r / (t_fold * 1e-3) / 1e12, 1)},
           "dense_gradient": {"us": round(t_dense * 1e3, 2),
                              "tflops": round(2.0 * d * T * k / (t_dense * 1e-3) / 1e12, 1)}}
    if fold_ms is not None:
        out["logra_fold_us"] = round(fold_ms * 1e3, 2)
    del sets
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, budget_s=15.0):
    """The oracle as it stands, timed on the host: the step's sketch-accumulate
    units (P = X A^T, then S += dY^T P over all rows, fp64) in the order the
    GPU step takes them, until about budget_s seconds have been spent."""
    import oracle
    from rank_gradient_sketching_sketch_amd import inputs
    done, flop, spent = 0, 0.0, 0.0
    S = {}
    for mb in range(wl.microbatches):
        for spec in wl.matrices:
            if spent >= budget_s:
                break
            X = inputs.activations(wl, spec, 0, mb).double().numpy()
            dY = inputs.output_grads(wl, spec, 0, mb).double().numpy()
            A = oracle.sign_matrix(0, 0, spec.matrix_id, wl.r, spec.k)
            t0 = time.perf_counter()
            P = oracle.project(X, A)
            S[spec.matrix_id] = oracle.sketch_rows(dY, P, S_rows=S.get(spec.matrix_id), accumulate=mb > 0)
            spent += time.perf_counter() - t0
            flop += 2.0 * wl.tokens * wl.r * (spec.d + spec.k)
            done += 1
    total = wl.microbatches * len(wl.matrices)
    out = {"value": round(flop / spent / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle", "seconds": round(spent, 2), "cpu": cpu_model(),
           "sample": "%d of the step's %d sketch-accumulate units (microbatch x matrix, %d tokens each), "
                     "all rows, fp64" % (done, total, wl.tokens)}
    # the same oracle on one thread, for one unit (the first microbatch of the
    # largest matrix)
    spec = max(wl.matrices, key=lambda s: s.d * s.k)
    X = inputs.activations(wl, spec, 0, 0).double().numpy()
    dY = inputs.output_grads(wl, spec, 0, 0).double().numpy()
    A = oracle.sign_matrix(0, 0, spec.matrix_id, wl.r, spec.k)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.sketch_rows(dY, oracle.project(X, A), accumulate=False)
        one = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    out["single_thread"] = {"value": round(2.0 * wl.tokens * wl.r * (spec.d + spec.k) / one / 1e12, 6),
                            "unit": "TFLOP/s", "seconds": round(one, 2),
                            "sample": "one sketch-accumulate unit, %d x %d, %d tokens, all rows, fp64"
                                      % (spec.d, spec.k, wl.tokens)}
    return out


if __name__ == "__main__":
    main()
