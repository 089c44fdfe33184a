"""Benchmark of the LoGRA sketch-accumulate + RowAdam-apply path on one GPU.

One step (rank_gradient_sketching_sketch_amd.step.Step) = every microbatch of
the step folded into the sketch (logra_sketch_project + logra_sketch_fold),
pass 1 (logra_update_sqnorm, v -> v') for every matrix, one device-to-host
read of the sqnorms for the step controller (the library's host controller
runs on them and its decision is reported; the update uses the workload's
drawn scale), pass 2 (logra_rowadam_apply) for every matrix, and the swap of
v and v'. Inputs are synthetic and already resident in HBM when the timed
region starts: the one-matrix workloads draw fresh X and dY for every step
and microbatch (all of them generated before timing), the layer stacks
rotate two sets per shape.

Prints one JSON line. value = sketch-accumulate TFLOP/s (algorithmic
2*T*r*(d+k) per microbatch call, over the HIP-event time of each step's
sketch phase, one event pair per phase; every timing event here is created
without the system-scope fence, which would add its cost to what it times);
the same line carries the RowAdam-apply GB/s (passes 1 and 2, the
device-to-host read excluded), the roofline of the dominant kernel (the
stage-2 fold, one accumulating launch per timed step: a pair around its
projection and it, less a pair around the projection before it alone, on
the stream they run on), its HBM
traffic from the committed profiler counters (when they were taken on the
current fold sources), and the CPU oracle timed on a bounded sample of the
same workload. Exits with status 3 if any fold workgroup gave up waiting for
its partner (its rows would be NaN).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "sketch-accum TFLOP/s + RowAdam-apply GB/s at 7B shapes, r=256; % of roofline"
# Sources that define the fold kernel: its HBM counters are reported only
# while these are unchanged since the counters were taken.
FOLD_SOURCES = ("rank_gradient_sketching_sketch_amd/csrc/fold_bf16.hip",
                "rank_gradient_sketching_sketch_amd/csrc/fold_body.hpp",
                "rank_gradient_sketching_sketch_amd/csrc/common.hpp",
                "rank_gradient_sketching_sketch_amd/build_lib.py")
# Predicted-KL controller run on every step's sqnorms and reported: an
# isotropic Fisher of scale 1 and a budget annealed from 1e-3 to 1e-4 nats
# over 1000 steps (the pages give no values). The update itself uses the
# workload's drawn scale.
KL_PHI = 1.0
# Device memory the one-matrix workloads may spend on fresh per-step inputs
# (beyond that, step input sets are reused in rotation).
INPUT_BUDGET_BYTES = 120 << 30


def sketch_flop_per_step(wl):
    """Algorithmic FLOPs of one step's sketch: both products, 2 T r (d + k)
    per matrix and microbatch (work the method avoids is not counted)."""
    return sum(2.0 * wl.tokens * wl.r * (s.d + s.k) for s in wl.matrices) * wl.microbatches


def fold_bytes_per_launch(T, d, r, accumulate):
    """Algorithmic bytes of one fold: dY and P read, S written, and S also
    read when the fold accumulates."""
    return 2 * T * d + 2 * T * r + 4 * d * r * (2 if accumulate else 1)


def fold_bytes_per_step(wl):
    """Algorithmic bytes of one step's folds (every microbatch but the first
    accumulates)."""
    return sum(fold_bytes_per_launch(wl.tokens, s.d, wl.r, mb > 0)
               for s in wl.matrices for mb in range(wl.microbatches))


def apply_bytes_per_matrix(d, k, r, wbytes):
    """Algorithmic bytes of one matrix's apply: W read and written at its
    dtype, S read once, v read, v' written (pass 1) and read (pass 2)."""
    return 2.0 * d * k * wbytes + 4.0 * d * r + 12.0 * d


def apply_bytes_per_step(wl):
    import torch
    wbytes = 2 if wl.w_dtype == torch.bfloat16 else 4
    return sum(apply_bytes_per_matrix(s.d, s.k, wl.r, wbytes) for s in wl.matrices)


def fold_sources_sha256():
    h = hashlib.sha256()
    for rel in FOLD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def fold_traffic_record(workload, call="logra_sketch_fold_parts"):
    """The fold's HBM bytes per dispatch from the committed counter summary
    (profiles/hbm_traffic_<workload>.md, JSON lines after 'traffic-record:',
    one per fold call), for the call the bench timed; None when there is
    none or it was taken on other fold sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % workload)
    try:
        text = open(path).read()
    except OSError:
        return None
    for m in re.finditer(r"traffic-record:\s*(\{.*\})", text):
        rec = json.loads(m.group(1))
        if rec.get("call", "logra_sketch_fold") != call:
            continue
        if rec.get("fold_sources_sha256") != fold_sources_sha256():
            return None
        return rec
    return None


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
    ap.add_argument("--parts", default="pair", choices=("pair", "all", "none"),
                    help="which matrices keep their sketch in parts during the step (logra_sketch_fold_parts)")
    ap.add_argument("--input-sets", type=int, default=0,
                    help="one-matrix workloads: distinct per-step input sets rotated over the steps "
                         "(0: as many as the input budget holds, up to one per step)")
    ap.add_argument("--no-batch", action="store_true",
                    help="pass 1 one matrix per call instead of batches of up to 16 per stream")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward dX product (alone and with the fold beside it)")
    ap.add_argument("--no-two-sided", action="store_true",
                    help="skip the two-sided sketch variant (rank 32) at the largest matrix's shape")
    ap.add_argument("--yardstick", action="store_true",
                    help="also time torch.mm (the vendor GEMM) on the fold's contraction and on the "
                         "dense dY^T X it replaces, for context")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (reference for HBM counters)")
    ap.add_argument("--fold-sha", action="store_true",
                    help="only print the hash of the fold sources (for the counter record)")
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
    if args.fold_sha:
        print(fold_sources_sha256())
        return
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    from rank_gradient_sketching_sketch_amd import binding as B
    from rank_gradient_sketching_sketch_amd import hip_timing, inputs
    from rank_gradient_sketching_sketch_amd.step import Matrix, Step

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
    n_steps = args.warmup + args.steps

    # ---- resident state and inputs -------------------------------------
    mats = [Matrix(s.d, s.k, s.matrix_id, W=inputs.weights(wl, s, device=dev),
                   v=inputs.second_moment(wl, s, device=dev), name="%s.%d" % (s.name, s.layer))
            for s in wl.matrices]
    step_runner = Step(mats, r, T, code, device=dev, sketch_lanes=args.streams,
                       apply_lanes=args.apply_streams, batch_pass1=not args.no_batch, parts=args.parts)

    # Microbatch buffers. One-matrix workloads: fresh X and dY for every
    # step and microbatch (as many step sets as the input budget holds,
    # reused in rotation beyond that). Layer stacks: two sets of per-layer
    # inputs (even and odd layers) for every microbatch, which keeps a 28-
    # or 64-layer step within memory while consecutive layers still read
    # different buffers. Projections that read the same activation share X.
    per_step_bytes = sum((T * s.k + T * s.d) * (2 if code == B.LOGRA_BF16 else 4)
                         for s in wl.matrices) * nmb
    fresh = len(wl.matrices) == 1
    step_sets = max(1, min(n_steps, INPUT_BUDGET_BYTES // max(1, per_step_bytes))) if fresh else 1
    if fresh and args.input_sets > 0:
        step_sets = min(step_sets, args.input_sets)

    def xkey(spec, step, mb):
        st = step % step_sets if fresh else 0
        return (st, spec.layer % 2, inputs.INPUT_GROUP.get(spec.name, spec.name), spec.k, mb)

    def ykey(spec, step, mb):
        st = step % step_sets if fresh else 0
        return (st, spec.layer % 2, spec.name, spec.d, mb)

    xbuf, ybuf = {}, {}
    for st in range(step_sets):
        for spec in wl.matrices:
            for mb in range(nmb):
                if xkey(spec, st, mb) not in xbuf:
                    xbuf[xkey(spec, st, mb)] = inputs.activations(wl, spec, st, mb, device=dev)
                if ykey(spec, st, mb) not in ybuf:
                    ybuf[ykey(spec, st, mb)] = inputs.output_grads(wl, spec, st, mb, device=dev)
    torch.cuda.synchronize()
    main_stream = torch.cuda.current_stream()

    sketch_flop = sketch_flop_per_step(wl)
    apply_bytes = apply_bytes_per_step(wl)

    # The roofline's kernel: one accumulating fold per timed step (the
    # largest matrix's, at the middle microbatch), timed on the stream it
    # runs on as the difference of two event pairs, one around that
    # microbatch's projection and fold, one around the projection before it
    # alone; the phases are bracketed on the main stream. Event records
    # cost GPU time, so nothing else is bracketed.
    big = max(range(len(mats)), key=lambda i: mats[i].d * mats[i].k)
    if nmb < 2:
        raise SystemExit("bench.py: the fold's timing needs at least two microbatches per step")
    probe_mb = nmb // 2
    fold_events, proj_events = [], []
    ev_log = []   # (kind, start_event, end_event)

    def ev(stream):
        return hip_timing.record(stream)

    def sketch_phase(step, timed):
        def get(i, mb):
            spec = wl.matrices[i]
            return xbuf[xkey(spec, step, mb)], ybuf[ykey(spec, step, mb)]
        marks = step_runner.sketch(step, nmb, get, probe=(big, probe_mb) if timed else None)
        if marks is not None:
            proj_events.append(marks[0])
            fold_events.append(marks[1])

    skipped = [0]
    ctl_log = []

    def one_step(step, timed):
        e0 = ev(main_stream) if timed else None
        sketch_phase(step, timed)
        e1 = ev(main_stream) if timed else None
        step_runner.pass1(wl.beta2, wl.eps)
        e2 = ev(main_stream) if timed else None
        # one device->host read of every sqnorm; the library's host controller
        # predicts the step's KL from them (reported, and timed on the host);
        # the update uses the workload's drawn scale, skipping non-finite ones
        sqs = step_runner.sqnorms()
        c0 = time.perf_counter()
        gamma, kl_pred, _ = B.logra_kl_step_scale(sqs, wl.lr, KL_PHI, B.logra_kl_budget_at(kl_budget, step))
        ctl_log.append((time.perf_counter() - c0, kl_pred, float(gamma.max()) if len(gamma) else 1.0))
        scales = Step.finite_scales(sqs, [inputs.step_scale(wl, s, step) for s in wl.matrices])
        skipped[0] += sum(1 for s in scales if s is None)
        e3 = ev(main_stream) if timed else None
        step_runner.pass2(wl.lr, scales, wl.eps)
        if timed:
            e4 = ev(main_stream)
            ev_log.append(("sketch", e0, e1))
            ev_log.append(("sqnorm", e1, e2))
            ev_log.append(("apply", e3, e4))

    for s in range(args.warmup):
        one_step(s, False)
    torch.cuda.synchronize()
    # Pass 2 is timed from an event the host records just before launching
    # it (after reading the sqnorms), so a host pause there would count as
    # GPU time: no garbage collection inside the timed steps.
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for s in range(args.steps):
            one_step(args.warmup + s, True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    timeouts = step_runner.fold_timeouts()

    tot = {"sketch": 0.0, "sqnorm": 0.0, "apply": 0.0}
    per_step = {"sketch": [], "sqnorm": [], "apply": []}
    for kind, a, b in ev_log:
        t = a.elapsed_time(b)
        tot[kind] += t
        per_step[kind].append(t)
    K = args.steps
    sketch_ms = tot["sketch"] / K
    apply_ms = (tot["sqnorm"] + tot["apply"]) / K
    sketch_tflops = sketch_flop / (sketch_ms * 1e-3) / 1e12
    apply_gbps = apply_bytes / (apply_ms * 1e-3) / 1e9
    # the fold: the projection + fold pair less the projection-alone pair
    # (each holds one event record's delay, which the difference cancels)
    both_ms = sum(a.elapsed_time(b) for a, b in fold_events) / len(fold_events)
    proj_ms = sum(a.elapsed_time(b) for a, b in proj_events) / len(proj_events)
    fold_ms = both_ms - proj_ms
    spec_big = wl.matrices[big]
    fold_bytes = fold_bytes_per_launch(T, spec_big.d, r, probe_mb > 0)
    fold_gbps = fold_bytes / (fold_ms * 1e-3) / 1e9
    probed_call = "logra_sketch_fold_parts" if mats[big].parts is not None else "logra_sketch_fold"
    rec = fold_traffic_record(wl.name, probed_call)
    traffic = None if rec is None else int(round(rec["fold_bytes_per_dispatch"]))
    dev_free, dev_total = torch.cuda.mem_get_info(dev)

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
        "data": "synthetic (seeded Gaussian inputs of the workload's shapes, generated on the GPU; "
                "no datasets or weights)",
        "config": {"workload": wl.name, "description": wl.description, "r": r,
                   "microbatches": nmb, "tokens": T, "matrices": len(mats),
                   "shapes": sorted({(s.d, s.k) for s in wl.matrices}),
                   "input_sets": ("fresh per step (%d distinct step sets)" % step_sets) if fresh
                   else "two rotating sets (even / odd layers)"},
        "sketch": {"tflops": round(sketch_tflops, 2),
                   "frac_mfma_peak": round(sketch_tflops / PEAK_BF16_TFLOPS, 4),
                   "ms_per_step": round(sketch_ms, 4),
                   "project_ms_per_launch": round(proj_ms, 5),
                   "fold_ms_per_launch": round(fold_ms, 5),
                   "ms_per_step_range": [round(min(per_step["sketch"]), 4), round(max(per_step["sketch"]), 4)]},
        "apply": {"GBps": round(apply_gbps, 1), "frac_hbm_peak": round(apply_gbps / PEAK_HBM_GBPS, 4),
                  "ms_per_step": round(apply_ms, 4),
                  "sqnorm_ms": round(tot["sqnorm"] / K, 5), "rowadam_ms": round(tot["apply"] / K, 5),
                  "rowadam_ms_range": [round(min(per_step["apply"]), 5), round(max(per_step["apply"]), 5)],
                  "skipped_nonfinite": skipped[0]},
        "roofline": {"kernel": ("fold_bf16_kernel (logra_sketch_fold_parts, a middle microbatch)"
                                if mats[big].parts is not None else "fold_bf16_kernel (logra_sketch_fold)"),
                     "bound": "hbm",
                     "achieved": round(fold_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(fold_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": fold_bytes,
                     "launch_us": round(fold_ms * 1e3, 2),
                     "timing": "fence-free HIP events on the fold's stream in every timed step: a pair around "
                               "the projection and accumulating fold of matrix %s, microbatch %d (%.2f us), less "
                               "a pair around the projection of microbatch %d alone (%.2f us); %d steps"
                               % (mats[big].name, probe_mb, both_ms * 1e3, probe_mb - 1, proj_ms * 1e3,
                                  len(fold_events)),
                     "traffic_source": None if rec is None else rec.get("source")},
        "fold_timeouts": timeouts,
        "state_bytes": {"sketch_plus_v": sum(4 * s.d * r + 4 * s.d for s in wl.matrices),
                        "dense_grad_fp32": sum(4 * s.d * s.k for s in wl.matrices)},
        "memory": {"peak_allocated": torch.cuda.max_memory_allocated(dev),
                   "device_in_use": dev_total - dev_free,
                   "weights": sum(m.W.numel() * m.W.element_size() for m in mats),
                   "microbatch_inputs": sum(t.numel() * t.element_size()
                                            for t in list(xbuf.values()) + list(ybuf.values())),
                   "workspaces": step_runner.workspace_bytes,
                   "sketch_parts": step_runner.parts_bytes},
        "streams": {"sketch": step_runner.n_sketch, "apply": step_runner.n_apply,
                    "pass1_batches": sum(1 for b in step_runner.batches if b[2] is not None)},
        "controller": {"fisher_scale": KL_PHI,
                       "budget": [kl_budget.delta_start, kl_budget.delta_end, kl_budget.anneal_steps],
                       "kl_pred_last_step": ctl_log[-1][1], "gamma_last_step": ctl_log[-1][2],
                       "host_us_per_step": round(1e6 * sum(c[0] for c in ctl_log) / len(ctl_log), 2),
                       "applied": False},
    }

    if code == B.LOGRA_BF16 and not args.no_backward:
        spec = wl.matrices[big]
        result["backward_dx"] = backward_dx(wl, spec, mats[big].W, xbuf[xkey(spec, 0, 0)],
                                            [ybuf[ykey(spec, 0, mb)] for mb in range(min(nmb, 3))], fold_ms)
    if code == B.LOGRA_BF16 and not args.no_two_sided:
        spec = wl.matrices[big]
        result["two_sided"] = two_sided(wl, spec, mats[big].W,
                                        [xbuf[xkey(spec, 0, mb)] for mb in range(min(nmb, 3))],
                                        [ybuf[ykey(spec, 0, mb)] for mb in range(min(nmb, 3))])
    if args.yardstick:
        result["yardstick"] = yardstick(wl, fold_ms if len(mats) == 1 else None)
    if not args.no_cpu_baseline:
        del xbuf, ybuf
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)
    if timeouts:
        print("fold time-outs: %d workgroups gave up waiting for their partner" % timeouts, file=sys.stderr)
        sys.exit(3)


def backward_dx(wl, spec, W, X, dYs, fold_ms, reps=15):
    """The backward input gradient dX = dY W of the largest matrix at the
    workload's token count: the library's product alone
    (logra_backward_dx) and the product with the sketch's fold beside it
    (logra_backward_dx_sketch), timed in alternation, one event pair per call
    (the projection made beforehand, as in the sketch step), medians; and
    torch.mm on the same operands for context."""
    import statistics
    import torch
    from rank_gradient_sketching_sketch_amd import binding as B
    from rank_gradient_sketching_sketch_amd import hip_timing
    T, d, k, r = wl.tokens, spec.d, spec.k, wl.r
    dev = W.device
    m = B.MatrixDesc(d, k, r, seed=0, step=0, matrix_id=spec.matrix_id)
    ws = torch.empty(B.logra_sketch_workspace_bytes(m, T, B.LOGRA_BF16), dtype=torch.uint8, device=dev)
    S = torch.zeros(d, r, dtype=torch.float32, device=dev)
    dX = torch.empty(T, k, dtype=torch.bfloat16, device=dev)
    B.logra_sketch_project(m, X, ws)
    auto = B.LaunchOpts()

    def timed(fn, i):
        a, b = hip_timing.FenceFreeEvent(), hip_timing.FenceFreeEvent()
        a.record()
        fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3

    runs = {"product": lambda i: B.logra_backward_dx(m, dYs[i % len(dYs)], W, dX),
            "fused": lambda i: B.logra_backward_dx_sketch(m, dYs[i % len(dYs)], W, dX, S, True, ws, opts=auto),
            "torch_mm": lambda i: torch.mm(dYs[i % len(dYs)], W)}
    for name, fn in runs.items():
        for i in range(3):
            fn(i)
    torch.cuda.synchronize()
    t = {name: [] for name in runs}
    for i in range(reps):
        for name, fn in runs.items():
            t[name].append(timed(fn, i))
    med = {name: statistics.median(v) for name, v in t.items()}
    flop = 2.0 * T * d * k
    out = {"shape_Tdk": [T, d, k], "r": r,
           "product_us": round(med["product"], 2),
           "product_tflops": round(flop / med["product"] / 1e6, 1),
           "product_frac_bf16_peak": round(flop / med["product"] / 1e6 / PEAK_BF16_TFLOPS, 4),
           "fused_us": round(med["fused"], 2),
           "sketch_incremental_us": round(med["fused"] - med["product"], 2),
           "fold_in_step_us": round(fold_ms * 1e3, 2),
           "placement": "in the product's launch" if _fuses(m, T) else "after the product",
           "torch_mm_us": round(med["torch_mm"], 2),
           "torch_mm_tflops": round(flop / med["torch_mm"] / 1e6, 1),
           "timing": "medians of %d alternating calls, one event pair each" % reps}
    del ws, S, dX
    torch.cuda.empty_cache()
    return out


def two_sided(wl, spec, W, Xs, dYs, reps=20):
    """The two-sided sketch variant (rank 32, fixed Gaussian projections) at
    the largest matrix's shape and the workload's token count: `reps`
    back-to-back sketch calls (alternating microbatches) between one event
    pair, then `reps` update calls (moments, coupling, sqnorm), then `reps`
    apply calls (on a copy of W), per-call averages; the projections'
    one-time construction; and the step at the workload's microbatch count.
    Byte rates count what the design moves: the sketch reads X and dY twice
    (once to project them, once in the two folds), the apply reads and
    writes W once."""
    import torch
    from rank_gradient_sketching_sketch_amd import binding as B
    from rank_gradient_sketching_sketch_amd import hip_timing
    R = 32
    T, d, k = wl.tokens, spec.d, spec.k
    dev = W.device
    m = B.MatrixDesc(d, k, R, seed=0, step=0, matrix_id=spec.matrix_id)
    pP = torch.empty(B.logra_ts_projection_bytes(m, 0), dtype=torch.uint8, device=dev)
    pQ = torch.empty(B.logra_ts_projection_bytes(m, 1), dtype=torch.uint8, device=dev)
    ws = torch.empty(B.logra_ts_sketch_workspace_bytes(m, T), dtype=torch.uint8, device=dev)
    uws = torch.empty(B.logra_ts_update_workspace_bytes(m), dtype=torch.uint8, device=dev)
    S_L = torch.zeros(k, R, device=dev)
    S_R = torch.zeros(d, R, device=dev)
    mom = [torch.zeros(n, R, device=dev) for n in (k, k, d, d)]
    sq = torch.zeros(1, device=dev)
    Wc = W.clone()

    def bracket(fn, n):
        a, b = hip_timing.FenceFreeEvent(), hip_timing.FenceFreeEvent()
        torch.cuda.synchronize()
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    proj_us = bracket(lambda i: (B.logra_ts_make_projection(m, 0, pP), B.logra_ts_make_projection(m, 1, pQ)), 1)
    runs = {"sketch": lambda i: B.logra_ts_sketch_accumulate(m, Xs[i % len(Xs)], dYs[i % len(dYs)], pP, pQ,
                                                             S_L, S_R, i > 0, ws),
            "update": lambda i: B.logra_ts_update(m, S_L, S_R, pP, *mom, 0.9, 0.999, 1e-8, sq, uws),
            "apply": lambda i: B.logra_ts_apply(m, uws, Wc, wl.lr, 1.0)}
    for fn in runs.values():
        bracket(fn, 3)
    us = {name: bracket(fn, reps) for name, fn in runs.items()}
    act = T * (d + k) * Xs[0].element_size()
    wbytes = 2 * d * k * W.element_size()
    nmb = wl.microbatches
    out = {"shape_Tdk": [T, d, k], "r": R,
           "projections_once_us": round(proj_us, 1),
           "sketch_us_per_microbatch": round(us["sketch"], 2),
           "sketch_GBps_two_reads": round(2 * act / us["sketch"] / 1e3, 1),
           "update_us": round(us["update"], 2),
           "apply_us": round(us["apply"], 2),
           "apply_GBps": round(wbytes / us["apply"] / 1e3, 1),
           "step_us": round(nmb * us["sketch"] + us["update"] + us["apply"], 1),
           "microbatches": nmb,
           "state_bytes": 3 * 4 * R * (d + k),
           "timing": "one event pair around %d back-to-back calls of each kind" % reps}
    del ws, uws, S_L, S_R, mom, Wc, pP, pQ
    torch.cuda.empty_cache()
    return out


def _fuses(m, T):
    """Whether logra_backward_dx_sketch runs the fold in the product's launch
    for this shape (the planner's rule, mirrored for the report: the fold
    workgroups' share of all-token tiles against three quarters of the
    product at 700 TFLOP/s, 60 GB/s per fold workgroup)."""
    G = -(-T // 256) * -(-m.k // 256)
    tiles = -(-(-(-m.d // 16)) // 10)
    spare = 0 if G % 256 == 0 else 256 - G % 256
    n_fold = min(max(spare, 32), tiles)
    per_wg = -(-tiles // n_fold) * 2.0 * T * (160 + m.r) / 60e9
    return per_wg <= 0.75 * (2.0 * T * m.d * m.k / 700e12)


def yardstick(wl, fold_ms):
    """Context only, not the product path: the vendor GEMM behind torch.mm on
    the largest matrix's shapes, (a) the fold's contraction dY^T P (d x T x r)
    and (b) the dense gradient dY^T X (d x T x k) that the sketch never forms.
    Operands are contiguous bf16 (dY^T materialised once), rotated over three
    sets so that no launch finds its inputs in the last-level cache."""
    import torch
    from rank_gradient_sketching_sketch_amd import hip_timing
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
            a, b = hip_timing.FenceFreeEvent(), hip_timing.FenceFreeEvent()
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
    """The oracle as it stands, timed on the host (input generation and
    conversion excluded): (a) the step's sketch-accumulate units (P = X A^T,
    then S += dY^T P over all rows, fp64) in the order the GPU step takes
    them, until about budget_s seconds have been spent; (b) one whole apply
    (rowsq, v', the sqnorm term and W') over every row of the largest
    matrix, from the sketch (a) left; (c) one sketch unit on one thread."""
    import numpy as np
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
    # (b) the apply of the largest matrix, every row
    spec = max(wl.matrices, key=lambda s: s.d * s.k)
    A = oracle.sign_matrix(0, 0, spec.matrix_id, wl.r, spec.k)
    S_big = S.get(spec.matrix_id)
    if S_big is None:
        S_big = np.zeros((spec.d, wl.r))
    v = inputs.second_moment(wl, spec).double().numpy()
    W = inputs.weights(wl, spec).double().numpy()
    t0 = time.perf_counter()
    oracle.rowadam_rows(S_big, A, v, W, beta2=wl.beta2, eps=wl.eps, lr=wl.lr,
                        scale=inputs.step_scale(wl, spec, 0))
    t_apply = time.perf_counter() - t0
    wbytes = 2 if wl.w_dtype.itemsize == 2 else 4
    out["apply"] = {"value": round(apply_bytes_per_matrix(spec.d, spec.k, wl.r, wbytes) / t_apply / 1e9, 4),
                    "unit": "GB/s", "seconds": round(t_apply, 2), "cores": oracle.num_threads(),
                    "sample": "one apply (passes 1 and 2, literal S A) of %d x %d, all %d rows, fp64; GB/s by "
                              "the GPU apply's algorithmic bytes" % (spec.d, spec.k, spec.d)}
    # (c) the same oracle on one thread, for one unit (the first microbatch of
    # the largest matrix)
    X = inputs.activations(wl, spec, 0, 0).double().numpy()
    dY = inputs.output_grads(wl, spec, 0, 0).double().numpy()
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
