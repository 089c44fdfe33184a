"""One optimizer step of the LoGRA path over many matrices, scheduled over
several HIP streams.

The sketched set is every attention and MLP projection of a model ("NVIDIA's
LoGRA fits RL post-training of a 27B model onto a single eight-GPU node",
section "Why it matters"), so a step is many independent matrices, most of
them too small to fill the chip alone. This module only schedules the C-ABI
calls: it holds no arithmetic of the method, and every number is produced by
the library's kernels.

A step, in the order the host drives it:
  1. sketch: for every microbatch (in order, as a backward pass produces
     them) and every matrix, logra_sketch_project then the fold: for a
     matrix that keeps its sketch in parts during the step (the `parts`
     policy), logra_sketch_fold_parts with LOGRA_FOLD_FIRST on the first
     microbatch and LOGRA_FOLD_LAST on the last, so that the workgroups
     sharing a tile of S never wait for each other; otherwise
     logra_sketch_fold (accumulate = 0 for the first microbatch). Matrix i
     runs on sketch lane i mod n_sketch; each lane is a stream with its own
     workspace.
  2. pass 1: logra_update_sqnorm for every matrix (v -> v'), in batches of
     up to 16 matrices per apply lane (logra_update_sqnorm_batch: two
     launches per batch), matrix i on apply lane i mod n_apply.
  3. one device-to-host read of every sqnorm (the host step controller's
     input).
  4. pass 2: logra_rowadam_apply for every matrix given a scale; a matrix
     that is given none (or whose sqnorm is not finite, when the caller asks
     to skip those) keeps W and v. Each applied matrix then swaps v and v'.
Every lane forks from the caller's current stream at the start of a phase
and joins it at the end, so the caller can time phases with events on its
own stream. The calls carry launch options that declare the lane counts to
the kernels (the projection and pass 2 size their grids for a 1/n share of
the chip) and a device counter of fold time-outs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence, Tuple

import torch

from . import binding as B
from . import hip_timing

MAX_SKETCH_LANES = 4   # HIP gives a process four hardware queues by default
DEFAULT_APPLY_LANES = 3


@dataclasses.dataclass
class Matrix:
    """One sketched projection W (d x k). W and v are the caller's state
    (updated in place by the step: W by pass 2, v by the swap with v')."""
    d: int
    k: int
    matrix_id: int
    W: torch.Tensor
    v: torch.Tensor
    name: str = ""
    # allocated by Step
    S: Optional[torch.Tensor] = None
    v_new: Optional[torch.Tensor] = None
    sq: Optional[torch.Tensor] = None
    rowsq: Optional[torch.Tensor] = None
    desc: Optional[B.MatrixDesc] = None
    parts: Optional[torch.Tensor] = None
    lane: int = 0
    alane: int = 0


def _event(stream):
    # timing only: no system-scope fence, which would add its cost to the
    # probed kernel's time and to the step
    return hip_timing.record(stream)


class Step:
    """Streams, workspaces and per-phase calls for a fixed set of matrices.

    matrices  the Matrix records (W, v on the device).
    r, tokens the sketch rank and the tokens of every microbatch.
    act_dtype B.LOGRA_BF16 or B.LOGRA_F32 (X, dY and the compute dtype).
    sketch_lanes / apply_lanes  stream counts (0: min(4, n) for the sketch;
              1 for a single matrix, else 3, for the apply).
    batch_pass1  pass 1 in batches of up to 16 matrices per apply lane.
    seed      the library seed of the sign matrices.
    rowsq     also keep every matrix's per-row sums of squares from pass 1
              (Matrix.rowsq), for callers that inspect them.
    parts     which matrices hold their sketch in parts during the step:
              "pair" (those whose fold tiles are shared by two workgroups:
              one extra d x r array each), "all" (every matrix whose fold
              splits its tiles: up to 31 arrays for small d), or "none".
    """

    def __init__(self, matrices: Sequence[Matrix], r: int, tokens: int, act_dtype: int,
                 device=None, sketch_lanes: int = 0, apply_lanes: int = 0,
                 batch_pass1: bool = True, seed: int = 0, rowsq: bool = False, parts: str = "pair"):
        if not matrices:
            raise ValueError("a step needs at least one matrix")
        self.mats: List[Matrix] = list(matrices)
        self.r, self.tokens, self.code, self.seed = int(r), int(tokens), int(act_dtype), int(seed)
        dev = torch.device(device) if device is not None else self.mats[0].W.device
        self.device = dev
        n = len(self.mats)
        self.n_sketch = max(1, min(sketch_lanes or min(MAX_SKETCH_LANES, n), n))
        self.n_apply = max(1, min(apply_lanes or (1 if n == 1 else DEFAULT_APPLY_LANES), n))
        self.timeouts = torch.zeros(1, dtype=torch.int32, device=dev)
        self.sketch_opts = B.LaunchOpts(sketch_concurrency=self.n_sketch, fold_timeouts=self.timeouts)
        self.apply_opts = B.LaunchOpts(apply_concurrency=self.n_apply)
        ws_bytes = max(B.logra_sketch_workspace_bytes(B.MatrixDesc(m.d, m.k, r), tokens, act_dtype)
                       for m in self.mats)
        sq_ws_bytes = max(B.logra_sqnorm_workspace_bytes(B.MatrixDesc(m.d, m.k, r), act_dtype)
                          for m in self.mats)
        self.main = torch.cuda.current_stream(dev)
        n_lanes = max(self.n_sketch, self.n_apply)
        self.lanes = []
        for i in range(n_lanes):
            self.lanes.append({
                "stream": self.main if i == 0 else torch.cuda.Stream(device=dev),
                "ws": torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev),
                "sq_ws": torch.empty(max(16, sq_ws_bytes), dtype=torch.uint8, device=dev),
            })
        if parts not in ("pair", "all", "none"):
            raise ValueError("parts must be 'pair', 'all' or 'none'")
        self.parts_bytes = 0
        for i, m in enumerate(self.mats):
            m.S = torch.empty(m.d, r, dtype=torch.float32, device=dev)
            pb = B.logra_sketch_parts_bytes(B.MatrixDesc(m.d, m.k, r), tokens, act_dtype)
            use = pb > 0 and (parts == "all" or (parts == "pair" and pb == 4 * m.d * r))
            m.parts = torch.empty(pb // 4, dtype=torch.float32, device=dev) if use else None
            self.parts_bytes += pb if use else 0
            m.v_new = torch.empty(m.d, dtype=torch.float32, device=dev)
            m.sq = torch.empty(1, dtype=torch.float32, device=dev)
            m.rowsq = torch.empty(m.d, dtype=torch.float32, device=dev) if rowsq else None
            m.lane = i % self.n_sketch
            m.alane = i % self.n_apply
        # Pass-1 batches: each apply lane's matrices in as few chunks of at
        # most MAX_BATCH as hold them, of equal size (65 matrices: 5 x 13,
        # not 4 x 16 + 1); a chunk of one matrix uses the single-matrix call.
        # A batched matrix's sqnorm is a view of its chunk's output.
        self.batches = []
        self.batch_ws_bytes = 0
        for li in range(self.n_apply):
            own = [m for m in self.mats if m.alane == li]
            if not batch_pass1:
                self.batches.extend((li, [m], None, None) for m in own)
                continue
            n_chunks = -(-len(own) // B.MAX_BATCH)
            bounds = [len(own) * c // max(1, n_chunks) for c in range(n_chunks + 1)]
            for c0, c1 in zip(bounds[:-1], bounds[1:]):
                chunk = own[c0:c1]
                if len(chunk) == 1:
                    self.batches.append((li, chunk, None, None))
                    continue
                sq = torch.empty(len(chunk), dtype=torch.float32, device=dev)
                for j, m in enumerate(chunk):
                    m.sq = sq[j:j + 1]
                wsb = B.logra_sqnorm_batch_workspace_bytes([B.MatrixDesc(m.d, m.k, r) for m in chunk],
                                                           act_dtype)
                self.batch_ws_bytes += wsb
                self.batches.append((li, chunk, sq, torch.empty(max(16, wsb), dtype=torch.uint8, device=dev)))
        self.workspace_bytes = n_lanes * (max(16, ws_bytes) + max(16, sq_ws_bytes)) + self.batch_ws_bytes

    # ---- streams ---------------------------------------------------------
    def _fork(self):
        if len(self.lanes) > 1:
            e = torch.cuda.Event()
            e.record(self.main)
            for ln in self.lanes[1:]:
                ln["stream"].wait_event(e)

    def _join(self):
        for ln in self.lanes[1:]:
            e = torch.cuda.Event()
            e.record(ln["stream"])
            self.main.wait_event(e)

    # ---- phases ----------------------------------------------------------
    def set_step(self, step: int):
        """The optimizer step whose sign matrices the calls use."""
        for m in self.mats:
            m.desc = B.MatrixDesc(m.d, m.k, self.r, seed=self.seed, step=step, matrix_id=m.matrix_id)

    def sketch(self, step: int, microbatches: int,
               inputs: Callable[[int, int], Tuple[torch.Tensor, torch.Tensor]],
               probe: Optional[Tuple[int, int]] = None):
        """Fold `microbatches` microbatches into every matrix's S, microbatch
        by microbatch; inputs(i, mb) returns (X, dY) of matrix i.

        probe = (i, mb), mb >= 1: time matrix i's projection and fold
        without an event between the two (an event record delays the next
        kernel by a few microseconds): one event pair on its stream around
        the projection of microbatch mb - 1 alone, one around the projection
        and fold of microbatch mb; returns those two pairs,
        ((project_start, project_end), (both_start, both_end)), else None.
        The fold's time is the second pair's less the first's: each holds
        one event record's delay."""
        if probe is not None and probe[1] < 1:
            raise ValueError("probe: the microbatch must have one before it")
        self.set_step(step)
        self._fork()
        events = None
        for mb in range(microbatches):
            for i, m in enumerate(self.mats):
                X, dY = inputs(i, mb)
                ln = self.lanes[m.lane]
                st = ln["stream"]
                alone = probe == (i, mb + 1)     # the projection before the probed one
                both = probe == (i, mb)
                if alone or both:
                    start = _event(st)
                B.logra_sketch_project(m.desc, X, ln["ws"], st, opts=self.sketch_opts)
                if alone:
                    proj_pair = (start, _event(st))
                if m.parts is not None:
                    phase = ((B.LOGRA_FOLD_FIRST if mb == 0 else 0)
                             | (B.LOGRA_FOLD_LAST if mb == microbatches - 1 else 0))
                    B.logra_sketch_fold_parts(m.desc, dY, m.S, m.parts, phase, ln["ws"], st,
                                              opts=self.sketch_opts)
                else:
                    B.logra_sketch_fold(m.desc, dY, m.S, mb > 0, ln["ws"], st, opts=self.sketch_opts)
                if both:
                    events = (proj_pair, (start, _event(st)))
        self._join()
        return events

    def pass1(self, beta2: float, eps: float):
        """v' and sqnorm of every matrix (v unchanged)."""
        self._fork()
        for li, chunk, sq, bws in self.batches:
            ln = self.lanes[li]
            if sq is None:
                m = chunk[0]
                B.logra_update_sqnorm(m.desc, self.code, m.S, m.v, beta2, eps, m.v_new, m.sq, m.rowsq,
                                      ln["sq_ws"], ln["stream"])
            else:
                rq = [m.rowsq for m in chunk] if chunk[0].rowsq is not None else None
                B.logra_update_sqnorm_batch([m.desc for m in chunk], self.code, [m.S for m in chunk],
                                            [m.v for m in chunk], beta2, eps, [m.v_new for m in chunk], sq,
                                            rq, bws, ln["stream"])
        self._join()

    def sqnorms(self) -> List[float]:
        """Every matrix's sqnorm on the host (one device-to-host copy)."""
        return torch.cat([m.sq for m in self.mats]).cpu().tolist()

    def pass2(self, lr: float, scales: Sequence[Optional[float]], eps: float) -> int:
        """W -= lr * scale * Ghat / (sqrt(v') + eps) for every matrix whose
        scale is not None, then v' becomes its v (buffer swap); the others
        keep W and v. Returns the number of matrices updated."""
        if len(scales) != len(self.mats):
            raise ValueError("one scale (or None) per matrix")
        self._fork()
        done = 0
        for m, sc in zip(self.mats, scales):
            if sc is None:
                continue
            B.logra_rowadam_apply(m.desc, self.code, m.S, m.v_new, m.W, lr, sc, eps,
                                  self.lanes[m.alane]["stream"], opts=self.apply_opts)
            m.v, m.v_new = m.v_new, m.v
            done += 1
        self._join()
        return done

    @staticmethod
    def finite_scales(sqnorms: Sequence[float], scales: Sequence[float]) -> List[Optional[float]]:
        """The scales with None where a matrix's sqnorm is not finite (its
        update is skipped)."""
        return [sc if math.isfinite(q) else None for q, sc in zip(sqnorms, scales)]

    def fold_timeouts(self) -> int:
        """Fold workgroups that gave up waiting for their partner since the
        counter was last cleared (0 in a healthy run)."""
        return int(self.timeouts.item())

    def clear_fold_timeouts(self):
        self.timeouts.zero_()
