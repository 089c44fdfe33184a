"""Oracle of the predicted-KL step controller (host side of a LoGRA step).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite and
the benchmark's CPU leg may call it; the library never does.

Sources: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
Sketches", paragraph "Step control." (the step is scaled so the predicted KL
change stays within a budget that is annealed); "NVIDIA's LoGRA fits RL
post-training of a 27B model onto a single eight-GPU node", section "Why it
matters" (the KL is predicted from the sketch itself); the walk-through page
on LoGRA, section "Predicted-KL Step Control" (a local quadratic model of the
KL with the Fisher matrix; a scalar shrink factor in closed form when the
prediction exceeds the budget).

Readings where the pages are silent: the Fisher matrix is taken isotropic,
F = phi * I, so for the RowAdam update dW = -lr * Ghat / (sqrt(v') + eps) the
quadratic model gives KL(dW) = 1/2 phi ||dW||^2 = 1/2 phi lr^2 sqnorm summed
over the step's matrices; one factor gamma per step; the budget goes
linearly from delta_start to delta_end over anneal_steps steps. Matrices whose
sqnorm is negative or not finite are skipped (scale 0) and left out of the
prediction.

Written in plain Python floats (double precision) with exact summation
(math.fsum).
"""
from __future__ import annotations

import math


def kl_budget(step: int, delta_start: float, delta_end: float, anneal_steps: int) -> float:
    """Budget of step `step`: linear from delta_start (step 0) to delta_end
    (step anneal_steps and later); delta_end throughout if anneal_steps is 0."""
    if anneal_steps == 0 or int(step) >= int(anneal_steps):
        return float(delta_end)
    t = int(step) / float(anneal_steps)
    return float(delta_start) + (float(delta_end) - float(delta_start)) * t


def predicted_kl(sqnorms, lr: float, phi: float) -> float:
    """1/2 phi lr^2 times the sum of the usable sqnorms."""
    kept = [float(q) for q in sqnorms if math.isfinite(float(q)) and float(q) >= 0.0]
    return 0.5 * phi * float(lr) ** 2 * math.fsum(kept)


def step_scale(sqnorms, lr: float, phi: float, delta: float):
    """Returns (scales per matrix, kl before scaling, kl after scaling)."""
    kl = predicted_kl(sqnorms, lr, phi)
    # KL(gamma dW) = gamma^2 KL(dW): the largest gamma <= 1 within the budget
    gamma = 1.0 if kl <= delta else math.sqrt(delta / kl)
    scales = [gamma if (math.isfinite(float(q)) and float(q) >= 0.0) else 0.0 for q in sqnorms]
    return scales, kl, gamma * gamma * kl
