"""Seeded synthetic inputs for the sketch + RowAdam workloads.

This module holds no arithmetic of the method: it only draws the tensors the
method consumes (activations X, output gradients dY, weights W, second
moments v, the per-step scale) with the shapes and distributions of the
Qwen-shaped workloads, so that the HIP path, the oracle and the benchmark all
see the same data. Random numbers come from torch generators seeded by a hash
of a descriptive key, so a tensor depends only on its key and size, never on
what was drawn before it.

Distributions ("N(0, s)" takes s as the standard deviation):
  X  ~ N(0, 1); in the 7B/27B-shaped workloads round(0.01 k) fixed columns
       (the first ones of a seeded permutation) are multiplied by 10 before
       rounding, standing in for outlier channels;
  dY ~ N(0, 1e-3) in the tiny fp32 case, N(0, 1e-4) otherwise;
  W  ~ N(0, 0.02);
  v  = 0 (tiny and 1.5B cases) or U(1e-10, 1e-8) (7B and 27B cases);
  scale ~ U(0.5, 1) per matrix per step (1.0 in the tiny case).
bf16 tensors are drawn in fp32 and rounded to nearest even by torch.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Tuple

import torch

# Projection order inside a layer; matrix_id = 7 * layer + index.
PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
# Which activation each projection reads: q/k/v share the attention input,
# gate/up share the MLP input.
INPUT_GROUP = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
               "gate": "mlp_in", "up": "mlp_in", "down": "down_in"}


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    layer: int
    d: int          # rows of W (output features)
    k: int          # columns of W (input features)
    matrix_id: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    r: int
    microbatches: int
    tokens: int             # tokens per microbatch
    steps: int
    act_dtype: torch.dtype  # dtype of X and dY
    w_dtype: torch.dtype
    dy_std: float
    outliers: bool          # 1% of X columns scaled x10
    v_init: str             # "zero" or "uniform"
    lr: float
    beta2: float
    eps: float
    scale_mode: str         # "one" or "uniform"
    matrices: Tuple[MatrixSpec, ...]


def _layer_set(layer: int, hidden: int, inter: int, kv: int, qo: Optional[int] = None):
    qo = hidden if qo is None else qo
    shapes = {"q": (qo, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, qo),
              "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    return [MatrixSpec(n, layer, shapes[n][0], shapes[n][1], 7 * layer + i)
            for i, n in enumerate(PROJ_NAMES)]


def _build() -> Dict[str, Workload]:
    w = {}
    w["tiny_fp32"] = Workload(
        "tiny_fp32", "single projection d=256 k=512 r=32, fp32, 4 x 128 tokens",
        r=32, microbatches=4, tokens=128, steps=1, act_dtype=torch.float32,
        w_dtype=torch.float32, dy_std=1e-3, outliers=False, v_init="zero",
        lr=1e-3, beta2=0.999, eps=1e-8, scale_mode="one",
        matrices=(MatrixSpec("proj", 0, 256, 512, 0),))
    w["qwen1.5b_set"] = Workload(
        "qwen1.5b_set", "Qwen-1.5B-shaped projection set (7 matrices), r=256, 8 x 2048 tokens",
        r=256, microbatches=8, tokens=2048, steps=1, act_dtype=torch.bfloat16,
        w_dtype=torch.bfloat16, dy_std=1e-4, outliers=False, v_init="zero",
        lr=1e-6, beta2=0.999, eps=1e-8, scale_mode="uniform",
        matrices=tuple(_layer_set(0, 1536, 8960, 256)))
    w["qwen7b_up"] = Workload(
        "qwen7b_up", "Qwen-7B-shaped MLP up projection d=18944 k=3584, r=256, 16 x 4096 tokens",
        r=256, microbatches=16, tokens=4096, steps=10, act_dtype=torch.bfloat16,
        w_dtype=torch.bfloat16, dy_std=1e-4, outliers=True, v_init="uniform",
        lr=1e-6, beta2=0.999, eps=1e-8, scale_mode="uniform",
        matrices=(MatrixSpec("up", 0, 18944, 3584, 5),))
    w["qwen7b_28layer"] = Workload(
        "qwen7b_28layer", "28-layer Qwen-7B-shaped step, all 196 projections, r=256, 8 x 4096 tokens",
        r=256, microbatches=8, tokens=4096, steps=1, act_dtype=torch.bfloat16,
        w_dtype=torch.bfloat16, dy_std=1e-4, outliers=True, v_init="uniform",
        lr=1e-6, beta2=0.999, eps=1e-8, scale_mode="uniform",
        matrices=tuple(m for L in range(28) for m in _layer_set(L, 3584, 18944, 512)))
    w["27b_64layer"] = Workload(
        "27b_64layer", "64-layer 27B-class stack, hidden 5120, inter 17408, r=256, 8 x 8192 tokens",
        r=256, microbatches=8, tokens=8192, steps=5, act_dtype=torch.bfloat16,
        w_dtype=torch.bfloat16, dy_std=1e-4, outliers=True, v_init="uniform",
        lr=1e-6, beta2=0.999, eps=1e-8, scale_mode="uniform",
        matrices=tuple(m for L in range(64) for m in _layer_set(L, 5120, 17408, 1024)))
    return w


WORKLOADS: Dict[str, Workload] = _build()


def _seed_of(*key) -> int:
    h = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(h[:8], "little") & 0x7FFFFFFFFFFFFFFF


def generator(*key, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(*key))
    return g


def outlier_columns(workload: str, k: int, data_seed: int = 0) -> torch.Tensor:
    """The round(0.01 k) columns scaled x10: the first entries of a seeded
    permutation of range(k)."""
    n_out = int(round(0.01 * k))
    g = generator("outlier-cols", workload, k, data_seed)
    return torch.randperm(k, generator=g)[:n_out]


def activations(wl: Workload, spec: MatrixSpec, step: int, mb: int, T: Optional[int] = None,
                data_seed: int = 0, device="cpu") -> torch.Tensor:
    """X (T x k) for one microbatch; projections that share an input share X."""
    T = wl.tokens if T is None else T
    g = generator("X", wl.name, spec.layer, INPUT_GROUP.get(spec.name, spec.name),
                  spec.k, step, mb, T, data_seed, device=device)
    X = torch.randn(T, spec.k, generator=g, device=device, dtype=torch.float32)
    if wl.outliers:
        cols = outlier_columns(wl.name, spec.k, data_seed).to(device)
        X[:, cols] *= 10.0
    return X.to(wl.act_dtype)


def output_grads(wl: Workload, spec: MatrixSpec, step: int, mb: int, T: Optional[int] = None,
                 data_seed: int = 0, device="cpu") -> torch.Tensor:
    """dY (T x d) for one microbatch."""
    T = wl.tokens if T is None else T
    g = generator("dY", wl.name, spec.matrix_id, spec.d, step, mb, T, data_seed, device=device)
    dY = torch.randn(T, spec.d, generator=g, device=device, dtype=torch.float32) * wl.dy_std
    return dY.to(wl.act_dtype)


def weights(wl: Workload, spec: MatrixSpec, data_seed: int = 0, device="cpu",
            dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    g = generator("W", wl.name, spec.matrix_id, spec.d, spec.k, data_seed, device=device)
    W = torch.randn(spec.d, spec.k, generator=g, device=device, dtype=torch.float32) * 0.02
    return W.to(wl.w_dtype if dtype is None else dtype)


def second_moment(wl: Workload, spec: MatrixSpec, data_seed: int = 0, device="cpu") -> torch.Tensor:
    if wl.v_init == "zero":
        return torch.zeros(spec.d, dtype=torch.float32, device=device)
    g = generator("v", wl.name, spec.matrix_id, spec.d, data_seed, device=device)
    u = torch.rand(spec.d, generator=g, device=device, dtype=torch.float32)
    return 1e-10 + u * (1e-8 - 1e-10)


def step_scale(wl: Workload, spec: MatrixSpec, step: int, data_seed: int = 0) -> float:
    """The step scale applied to one matrix in one step, drawn U(0.5, 1)
    per the workload recipe (the predicted-KL controller's factor is
    computed and reported alongside, not applied)."""
    if wl.scale_mode == "one":
        return 1.0
    g = generator("scale", wl.name, spec.matrix_id, step, data_seed)
    return float(0.5 + 0.5 * torch.rand(1, generator=g).item())


def random_case(seed: int, T: int, d: int, k: int, dtype=torch.float32,
                dy_std: float = 1.0, outlier_cols: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """A free-form (X, dY) pair for tests at arbitrary (ragged) sizes."""
    g = generator("case", seed, T, d, k)
    X = torch.randn(T, k, generator=g, dtype=torch.float32)
    if outlier_cols:
        X[:, torch.randperm(k, generator=g)[:outlier_cols]] *= 10.0
    dY = torch.randn(T, d, generator=g, dtype=torch.float32) * dy_std
    return X.to(dtype), dY.to(dtype)


def list_workloads() -> List[str]:
    return list(WORKLOADS)
