"""LoGRA sketch-accumulate + RowAdam-apply on MI355X (gfx950).

The compute path is the C-ABI library ``liblogra.so`` (HIP kernels); the
functions here are a thin ctypes binding over it. Importing the package does
not load the library; the first call does, and fails loudly if it is not
built.
"""
from __future__ import annotations

__all__ = [
    "logra_abi_version", "logra_status_string", "logra_sign_words",
    "logra_sketch_workspace_bytes", "logra_sketch_accumulate",
    "logra_sketch_project", "logra_sketch_fold", "LaunchOpts",
    "logra_backward_dx", "logra_backward_dx_sketch",
    "logra_sqnorm_workspace_bytes", "logra_update_sqnorm", "logra_rowadam_apply",
    "logra_sqnorm_prepare", "logra_update_sqnorm_prepared", "logra_update_sqnorm_noalloc",
    "logra_sqnorm_batch_workspace_bytes", "logra_update_sqnorm_batch",
    "logra_kl_budget_at", "logra_kl_step_scale", "KLBudget",
    "LograError", "MatrixDesc", "library_path", "load_library",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
