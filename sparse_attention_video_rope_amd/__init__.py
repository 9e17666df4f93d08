"""SCOPE sparse attention for video DiTs on MI355X (gfx950).

The hot path (3D RoPE, query / key-subspace k-means, LUT proxy scoring,
hybrid Top-p with online per-head k_head, gathered exact attention) runs in
the HIP library libscope.so behind the C ABI of include/scope.h; this package
is its Python binding.
"""
from ._lib import (SCOPE_BF16, SCOPE_DENSE, SCOPE_F32, SCOPE_FULL_DIM_KEYS, SCOPE_FIXED_TOPK_ONLY, SCOPE_PERMUTE_CHANNELS, SCOPE_USE_INIT_CENTROIDS, Params, Plan, ScopeError,
                   STAGES, attend, load, make_params, params_for, plan, plan_finalize, plan_noalloc, plan_timed,
                   sizes)

__all__ = ["SCOPE_BF16", "SCOPE_DENSE", "SCOPE_F32", "SCOPE_FULL_DIM_KEYS", "SCOPE_FIXED_TOPK_ONLY", "SCOPE_PERMUTE_CHANNELS", "SCOPE_USE_INIT_CENTROIDS", "Params", "Plan",
           "STAGES", "ScopeError", "attend", "load", "make_params", "params_for", "plan", "plan_finalize", "plan_noalloc",
           "plan_timed",
           "sizes"]
