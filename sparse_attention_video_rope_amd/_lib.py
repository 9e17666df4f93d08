"""ctypes binding of libscope.so (include/scope.h): argument marshalling only.

Every stage of the path runs in the HIP library; this module allocates the
caller-owned buffers with torch (device memory and streams) and passes raw
pointers.  There is no fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_int32, c_int64, c_uint32, c_uint64, c_void_p, c_size_t
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libscope.so")

SCOPE_F32 = 0
SCOPE_BF16 = 1
SCOPE_USE_INIT_CENTROIDS = 0x1
SCOPE_PERMUTE_CHANNELS = 0x2
SCOPE_FIXED_TOPK_ONLY = 0x4
SCOPE_DENSE = 0x8
SCOPE_FULL_DIM_KEYS = 0x10

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace too small",
          4: "plan buffer too small", 5: "HIP error"}


class ScopeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} (status {code})")
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("T", c_int32), ("Hg", c_int32), ("Wg", c_int32),
                ("d", c_int32), ("d_t", c_int32), ("d_h", c_int32), ("d_w", c_int32),
                ("Cq", c_int32), ("Cm", c_int32), ("iters", c_int32),
                ("rope_base", c_double), ("rho", c_double), ("alpha", c_double),
                ("seed", c_uint64), ("dtype", c_int32), ("flags", c_uint32),
                ("channel_perm", ctypes.c_uint8 * 128)]

    @property
    def N(self) -> int:
        return self.T * self.Hg * self.Wg

    @property
    def BH(self) -> int:
        return self.B * self.H


class PlanStruct(ctypes.Structure):
    _fields_ = [("perm_q", c_void_p), ("q_off", c_void_p), ("counts_t", c_void_p), ("counts_b", c_void_p),
                ("counts_r", c_void_p), ("k_head", c_void_p), ("sel_off", c_void_p), ("sel_idx", c_void_p),
                ("sel_capacity", c_int64), ("work", c_void_p), ("work_capacity", c_int64), ("status", c_void_p),
                ("q_centroids", c_void_p), ("k_centroids", c_void_p), ("q_labels", c_void_p),
                ("k_codes", c_void_p), ("seeds", c_void_p), ("lut", c_void_p), ("k_norm_max", c_void_p)]


_lib = None


def load():
    """Loads libscope.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m sparse_attention_video_rope_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, PL = ctypes.POINTER(Params), ctypes.POINTER(PlanStruct)
        lib.scope_workspace_size.argtypes = [P, ctypes.POINTER(c_size_t), ctypes.POINTER(c_int64),
                                             ctypes.POINTER(c_int64)]
        lib.scope_workspace_size.restype = c_int32
        lib.scope_plan.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, PL, c_void_p, c_size_t, c_void_p]
        lib.scope_plan.restype = c_int32
        lib.scope_plan_noalloc.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, PL, c_void_p]
        lib.scope_plan_noalloc.restype = c_int32
        lib.scope_plan_timed.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, PL, c_void_p, c_size_t,
                                         ctypes.POINTER(c_void_p), c_int32, c_void_p]
        lib.scope_plan_timed.restype = c_int32
        lib.scope_plan_finalize.argtypes = [P, PL, c_void_p]
        lib.scope_plan_finalize.restype = c_int32
        lib.scope_attend.argtypes = [P, PL, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        lib.scope_attend.restype = c_int32
        lib.scope_status_string.argtypes = [c_int32]
        lib.scope_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def make_params(*, B, H, T, Hg, Wg, d, split, Cq, Cm, iters=10, rope_base=10000.0, rho=0.9, alpha=0.0,
                seed=0, dtype="bf16", init_centroids=False, channel_perm=None, online_khead=True,
                dense=False, full_dim_keys=False) -> Params:
    """channel_perm: None, or the channel order of the proxy subspaces (a
    permutation of 0..d-1; sets SCOPE_PERMUTE_CHANNELS); online_khead=False
    sets SCOPE_FIXED_TOPK_ONLY (r_c = b_c); dense=True sets SCOPE_DENSE
    (dense attention: RoPE and a plan of all keys for every query);
    full_dim_keys=True sets SCOPE_FULL_DIM_KEYS (one key codebook over all d
    channels instead of the T/H/W subspaces)."""
    p = Params()
    p.B, p.H, p.T, p.Hg, p.Wg, p.d = B, H, T, Hg, Wg, d
    p.d_t, p.d_h, p.d_w = split
    p.Cq, p.Cm, p.iters = Cq, Cm, iters
    p.rope_base, p.rho, p.alpha, p.seed = float(rope_base), float(rho), float(alpha), int(seed)
    p.dtype = SCOPE_BF16 if dtype == "bf16" else SCOPE_F32
    p.flags = SCOPE_USE_INIT_CENTROIDS if init_centroids else 0
    if not online_khead:
        p.flags |= SCOPE_FIXED_TOPK_ONLY
    if dense:
        p.flags |= SCOPE_DENSE
    if full_dim_keys:
        p.flags |= SCOPE_FULL_DIM_KEYS
    if channel_perm is not None:
        cp = [int(c) for c in channel_perm]
        if len(cp) != d:
            raise ValueError(f"channel_perm: expected {d} entries, got {len(cp)}")
        for i, c in enumerate(cp):
            p.channel_perm[i] = c
        p.flags |= SCOPE_PERMUTE_CHANNELS
    return p


def params_for(w, rho: Optional[float] = None, **kw) -> Params:
    """Params of a workloads.Workload."""
    args = dict(B=w.B, H=w.H, T=w.T, Hg=w.Hg, Wg=w.Wg, d=w.d, split=w.split, Cq=w.Cq, Cm=w.Cm, iters=w.iters,
                rope_base=w.rope_base, rho=w.rho if rho is None else rho, alpha=w.alpha, seed=w.kmeans_seed,
                dtype=w.dtype)
    args.update(kw)
    return make_params(**args)


def sizes(p: Params):
    ws, sel, work = c_size_t(), c_int64(), c_int64()
    st = load().scope_workspace_size(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(sel), ctypes.byref(work))
    if st:
        raise ScopeError(st, "scope_workspace_size")
    return ws.value, sel.value, work.value


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Plan:
    """Caller-owned device buffers of one plan (torch tensors) plus the C struct."""

    def __init__(self, p: Params, device="cuda", debug: bool = True, sel_capacity: Optional[int] = None,
                 norm_bound: bool = True, centroids: Optional[bool] = None, workspace: bool = True):
        """debug: also keep labels, codes, seeds and LUT; centroids (default:
        debug): keep the final centroids, which a later plan can start from
        with SCOPE_USE_INIT_CENTROIDS; workspace=False: no workspace (for
        plan_noalloc only)."""
        import torch
        ws, sel_worst, work_cap = sizes(p)
        BH, N, Cq, Cm, d = p.BH, p.N, p.Cq, p.Cm, p.d
        i32 = dict(dtype=torch.int32, device=device)
        self.params = p
        self.perm_q = torch.empty(BH * N, **i32)
        self.q_off = torch.empty(BH * (Cq + 1), **i32)
        self.counts_t = torch.empty(BH * Cq, **i32)
        self.counts_b = torch.empty(BH * Cq, **i32)
        self.counts_r = torch.empty(BH * Cq, **i32)
        self.k_head = torch.empty(BH, **i32)
        self.sel_off = torch.empty(BH * Cq + 1, dtype=torch.int64, device=device)
        cap = sel_worst if sel_capacity is None else sel_capacity
        self.sel_idx = torch.empty(max(cap, 1), **i32)
        self.work = torch.empty(2 * max(work_cap, 1), **i32)
        self.status = torch.zeros(4, **i32)
        # per-head bound of ||k'|| (lets scope_attend drop the running softmax maximum); None: not provided
        self.k_norm_max = torch.zeros(BH, dtype=torch.float32, device=device) if norm_bound else None
        self.workspace = torch.empty(ws if workspace else 0, dtype=torch.uint8, device=device)
        self.debug = debug
        self.q_centroids = self.k_centroids = None
        if debug if centroids is None else centroids:
            self.q_centroids = torch.zeros(BH * Cq * d, dtype=torch.float32, device=device)
            self.k_centroids = torch.zeros(BH * Cm * d, dtype=torch.float32, device=device)
        if debug:
            self.q_labels = torch.empty(BH * N, **i32)
            self.k_codes = torch.empty(BH * N * 4, dtype=torch.int16, device=device)
            self.seeds = torch.empty(BH * 4 * max(Cq, Cm), **i32)
            self.lut = torch.empty(BH * Cq * 3 * Cm, dtype=torch.float64, device=device)
        else:
            self.q_labels = self.k_codes = self.seeds = self.lut = None
        s = PlanStruct()
        for name in ("perm_q", "q_off", "counts_t", "counts_b", "counts_r", "k_head", "sel_off", "sel_idx", "work",
                     "status", "q_centroids", "k_centroids", "q_labels", "k_codes", "seeds", "lut", "k_norm_max"):
            setattr(s, name, _ptr(getattr(self, name)))
        s.sel_capacity = cap
        s.work_capacity = work_cap
        self.struct = s


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check_tensor(t, p: Params, name: str):
    import torch
    want = torch.bfloat16 if p.dtype == SCOPE_BF16 else torch.float32
    if t.dtype != want or not t.is_contiguous() or not t.is_cuda or t.numel() != p.BH * p.N * p.d:
        raise ValueError(f"{name}: expected a contiguous {want} CUDA tensor with {p.BH * p.N * p.d} elements")


def plan(p: Params, q, k, pl: Optional[Plan] = None, q_rope=None, k_rope=None):
    """scope_plan: returns (q_rope, k_rope, plan)."""
    import torch
    _check_tensor(q, p, "q")
    _check_tensor(k, p, "k")
    pl = pl or Plan(p, device=q.device)
    q_rope = torch.empty_like(q) if q_rope is None else q_rope
    k_rope = torch.empty_like(k) if k_rope is None else k_rope
    st = load().scope_plan(ctypes.byref(p), q.data_ptr(), k.data_ptr(), q_rope.data_ptr(), k_rope.data_ptr(),
                           ctypes.byref(pl.struct), pl.workspace.data_ptr(), pl.workspace.numel(), _stream())
    if st:
        raise ScopeError(st, "scope_plan")
    return q_rope, k_rope, pl


NOALLOC_MAX_WORKSPACE = 64 << 20       # SCOPE_NOALLOC_MAX_WORKSPACE of include/scope.h


def plan_noalloc(p: Params, q, k, pl: Plan, q_rope, k_rope):
    """scope_plan_noalloc: the plan in the library's fixed per-GPU scratch
    array (no workspace; the caller still passes every input and output)."""
    _check_tensor(q, p, "q")
    _check_tensor(k, p, "k")
    st = load().scope_plan_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), q_rope.data_ptr(),
                                   k_rope.data_ptr(), ctypes.byref(pl.struct), _stream())
    if st:
        raise ScopeError(st, "scope_plan_noalloc")
    return q_rope, k_rope, pl


STAGES = ("rope", "kmeanspp", "lloyd", "perm_lut", "score_select")


def plan_timed(p: Params, q, k, pl: Plan, q_rope, k_rope):
    """scope_plan_timed: the same plan, with HIP events after each stage.

    Returns {stage: ms} (synchronises the stream to read the events)."""
    import torch
    _check_tensor(q, p, "q")
    _check_tensor(k, p, "k")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
    for e in ev:
        e.record()          # creates the HIP event behind each torch event
    ev[0].record()
    arr = (c_void_p * len(STAGES))(*[e.cuda_event for e in ev[1:]])
    st = load().scope_plan_timed(ctypes.byref(p), q.data_ptr(), k.data_ptr(), q_rope.data_ptr(), k_rope.data_ptr(),
                                 ctypes.byref(pl.struct), pl.workspace.data_ptr(), pl.workspace.numel(), arr,
                                 len(STAGES), _stream())
    if st:
        raise ScopeError(st, "scope_plan_timed")
    ev[-1].synchronize()
    return {name: ev[i].elapsed_time(ev[i + 1]) for i, name in enumerate(STAGES)}


def plan_finalize(p: Params, pl: Plan):
    st = load().scope_plan_finalize(ctypes.byref(p), ctypes.byref(pl.struct), _stream())
    if st:
        raise ScopeError(st, "scope_plan_finalize")


def attend(p: Params, pl: Plan, q_rope, k_rope, v, out=None):
    """scope_attend: returns out [B*H*N*d] in the storage dtype."""
    import torch
    for t, n in ((q_rope, "q_rope"), (k_rope, "k_rope"), (v, "v")):
        _check_tensor(t, p, n)
    out = torch.empty_like(v) if out is None else out
    st = load().scope_attend(ctypes.byref(p), ctypes.byref(pl.struct), q_rope.data_ptr(), k_rope.data_ptr(),
                             v.data_ptr(), out.data_ptr(), _stream())
    if st:
        raise ScopeError(st, "scope_attend")
    return out
