"""C-ABI checks that need no GPU: the library loads, exports every declared entry
point, and rejects bad parameters before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_video_rope_amd as sav
from sparse_attention_video_rope_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scope.h")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(scope_[a-z_]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = sav.load()
    names = declared_symbols()
    assert names == ["scope_attend", "scope_plan", "scope_plan_finalize", "scope_plan_noalloc", "scope_plan_timed",
                     "scope_status_string", "scope_workspace_size"]
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(tmp_path):
    """Every field of the ctypes mirrors sits at the offset the C compiler gives it in include/scope.h."""
    assert ctypes.sizeof(_lib.Params) == 216
    structs = {"scope_params": _lib.Params, "scope_plan_t": _lib.PlanStruct}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "scope.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER), "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, fname, val = line.split()
        got[(cname, fname)] = int(val)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_status_strings():
    lib = sav.load()
    assert lib.scope_status_string(0) == b"ok"
    assert lib.scope_status_string(3) == b"workspace too small"
    assert lib.scope_status_string(99) == b"unknown status"


def good(**kw):
    args = dict(B=1, H=2, T=4, Hg=8, Wg=8, d=64, split=(16, 24, 24), Cq=8, Cm=8)
    args.update(kw)
    return sav.make_params(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(split=(16, 24, 22)), 1),            # split does not sum to d
    (dict(split=(15, 25, 24)), 1),            # odd range
    (dict(d=96, split=(32, 32, 32)), 2),      # unsupported head dim
    (dict(Cq=0), 1), (dict(Cm=257), 1),       # Cm > N
    (dict(Cq=300, T=8, Hg=16, Wg=16, Cm=2000), 2),   # beyond the supported cluster count
    (dict(Cq=600, T=8, Hg=16, Wg=16, d=128, split=(44, 42, 42)), 2),   # query table beyond one CU's LDS
    (dict(Cq=8, Cm=999, T=8, Hg=16, Wg=16, d=128, split=(44, 42, 42), full_dim_keys=True), 2),
    (dict(rho=0.0), 1), (dict(rho=1.5), 1), (dict(alpha=-0.1), 1),
    (dict(iters=-1), 1), (dict(rope_base=1.0), 1),
])
def test_invalid_parameters(kw, code):
    p = good(**kw)
    st = sav.load().scope_workspace_size(ctypes.byref(p), None, None, None)
    assert st == code


def test_channel_permutation_validation():
    lib = sav.load()
    perm = list(range(63, -1, -1))
    p = good(channel_perm=perm)
    assert lib.scope_workspace_size(ctypes.byref(p), None, None, None) == 0
    for bad in (perm[:-1] + [perm[0]], [64] + perm[1:]):     # repeated channel; channel >= d
        q = good()
        for i, c in enumerate(bad):
            q.channel_perm[i] = c
        q.flags = _lib.SCOPE_PERMUTE_CHANNELS
        assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 1
    q = good(online_khead=False)
    assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 0
    q.flags = _lib.SCOPE_FULL_DIM_KEYS | _lib.SCOPE_FIXED_TOPK_ONLY   # one key codebook
    assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 0
    q.flags = _lib.SCOPE_FULL_DIM_KEYS | _lib.SCOPE_PERMUTE_CHANNELS   # not combinable
    assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 1
    q.flags = 0x20                                          # unknown flag
    assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 1
    q.flags = _lib.SCOPE_DENSE                              # dense attention alone
    assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 0
    for other in (_lib.SCOPE_FIXED_TOPK_ONLY, _lib.SCOPE_USE_INIT_CENTROIDS, _lib.SCOPE_PERMUTE_CHANNELS,
                  _lib.SCOPE_FULL_DIM_KEYS):
        q.flags = _lib.SCOPE_DENSE | other                  # not combinable
        assert lib.scope_workspace_size(ctypes.byref(q), None, None, None) == 1
    # entries beyond d are not read; the reordered copies of q_rope / k_rope (bf16) enlarge the workspace
    p.channel_perm[100] = 200
    ws_p, _, _ = sav.sizes(p)
    ws, _, _ = sav.sizes(good())
    assert ws_p >= ws + 2 * (2 * 2 * 256 * 64)


def test_workspace_size_and_capacities():
    p = good()
    ws, sel, work = sav.sizes(p)
    # work items: BH * (Cq + ceil(N / chunk)); chunk = 128 queries, 256 for bf16 with d = 128
    assert ws > 0 and sel == 2 * 8 * 256 and work == 2 * (8 + 2)
    assert sav.sizes(good(dtype="f32"))[2] == 2 * (8 + 2)
    assert sav.sizes(good(d=128, split=(44, 42, 42)))[2] == 2 * (8 + 1)
    assert sav.sizes(good(d=128, split=(44, 42, 42), dtype="f32"))[2] == 2 * (8 + 2)
    # monotone in the token count
    ws2, _, _ = sav.sizes(good(T=8))
    assert ws2 > ws


def test_plan_rejects_null_pointers_before_launch():
    lib = sav.load()
    p = good()
    plan = _lib.PlanStruct()
    st = lib.scope_plan(ctypes.byref(p), None, None, None, None, ctypes.byref(plan), None, 0, None)
    assert st == 1
    st = lib.scope_attend(ctypes.byref(p), ctypes.byref(plan), None, None, None, None, None)
    assert st == 1
    st = lib.scope_plan_finalize(ctypes.byref(p), None, None)
    assert st == 1


def test_plan_rejects_misaligned_and_small_workspace():
    lib = sav.load()
    p = good()
    plan = _lib.PlanStruct()
    fake = 1 << 20                     # never dereferenced: validation fails first
    for name in ("perm_q", "q_off", "counts_t", "counts_b", "counts_r", "k_head", "sel_off", "sel_idx", "work",
                 "status"):
        setattr(plan, name, fake)
    _, _, work = sav.sizes(p)
    plan.work_capacity = work
    plan.sel_capacity = 10
    st = lib.scope_plan(ctypes.byref(p), fake + 2, fake, fake, fake, ctypes.byref(plan), fake, 1 << 40, None)
    assert st == 1                      # q misaligned
    st = lib.scope_plan(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 16, None)
    assert st == 3                      # workspace too small
    plan.work_capacity = work - 1
    st = lib.scope_plan(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 1 << 40, None)
    assert st == 4                      # work list too small
    p.flags = _lib.SCOPE_USE_INIT_CENTROIDS
    plan.work_capacity = work
    st = lib.scope_plan(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 1 << 40, None)
    assert st == 1                      # init centroids requested but not given


def test_plan_timed_rejects_bad_event_arrays_before_launch():
    lib = sav.load()
    p = good()
    plan = _lib.PlanStruct()
    fake = 1 << 20                     # never dereferenced: validation fails first
    for name in ("perm_q", "q_off", "counts_t", "counts_b", "counts_r", "k_head", "sel_off", "sel_idx", "work",
                 "status"):
        setattr(plan, name, fake)
    _, _, work = sav.sizes(p)
    plan.work_capacity = work
    ev = (ctypes.c_void_p * 5)(*([fake] * 5))
    for arr, n in ((None, 5), (ev, 0), (ev, 6)):
        st = lib.scope_plan_timed(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 1 << 40,
                                  arr, n, None)
        assert st == 1
    ev[2] = None                       # a null event
    st = lib.scope_plan_timed(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 1 << 40, ev, 5, None)
    assert st == 1
    st = lib.scope_plan_timed(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(plan), fake, 16, ev, 5, None)
    assert st == 3                     # the workspace check comes first, as in scope_plan


def test_plan_noalloc_rejects_parameters_beyond_its_scratch_before_launch():
    """The no-allocation entry point: a parameter set whose workspace exceeds
    the fixed scratch array is refused with SCOPE_ERR_WORKSPACE before any HIP
    call; invalid parameters still give SCOPE_ERR_INVALID."""
    lib = sav.load()
    big = good(H=40, T=21, Hg=45, Wg=80, d=128, split=(44, 42, 42), Cq=300, Cm=333)
    assert sav.sizes(big)[0] > _lib.NOALLOC_MAX_WORKSPACE
    plan = _lib.PlanStruct()
    assert lib.scope_plan_noalloc(ctypes.byref(big), None, None, None, None, ctypes.byref(plan), None) == 3
    assert lib.scope_plan_noalloc(ctypes.byref(good(rho=0.0)), None, None, None, None, ctypes.byref(plan), None) == 1
    assert sav.sizes(good())[0] <= _lib.NOALLOC_MAX_WORKSPACE


def test_largest_supported_centroid_tables():
    """The bf16 centroid table of a clustering must fit in one CU's LDS: 576
    centroids of 128 channels do, 577 do not; fp32 runs take no table."""
    lib = sav.load()
    kw = dict(T=8, Hg=16, Wg=16, d=128, split=(44, 42, 42))
    for cq, code in ((576, 0), (577, 2)):
        p = good(Cq=cq, **kw)
        assert lib.scope_workspace_size(ctypes.byref(p), None, None, None) == code
        p = good(Cq=8, Cm=cq, full_dim_keys=True, **kw)
        assert lib.scope_workspace_size(ctypes.byref(p), None, None, None) == code
    p = good(Cq=1000, dtype="f32", **kw)
    assert lib.scope_workspace_size(ctypes.byref(p), None, None, None) == 0
    p = good(Cq=1024, Cm=1024, T=16, Hg=16, Wg=16)        # d = 64: 1024-centroid tables fit
    assert lib.scope_workspace_size(ctypes.byref(p), None, None, None) == 0
