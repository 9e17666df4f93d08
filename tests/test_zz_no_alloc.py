"""The no-allocation entry point (scope_plan_noalloc, scratch in the library)
against scope_plan with a caller workspace, through the C ABI, on two calls in
a row, the second with a smaller input.  The same kernels run in both, so the
plans and the attention outputs must be bit-identical."""
import numpy as np
import pytest
import torch

import sparse_attention_video_rope_amd as sav
import workloads
from tests.scope_gpu import say, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("q_centroids", "k_centroids", "q_labels", "lut", "perm_q", "q_off", "counts_t", "counts_b", "counts_r",
          "k_head", "sel_off", "k_norm_max", "status")


def _plan_both(w):
    q, k, v = workloads.generate(w)
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    p = sav.params_for(w)
    assert sav.sizes(p)[0] <= sav._lib.NOALLOC_MAX_WORKSPACE
    ref = sav.Plan(p, debug=True)
    qr0, kr0, _ = sav.plan(p, qd, kd, ref)
    out0 = sav.attend(p, ref, qr0, kr0, vd)
    pl = sav.Plan(p, debug=True, workspace=False)
    assert pl.workspace.numel() == 0
    qr1, kr1 = torch.empty_like(qd), torch.empty_like(kd)
    sav.plan_noalloc(p, qd, kd, pl, qr1, kr1)
    out1 = sav.attend(p, pl, qr1, kr1, vd)
    torch.cuda.synchronize()
    return w, p, ref, pl, (qr0, kr0, out0), (qr1, kr1, out1)


def _assert_same(w, ref, pl, a, b):
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for f in FIELDS:
        assert torch.equal(getattr(pl, f), getattr(ref, f)), f
    sa, sb = (t.view(w.BH, 4, max(w.Cq, w.Cm)) for t in (pl.seeds, ref.seeds))
    assert torch.equal(sa[:, 0, :w.Cq], sb[:, 0, :w.Cq]) and torch.equal(sa[:, 1:, :w.Cm], sb[:, 1:, :w.Cm])
    assert torch.equal(pl.k_codes.view(-1, 4)[:, :3], ref.k_codes.view(-1, 4)[:, :3])
    n = int(ref.sel_off[-1])
    assert torch.equal(pl.sel_idx[:n], ref.sel_idx[:n])
    items = int(ref.status[0])
    assert torch.equal(pl.work[:2 * items], ref.work[:2 * items])


def test_noalloc_plan_equals_workspace_plan_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sav.load()
    # first call: 2 heads of 2400 tokens, d = 128 (several k-means++ workgroups' worth of points)
    big = workloads.small("noalloc1", 5, 20, 24, 128, (44, 42, 42), "bf16", 40, 33, H=2, index=120)
    # second call, smaller: 1 head of 297 tokens, d = 64 (the scratch keeps the first call's contents)
    small = workloads.small("noalloc2", 3, 9, 11, 64, (16, 24, 24), "bf16", 7, 9, H=1, index=121)
    assert sav.sizes(sav.params_for(small))[0] < sav.sizes(sav.params_for(big))[0]
    for w in (big, small):
        say("noalloc", w.name, w.N)
        w, p, ref, pl, a, b = _plan_both(w)
        _assert_same(w, ref, pl, a, b)
        say(f"  {w.name}: identical ({int(ref.sel_off[-1])} selected keys)")
