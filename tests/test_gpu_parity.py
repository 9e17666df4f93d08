"""GPU parity of every stage against the oracle, at sizes the oracle finishes in
seconds.  The shapes span several tiles of each kernel with ragged tails
(128- and 256-query attention chunks, 64-key gather chunks, 32-centroid MFMA blocks,
256-point assignment tiles)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import sparse_attention_video_rope_amd as sav
import workloads
from oracle import scope_oracle as O
from tests.scope_gpu import (assert_attention, assert_rope, gpu_sel, labels_match_or_near_tie, run_gpu, say, to_dev,
                             to_np)

pytestmark = pytest.mark.gpu

SMALL = [
    workloads.small("s64", 5, 9, 11, 64, (16, 24, 24), "bf16", 3, 40, index=101),
    workloads.small("s128", 4, 10, 13, 128, (44, 42, 42), "bf16", 4, 37, index=102),
    workloads.small("s128h", 3, 11, 17, 128, (16, 56, 56), "bf16", 5, 33, index=103),
    workloads.small("s64f", 3, 6, 7, 64, (16, 24, 24), "f32", 4, 9, index=104),
    workloads.small("s128f", 2, 5, 9, 128, (44, 42, 42), "f32", 3, 7, index=105, H=1),
    # 300 query clusters at d = 128: the query assignment's centroid table
    # fills a CU's LDS, so the key clusterings are assigned in a launch of their own
    workloads.small("s128c", 3, 10, 12, 128, (44, 42, 42), "bf16", 300, 60, index=112),
    # 600 query clusters: the centroid updates take 16-channel slices
    workloads.small("s64c", 4, 20, 24, 64, (16, 24, 24), "bf16", 600, 40, H=1, index=114),
]
IDS = [w.name for w in SMALL]

_cache = {}


def oracle_heads(w, rho=None, **kw):
    key = (w, rho, tuple(sorted(kw.items())))
    if key not in _cache:
        q, k, v = workloads.generate(w)
        _cache[key] = [O.workload_head(w, bh, q[bh], k[bh], v[bh], rho=rho, **kw) for bh in range(w.BH)]
    return _cache[key]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sav.load()


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_rope_matches_oracle(w):
    say("rope", w.name)
    g = run_gpu(w)
    for bh, o in enumerate(oracle_heads(w)):
        n = assert_rope(g["q_rope"][bh], o["q_rope"], w.dtype) + assert_rope(g["k_rope"][bh], o["k_rope"], w.dtype)
        say(f"  head {bh}: {n} RoPE elements differ (within 1 ulp)")


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_kmeanspp_seeds_match_oracle(w):
    say("seeds", w.name)
    g = run_gpu(w)
    for bh, o in enumerate(oracle_heads(w)):
        assert g["seeds"][bh, 0, :w.Cq].tolist() == list(o["q_seeds"])
        for m in range(3):
            assert g["seeds"][bh, 1 + m, :w.Cm].tolist() == list(o["k_seeds"][m]), f"head {bh} subspace {m}"


@pytest.mark.parametrize("iters", [0, 1, 3])
@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_lloyd_teacher_forced(w, iters):
    """Same initial centroids on both sides: assignments and centroids after `iters` rounds."""
    say("lloyd", w.name, iters)
    q, k, v = workloads.generate(w)
    wi = w.with_(iters=iters)
    init_q, init_k = [], []
    for bh, o in enumerate(oracle_heads(w)):
        init_q.append(o["q_rope"][o["q_seeds"]])
        kc = np.zeros((w.Cm, w.d))
        offs = O.subspace_offsets(w.split)
        for m, (off, dm) in enumerate(zip(offs, w.split)):
            kc[:, off:off + dm] = o["k_rope"][o["k_seeds"][m], off:off + dm]
        init_k.append(kc)
    g = run_gpu(wi, init_q=np.stack(init_q), init_k=np.stack(init_k), inputs=(q, k, v))
    offs = O.subspace_offsets(w.split)
    for bh, o in enumerate(oracle_heads(w)):
        qr, kr = o["q_rope"], o["k_rope"]
        ref = O.kmeans(qr, w.Cq, iters, w.dtype, 0, bh, 0, init=init_q[bh])
        np.testing.assert_allclose(g["q_centroids"][bh], ref["centroids"], rtol=1e-6, atol=0)
        n_bad = labels_match_or_near_tie(g["q_labels"][bh], ref["labels"], qr, ref["centroids"], w.dtype)
        for m, (off, dm) in enumerate(zip(offs, w.split)):
            X = kr[:, off:off + dm]
            refk = O.kmeans(X, w.Cm, iters, w.dtype, 0, bh, 1 + m, init=init_k[bh][:, off:off + dm])
            np.testing.assert_allclose(g["k_centroids"][bh][:, off:off + dm], refk["centroids"], rtol=1e-6, atol=0)
            n_bad += labels_match_or_near_tie(g["k_codes"][bh][:, m], refk["labels"], X, refk["centroids"], w.dtype)
        say(f"  head {bh}: {n_bad} near-tie label differences")


def upload_oracle_plan(w, heads, pl):
    """Writes the oracle's clustering and key sets into a plan's buffers."""
    BH, N, Cq = w.BH, w.N, w.Cq
    perm = np.concatenate([h["perm_q"] for h in heads]).astype(np.int32)
    qoff = np.concatenate([h["q_off"] for h in heads]).astype(np.int32)
    t = np.concatenate([h["t"] for h in heads]).astype(np.int32)
    b = np.concatenate([h["b"] for h in heads]).astype(np.int32)
    r = np.concatenate([h["r"] for h in heads]).astype(np.int32)
    kh = np.array([h["k_head"] for h in heads], dtype=np.int32)
    sels = [s for h in heads for s in h["sel"]]
    off = np.concatenate([[0], np.cumsum([len(s) for s in sels])]).astype(np.int64)
    idx = np.concatenate(sels).astype(np.int32) if off[-1] else np.zeros(1, np.int32)
    for name, arr in (("perm_q", perm), ("q_off", qoff), ("counts_t", t), ("counts_b", b), ("counts_r", r),
                      ("k_head", kh), ("sel_off", off)):
        getattr(pl, name).copy_(torch.from_numpy(arr).cuda())
    pl.sel_idx[:len(idx)].copy_(torch.from_numpy(idx).cuda())
    pl.status.zero_()


@pytest.mark.parametrize("w", [w for w in SMALL if w.name in ("s128c", "s64c")], ids=["s128c", "s64c"])
def test_lloyd_ties_across_blocks_exact(w):
    """Assignment to centroids with exact and near duplicates in other 32-centroid blocks.

    The initial centroids repeat a set of points three times, so the copies of a
    centroid sit in different MFMA blocks.  In each copy one channel is set to
    0, except in the last third, where it is 2^-20: the first two thirds are
    exact duplicates (every point ties; the lowest index must win), and a point
    is nearer the last copy exactly when that channel of it is positive, by
    about 2^-19 |x_ch|, far below what the bf16 filter resolves.  With no Lloyd
    round the labels must equal the oracle's fp64 argmin exactly, with no
    near-tie allowance: these points are decided by the exact re-decision and
    its block marks alone.
    """
    say("lloyd ties across blocks", w.name)
    q, k, v = workloads.generate(w)
    offs = O.subspace_offsets(w.split)
    rng = np.random.default_rng(7)
    init_q, init_k = [], []
    heads = oracle_heads(w)
    for bh, o in enumerate(heads):
        def tripled(X, C):
            nb = C // 3
            base = X[rng.choice(X.shape[0], nb, replace=False)].astype(np.float64)
            ch = rng.integers(0, X.shape[1], size=nb)
            base[np.arange(nb), ch] = 0.0
            near = base.copy()
            near[np.arange(nb), ch] = 2.0 ** -20
            return np.concatenate([base, base, near, base[: C - 3 * nb]], axis=0)[:C]
        init_q.append(tripled(o["q_rope"], w.Cq))
        kc = np.zeros((w.Cm, w.d))
        for off, dm in zip(offs, w.split):
            kc[:, off:off + dm] = tripled(o["k_rope"][:, off:off + dm], w.Cm)
        init_k.append(kc)
    g = run_gpu(w.with_(iters=0), init_q=np.stack(init_q), init_k=np.stack(init_k), inputs=(q, k, v))
    for bh in range(w.BH):
        # the reference assigns the GPU's own RoPE output (the RoPE comparison
        # is a test of its own)
        ref = O.kmeans(g["q_rope"][bh], w.Cq, 0, w.dtype, 0, bh, 0, init=init_q[bh])
        assert np.array_equal(g["q_labels"][bh], ref["labels"]), f"head {bh} query labels"
        for m, (off, dm) in enumerate(zip(offs, w.split)):
            X = g["k_rope"][bh][:, off:off + dm]
            refk = O.kmeans(X, w.Cm, 0, w.dtype, 0, bh, 1 + m, init=init_k[bh][:, off:off + dm])
            assert np.array_equal(g["k_codes"][bh][:, m], refk["labels"]), f"head {bh} key codes {m}"
        # the duplicates really tie (no label of the second third), and both
        # sides of the near pairs occur
        nb = w.Cq // 3
        lab = g["q_labels"][bh]
        assert not np.any((lab >= nb) & (lab < 2 * nb))
        assert np.any(lab < nb) and np.any((lab >= 2 * nb) & (lab < 3 * nb))


@pytest.mark.parametrize("rho", [0.9, 1.0, 0.3])
@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_attend_on_oracle_plan(w, rho):
    say("attend", w.name, rho)
    heads = oracle_heads(w, rho=rho)
    q, k, v = workloads.generate(w)
    p = sav.params_for(w, rho=rho)
    pl = sav.Plan(p, debug=False)
    upload_oracle_plan(w, heads, pl)
    sav.plan_finalize(p, pl)
    qr = to_dev(np.stack([h["q_rope"] for h in heads]), w.dtype)
    kr = to_dev(np.stack([h["k_rope"] for h in heads]), w.dtype)
    out = to_np(sav.attend(p, pl, qr, kr, to_dev(v, w.dtype))).reshape(w.BH, w.N, w.d)
    for bh, h in enumerate(heads):
        mx, mn = assert_attention(out[bh], h["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


BF16_SMALL = [w for w in SMALL if w.dtype == "bf16"]


@pytest.mark.parametrize("w", BF16_SMALL, ids=[w.name for w in BF16_SMALL])
def test_attend_softmax_reference_paths(w):
    """The per-head key-norm bound written by scope_plan, and all three softmax paths of the
    attention kernel: fixed reference (bound given and tight), running maximum (no bound), and
    running maximum after a rejected bound (10^4 times too loose)."""
    say("softmax paths", w.name)
    heads = oracle_heads(w)
    q, k, v = workloads.generate(w)
    p = sav.params_for(w)
    pl = sav.Plan(p, debug=False)
    qr, kr, pl = sav.plan(p, to_dev(q, w.dtype), to_dev(k, w.dtype), pl)
    kn = pl.k_norm_max.clone()
    for bh, h in enumerate(heads):
        exact = float(np.sqrt((h["k_rope"] ** 2).sum(1)).max())
        got = float(kn[bh])
        assert exact <= got <= exact * (1 + 2**-10), (bh, got, exact)
    vd = to_dev(v, w.dtype)
    for name, scale in (("bound", 1.0), ("no bound", 0.0), ("loose bound", 1e4)):
        pl.k_norm_max.copy_(kn * scale)
        out = to_np(sav.attend(p, pl, qr, kr, vd)).reshape(w.BH, w.N, w.d)
        for bh, h in enumerate(heads):
            mx, mn = assert_attention(out[bh], h["out"], w.dtype, f"{w.name} head {bh} ({name})")
            say(f"  {name} head {bh}: max {mx:.2e} mean {mn:.2e}")


def assert_plan_equal(w, g, heads):
    """End-to-end plan equality (exact) on every head."""
    for bh, o in enumerate(heads):
        assert g["q_labels"][bh].tolist() == o["q_labels"].tolist(), f"head {bh} query labels"
        assert np.array_equal(g["k_codes"][bh], o["k_codes"]), f"head {bh} key codes"
        np.testing.assert_array_equal(g["q_centroids"][bh], o["q_centroids"])
        np.testing.assert_array_equal(g["k_centroids"][bh], o["k_centroids"])
        np.testing.assert_allclose(g["lut"][bh], np.transpose(o["lut"], (1, 0, 2)), rtol=1e-12, atol=1e-12)
        assert g["perm_q"][bh].tolist() == o["perm_q"].tolist()
        assert g["q_off"][bh].tolist() == o["q_off"].tolist()
        assert g["t"][bh].tolist() == o["t"].tolist(), f"head {bh} t_c"
        assert g["b"][bh].tolist() == o["b"].tolist()
        assert int(g["k_head"][bh]) == o["k_head"]
        assert g["r"][bh].tolist() == o["r"].tolist()
        for c, (gs, os_) in enumerate(zip(gpu_sel(g, bh, w.Cq), o["sel"])):
            assert np.array_equal(gs, os_), f"head {bh} cluster {c}: |S| {len(gs)} vs {len(os_)}"


@pytest.mark.parametrize("rho", [0.9, 0.5])
@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_end_to_end_matches_oracle(w, rho):
    say("e2e", w.name, rho)
    heads = oracle_heads(w, rho=rho)
    g = run_gpu(w, rho=rho)
    assert g["status"][1] == 0
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e} density {np.sum(o['n'] * o['r']) / w.N**2:.3f}")


@pytest.mark.parametrize("iters", [0, 2])
@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_warm_start_end_to_end(w, iters):
    """Codebook reuse across denoising steps: the plan of the step-1 stand-in
    inputs with Lloyd started from the oracle's final step-0 centroids (in the
    plan's fp32 centroid format) instead of k-means++."""
    say("warm start", w.name, iters)
    heads0 = oracle_heads(w)
    init_q = np.stack([h["q_centroids"] for h in heads0]).astype(np.float32).astype(np.float64)
    init_k = np.stack([h["k_centroids"] for h in heads0]).astype(np.float32).astype(np.float64)
    q, k, v = workloads.generate(w, step=1)
    wi = w.with_(iters=iters)
    heads = [O.workload_head(wi, bh, q[bh], k[bh], v[bh], init_q=init_q[bh], init_k=init_k[bh])
             for bh in range(w.BH)]
    g = run_gpu(wi, init_q=init_q, init_k=init_k, inputs=(q, k, v))
    assert g["status"][1] == 0
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


def test_tiny_config_end_to_end():
    w = workloads.CONFIGS["tiny"]
    say("tiny")
    heads = oracle_heads(w)
    g = run_gpu(w)
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        assert_attention(g["out"][bh], o["out"], w.dtype, f"tiny head {bh}")


def test_alpha_floor_end_to_end():
    w = SMALL[0].with_(alpha=0.4)
    heads = oracle_heads(w)
    g = run_gpu(w)
    assert_plan_equal(w, g, heads)


# Above 8192 tokens the k-means++ kernel keeps D^2 and the nearest-centre ids
# in global memory between draws instead of registers; these shapes take that
# path, with a last group of point rounds that is only partly filled.
LARGE = [
    workloads.small("m64", 5, 43, 45, 64, (16, 24, 24), "bf16", 6, 12, index=106, H=1),
    workloads.small("m128", 3, 37, 83, 128, (44, 42, 42), "bf16", 5, 9, index=107, H=1),
    workloads.small("m64f", 2, 67, 71, 64, (16, 24, 24), "f32", 4, 6, index=108, H=1),
]
LARGE_IDS = [w.name for w in LARGE]


@pytest.mark.parametrize("w", LARGE, ids=LARGE_IDS)
def test_end_to_end_large_token_count(w):
    say("e2e large", w.name, w.N)
    heads = oracle_heads(w)
    g = run_gpu(w)
    assert g["status"][1] == 0
    for bh, o in enumerate(heads):
        assert g["seeds"][bh, 0, :w.Cq].tolist() == list(o["q_seeds"])
        for m in range(3):
            assert g["seeds"][bh, 1 + m, :w.Cm].tolist() == list(o["k_seeds"][m]), f"head {bh} subspace {m}"
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("w", SMALL + LARGE[:1], ids=IDS + LARGE_IDS[:1])
def test_random_channel_partition_end_to_end(w):
    """The partition ablation: proxy subspaces from a seeded random channel
    order (SCOPE_PERMUTE_CHANNELS) instead of the 3D-RoPE ranges."""
    perm = tuple(int(c) for c in np.random.default_rng([w.index, 11]).permutation(w.d))
    say("random partition", w.name)
    heads = oracle_heads(w, channel_perm=perm)
    g = run_gpu(w, channel_perm=perm)
    assert g["status"][1] == 0
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_fixed_topk_only_end_to_end(w):
    """The selection without the online per-head Top-k (SCOPE_FIXED_TOPK_ONLY,
    r_c = b_c) at the alpha = 0.1 floor."""
    wa = w.with_(alpha=0.1)
    say("fixed top-k only", w.name)
    heads = oracle_heads(wa, online_khead=False)
    g = run_gpu(wa, online_khead=False)
    assert g["status"][1] == 0
    assert_plan_equal(wa, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("grid", [(4, 61, 71), (7, 50, 77), (9, 61, 67)])
def test_kmeanspp_seeds_three_or_more_point_groups(grid):
    """Seeds only, at 17324, 26950 and 36783 tokens (3, 4 and 5 groups of 8192
    points); from 18433 tokens on, one clustering spans several workgroups."""
    w = workloads.small("seedN", *grid, 64, (16, 24, 24), "bf16", 24, 24, index=109, H=1, iters=0)
    say("seeds", grid, w.N)
    q, k, _ = workloads.generate(w)
    g = run_gpu(w, inputs=(q, k, k))
    gridt = (w.T, w.Hg, w.Wg)
    qr = O.round_storage(O.rope_3d(q[0], gridt, w.split, w.rope_base), w.dtype)
    kr = O.round_storage(O.rope_3d(k[0], gridt, w.split, w.rope_base), w.dtype)
    assert g["seeds"][0, 0, :w.Cq].tolist() == list(O.kmeanspp_seeds(qr, w.Cq, w.kmeans_seed, 0, 0))
    for m, (off, dm) in enumerate(zip(O.subspace_offsets(w.split), w.split)):
        want = O.kmeanspp_seeds(kr[:, off:off + dm], w.Cm, w.kmeans_seed, 0, 1 + m)
        assert g["seeds"][0, 1 + m, :w.Cm].tolist() == list(want), f"subspace {m}"


def _seeds_vs_oracle(w, q, k, g):
    gridt = (w.T, w.Hg, w.Wg)
    qr = O.round_storage(O.rope_3d(q[0], gridt, w.split, w.rope_base), w.dtype)
    kr = O.round_storage(O.rope_3d(k[0], gridt, w.split, w.rope_base), w.dtype)
    assert g["seeds"][0, 0, :w.Cq].tolist() == list(O.kmeanspp_seeds(qr, w.Cq, w.kmeans_seed, 0, 0))
    for m, (off, dm) in enumerate(zip(O.subspace_offsets(w.split), w.split)):
        want = O.kmeanspp_seeds(kr[:, off:off + dm], w.Cm, w.kmeans_seed, 0, 1 + m)
        assert g["seeds"][0, 1 + m, :w.Cm].tolist() == list(want), f"subspace {m}"


def test_kmeanspp_seeds_d128_split_over_workgroups():
    """d = 128 at 36783 tokens (5 groups of 8192 points, one workgroup each)."""
    w = workloads.small("seedN128", 9, 61, 67, 128, (44, 42, 42), "bf16", 40, 33, index=110, H=1, iters=0)
    say("seeds d128", w.N)
    q, k, _ = workloads.generate(w)
    g = run_gpu(w, inputs=(q, k, k))
    assert g["status"][2] == 0
    _seeds_vs_oracle(w, q, k, g)


def test_kmeanspp_seeds_all_points_coincide():
    """Queries all zero (every RoPE'd query is the origin): after the first
    draw every D^2 is 0 and each later centre is the lowest index not chosen
    yet, found across the workgroups that share the clustering."""
    w = workloads.small("seedZ", 9, 61, 67, 64, (16, 24, 24), "bf16", 30, 12, index=111, H=1, iters=0)
    say("seeds zero", w.N)
    q, k, _ = workloads.generate(w)
    q = np.zeros_like(q)
    g = run_gpu(w, inputs=(q, k, k))
    assert g["status"][2] == 0
    _seeds_vs_oracle(w, q, k, g)


def _assert_all_ties(w, g, rho):
    """Every key of every cluster has the same proxy logit: t_c = ceil(rho N)
    (the Cm = 1 closed form) and S_c the lowest-index keys."""
    t_want = math.ceil(Fraction(rho) * w.N)
    for bh in range(w.BH):
        assert g["t"][bh].tolist() == [t_want] * w.Cq, f"head {bh}: t_c {sorted(set(g['t'][bh].tolist()))}"
        for c, s in enumerate(gpu_sel(g, bh, w.Cq)):
            assert np.array_equal(s, np.arange(g["r"][bh, c])), f"head {bh} cluster {c}"


@pytest.mark.parametrize("rho", [0.9, 0.5])
def test_tie_walk_all_queries_at_the_origin(rho):
    """Queries all zero: every LUT row is 0 and all N = 36783 logits of every
    cluster tie, far more than the 1024 boundary candidates the selection
    sorts, so the Top-p pass and the final selection resolve the boundary by
    their walk over distinct logits.  Plan and attention against the oracle."""
    w = workloads.small("tieZ", 9, 61, 67, 64, (16, 24, 24), "bf16", 30, 12, index=111, H=1, rhos=(rho,))
    say("tie walk, zero queries", w.N, rho)
    q, k, v = workloads.generate(w)
    q = np.zeros_like(q)
    heads = [O.workload_head(w, 0, q[0], k[0], v[0])]
    g = run_gpu(w, inputs=(q, k, v))
    assert g["status"][1] == 0 and g["status"][2] == 0
    _assert_all_ties(w, g, rho)
    assert_plan_equal(w, g, heads)
    mx, mn = assert_attention(g["out"][0], heads[0]["out"], w.dtype, "zero queries")
    say(f"  max {mx:.2e} mean {mn:.2e}")


def _boundary_bin_sizes(s_row, count):
    """Keys in the level-1 selection bin (2048 equal bins over [min, max] of the
    row, highest logits first) of the count-th key in (s desc, j asc) order."""
    smax, smin = s_row.max(), s_row.min()
    x = (smax - s_row) * (2048.0 / (smax - smin))
    bins = np.clip(x.astype(np.int64), 0, 2047)
    order = np.lexsort((np.arange(s_row.size), -s_row))
    return int(np.sum(bins == bins[order[count - 1]]))


@pytest.mark.parametrize("rho", [0.9, 0.5])
def test_boundary_in_level2_bins(rho):
    """One key 2^10 times longer than the others (all keys scaled by powers of
    two, so the inputs stay exact) stretches every cluster's logit range: the
    other keys crowd into a few of the 2048 level-1 bins, the boundary bin holds
    more than the 1024 keys the selection sorts directly, and the Top-p pass
    and the final selection find the boundary in the level-2 bins.  Plan and
    attention against the oracle."""
    w = workloads.small("lvl2", 9, 61, 67, 64, (16, 24, 24), "bf16", 30, 12, index=115, H=1, rhos=(rho,))
    say("level-2 boundary bins", w.N, rho)
    q, k, v = workloads.generate(w)
    k = k * 2.0 ** -6
    k[0, 4321] *= 2.0 ** 10
    heads = [O.workload_head(w, 0, q[0], k[0], v[0])]
    o = heads[0]
    big_t = sum(_boundary_bin_sizes(o["scores"][c], o["t"][c]) > 1024 for c in range(w.Cq) if o["n"][c] > 0)
    big_r = sum(_boundary_bin_sizes(o["scores"][c], o["r"][c]) > 1024
                for c in range(w.Cq) if 0 < o["r"][c] < w.N and o["r"][c] != o["t"][c])
    say(f"  clusters with a boundary bin of more than 1024 keys: Top-p {big_t}, final count {big_r}")
    assert big_t > 0
    g = run_gpu(w, inputs=(q, k, v))
    assert g["status"][1] == 0 and g["status"][3] == 0
    assert_plan_equal(w, g, heads)
    mx, mn = assert_attention(g["out"][0], o["out"], w.dtype, "level-2 bins")
    say(f"  max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("rho", [0.9, 0.5])
def test_tie_walk_one_key_centroid(rho):
    """Cm = 1: every key has the same code triple, so inside each query
    cluster all N = 4991 logits are equal (the closed form t_c = ceil(rho N),
    S_c = the lowest indices), with 20 distinct query clusters."""
    w = workloads.small("tieC1", 7, 23, 31, 128, (44, 42, 42), "bf16", 20, 1, index=113, H=2, rhos=(rho,))
    say("tie walk, Cm = 1", w.N, rho)
    heads = oracle_heads(w)
    g = run_gpu(w)
    assert g["status"][1] == 0
    _assert_all_ties(w, g, rho)
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"Cm = 1 head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("w", SMALL + [workloads.CONFIGS["tiny"]], ids=IDS + ["tiny"])
def test_dense_mode_matches_oracle_dense_attention(w):
    """SCOPE_DENSE (the dense prefix of the schedule): RoPE and a plan of all
    N keys for every query, then the same attention kernel; output against the
    oracle's dense softmax attention, plan structure exact."""
    say("dense", w.name)
    q, k, v = workloads.generate(w)
    p = sav.params_for(w, dense=True)
    pl = sav.Plan(p, debug=False)
    qr, kr, _ = sav.plan(p, to_dev(q, w.dtype), to_dev(k, w.dtype), pl)
    out = to_np(sav.attend(p, pl, qr, kr, to_dev(v, w.dtype))).reshape(w.BH, w.N, w.d)
    BH, N, Cq = w.BH, w.N, w.Cq
    assert to_np(pl.status)[1] == 0
    assert np.array_equal(to_np(pl.perm_q).reshape(BH, N), np.tile(np.arange(N), (BH, 1)))
    assert np.array_equal(to_np(pl.q_off).reshape(BH, Cq + 1), np.tile([0] + [N] * Cq, (BH, 1)))
    for name in ("counts_t", "counts_b", "counts_r"):
        assert np.array_equal(to_np(getattr(pl, name)).reshape(BH, Cq), np.tile([N] + [0] * (Cq - 1), (BH, 1)))
    assert to_np(pl.k_head).tolist() == [N] * BH
    so = to_np(pl.sel_off)
    assert so[-1] == BH * N
    assert np.array_equal(to_np(pl.sel_idx[:BH * N]).reshape(BH, N), np.tile(np.arange(N), (BH, 1)))
    grid = (w.T, w.Hg, w.Wg)
    for bh in range(BH):
        o = O.dense_head(q[bh], k[bh], v[bh], grid=grid, split=w.split, dtype=w.dtype, rope_base=w.rope_base)
        mx, mn = assert_attention(out[bh], o["out"], w.dtype, f"{w.name} dense head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


@pytest.mark.parametrize("w", SMALL + LARGE[:2], ids=IDS + LARGE_IDS[:2])
def test_full_dim_key_codebook_end_to_end(w):
    """The cluster-level ablation proxy (SCOPE_FULL_DIM_KEYS): one key
    codebook over all d channels; plan and attention against the oracle."""
    say("full-dim keys", w.name)
    heads = oracle_heads(w, full_dim_keys=True)
    g = run_gpu(w, full_dim_keys=True)
    assert g["status"][1] == 0 and g["status"][2] == 0
    for bh, o in enumerate(heads):
        assert g["seeds"][bh, 1, :w.Cm].tolist() == list(o["k_seeds"][0]), f"head {bh} key seeds"
        assert not g["k_codes"][bh][:, 1:].any()
    assert_plan_equal(w, g, heads)
    for bh, o in enumerate(heads):
        mx, mn = assert_attention(g["out"][bh], o["out"], w.dtype, f"{w.name} head {bh}")
        say(f"  head {bh}: max {mx:.2e} mean {mn:.2e}")


# cluster sizes around the 32-query wave groups and the 128- / 256-query work
# items (one empty cluster), and key-set sizes around the 32-key subtiles and the
# 64-key chunks of the attention kernel
ITEM_SIZES = [1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 191, 192, 193, 0, 256, 257, 255, 445]
KEY_SIZES = [1, 7, 31, 32, 33, 63, 64, 65, 97, 128, 129, 255, 300, 1000, 2560]


@pytest.mark.parametrize("shift", [0, 4, 9])
@pytest.mark.parametrize("d", [64, 128])
def test_attend_item_shapes(d, shift):
    """Hand-built plans: every query count around the wave groups and work items
    paired with key sets of every size around the subtiles and chunks (shifted
    per case), with and without the logit bound; output against the oracle's
    attention over the same sets."""
    split = (16, 24, 24) if d == 64 else (44, 42, 42)
    w = workloads.small("shapes", 4, 16, 40, d, split, "bf16", len(ITEM_SIZES), 8, H=1, index=115)
    N, Cq = w.N, w.Cq
    assert sum(ITEM_SIZES) == N
    say("item shapes", d, shift)
    q, k, v = workloads.generate(w)
    rng = np.random.default_rng(1000 + shift)
    tokens = rng.permutation(N)
    labels = np.empty(N, dtype=np.int64)
    labels[tokens] = np.repeat(np.arange(Cq), ITEM_SIZES)
    sel = [np.sort(rng.choice(N, size=KEY_SIZES[(c + shift) % len(KEY_SIZES)], replace=False)) for c in range(Cq)]
    r = np.array([len(s) if ITEM_SIZES[c] else 0 for c, s in enumerate(sel)])
    sel = [s if ITEM_SIZES[c] else s[:0] for c, s in enumerate(sel)]
    perm, off = O.cluster_permutation(labels, Cq)
    head = {"perm_q": perm, "q_off": off, "t": r, "b": r, "r": r, "k_head": int(r.max()), "sel": sel}
    p = sav.params_for(w)
    pl = sav.Plan(p, debug=False)
    upload_oracle_plan(w, [head], pl)
    sav.plan_finalize(p, pl)
    want = O.sparse_attention(q[0], k[0], v[0], labels, sel)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kn = float(np.sqrt((k[0] ** 2).sum(1)).max()) * (1 + 2**-10)
    for name, bound in (("bound", kn), ("no bound", 0.0)):
        pl.k_norm_max.fill_(bound)
        out = to_np(sav.attend(p, pl, qd, kd, vd)).reshape(N, d)
        for c in range(Cq):
            rows = labels == c
            if rows.any():
                assert_attention(out[rows], want[rows], "bf16",
                                 f"{name}: cluster {c} n {ITEM_SIZES[c]} r {r[c]}")
        mx, mn = assert_attention(out, want, "bf16", name)
        say(f"  {name}: max {mx:.2e} mean {mn:.2e}")
