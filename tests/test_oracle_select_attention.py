"""Pins of the oracle's LUT/proxy (Eq. (6), (27)), hybrid selection (Eq. (7)-(10)) and attention."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import scope_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- Eq. (27) and check (a) -------------------------------------------------

def test_eq27_lut_sum_equals_product_code_inner_product():
    rng = np.random.default_rng(0)
    split, d, N, Cq, Cm = (16, 24, 24), 64, 300, 7, 9
    qc = rng.standard_normal((Cq, d))
    kc = rng.standard_normal((Cm, d))
    codes = rng.integers(0, Cm, (N, 3))
    P = O.lookup_tables(qc, kc, split)
    s = O.proxy_logits(P, codes, d)
    offs = [0, 16, 40]
    khat = np.concatenate([kc[codes[:, m], o:o + dm] for m, (o, dm) in enumerate(zip(offs, split))], 1)
    np.testing.assert_allclose(s, qc @ khat.T / 8.0, rtol=1e-12, atol=1e-12)


def test_check_a_proxy_is_exact_logit_when_every_key_is_its_own_centroid():
    w = workloads.small("a", 2, 3, 4, 64, (16, 24, 24), "f32", 24, 24, H=1, iters=3)
    q, k, v = workloads.generate(w)
    r = O.workload_head(w, 0, q[0], k[0], v[0])
    # every query / key sub-vector is its own centroid
    np.testing.assert_array_equal(np.sort(r["q_labels"]), np.arange(24))
    exact = r["q_rope"] @ r["k_rope"].T / 8.0
    qc = r["q_centroids"][r["q_labels"]]         # row i -> centroid of query i == query i
    np.testing.assert_array_equal(qc, r["q_rope"])
    s_rows = r["scores"][r["q_labels"]]          # proxy logits of each query's own cluster
    np.testing.assert_allclose(s_rows, exact, rtol=1e-12, atol=1e-12)


# --- without the online per-head Top-k (the Fig. 7 ablation) ---------------

def test_fixed_topk_only_keeps_the_base_counts():
    """r_c = b_c without the Eq. (10) extension; the key sets are prefixes of
    the full method's (same order), and only clusters with b_c < k_head shrink."""
    rng = np.random.default_rng(4)
    Cq, N = 6, 200
    s = rng.standard_normal((Cq, N)) * np.array([[0.1], [3.0], [1.0], [8.0], [0.5], [2.0]])
    n = np.array([30, 5, 0, 60, 10, 95])
    t, b, kh, r, sel = O.hybrid_select(s, n, 0.8, 0.05)
    t2, b2, kh2, r2, sel2 = O.hybrid_select(s, n, 0.8, 0.05, online_khead=False)
    assert np.array_equal(t, t2) and np.array_equal(b, b2) and kh == kh2
    assert np.array_equal(r2, np.where(n > 0, b, 0))
    assert r2[2] == 0 and r[2] == 0
    for c in range(Cq):
        assert set(sel2[c].tolist()) <= set(sel[c].tolist())
        assert len(sel2[c]) == r2[c]
    assert np.any(r2 < r)                       # the extension matters on this example
    assert np.array_equal(r2[b >= kh], r[b >= kh])


# --- the partition ablation (a reordered channel partition) -----------------

def test_check_a_holds_for_a_random_channel_partition():
    """Every key its own centroid: with any channel partition the proxy of a
    query's own cluster is its exact logit row (a reordering applied to one
    side only, or to different channels on the two sides, breaks this)."""
    w = workloads.small("a", 2, 3, 4, 64, (16, 24, 24), "f32", 24, 24, H=1, iters=3)
    q, k, v = workloads.generate(w)
    perm = np.random.default_rng(5).permutation(64)
    r = O.workload_head(w, 0, q[0], k[0], v[0], channel_perm=perm)
    exact = r["q_rope"] @ r["k_rope"].T / 8.0
    np.testing.assert_allclose(r["scores"][r["q_labels"]], exact, rtol=1e-12, atol=1e-12)
    # the centroids live in the reordered channel space
    np.testing.assert_array_equal(r["q_centroids"][r["q_labels"]], r["q_rope"][:, perm])


def test_channel_order_inside_each_rope_range_does_not_change_the_plan():
    """Reordering channels only inside each 3D-RoPE range leaves every
    distance, and so the clustering, the proxy and the key sets, as they are;
    the identity reordering reproduces the plain path exactly."""
    w = workloads.small("p", 3, 5, 6, 64, (16, 24, 24), "bf16", 6, 10, H=1, iters=3)
    q, k, v = workloads.generate(w)
    base = O.workload_head(w, 0, q[0], k[0], v[0])
    ident = O.workload_head(w, 0, q[0], k[0], v[0], channel_perm=np.arange(64))
    rng = np.random.default_rng(9)
    inside = np.concatenate([o + rng.permutation(dm) for o, dm in zip((0, 16, 40), (16, 24, 24))])
    r = O.workload_head(w, 0, q[0], k[0], v[0], channel_perm=inside)
    for x in (ident, r):
        np.testing.assert_array_equal(x["q_labels"], base["q_labels"])
        np.testing.assert_array_equal(x["k_codes"], base["k_codes"])
        np.testing.assert_allclose(x["scores"], base["scores"], rtol=1e-12, atol=1e-12)
        for a, b in zip(x["sel"], base["sel"]):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_allclose(x["out"], base["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["q_centroids"], base["q_centroids"][:, inside])
    np.testing.assert_array_equal(ident["k_centroids"], base["k_centroids"])
    # a partition that mixes the ranges is a different proxy
    mixed = O.workload_head(w, 0, q[0], k[0], v[0], channel_perm=rng.permutation(64))
    assert not np.array_equal(mixed["k_codes"], base["k_codes"])


# --- Top-p (Eq. (7)) --------------------------------------------------------

def test_top_p_closed_form_when_all_scores_tie():
    for N, rho in [(256, 0.9), (100, 0.5), (17, 0.31)]:
        t = O.top_p_count(np.full(N, 0.37), rho)
        assert t == math.ceil(Fraction(rho).limit_denominator(1000) * N)
    s = np.zeros((1, 256))
    t, b, kh, r, sel = O.hybrid_select(s, np.array([5]), 0.9, 0.0)
    assert t[0] == 231 and r[0] == 231
    np.testing.assert_array_equal(sel[0], np.arange(231))


def test_top_p_limits():
    s = np.array([0.1, 3.0, 3.0, -1.0, 2.0])
    assert O.top_p_count(s, 1e-12) == 1
    assert O.key_order(s)[0] == 1                  # equal logits: lower index first
    assert O.top_p_count(s, 1.0) == 5


def _top_p_brute(s, rho):
    # t = 1 + #{positions whose inclusive prefix mass < rho}, prefix by (s desc, j asc)
    p = np.exp(s - s.max())
    p /= p.sum()
    N = len(s)
    cnt = 0
    for j in range(N):
        before = [(s[i] > s[j]) or (s[i] == s[j] and i <= j) for i in range(N)]
        if math.fsum(p[before]) < rho:
            cnt += 1
    return min(cnt + 1, N)


def test_top_p_matches_sort_free_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(30):
        N = int(rng.integers(2, 40))
        s = np.round(rng.standard_normal(N) * 2, 1)   # rounding makes ties
        rho = float(rng.uniform(0.05, 0.99))
        assert O.top_p_count(s, rho) == _top_p_brute(s, rho)


def test_golden_hand_examples():
    with open(os.path.join(GOLDEN, "select_worked_example.json")) as f:
        doc = json.load(f)
    for ex in doc["examples"]:
        s = np.log(np.array(ex["weights"], dtype=np.float64))
        n = np.array(ex["n"])
        t, b, kh, r, sel = O.hybrid_select(s, n, ex["rho"], ex["alpha"])
        assert t.tolist() == ex["t"]
        assert b.tolist() == ex["b"]
        assert kh == ex["k_head"]
        assert r.tolist() == ex["r"]
        assert [x.tolist() for x in sel] == ex["sel"]


# --- k_head (Eq. (9)) and r_c (Eq. (10)) -------------------------------------

def test_k_head_examples_and_bounds():
    assert O.k_head_of([3, 1], [2, 7]) == 4          # 13/4 -> 4
    assert O.k_head_of([2, 2], [3, 5]) == 4          # exactly 4
    assert O.k_head_of([1, 0, 5], [100, 1, 1]) == 18  # 105/6 = 17.5 -> 18
    rng = np.random.default_rng(8)
    for _ in range(200):
        n = rng.integers(0, 50, 20)
        n[0] += 1
        b = rng.integers(1, 10000, 20)
        kh = O.k_head_of(n, b)
        mean = Fraction(int((n * b).sum()), int(n.sum()))
        assert kh - 1 < mean <= kh
        assert b[n > 0].min() <= kh <= b[n > 0].max()


def test_selection_invariants_and_nesting():
    rng = np.random.default_rng(9)
    Cq, N = 6, 200
    s = rng.standard_normal((Cq, N)) * 1.5
    s[:, 50:60] = s[:, 50:51]                        # a tie group
    n = np.array([10, 0, 40, 3, 70, 77])
    prev = None
    for rho in (0.5, 0.7, 0.9, 0.95):
        t, b, kh, r, sel = O.hybrid_select(s, n, rho, 0.05)
        assert np.all(b >= t) and np.all(b >= math.ceil(0.05 * N))
        assert r[1] == 0 and len(sel[1]) == 0
        for c in range(Cq):
            if n[c]:
                assert r[c] == max(b[c], kh) and len(sel[c]) == r[c]
                assert np.all(np.diff(sel[c]) > 0)
                # selected keys score at least as high as every key left out
                out = np.setdiff1d(np.arange(N), sel[c])
                if len(out):
                    assert s[c, sel[c]].min() >= s[c, out].max()
        if prev is not None:
            for c in range(Cq):
                assert set(prev[c]).issubset(set(sel[c]))
        prev = sel


# --- attention ----------------------------------------------------------------

def test_rho_one_is_dense_attention():
    rng = np.random.default_rng(10)
    N, d, Cq = 90, 64, 4
    q, k, v = rng.standard_normal((3, N, d))
    labels = rng.integers(0, Cq, N)
    sel = [np.arange(N)] * Cq
    out = O.sparse_attention(q, k, v, labels, sel)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_single_key_gives_that_value_and_convexity():
    rng = np.random.default_rng(11)
    N, d = 40, 64
    q, k, v = rng.standard_normal((3, N, d))
    labels = np.arange(N) % 3
    out = O.sparse_attention(q, k, v, labels, [np.array([7]), np.array([2, 9, 30]), np.array([5])])
    np.testing.assert_array_equal(out[labels == 0], np.broadcast_to(v[7], out[labels == 0].shape))
    sub = v[[2, 9, 30]]
    o1 = out[labels == 1]
    assert np.all(o1 <= sub.max(0) + 1e-12) and np.all(o1 >= sub.min(0) - 1e-12)


def test_tiny_end_to_end_invariants():
    w = workloads.CONFIGS["tiny"]
    q, k, v = workloads.generate(w)
    for bh in range(w.BH):
        r = O.workload_head(w, bh, q[bh], k[bh], v[bh])
        n = r["n"]
        assert n.sum() == w.N and r["k_head"] == O.k_head_of(n, r["b"])
        assert np.all(r["t"] >= 1) and np.all(r["r"] <= w.N)
        assert sorted(r["perm_q"].tolist()) == list(range(w.N))
        assert r["q_off"][-1] == w.N
        # rho = 1 on the same clustering is dense attention
        d = O.workload_head(w, bh, q[bh], k[bh], v[bh], rho=1.0)
        logit = d["q_rope"] @ d["k_rope"].T / 8.0
        p = np.exp(logit - logit.max(1, keepdims=True))
        dense = (p @ v[bh]) / p.sum(1, keepdims=True)
        np.testing.assert_allclose(d["out"], dense, atol=1e-12)


# --- queries grouped by cluster (the attention work order) ---------------------

def test_cluster_permutation_hand_built_example():
    """Labels worked by hand: members of each cluster listed in ascending token
    order, clusters in ascending label order, empty clusters give equal offsets,
    and the offsets start at 0 and end at N."""
    labels = np.array([2, 0, 2, 3, 0, 2, 0, 3, 2, 0])
    perm, off = O.cluster_permutation(labels, 5)
    #           cluster 0       cluster 2        cluster 3   (1 and 4 empty)
    assert perm.tolist() == [1, 4, 6, 9, 0, 2, 5, 8, 3, 7]
    assert off.tolist() == [0, 4, 4, 8, 10, 10]


def test_cluster_permutation_is_stable_inside_each_cluster():
    """Against a brute-force grouping: for every cluster c the slice
    perm[off[c]:off[c+1]] is exactly the ascending list of tokens with label c."""
    rng = np.random.default_rng(12)
    for Cq, N in ((1, 7), (5, 64), (40, 33)):
        labels = rng.integers(0, Cq, N)
        perm, off = O.cluster_permutation(labels, Cq)
        assert len(off) == Cq + 1 and off[0] == 0 and off[-1] == N
        for c in range(Cq):
            assert perm[off[c]:off[c + 1]].tolist() == [i for i in range(N) if labels[i] == c]


def test_dense_head_is_softmax_attention_over_all_keys():
    """The dense-prefix oracle: RoPE'd rows (the same rounding as the sparse
    path) and full softmax attention, against torch's fp64 attention on those
    rows, and equal to the sparse path at rho = 1 (every key kept)."""
    w = workloads.small("dn", 3, 4, 5, 64, (16, 24, 24), "bf16", 4, 5, H=1, iters=2)
    q, k, v = workloads.generate(w)
    d = O.dense_head(q[0], k[0], v[0], grid=(w.T, w.Hg, w.Wg), split=w.split, dtype=w.dtype)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(d["q_rope"])[None], torch.from_numpy(d["k_rope"])[None], torch.from_numpy(v[0])[None])
    np.testing.assert_allclose(d["out"], ref[0].numpy(), rtol=1e-12, atol=1e-12)
    full = O.workload_head(w, 0, q[0], k[0], v[0], rho=1.0)
    np.testing.assert_array_equal(full["q_rope"], d["q_rope"])
    np.testing.assert_allclose(full["out"], d["out"], rtol=0, atol=1e-13)


# --- the full-dimensional key codebook (the cluster-level ablation proxy) ---

def test_full_dim_proxy_is_exact_logit_when_every_key_is_its_own_centroid():
    """Check (a) for the one-codebook proxy: with Cq = Cm = N every query and
    key is its own centroid, so P[c, z_j] / sqrt(d) is the exact logit."""
    w = workloads.small("fa", 2, 3, 4, 64, (16, 24, 24), "f32", 24, 24, H=1, iters=3)
    q, k, v = workloads.generate(w)
    r = O.workload_head(w, 0, q[0], k[0], v[0], full_dim_keys=True)
    np.testing.assert_array_equal(np.sort(r["q_labels"]), np.arange(24))
    np.testing.assert_array_equal(np.sort(r["k_codes"][:, 0]), np.arange(24))
    assert not r["k_codes"][:, 1:].any() and not r["lut"][1:].any()
    np.testing.assert_array_equal(r["k_centroids"][r["k_codes"][:, 0]], r["k_rope"])
    exact = r["q_rope"] @ r["k_rope"].T / 8.0
    np.testing.assert_allclose(r["scores"][r["q_labels"]], exact, rtol=1e-12, atol=1e-12)


def test_full_dim_lut_is_the_inner_product_with_the_key_centroid():
    """The one-term table: s[c, j] = <qbar_c, mu_{z_j}> / sqrt(d) computed
    directly, and the key codebook is a k-means of whole key vectors (every
    key nearest its own centroid over all d channels)."""
    w = workloads.small("fb", 3, 4, 5, 128, (44, 42, 42), "bf16", 5, 7, H=1, iters=3)
    q, k, v = workloads.generate(w)
    r = O.workload_head(w, 0, q[0], k[0], v[0], full_dim_keys=True)
    mu = r["k_centroids"][r["k_codes"][:, 0]]
    direct = r["q_centroids"] @ mu.T / np.sqrt(128)
    np.testing.assert_allclose(r["scores"], direct, rtol=1e-12, atol=1e-12)
    Mr = O.round_bf16(r["k_centroids"])
    dist = ((r["k_rope"][:, None, :] - Mr[None]) ** 2).sum(2)
    np.testing.assert_array_equal(r["k_codes"][:, 0], np.argmin(dist, 1))
