"""SCOPE oracle: a plain, slow fp64 CPU implementation of the sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module.  It shares no code
with the HIP library (no kernels, headers, helpers or tables) and never takes
an input produced by it.

Method source: "SCOPE: Subspace Clustering with Online Per-Head Top-K
Estimation for Sparse Video Attention" (arXiv 2608.12780).  The abstract
(aipentium.com and mlsanity.com pages) fixes the pipeline; the pith.science
review page of 2608.12780 quotes the equations: Eq. (3) per-subspace k-means,
Eq. (6) the proxy logit, Eq. (7)-(10) Top-p, base count, k_head and final
count, Eq. (27) the product-code identity, and the hyper-parameters
(Cq = 300, CT = CH = CW = 333, alpha = 0.1).  Where the pages are silent the
readings below are used; each one is listed with its reason in the design
notes of the repository.

Precision: everything is fp64.  Where the GPU path feeds bf16 operands to a
matrix core, the same quantity is rounded to bf16 (round to nearest even,
a single rounding from the exact value) at the same point, then used in fp64:
post-RoPE Q/K and the centroids used for assignment.  RoPE output and the
centroid means are rounded to the run's storage type (bf16 or fp32).

Parity pins: every function here is pinned by tests under tests/ against
closed forms, invariants, brute force or an independent library routine
(see tests/test_oracle_*.py).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even (one rounding).

    bf16 keeps 8 significant bits: in the binade [2^(e-1), 2^e) the spacing is
    2^(e-8); below the smallest normal (2^-126) the spacing is 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(x[nz] / q) * q            # np.round: half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Counter-based random numbers for k-means++ (SplitMix64, Steele/Lea/Flood 2014)
# ---------------------------------------------------------------------------

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, i: int) -> int:
    """Output number i (0-based) of the SplitMix64 generator seeded with `seed`."""
    z = (seed + (i + 1) * _GAMMA) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def seeding_draw(seed: int, bh: int, clustering: int, step: int):
    """53-bit draw for step `step` of clustering `clustering` (0=Q, 1=T, 2=H, 3=W) of head bh.

    Returns (k, u) with k in [0, 2^53) and u = k / 2^53 in [0, 1).
    """
    i = ((bh * 4 + clustering) << 20) + step
    k = splitmix64(seed, i) >> 11
    return k, k * 2.0 ** -53


# ---------------------------------------------------------------------------
# Stage 1: 3D RoPE
# ---------------------------------------------------------------------------

def token_positions(T: int, Hg: int, Wg: int) -> np.ndarray:
    """[N, 3] (t, h, w) of token n = (t*Hg + h)*Wg + w (reading: row-major, t slowest, origin 0)."""
    n = np.arange(T * Hg * Wg)
    return np.stack([n // (Hg * Wg), (n // Wg) % Hg, n % Wg], axis=1)


def rope_3d(x: np.ndarray, grid, split, base: float = 10000.0) -> np.ndarray:
    """3D rotary embedding of one head, x: [N, d] fp64, returned in fp64 (unrounded).

    The channels are the concatenation [T | H | W] of the three 3D-RoPE
    channel ranges (temporal, height, width), which are the key subspaces
    of SCOPE (core discovery, pith.science page).  Inside range m (offset o, width d_m) channel pairs
    (o+2i, o+2i+1) rotate by angle p_m * base^(-2i/d_m), p_m being the
    token's t, h or w index (RoFormer's interleaved-pair form, applied per
    range; reading, the pages fix only the split).
    """
    pos = token_positions(*grid)
    out = np.array(x, dtype=np.float64, copy=True)
    off = 0
    for m, dm in enumerate(split):
        i = np.arange(dm // 2)
        theta = base ** (-2.0 * i / dm)
        ang = pos[:, m][:, None] * theta[None, :]
        c, s = np.cos(ang), np.sin(ang)
        x0 = x[:, off + 2 * i]
        x1 = x[:, off + 2 * i + 1]
        out[:, off + 2 * i] = x0 * c - x1 * s
        out[:, off + 2 * i + 1] = x0 * s + x1 * c
        off += dm
    return out


# ---------------------------------------------------------------------------
# Stage 2: k-means (Eq. (3)): seeded k-means++ then Lloyd iterations
# ---------------------------------------------------------------------------

def sq_dist_to_point(X: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Squared Euclidean distance of every row of X to c, in difference form."""
    diff = X - c[None, :]
    return np.sum(diff * diff, axis=1)


def kmeanspp_seeds(X: np.ndarray, C: int, seed: int, bh: int, clustering: int) -> List[int]:
    """Seeded k-means++ (Arthur and Vassilvitskii 2007): indices of the C initial centres.

    Centre 0 is floor(u_0 * N) (exact integer arithmetic on the 53-bit draw).
    Centre s is the smallest i with cumsum(D^2)[i] > u_s * sum(D^2), D^2 being
    the squared distance to the nearest centre chosen so far.  If every D^2 is
    zero the lowest-index point not chosen yet is taken; if rounding leaves no
    i above the target, the last point with D^2 > 0 is taken.
    """
    N = X.shape[0]
    k0, _ = seeding_draw(seed, bh, clustering, 0)
    first = (k0 * N) >> 53
    chosen = [first]
    D2 = sq_dist_to_point(X, X[first])
    for s in range(1, C):
        cum = np.cumsum(D2)
        total = cum[-1]
        if total == 0.0:
            taken = set(chosen)
            i = next(j for j in range(N) if j not in taken)
        else:
            _, u = seeding_draw(seed, bh, clustering, s)
            above = np.nonzero(cum > u * total)[0]
            i = int(above[0]) if len(above) else int(np.nonzero(D2 > 0)[0][-1])
        chosen.append(int(i))
        D2 = np.minimum(D2, sq_dist_to_point(X, X[i]))
    return chosen


def assign(X: np.ndarray, M: np.ndarray, chunk: int = 512) -> np.ndarray:
    """argmin_c ||x - M_c||^2 for every row x (difference form, ties to the lowest c)."""
    N = X.shape[0]
    labels = np.empty(N, dtype=np.int64)
    for a in range(0, N, chunk):
        diff = X[a:a + chunk, None, :] - M[None, :, :]
        labels[a:a + chunk] = np.argmin(np.sum(diff * diff, axis=2), axis=1)
    return labels


def centroid_means(X: np.ndarray, labels: np.ndarray, M_prev: np.ndarray) -> np.ndarray:
    """Per-cluster mean rounded to fp32: exact sum (math.fsum) / n_c; empty clusters keep M_prev."""
    C, dm = M_prev.shape
    M = np.array(M_prev, dtype=np.float64, copy=True)
    order = np.argsort(labels, kind="stable")
    Xs = X[order]
    bounds = np.searchsorted(labels[order], np.arange(C + 1))
    for c in range(C):
        a, b = bounds[c], bounds[c + 1]
        if b == a:
            continue
        M[c] = [math.fsum(Xs[a:b, ch]) / (b - a) for ch in range(dm)]
    return round_f32(M)


def kmeans(X: np.ndarray, C: int, iters: int, dtype: str, seed: int, bh: int, clustering: int,
           init: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """k-means of the rows of X: k-means++ (or given init), then `iters` Lloyd rounds.

    labels_0 = assign(init); for it = 1..iters: M = mean(labels); labels = assign(M).
    The returned (centroids, labels) are consistent: labels = assign(centroids).
    The distance uses M rounded to bf16 in bf16 runs (the matrix-core operand).
    """
    rnd = round_bf16 if dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float64))
    if init is None:
        seeds = kmeanspp_seeds(X, C, seed, bh, clustering)
        M = X[seeds].astype(np.float64)
    else:
        seeds = None
        M = np.asarray(init, dtype=np.float64)
    labels = assign(X, rnd(M))
    for _ in range(iters):
        M = centroid_means(X, labels, M)
        labels = assign(X, rnd(M))
    return {"centroids": M, "labels": labels, "seeds": seeds}


# ---------------------------------------------------------------------------
# Stages 3-4: lookup tables and proxy logits (Eq. (6))
# ---------------------------------------------------------------------------

def subspace_offsets(split) -> List[int]:
    return [0, split[0], split[0] + split[1]]


def lookup_tables(q_centroids: np.ndarray, k_centroids: np.ndarray, split) -> np.ndarray:
    """P^m[c, z] = <qbar_c restricted to range m, mu^m_z>; returns [3, Cq, Cm].

    k_centroids is [Cm, d] with row z = (mu^T_z | mu^H_z | mu^W_z).
    """
    offs = subspace_offsets(split)
    return np.stack([
        q_centroids[:, o:o + dm] @ k_centroids[:, o:o + dm].T for o, dm in zip(offs, split)
    ])


def lookup_table_full(q_centroids: np.ndarray, k_centroids: np.ndarray) -> np.ndarray:
    """The cluster-level proxy of the ablation that clusters the keys in all d
    channels at once (one codebook instead of the T/H/W product code):
    P[c, z] = <qbar_c, mu_z> over every channel; [Cq, Cm]."""
    return q_centroids @ k_centroids.T


def proxy_logits(P: np.ndarray, codes: np.ndarray, d: int) -> np.ndarray:
    """Eq. (6): s[c, j] = (P^T[c, zT_j] + P^H[c, zH_j] + P^W[c, zW_j]) / sqrt(d); [Cq, N]."""
    return (P[0][:, codes[:, 0]] + P[1][:, codes[:, 1]] + P[2][:, codes[:, 2]]) / np.sqrt(d)


# ---------------------------------------------------------------------------
# Stage 5: hybrid selection (Eq. (7)-(10))
# ---------------------------------------------------------------------------

def key_order(s_row: np.ndarray) -> np.ndarray:
    """Keys by proxy logit descending, equal logits by index ascending (reading)."""
    return np.lexsort((np.arange(len(s_row)), -s_row))


def top_p_count(s_row: np.ndarray, rho: float) -> int:
    """Eq. (7): smallest t whose first t keys (in key_order) hold softmax mass >= rho."""
    N = len(s_row)
    if rho >= 1.0:
        return N
    p = np.exp(s_row - s_row.max())
    p /= p.sum()
    cum = np.cumsum(p[key_order(s_row)])
    hit = np.nonzero(cum >= rho)[0]
    return int(hit[0]) + 1 if len(hit) else N


def k_head_of(n: Sequence[int], b: Sequence[int]) -> int:
    """Eq. (9): ceil(sum_c n_c b_c / sum_c n_c), exact integer arithmetic."""
    num = sum(int(x) * int(y) for x, y in zip(n, b))
    den = sum(int(x) for x in n)
    return -((-num) // den)


def hybrid_select(s: np.ndarray, n: np.ndarray, rho: float, alpha: float, online_khead: bool = True):
    """Top-p counts t, base counts b (Eq. 8), k_head (Eq. 9), final counts r (Eq. 10), key sets.

    b_c = max(t_c, ceil(alpha*N)) (reading: alpha is the fixed Top-k floor as a
    fraction of N); r_c = max(b_c, k_head) for non-empty clusters, 0 for empty
    ones; the keys of cluster c are its first r_c keys in key_order, returned
    in ascending index order.  online_khead=False: r_c = b_c (the hybrid
    Top-p / fixed Top-k selection the method extends, as in the SCOPE
    paper's Fig. 7 ablation); k_head is still returned.
    """
    Cq, N = s.shape
    floor = math.ceil(alpha * N)
    t = np.array([top_p_count(s[c], rho) for c in range(Cq)], dtype=np.int64)
    b = np.maximum(t, floor)
    kh = k_head_of(n, b)
    # without the online extension (the Fig. 7 ablation): the base counts alone
    r = np.where(n > 0, np.maximum(b, kh) if online_khead else b, 0)
    sel = [np.sort(key_order(s[c])[: r[c]]) for c in range(Cq)]
    return t, b, kh, r, sel


# ---------------------------------------------------------------------------
# Stage 6: exact attention over the selected original keys and values
# ---------------------------------------------------------------------------

def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_labels: np.ndarray,
                     sel: Sequence[np.ndarray], only_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """o_i = softmax_j in S_c(i) (<q_i, k_j>/sqrt(d)) v_j, fp64.

    only_rows: compute just these query rows (the others stay zero).
    """
    N, d = q.shape
    out = np.zeros((N, v.shape[1]), dtype=np.float64)
    wanted = None if only_rows is None else np.zeros(N, dtype=bool)
    if wanted is not None:
        wanted[np.asarray(only_rows)] = True
    for c, keys in enumerate(sel):
        rows = np.nonzero((q_labels == c) & (True if wanted is None else wanted))[0]
        if len(rows) == 0:
            continue
        logit = (q[rows] @ k[keys].T) / np.sqrt(d)
        logit -= logit.max(axis=1, keepdims=True)
        w = np.exp(logit)
        out[rows] = (w @ v[keys]) / w.sum(axis=1, keepdims=True)
    return out


def dense_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, grid, split, dtype: str,
               rope_base: float = 10000.0) -> Dict[str, np.ndarray]:
    """Dense attention of one head (the dense prefix of the SCOPE paper's
    schedule, referee report of the pith.science page, major comment 3: the
    first layer at every step and the first denoising steps skip the sparse
    selection): RoPE, then o_i = softmax_j over all N keys (<q'_i, k'_j>/sqrt(d)) v_j."""
    qr = round_storage(rope_3d(q, grid, split, rope_base), dtype)
    kr = round_storage(rope_3d(k, grid, split, rope_base), dtype)
    N = q.shape[0]
    out = sparse_attention(qr, kr, v, np.zeros(N, dtype=np.int64), [np.arange(N)])
    return {"q_rope": qr, "k_rope": kr, "out": out}


def cluster_permutation(q_labels: np.ndarray, Cq: int):
    """Tokens grouped by cluster, ascending index inside a cluster; offsets [Cq+1]."""
    perm = np.argsort(q_labels, kind="stable")
    off = np.concatenate([[0], np.cumsum(np.bincount(q_labels, minlength=Cq))])
    return perm, off


# ---------------------------------------------------------------------------
# One head, end to end
# ---------------------------------------------------------------------------

def scope_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, grid, split, dtype: str,
               Cq: int, Cm: int, iters: int, rho: float, alpha: float = 0.0,
               seed: int = 0, bh: int = 0, rope_base: float = 10000.0,
               init_q: Optional[np.ndarray] = None, init_k: Optional[np.ndarray] = None,
               with_attention: bool = True, channel_perm: Optional[np.ndarray] = None,
               online_khead: bool = True, full_dim_keys: bool = False) -> Dict[str, object]:
    """The whole path for one head; inputs are fp64 arrays holding `dtype` values.

    init_q [Cq, d] / init_k [Cm, d] replace k-means++ when given.

    channel_perm (the partition ablation of the SCOPE paper's experiments,
    Table 3: a random channel partition in place of the 3D-RoPE one): the
    clustering, centroids, LUT and proxy use the RoPE'd rows with their
    channels reordered, row[:, channel_perm], so key subspace m is the m-th
    run of split[m] reordered channels; attention uses the rows as they are.

    full_dim_keys (the other ablation of the pages' forward implications: a
    cluster-level proxy over whole key vectors, as in SVG2, instead of the
    subspace partition): the keys form one k-means clustering of Cm centroids
    over all d channels (k-means++ draws of clustering 1), the proxy is
    P[c, z_j] / sqrt(d) with the one-term table of lookup_table_full; the
    codes of the two other terms are 0 and their tables are zero, so the
    same three-term Eq. (6) sum gives that value exactly.
    """
    N, d = q.shape
    qr = round_storage(rope_3d(q, grid, split, rope_base), dtype)
    kr = round_storage(rope_3d(k, grid, split, rope_base), dtype)
    qc, kc = qr, kr
    if channel_perm is not None:
        channel_perm = np.asarray(channel_perm)
        assert sorted(channel_perm.tolist()) == list(range(d))
        qc, kc = qr[:, channel_perm], kr[:, channel_perm]

    kq = kmeans(qc, Cq, iters, dtype, seed, bh, 0, init_q)
    offs = subspace_offsets(split)
    k_cent = np.zeros((Cm, d))
    codes = np.zeros((N, 3), dtype=np.int64)
    k_seeds = []
    if full_dim_keys:
        assert channel_perm is None
        km = kmeans(kc, Cm, iters, dtype, seed, bh, 1, init_k)
        k_cent = km["centroids"]
        codes[:, 0] = km["labels"]
        k_seeds = [km["seeds"], None, None]
        P = np.stack([lookup_table_full(kq["centroids"], k_cent), np.zeros((Cq, Cm)), np.zeros((Cq, Cm))])
    else:
        for m, (o, dm) in enumerate(zip(offs, split)):
            init = None if init_k is None else init_k[:, o:o + dm]
            km = kmeans(kc[:, o:o + dm], Cm, iters, dtype, seed, bh, 1 + m, init)
            k_cent[:, o:o + dm] = km["centroids"]
            codes[:, m] = km["labels"]
            k_seeds.append(km["seeds"])
        P = lookup_tables(kq["centroids"], k_cent, split)
    s = proxy_logits(P, codes, d)
    n = np.bincount(kq["labels"], minlength=Cq)
    t, b, kh, r, sel = hybrid_select(s, n, rho, alpha, online_khead)
    perm, q_off = cluster_permutation(kq["labels"], Cq)
    res = {
        "q_rope": qr, "k_rope": kr,
        "q_seeds": kq["seeds"], "k_seeds": k_seeds,
        "q_centroids": kq["centroids"], "q_labels": kq["labels"],
        "k_centroids": k_cent, "k_codes": codes,
        "lut": P, "scores": s, "n": n,
        "t": t, "b": b, "k_head": kh, "r": r, "sel": sel,
        "perm_q": perm, "q_off": q_off,
    }
    if with_attention:
        res["out"] = sparse_attention(qr, kr, v, kq["labels"], sel)
    return res


def workload_head(w, bh: int, q, k, v, rho: Optional[float] = None, **kw) -> Dict[str, object]:
    """scope_head with the parameters of a workloads.Workload."""
    return scope_head(q, k, v, grid=(w.T, w.Hg, w.Wg), split=w.split, dtype=w.dtype,
                      Cq=w.Cq, Cm=w.Cm, iters=w.iters, rho=w.rho if rho is None else rho,
                      alpha=w.alpha, seed=w.kmeans_seed, bh=bh, rope_base=w.rope_base, **kw)
