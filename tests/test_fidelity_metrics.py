"""The proxy-fidelity measures (recall of the true top keys, softmax mass on
the selected set, Spearman correlation of the proxy with the exact logits,
error against dense attention) on cases whose answers are fixed by hand."""
import math

import numpy as np
import torch

from bench import _avg_ranks, proxy_fidelity_rows


def _case(N=40, d=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(N, d, generator=g, dtype=torch.float64) for _ in range(3))
    return q, k, v


def _own_centroid_tables(q, k):
    """Every query its own cluster, every key sub-vector its own code: the
    lookup tables then hold the exact partial products of Eq. (27)."""
    N, d = q.shape
    offs = [(0, 2), (2, 3), (5, 3)]
    lut = torch.stack([q[:, o:o + w] @ k[:, o:o + w].t() for o, w in offs], dim=1)   # [N, 3, N]
    codes = torch.arange(N).repeat(3, 1).t().contiguous()
    return lut, codes, torch.arange(N)


def _dense(q, k, v):
    return torch.softmax(q @ k.t() / math.sqrt(q.shape[1]), dim=1) @ v


def test_average_ranks():
    r = _avg_ranks(torch.tensor([3.0, 1.0, 3.0, 2.0, 3.0]))
    assert r.tolist() == [3.0, 0.0, 3.0, 1.0, 3.0]


def test_exact_proxy_and_all_keys():
    q, k, v = _case()
    lut, codes, labels = _own_centroid_tables(q, k)
    N = q.shape[0]
    rows = torch.arange(0, N, 3)
    r = proxy_fidelity_rows(q, k, v, labels, lut, codes, lambda c: torch.arange(N), _dense(q, k, v), rows)
    np.testing.assert_allclose(r["spearman"], 1.0, atol=1e-12)
    assert np.all(r["recall"] == 1.0)
    np.testing.assert_allclose(r["mass"], 1.0, atol=1e-12)
    assert r["err2"] < 1e-24 * r["ref2"]


def test_reversed_proxy_and_exact_top_sets():
    q, k, v = _case(seed=1)
    lut, codes, labels = _own_centroid_tables(q, k)
    N, d = q.shape
    lg = q @ k.t() / math.sqrt(d)
    kt = math.ceil(0.1 * N)
    top = lg.topk(kt, dim=1).indices
    rows = torch.arange(N)
    r = proxy_fidelity_rows(q, k, v, labels, -lut, codes, lambda c: top[c], _dense(q, k, v), rows)
    np.testing.assert_allclose(r["spearman"], -1.0, atol=1e-12)
    assert np.all(r["recall"] == 1.0)
    want = torch.softmax(lg, dim=1).gather(1, top).sum(1)
    np.testing.assert_allclose(r["mass"], want.numpy(), rtol=1e-12)


def test_half_recall_and_mass_of_a_hand_set():
    # 20 keys, one query with logits 19, 18, ..., 0 (key j: 19 - j) times 1/sqrt(d)
    N, d = 20, 1
    q = torch.ones(1, d, dtype=torch.float64)
    k = (19.0 - torch.arange(N, dtype=torch.float64)).view(N, d)
    v = torch.randn(N, d, dtype=torch.float64)
    lut = torch.zeros(1, 3, N, dtype=torch.float64)
    lut[0, 0] = k[:, 0]                       # proxy = exact logits
    codes = torch.stack([torch.arange(N), torch.zeros(N, dtype=torch.long), torch.zeros(N, dtype=torch.long)], 1)
    S = torch.tensor([0, 5, 6])               # top-2 keys are 0 and 1: recall 1/2
    p = torch.softmax(k[:, 0], dim=0)
    out = (p[S] @ v[S]).view(1, d) / p[S].sum()
    r = proxy_fidelity_rows(q, k, v, torch.zeros(1, dtype=torch.long), lut, codes, lambda c: S, out,
                            torch.tensor([0]))
    assert r["recall"].tolist() == [0.5]
    np.testing.assert_allclose(r["mass"], float(p[S].sum()), rtol=1e-12)
    np.testing.assert_allclose(r["spearman"], 1.0, atol=1e-12)
