"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare its outputs with the oracle under the tolerance rules.

Comparison rules (numbers from the measurement definition of the path):
  * RoPE output: at most 1 bf16 ulp (1e-6 relative in fp32) per element;
  * k-means++ seeds, assignments, codes: identical, except a point whose two
    nearest centroids are within 1e-6 * (||x||^2 + max ||mu~||^2) (a near tie);
  * centroids: relative error <= 1e-6;
  * t_c: identical, or the oracle's fp64 prefix mass satisfies
    cum(t_c) >= rho (1 - 1e-6) and cum(t_c - 1) < rho (1 + 1e-6);
  * k_head, r_c: identical when every t_c matches (then also S_c, except keys
    at the boundary whose logit gap is < 1e-6 * sum_m |P^m| / sqrt(d));
  * attention: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 max-abs <= 1e-4.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_attention_video_rope_amd as sav
import workloads
from oracle import scope_oracle as O

TOL_BF16_MAX, TOL_BF16_MEAN, TOL_F32 = 2e-2, 2e-3, 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x).reshape(-1))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def run_gpu(w, rho=None, init_q=None, init_k=None, iters=None, inputs=None, debug=True, **kw):
    """Runs plan + attend on the GPU; returns a dict of numpy arrays (per head leading dim)."""
    q, k, v = inputs if inputs is not None else workloads.generate(w)
    extra = dict(kw)
    if iters is not None:
        extra["iters"] = iters
    if init_q is not None:
        extra["init_centroids"] = True
    p = sav.params_for(w, rho=rho, **extra)
    pl = sav.Plan(p, debug=debug)
    if init_q is not None:
        pl.q_centroids.copy_(torch.from_numpy(np.ascontiguousarray(init_q, dtype=np.float32).reshape(-1)).cuda())
        pl.k_centroids.copy_(torch.from_numpy(np.ascontiguousarray(init_k, dtype=np.float32).reshape(-1)).cuda())
    qd, kd, vd = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    qr, kr, _ = sav.plan(p, qd, kd, pl)
    out = sav.attend(p, pl, qr, kr, vd)
    torch.cuda.synchronize()
    BH, N, Cq, Cm, d = w.BH, w.N, w.Cq, w.Cm, w.d
    r = {
        "q_rope": to_np(qr).reshape(BH, N, d), "k_rope": to_np(kr).reshape(BH, N, d),
        "out": to_np(out).reshape(BH, N, d),
        "perm_q": to_np(pl.perm_q).reshape(BH, N), "q_off": to_np(pl.q_off).reshape(BH, Cq + 1),
        "t": to_np(pl.counts_t).reshape(BH, Cq), "b": to_np(pl.counts_b).reshape(BH, Cq),
        "r": to_np(pl.counts_r).reshape(BH, Cq), "k_head": to_np(pl.k_head),
        "sel_off": to_np(pl.sel_off), "status": to_np(pl.status),
    }
    total = int(r["sel_off"][-1])
    r["sel_idx"] = to_np(pl.sel_idx[:total])
    if debug:
        r.update({
            "q_centroids": to_np(pl.q_centroids).reshape(BH, Cq, d),
            "k_centroids": to_np(pl.k_centroids).reshape(BH, Cm, d),
            "q_labels": to_np(pl.q_labels).reshape(BH, N),
            "k_codes": to_np(pl.k_codes).astype(np.uint16).astype(np.int64).reshape(BH, N, 4)[:, :, :3],
            "seeds": to_np(pl.seeds).reshape(BH, 4, max(Cq, Cm)),
            "lut": to_np(pl.lut).reshape(BH, Cq, 3, Cm),
        })
    return r


def gpu_sel(r, bh, Cq):
    off = r["sel_off"]
    return [r["sel_idx"][off[bh * Cq + c]:off[bh * Cq + c + 1]] for c in range(Cq)]


def ulp_bf16(x):
    ax = np.abs(x)
    _, e = np.frexp(np.where(ax > 0, ax, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def assert_rope(got, want, dtype):
    if dtype == "bf16":
        diff = np.abs(got - want)
        assert np.all(diff <= ulp_bf16(want) * 1.0001), f"RoPE: {np.sum(diff > 0)} elements beyond 1 ulp"
        return int(np.sum(diff > 0))
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-30)
    return int(np.sum(got != want))


def labels_match_or_near_tie(got, want, X, M, dtype):
    """Identical labels except at near ties (relative gap < 1e-6)."""
    bad = np.nonzero(got != want)[0]
    if len(bad) == 0:
        return 0
    Mr = O.round_bf16(M) if dtype == "bf16" else M
    scale = np.max(np.sum(Mr * Mr, axis=1))
    for p in bad:
        dist = np.sum((X[p][None, :] - Mr) ** 2, axis=1)
        gap = abs(dist[got[p]] - dist[want[p]])
        assert gap <= 1e-6 * (np.sum(X[p] ** 2) + scale), f"point {p}: label {got[p]} vs {want[p]}, gap {gap}"
    return len(bad)


def assert_attention(got, want, dtype, what=""):
    err = np.abs(got - want)
    if dtype == "bf16":
        assert err.max() <= TOL_BF16_MAX and err.mean() <= TOL_BF16_MEAN, \
            f"{what}: max {err.max():.3e} mean {err.mean():.3e}"
    else:
        assert err.max() <= TOL_F32, f"{what}: max {err.max():.3e}"
    return float(err.max()), float(err.mean())
