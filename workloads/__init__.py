"""Seeded synthetic workloads for the SCOPE sparse-attention hot path.

This module only describes and generates inputs: the named configurations
(latent grid, head count, 3D-RoPE channel split, cluster counts, Top-p
threshold) and pre-RoPE Q/K plus V for one (batch, head).  It holds none of
the method's arithmetic (no RoPE, no clustering, no scoring, no selection,
no attention), so both the CPU oracle and the HIP path can take their inputs
from here without sharing any computation.

Input recipe (the pages evaluate on real video-DiT latents that are not
available; these fields stand in for them with the same shapes):

* token n <-> grid position (t, h, w) with n = (t*Hg + h)*Wg + w;
* pre-RoPE Q and K of one head are rank-R smooth fields over (t, h, w):
  R Gaussian bumps shared by Q and K, each with its own N(0, I_d)
  coefficient vector per tensor, scaled to unit RMS, plus i.i.d.
  N(0, 0.1^2) noise;
* V ~ N(0, 1);
* step s > 0 stands in for a later denoising step of the same head (for
  codebook reuse across steps): the same bumps, and every Gaussian draw of
  Q and K (coefficients and noise) replaced by cos(a) x + sin(a) z, with x
  step 0's draw, z a fresh one of step s and a = drift * s radians
  (drift = 0.05 by default), so the draws stay N(0, 1) and move by about
  5% per step; V is unchanged;
* bf16 configurations round every input element to bf16 (through fp32,
  round-to-nearest-even at each step); the values handed out are exactly
  representable in the configuration's dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

BASE_SEED = 20260813


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # selects the seed: BASE_SEED + index
    B: int
    H: int
    T: int
    Hg: int
    Wg: int
    d: int
    split: Tuple[int, int, int]   # (d_t, d_h, d_w)
    dtype: str                    # "f32" or "bf16"
    Cq: int
    Cm: int
    iters: int = 10
    rhos: Tuple[float, ...] = (0.9,)
    alpha: float = 0.0
    R: int = 8                    # number of Gaussian bumps of the smooth field
    rope_base: float = 10000.0

    @property
    def N(self) -> int:
        return self.T * self.Hg * self.Wg

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def kmeans_seed(self) -> int:
        """Seed of the k-means++ draws of this workload."""
        return BASE_SEED + self.index

    @property
    def rho(self) -> float:
        return self.rhos[0]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five configurations the measurements are defined on.
CONFIGS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 0, 1, 2, 4, 8, 8, 64, (16, 24, 24), "f32", 8, 8),
        Workload("cogvideox", 1, 1, 48, 13, 30, 45, 64, (16, 24, 24), "bf16", 100, 128),
        Workload("wan13b_480p", 2, 1, 12, 21, 30, 52, 128, (44, 42, 42), "bf16", 300, 333),
        Workload("wan14b_720p", 3, 1, 40, 21, 45, 80, 128, (44, 42, 42), "bf16", 300, 333,
                 rhos=(0.7, 0.9, 0.95)),
        Workload("hunyuan_720p", 4, 1, 24, 33, 45, 80, 128, (16, 56, 56), "bf16", 300, 333, R=16),
    ]
}


def small(name: str, T: int, Hg: int, Wg: int, d: int, split, dtype: str, Cq: int, Cm: int,
          H: int = 2, index: int = 100, **kw) -> Workload:
    """A reduced workload for parity tests (same generator, custom sizes)."""
    return Workload(name, index, 1, H, T, Hg, Wg, d, tuple(split), dtype, Cq, Cm, **kw)


def grid_positions(T: int, Hg: int, Wg: int) -> np.ndarray:
    """[N, 3] integer (t, h, w) of every token, t slowest, w fastest."""
    n = np.arange(T * Hg * Wg)
    return np.stack([n // (Hg * Wg), (n // Wg) % Hg, n % Wg], axis=1)


def _to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Input quantisation: fp64 -> fp32 (RNE) -> bf16 (RNE on the fp32 bits)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _to_bf16_values(x)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def generate_head(w: Workload, b: int, h: int, step: int = 0,
                  drift: float = 0.05) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Pre-RoPE q, k and v of head (b, h) as fp64 arrays [N, d] holding dtype values.

    step > 0: the later-step stand-in (same bumps, every Gaussian draw of Q
    and K rotated towards a fresh one by drift * step radians)."""
    seed = BASE_SEED + w.index
    N, d = w.N, w.d
    pos = grid_positions(w.T, w.Hg, w.Wg).astype(np.float64)
    extent = np.array([w.T, w.Hg, w.Wg], dtype=np.float64)

    geo = np.random.default_rng([seed, b, h, 3])
    centres = geo.uniform(0.0, 1.0, size=(w.R, 3)) * extent
    sigma = np.maximum(geo.uniform(0.1, 0.3, size=(w.R, 3)) * extent, 0.5)
    z = (pos[None, :, :] - centres[:, None, :]) / sigma[:, None, :]
    phi = np.exp(-0.5 * np.sum(z * z, axis=2))          # [R, N]

    out = []
    for tensor_id in (0, 1):
        rng = np.random.default_rng([seed, b, h, tensor_id])
        coef = rng.standard_normal((w.R, d))
        noise = rng.standard_normal((N, d))
        if step:
            a = drift * step
            fresh = np.random.default_rng([seed, b, h, tensor_id, 5, step])
            coef = np.cos(a) * coef + np.sin(a) * fresh.standard_normal((w.R, d))
            noise = np.cos(a) * noise + np.sin(a) * fresh.standard_normal((N, d))
        field = phi.T @ coef                              # [N, d], rank R over (t, h, w)
        field /= np.sqrt(np.mean(field * field))
        field += 0.1 * noise
        out.append(_cast(field, w.dtype))
    v = np.random.default_rng([seed, b, h, 2]).standard_normal((N, d))
    out.append(_cast(v, w.dtype))
    return out[0], out[1], out[2]


def generate(w: Workload, heads: Optional[list] = None, step: int = 0):
    """Stacked inputs [len(heads), N, d] for the given flat head indices bh = b*H + h."""
    if heads is None:
        heads = list(range(w.BH))
    qs, ks, vs = [], [], []
    for bh in heads:
        q, k, v = generate_head(w, bh // w.H, bh % w.H, step)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return np.stack(qs), np.stack(ks), np.stack(vs)
