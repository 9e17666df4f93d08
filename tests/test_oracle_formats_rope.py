"""Pins of the oracle's number formats, random draws and 3D RoPE (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import scope_oracle as O


# --- bf16 rounding ----------------------------------------------------------

def test_bf16_ties_to_even_closed_forms():
    one = 1.0
    assert O.round_bf16(one + 2.0**-8) == 1.0                    # tie, 1.0 is even
    assert O.round_bf16(one + 3 * 2.0**-8) == one + 2.0**-6      # tie, odd neighbour loses
    assert O.round_bf16(one + 2.0**-8 + 2.0**-40) == one + 2.0**-7
    assert O.round_bf16(-(one + 2.0**-8 + 2.0**-40)) == -(one + 2.0**-7)
    assert O.round_bf16(1.5 * 2.0**-133) == 2.0**-132            # subnormal tie
    assert O.round_bf16(2.0**-134) == 0.0                        # tie to the even zero
    assert O.round_bf16(float.fromhex("0x1.ff8p127")) == np.inf  # above max + half ulp
    assert O.round_bf16(0.0) == 0.0


def test_bf16_matches_torch_on_fp32_values():
    # torch rounds fp32 -> bf16 to nearest even; on fp32 inputs that is one rounding
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        rng.standard_normal(2000) * 1e-39])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_single_rounding_brute_force():
    # nearest of the two bracketing bf16 values, ties to the even bit pattern
    rng = np.random.default_rng(2)
    for x in rng.standard_normal(500) * 7.0:
        lo32 = np.float32(x)
        bits = int(np.array([lo32]).view(np.uint32)[0]) & 0xFFFF0000
        cands = []
        for b in (bits - 0x10000, bits, bits + 0x10000, bits + 0x20000):
            v = float(np.array([b & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0])
            cands.append((abs(v - x), (b >> 16) & 1, v))
        cands.sort()
        best = cands[0]
        if cands[1][0] == best[0] and best[1] == 1:
            best = cands[1]
        assert O.round_bf16(x) == best[2]


# --- SplitMix64 -------------------------------------------------------------

def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 seeded with 0 (Vigna's reference generator).
    assert O.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert O.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert O.splitmix64(0, 2) == 0x06C45D188009454F


def test_seeding_draw_range_and_streams():
    ks = [O.seeding_draw(7, bh, c, s)[0] for bh in range(3) for c in range(4) for s in range(50)]
    assert all(0 <= k < 2**53 for k in ks)
    assert len(set(ks)) == len(ks)
    u = np.array([O.seeding_draw(11, 0, 0, s)[1] for s in range(4000)])
    assert abs(u.mean() - 0.5) < 0.02 and u.min() >= 0.0 and u.max() < 1.0


# --- 3D RoPE ----------------------------------------------------------------

GRID = (3, 4, 5)
SPLIT = (16, 24, 24)


def _x(n=60, d=64, seed=0):
    return np.random.default_rng(seed).standard_normal((n, d))


def test_rope_identity_at_origin_and_pair_norms():
    x = _x()
    y = O.rope_3d(x, GRID, SPLIT)
    np.testing.assert_array_equal(y[0], x[0])
    nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


def test_rope_complex_form():
    x = _x()
    y = O.rope_3d(x, GRID, SPLIT, base=10000.0)
    pos = np.stack(np.unravel_index(np.arange(60), GRID), axis=1)
    off = 0
    for m, dm in enumerate(SPLIT):
        z = x[:, off:off + dm:2] + 1j * x[:, off + 1:off + dm:2]
        freq = np.exp(-np.log(10000.0) * np.arange(0, dm, 2) / dm)
        zr = z * np.exp(1j * pos[:, m:m + 1] * freq[None, :])
        np.testing.assert_allclose(y[:, off:off + dm:2], zr.real, atol=1e-12)
        np.testing.assert_allclose(y[:, off + 1:off + dm:2], zr.imag, atol=1e-12)
        off += dm


def test_rope_relative_position_property():
    # <R(p) q, R(p') k> depends only on p - p' in every subspace
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    N = int(np.prod(GRID))
    tok = lambda t, h, w: (t * GRID[1] + h) * GRID[2] + w
    X = np.zeros((N, 64))
    X[:] = q
    Y = np.zeros((N, 64))
    Y[:] = k
    rq = O.rope_3d(X, GRID, SPLIT)
    rk = O.rope_3d(Y, GRID, SPLIT)
    a = rq[tok(2, 3, 4)] @ rk[tok(1, 1, 2)]
    b = rq[tok(1, 2, 2)] @ rk[tok(0, 0, 0)]
    assert abs(a - b) < 1e-11
    c = rq[tok(2, 3, 4)] @ rk[tok(1, 1, 3)]
    assert abs(a - c) > 1e-6


def test_rope_subspaces_do_not_mix():
    # a vector living in one channel range stays in it
    x = np.zeros((60, 64))
    x[:, 16:40] = _x()[:, :24]
    y = O.rope_3d(x, GRID, SPLIT)
    assert np.all(y[:, :16] == 0) and np.all(y[:, 40:] == 0)


def test_token_positions_row_major():
    p = O.token_positions(3, 4, 5)
    assert p[0].tolist() == [0, 0, 0]
    assert p[1].tolist() == [0, 0, 1]
    assert p[5].tolist() == [0, 1, 0]
    assert p[20].tolist() == [1, 0, 0]
    assert p[59].tolist() == [2, 3, 4]
