"""Pins of the oracle's seeded k-means++ and Lloyd iterations (Eq. (3)), CPU only."""
import itertools
from fractions import Fraction

import numpy as np

from oracle import scope_oracle as O


def test_first_seed_is_floor_u0_times_n():
    X = np.random.default_rng(0).standard_normal((37, 4))
    for seed in range(5):
        s = O.kmeanspp_seeds(X, 3, seed, 1, 2)
        _, u0 = O.seeding_draw(seed, 1, 2, 0)
        assert s[0] == int(np.floor(Fraction(u0) * 37))


def test_kmeanspp_all_points_when_c_equals_n():
    X = np.random.default_rng(1).standard_normal((25, 3))
    s = O.kmeanspp_seeds(X, 25, 4, 0, 0)
    assert sorted(s) == list(range(25))


def test_kmeanspp_duplicates_take_lowest_unchosen():
    X = np.ones((6, 2))
    s = O.kmeanspp_seeds(X, 4, 9, 0, 0)
    rest = [j for j in range(6) if j != s[0]][:3]
    assert s[1:] == rest


def test_kmeanspp_second_centre_follows_d_squared():
    # points 0, 1, 3 on a line, first centre at point 0: D^2 = [0, 1, 9]
    # -> P(second = 1) = 0.1, P(second = 2) = 0.9 (0.25/0.75 if D were used)
    X = np.array([[0.0], [1.0], [3.0]])
    picks = []
    for seed in range(20000):
        if O.seeding_draw(seed, 0, 0, 0)[0] * 3 >> 53 != 0:
            continue
        picks.append(O.kmeanspp_seeds(X, 2, seed, 0, 0)[1])
        if len(picks) == 3000:
            break
    frac = np.mean(np.array(picks) == 2)
    assert abs(frac - 0.9) < 4 * np.sqrt(0.09 / len(picks))


def test_assign_ties_to_lowest_index_and_difference_form():
    X = np.array([[0.0, 0.0], [2.0, 0.0], [1.0, 0.0]])
    M = np.array([[2.0, 0.0], [0.0, 0.0], [0.0, 0.0]])
    assert O.assign(X, M).tolist() == [1, 0, 0]


def test_centroid_means_exact_then_fp32():
    rng = np.random.default_rng(5)
    X = np.concatenate([rng.standard_normal((40, 3)) * 1e8, rng.standard_normal((40, 3))])
    X = X.astype(np.float32).astype(np.float64)
    labels = rng.integers(0, 4, 80)
    labels[labels == 3] = 0                      # cluster 3 empty
    prev = np.full((4, 3), 0.25)
    M = O.centroid_means(X, labels, prev)
    for c in range(3):
        rows = X[labels == c]
        for ch in range(3):
            exact = sum(Fraction(v) for v in rows[:, ch]) / len(rows)
            want = np.float32(float(exact))     # Fraction -> float is correctly rounded
            assert M[c, ch] == want or abs(M[c, ch] - float(exact)) <= abs(float(want) - float(exact))
    np.testing.assert_array_equal(M[3], np.float32(0.25))


def _sse(X, labels):
    return sum(((X[labels == c] - X[labels == c].mean(0)) ** 2).sum() for c in np.unique(labels))


def test_lloyd_recovers_brute_force_optimum_on_separated_data():
    rng = np.random.default_rng(6)
    X = np.concatenate([rng.normal(0, 0.1, (4, 2)), rng.normal(5, 0.1, (4, 2))])
    res = O.kmeans(X, 2, 10, "f32", seed=3, bh=0, clustering=0)
    best = min(_sse(X, np.array(p)) for p in itertools.product([0, 1], repeat=8) if len(set(p)) == 2)
    assert abs(_sse(X, res["labels"]) - best) < 1e-9


def test_lloyd_fixed_point_and_monotone_objective():
    rng = np.random.default_rng(7)
    centres = rng.standard_normal((5, 6)) * 4
    X = (centres[rng.integers(0, 5, 300)] + 0.3 * rng.standard_normal((300, 6)))
    X = X.astype(np.float32).astype(np.float64)
    objs = []
    for it in range(0, 8):
        r = O.kmeans(X, 5, it, "f32", seed=11, bh=0, clustering=1)
        M = r["centroids"]
        objs.append(np.sum((X - M[r["labels"]]) ** 2))
    assert all(b <= a + 1e-9 for a, b in zip(objs, objs[1:]))
    r = O.kmeans(X, 5, 20, "f32", seed=11, bh=0, clustering=1)
    np.testing.assert_array_equal(O.assign(X, r["centroids"]), r["labels"])
    np.testing.assert_array_equal(O.centroid_means(X, r["labels"], r["centroids"]), r["centroids"])


def test_bf16_run_assigns_with_rounded_centroids():
    # a point exactly between a centroid and its bf16 rounding decides by the rounded value
    X = np.array([[1.0 + 2.0**-9, 0.0]])
    M = np.array([[1.0 + 2.0**-8 + 2.0**-12, 0.0], [1.0 - 2.0**-12 + 2.0**-9 - 2.0**-20, 0.0]])
    # rounded: row 0 -> 1 + 2^-7, row 1 -> 1.0; x is closer to 1.0
    r = O.kmeans(X, 2, 0, "bf16", seed=0, bh=0, clustering=0, init=M)
    assert r["labels"].tolist() == [1]
