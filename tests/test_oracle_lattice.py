"""Pins of the oracle's lattice steps against facts the mathematics fixes.

Nearest-point property by brute force, the E8 covering radius, kissing number
and normalised second moment (Conway & Sloane, tests/golden/e8_constants.json),
coset parity invariants, field round trips, and the one-bit saving of the
parity reduction (EntroPack paper, appendix A.3 / Table 4).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e8_candidates(v):
    """All E8 points whose coordinates are within distance 1 of v's (brute force).

    Every nearest point lies within the covering radius 1, so each coordinate is
    within 1 of v's; we enumerate both cosets independently of the oracle.
    """
    out = []
    for half in (0.0, 0.5):
        opts = []
        for vi in v:
            lo = np.ceil(vi - 1.0 - half) + half
            opts.append([lo + k for k in range(3) if abs(lo + k - vi) <= 1.0 + 1e-12])
        for combo in itertools.product(*opts):
            z = np.array(combo) - half
            if int(round(z.sum())) % 2 == 0:
                out.append(np.array(combo))
    return np.array(out)


def test_round_half_even_matches_numpy():
    x = np.array([-2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 0.49999999, -3.7, 1e9 + 0.5, 7.0])
    assert np.array_equal(oracle.round_half_even(x), np.rint(x))


def test_d8_nearest_brute_force():
    rng = np.random.default_rng(11)
    v = rng.normal(0, 2.0, size=(300, 8))
    y = oracle.d8_nearest(v)
    for i in range(v.shape[0]):
        assert int(round(y[i].sum())) % 2 == 0
        best = np.inf
        base = np.floor(v[i]).astype(int)
        for offs in itertools.product((-1, 0, 1, 2), repeat=8) if i < 3 else []:
            z = base + np.array(offs)
            if z.sum() % 2 == 0:
                best = min(best, ((v[i] - z) ** 2).sum())
        if i < 3:
            assert ((v[i] - y[i]) ** 2).sum() <= best + 1e-12
        # cheaper check for the rest: no single +-1 move pair improves it
        d = ((v[i] - y[i]) ** 2).sum()
        for a in range(8):
            for b in range(a + 1, 8):
                for sa in (-1, 1):
                    for sb in (-1, 1):
                        z = y[i].copy()
                        z[a] += sa
                        z[b] += sb
                        assert ((v[i] - z) ** 2).sum() >= d - 1e-12


def test_e8_nearest_brute_force():
    rng = np.random.default_rng(1)
    v = rng.normal(0, 1.7, size=(120, 8))
    x, c = oracle.e8_nearest(v)
    for i in range(v.shape[0]):
        cand = _e8_candidates(v[i])
        best = ((cand - v[i]) ** 2).sum(axis=1).min()
        d = ((x[i] - v[i]) ** 2).sum()
        assert d <= best + 1e-12, (i, d, best)
        # the returned point is in E8 and c names its coset
        z = x[i] - 0.5 * c[i]
        assert np.all(z == np.round(z))
        assert int(round(z.sum())) % 2 == 0


def test_e8_covering_radius_and_second_moment():
    gold = json.load(open(os.path.join(GOLD, "e8_constants.json")))
    rng = np.random.default_rng(7)
    v = rng.uniform(-40, 40, size=(200_000, 8))
    x, _ = oracle.e8_nearest(v)
    d2 = ((x - v) ** 2).sum(axis=1)
    assert d2.max() <= gold["covering_radius_sq"] + 1e-9
    # determinant 1: mean squared error per dimension -> G(E8)
    g = d2.mean() / 8.0
    assert abs(g - gold["normalized_second_moment"]) < 0.003 * gold["normalized_second_moment"] + 2e-4


def test_e8_minimal_vectors_kissing_number():
    gold = json.load(open(os.path.join(GOLD, "e8_constants.json")))
    # lattice points at squared norm 2 around the origin: nudge towards each and check
    pts = []
    for combo in itertools.product((-1, 0, 1), repeat=8):
        z = np.array(combo, float)
        if (z ** 2).sum() == 2 and int(z.sum()) % 2 == 0:
            pts.append(z)
    for signs in itertools.product((-0.5, 0.5), repeat=8):
        z = np.array(signs)
        if int(round((z - 0.5).sum())) % 2 == 0:
            pts.append(z)
    pts = np.array(pts)
    assert len(pts) == gold["kissing_number"]
    # each minimal vector is its own nearest point, and 0.4 of the way there the origin wins
    x, _ = oracle.e8_nearest(pts)
    assert np.array_equal(x, pts)
    x, _ = oracle.e8_nearest(0.4 * pts)
    assert np.all(x == 0)


def test_fields_parity_and_round_trip():
    rng = np.random.default_rng(3)
    v = rng.normal(0, 25.0, size=(20000, 8))
    x, c = oracle.e8_nearest(v)
    f = oracle.point_to_fields(x)
    assert np.array_equal(f[:, 0], c)
    # z = x - c/2 has an even coordinate sum in both cosets
    z = x - 0.5 * c[:, None]
    assert np.all(np.mod(np.round(z.sum(axis=1)).astype(np.int64), 2) == 0)
    # m = floor(z8 / 2) and the inverse recovers every coordinate
    assert np.array_equal(f[:, 8], np.floor(z[:, 7] / 2).astype(np.int32))
    assert np.array_equal(f[:, 1:8], z[:, :7].astype(np.int32))
    assert np.array_equal(oracle.fields_to_point(f), x)


def test_fields_round_trip_exhaustive_box():
    # every E8 point with coordinates in [-2, 2] (both cosets)
    pts = []
    for combo in itertools.product(range(-2, 3), repeat=4):
        for tail in itertools.product(range(-2, 3), repeat=4):
            z = np.array(combo + tail)
            if z.sum() % 2 == 0:
                pts.append(z.astype(float))
    pts = np.array(pts[::7])
    half = pts[np.all(np.abs(pts + 0.5) <= 2, axis=1)] + 0.5
    allp = np.concatenate([pts, half])
    f = oracle.point_to_fields(allp)
    assert np.array_equal(oracle.fields_to_point(f), allp)


def _cond_entropy_bits(values, cond):
    tot = 0.0
    n = len(values)
    for cc in np.unique(cond):
        sel = values[cond == cc]
        _, cnt = np.unique(sel, return_counts=True)
        p = cnt / cnt.sum()
        tot += len(sel) / n * -(p * np.log2(p)).sum()
    return tot


def test_parity_reduction_saves_about_one_bit_per_vector():
    """Coding m instead of z8 saves ~1 bit per 8 weights (Table 4: 0.10-0.13 bpp)."""
    gold = json.load(open(os.path.join(GOLD, "table4_coding_ablation.json")))
    rng = np.random.default_rng(5)
    w = rng.standard_t(5, size=(200_000, 8))
    for s in (0.3, 0.05):   # ~4 and ~8 bpp resolutions
        x, c = oracle.e8_nearest(w / s)
        f = oracle.point_to_fields(x)
        z8 = (x[:, 7] - 0.5 * c).astype(np.int64)
        saving_bpp = (_cond_entropy_bits(z8, c) - _cond_entropy_bits(f[:, 8], c)) / 8.0
        paper = np.array(gold["direct_z8"]) - np.array(gold["entropack_17_tables_parity_reduced"])
        assert 0.115 <= saving_bpp <= 0.126, saving_bpp
        assert paper.min() - 0.01 <= saving_bpp <= paper.max() + 0.01


def test_coset_conditioning_never_hurts():
    """17 coset-conditioned tables never cost more than 9 pooled ones (Table 4)."""
    rng = np.random.default_rng(6)
    w = rng.standard_t(5, size=(100_000, 8))
    x, c = oracle.e8_nearest(w / 0.6)
    f = oracle.point_to_fields(x)
    for k in range(1, 9):
        pooled = _cond_entropy_bits(f[:, k], np.zeros_like(c))
        cond = _cond_entropy_bits(f[:, k], c)
        assert cond <= pooled + 1e-12


def test_row_rms():
    W = np.array([[3.0, 4.0, 0.0, 0.0, 0, 0, 0, 0], [0] * 8], np.float32)
    n = oracle.row_rms(W)
    assert n[0] == pytest.approx(np.sqrt(25.0 / 8.0), rel=1e-15)
    assert n[1] == 0.0
    # closed forms of the root-mean-square (not the standard deviation, not the mean |w|):
    # a constant row has RMS |a|; a lone nonzero a among 16 columns has RMS |a| / 4
    V = np.zeros((2, 16), np.float32)
    V[0, :] = -2.5
    V[1, 5] = 6.0
    assert list(oracle.row_rms(V)) == [2.5, 1.5]
