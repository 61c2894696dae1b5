"""Pins of the oracle's per-row rate-distortion refinement (paper, section 3.5
"Per-row rate-distortion refinement", appendix C.2, appendix A.4).

What the pages fix is pinned directly: candidate ratios start at 1, stay inside
[0.70, 1.45] and are nested geometric bisections of the widest interval; each
row's candidates use the scale rho_k * s with a fitted row scale; the selection
trades distortion against rate under a common penalty and keeps the baseline's
storage; the refinement only changes what the encoder chooses, so its
container decodes like any other.  The distortions are recomputed here from
the lattice primitives, the rates are checked against the baseline's actual
payload, and the selection is checked against brute force on a tiny tensor.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synthgen


def _w(rows, cols, seed):
    return synthgen.student_t_weights(rows, cols, seed).numpy()


def _rel_l2(ct, W):
    y, st = oracle.decode(ct, "fp32")
    assert np.all(st == 0)
    W = W.astype(np.float64)
    return math.sqrt(((y.astype(np.float64) - W) ** 2).sum() / (W ** 2).sum())


def test_candidate_ratios_are_nested_log_bisections():
    r = oracle.rdo_ratios(7)
    # ln 1.45 = 0.372 is wider than ln(1/0.70) = 0.357, so the upper interval goes first
    want = [1.0, 1.45 ** 0.5, 0.70 ** 0.5, 1.45 ** 0.25, 1.45 ** 0.75, 0.70 ** 0.75, 0.70 ** 0.25]
    np.testing.assert_allclose(r, want, rtol=1e-13)
    for K in range(1, 20):
        rk = oracle.rdo_ratios(K)
        assert np.array_equal(rk, oracle.rdo_ratios(K + 1)[:K])       # nested sets
        assert rk.min() > 0.70 and rk.max() < 1.45 and rk[0] == 1.0
        assert len(set(rk.tolist())) == K


@pytest.mark.parametrize("K, sweeps", [(1, 1), (5, 0)])
def test_no_refinement_is_the_baseline_container(K, sweeps):
    W = _w(64, 256, 41)
    base = oracle.encode(W, 3.0)
    ct = oracle.encode_rdo(W, 3.0, K=K, sweeps=sweeps)
    for f in ("s", "b", "V", "T"):
        assert getattr(ct, f) == getattr(base, f)
    for a in ("row_scales", "states", "offsets", "payload", "freqs", "alphabet", "minval"):
        assert getattr(ct, a).tobytes() == getattr(base, a).tobytes(), a


def test_candidate_distortions_and_row_scales_recomputed():
    W = _w(48, 256, 42)
    K = 4
    tr = oracle.rdo_trace(W, 3.0, K=K)
    s = np.float32(tr["s"])
    rho = oracle.rdo_ratios(K)
    n = oracle.row_rms(W)
    W64 = W.astype(np.float64)
    for k in range(K):
        sk = float(s) * rho[k]
        v = (W64 / n[:, None]) / sk
        x, _ = oracle.e8_nearest(v.reshape(-1, 8))
        x = x.reshape(W.shape)
        sx = float(s) * x
        r = ((W64 * sx).sum(1) / (sx * sx).sum(1)).astype(np.float32)
        np.testing.assert_allclose(tr["row_scales"][:, k], r, rtol=2e-6)
        g = (s * tr["row_scales"][:, k]).astype(np.float32)
        y = (x.astype(np.float32) * g[:, None]).astype(np.float32)
        d = ((W64 - y.astype(np.float64)) ** 2).sum(1)
        np.testing.assert_allclose(tr["D"][:, k], d, rtol=1e-9)


def test_budget_is_the_baselines_code_length():
    W = _w(128, 512, 43)
    tr = oracle.rdo_trace(W, 3.0, K=3)
    base = oracle.encode(W, 3.0)
    assert tr["budget"] == tr["R"][:, 0].sum()
    model_bits = tr["budget"] / 65536.0
    payload_bits = 16.0 * base.payload.size
    # rANS stays within a few words per tile of the tables' code length
    assert abs(payload_bits - model_bits) <= 0.01 * model_bits + 64 * base.T
    # the selection fits the budget
    assert tr["R"][np.arange(W.shape[0]), tr["sel"]].sum() <= tr["budget"]


def test_selection_is_lagrangian_optimal_by_brute_force():
    W = _w(5, 64, 44)
    K = 3
    tr = oracle.rdo_trace(W, 3.0, K=K)
    D, R, lam, sel, budget = tr["D"], tr["R"], tr["lambda"], tr["sel"], tr["budget"]
    rows = np.arange(W.shape[0])
    r_sel, d_sel = R[rows, sel].sum(), D[rows, sel].sum()
    assert r_sel <= budget
    best_at_rate = min(D[rows, list(c)].sum() for c in itertools.product(range(K), repeat=len(rows))
                       if R[rows, list(c)].sum() <= r_sel)
    assert d_sel <= best_at_rate * (1 + 1e-12)
    # lambda is the smallest feasible penalty: a slightly smaller one overspends
    if lam > 0:
        lo = lam * (1 - 1e-6)
        ch = np.argmin(D + lo * (R / 65536.0), axis=1)
        assert R[rows, ch].sum() > budget


def test_refinement_lowers_error_at_the_same_rate():
    W = _w(256, 512, 3)
    base = oracle.encode(W, 3.0)
    e0 = _rel_l2(base, W)
    for K, sweeps in ((5, 1), (9, 2)):
        ct = oracle.encode_rdo(W, 3.0, K=K, sweeps=sweeps)
        assert abs(ct.bpp / base.bpp - 1) < 0.01, (K, sweeps, ct.bpp, base.bpp)
        assert _rel_l2(ct, W) < 0.97 * e0, (K, sweeps)
        # same scale and tiling: only the encoder's choices changed
        assert (ct.s, ct.V, ct.T) == (base.s, base.V, base.T)
