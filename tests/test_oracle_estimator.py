"""Pins of the scale search's row sample and its stored-size estimate.

EntroPack paper, Appendix C.1: the scale search evaluates candidate scales on a
nominal budget of 2^18 eight-dimensional vectors, drawn as complete rows with a
shape-dependent seed and held fixed through the search.  Section 3.4
("Stored-size estimate") and section 3.6 ("Stored representation"): the
estimate counts the coded fields and the side information of the stored
representation.

The row sample is pinned by its count, by being a set of distinct, sorted,
complete rows, by determinism per shape and dependence on the shape, and by
covering the whole row range.  The estimate is pinned exactly: with the sample
covering every row (and, separately, with a partial sample of a tensor whose
rows are identical, so that the sample's statistics are exactly the tensor's),
estimate x numel / 8 must equal the ideal code length of the encoded fields
under the container's own tables (computed here with numpy) plus the stored
bytes of everything but the payload.  Dropping or miscounting the side term,
or scaling the sampled code length wrongly, fails these equalities.
"""
import math

import numpy as np
import pytest

import oracle
import synthgen


def _expected_count(rows, cols):
    per_row = cols // 8
    return min(rows, max(1, math.ceil(2 ** 18 / per_row)))


@pytest.mark.parametrize("rows,cols", [(256, 512), (10240, 3840), (3840, 10240), (11520, 3840), (7, 8),
                                       (5, 4 * 2 ** 20), (100000, 16), (3, 2 ** 21 * 8)])
def test_sample_rows_count_distinct_sorted_complete(rows, cols):
    s = oracle.sample_rows(rows, cols)
    assert s.size == _expected_count(rows, cols)
    assert s.dtype == np.int64
    assert np.all(s >= 0) and np.all(s < rows)
    assert np.all(np.diff(s) > 0)          # sorted and distinct
    # the vectors of the sampled rows reach the 2^18 budget unless every row is taken
    if s.size < rows:
        assert s.size * (cols // 8) >= 2 ** 18 > (s.size - 1) * (cols // 8)


def test_sample_rows_takes_every_row_when_the_tensor_is_small():
    for rows, cols in ((256, 512), (64, 4096), (512, 4096)):
        assert np.array_equal(oracle.sample_rows(rows, cols), np.arange(rows))


def test_sample_rows_deterministic_and_shape_dependent():
    a = oracle.sample_rows(10240, 3840)
    assert np.array_equal(a, oracle.sample_rows(10240, 3840))
    # same count (ceil(2^18 / 480) = 547 rows), different shapes: different rows
    b = oracle.sample_rows(10241, 3840)
    c = oracle.sample_rows(10240, 3848)
    assert a.size == b.size == 547 and c.size == _expected_count(10240, 3848) == 545
    assert not np.array_equal(a, b)
    assert len(np.intersect1d(a, b)) < a.size // 4       # not a shifted copy of the same draw
    assert not np.array_equal(a[: c.size], c)


def test_sample_rows_cover_the_row_range():
    # a uniform draw of k of R rows: mean index (R - 1)/2, about k/2 in each half,
    # and both ends of the range reached (a "first k rows" or "every m-th row" rule fails)
    means, lows = [], []
    for rows in range(20000, 20040):
        s = oracle.sample_rows(rows, 8192)        # 256 of ~20000 rows
        assert s.size == 256
        means.append(s.mean() / (rows - 1))
        lows.append(np.mean(s < rows / 2))
        assert s[0] < rows * 0.05 and s[-1] > rows * 0.95
        assert len(set(np.diff(s))) > 100           # not evenly strided
    assert abs(np.mean(means) - 0.5) < 0.01
    assert abs(np.mean(lows) - 0.5) < 0.02


def _ideal_payload_bits(ct):
    """Ideal code length of the container's fields under its own tables: sum n (b - log2 f)."""
    fields, st = oracle.decode(ct, "fields")
    assert np.all(st == 0)
    c = fields[:, 0]
    bits = 0.0
    # coset bit: table 0 over values 0..1
    f0 = ct.table(0).astype(np.float64)
    n0 = np.bincount(c, minlength=2)
    bits += float(np.sum(n0 * (ct.b - np.log2(np.where(n0 > 0, f0, 1.0)))))
    for field in range(1, 9):
        for cs in (0, 1):
            k = 1 + 2 * (field - 1) + cs
            vals = fields[c == cs, field]
            if vals.size == 0:
                continue
            idx = vals.astype(np.int64) - int(ct.minval[k])
            assert idx.min() >= 0 and idx.max() < int(ct.alphabet[k])
            n = np.bincount(idx, minlength=int(ct.alphabet[k])).astype(np.float64)
            f = ct.table(k).astype(np.float64)
            assert np.all(f[n > 0] > 0)
            bits += float(np.sum(n[n > 0] * (ct.b - np.log2(f[n > 0]))))
    return bits


@pytest.mark.parametrize("s,b,V", [(0.12, 11, 64), (0.35, 12, 455), (0.05, 13, 32)])
def test_estimate_equals_ideal_code_length_plus_side_information(s, b, V):
    # 96 x 1024: 12,288 vectors, so the sample is the whole tensor
    W = synthgen.student_t_weights(96, 1024, 71, bf16=True).numpy()
    assert oracle.sample_rows(96, 1024).size == 96
    s = float(np.float32(s))       # the fixed-scale encoder takes s as fp32
    est = oracle.estimate_bpp(W, s, b, V)
    ct = oracle.encode_fixed_scale(W, s, V, b)
    side = oracle.stored_bytes(ct.rows, ct.T, 0, ct.alphabet)        # header, tables, scales, metadata
    ideal = _ideal_payload_bits(ct)
    assert est * W.size / 8.0 == pytest.approx(ideal / 8.0 + side, rel=1e-12)
    # the side term is a few percent of the stored size here: dropping it fails by far more than the tolerance
    assert side / (ideal / 8.0 + side) > 0.01
    # the coded payload is the ideal length up to the per-tile state overhead (32 states of at most 31 bits)
    payload = 2 * ct.nwords
    assert ideal / 8.0 - 4 * 32 * ct.T <= payload <= ideal / 8.0 + 2 * 32 * ct.T + 0.002 * ideal / 8.0


def test_estimate_scales_a_partial_sample_to_the_whole_tensor():
    # identical rows: any sample of complete rows has exactly the tensor's symbol
    # statistics, so the scaled sample code length equals the full ideal length
    row = synthgen.student_t_weights(1, 4096, 72, bf16=True).numpy()
    W = np.ascontiguousarray(np.tile(row, (600, 1)))
    samp = oracle.sample_rows(600, 4096)
    assert 0 < samp.size < 600                      # 512 of 600 rows
    s, b, V = float(np.float32(0.2)), 11, 1820
    est = oracle.estimate_bpp(W, s, b, V)
    ct = oracle.encode_fixed_scale(W, s, V, b)
    side = oracle.stored_bytes(ct.rows, ct.T, 0, ct.alphabet)
    ideal = _ideal_payload_bits(ct)
    assert est * W.size / 8.0 == pytest.approx(ideal / 8.0 + side, rel=1e-12)
