"""Pins of the oracle's frequency tables and tiled rANS coder.

Round-trip identity (the paper's own check, appendix A.3), end-of-tile
invariants, at most one payload word per symbol (appendix C.3), the payload
length against the ideal code length, and adversarial tables: every precision
b = 9..15, single-symbol tables, full 2^b alphabets, partial tiles.
"""
import numpy as np
import pytest

import oracle


def _random_tables(rng, b, alphabets, skew=1.0):
    """17 normalised tables; table 0 (coset bit) always has two symbols."""
    tabs = []
    for k, A in enumerate(alphabets):
        if A == 0:
            tabs.append(np.zeros(0, np.uint16))
            continue
        w = rng.random(A) ** (3.0 * skew) + 1e-3
        counts = np.maximum(1, (w / w.sum() * 10 * (1 << b)).astype(np.uint64))
        f = oracle.normalize_freqs(counts, b)
        assert f is not None
        tabs.append(f)
    return tabs


def _draw_symbols(rng, n, tabs, b):
    """Symbols drawn from the tables' own distributions (coset bit first)."""
    sym = np.zeros((n, 9), np.int32)
    M = 1 << b
    p0 = tabs[0].astype(float) / M
    sym[:, 0] = (rng.random(n) >= p0[0]).astype(np.int32) if tabs[0][1] > 0 else 0
    for f in range(1, 9):
        for c in (0, 1):
            k = 1 + 2 * (f - 1) + c
            sel = sym[:, 0] == c
            if sel.sum() == 0:
                continue
            p = tabs[k].astype(float) / M
            sym[sel, f] = rng.choice(len(p), size=sel.sum(), p=p)
    return sym


def _ideal_bits(sym, tabs, b):
    bits = 0.0
    for f in range(9):
        for v in range(sym.shape[0]):
            c = sym[v, 0]
            k = 0 if f == 0 else 1 + 2 * (f - 1) + c
            bits += b - np.log2(float(tabs[k][sym[v, f]]))
    return bits


def test_normalize_freqs_invariants():
    rng = np.random.default_rng(0)
    for b in range(9, 16):
        M = 1 << b
        for A in (1, 2, 7, 300, M):
            counts = rng.integers(0, 50, size=A).astype(np.uint64)
            counts[rng.integers(0, A)] += 1
            if rng.random() < 0.5:
                counts[rng.integers(0, A)] += 10 ** 6   # a dominant symbol
            f = oracle.normalize_freqs(counts, b)
            if (counts > 0).sum() > M:
                assert f is None
                continue
            assert f is not None
            assert int(f.astype(np.int64).sum()) == M
            assert np.array_equal(f > 0, counts > 0)
    # more observed symbols than 2^b cannot be normalised
    assert oracle.normalize_freqs(np.ones(1 << 9 + 1, np.uint64), 9) is None
    # a single symbol takes all of M, even M = 2^15
    assert oracle.normalize_freqs(np.array([5], np.uint64), 15)[0] == 1 << 15
    # an empty table stays empty
    assert np.all(oracle.normalize_freqs(np.zeros(4, np.uint64), 11) == 0)


def test_normalize_freqs_close_to_empirical():
    rng = np.random.default_rng(1)
    counts = np.round(1e6 * np.exp(-0.5 * (np.arange(-40, 41) / 6.0) ** 2)).astype(np.uint64) + 1
    f = oracle.normalize_freqs(counts, 12).astype(float)
    p = counts / counts.sum()
    q = f / f.sum()
    kl = (p * np.log2(p / q)).sum()
    # symbols whose share is below 1/M are lifted to f = 1; that mass is taken from
    # the rest, costing about -log2(1 - lifted/M) bits; rounding adds a little more
    lifted = int((counts.astype(float) * 4096 / counts.sum() < 1).sum())
    bound = -np.log2(1 - lifted / 4096.0) + 0.002
    assert kl < bound, (kl, bound)
    assert kl > 0.5 * (bound - 0.002)


@pytest.mark.parametrize("b", list(range(9, 16)))
def test_tile_round_trip_all_precisions(b):
    rng = np.random.default_rng(100 + b)
    alph = [2] + [int(a) for a in rng.integers(1, min(1 << b, 600), size=16)]
    tabs = _random_tables(rng, b, alph)
    for n in (1, 4, 31, 32, 33, 455, 512, 1000):
        sym = _draw_symbols(rng, n, tabs, b)
        states, words = oracle.tile_encode(sym, tabs, b)
        assert len(words) <= 9 * n                     # at most one word per symbol
        assert np.all(states >= 1 << 15) and np.all(states < 1 << 31)
        rc, dec = oracle.tile_decode(n, states, words, tabs, b)
        assert rc == oracle.TILE_OK
        assert np.array_equal(dec, sym)
        # lanes without vectors keep the initial state
        assert np.all(states[n:] == 1 << 15) if n < 32 else True


def test_tile_payload_matches_ideal_code_length():
    rng = np.random.default_rng(9)
    b = 11
    tabs = _random_tables(rng, b, [2] + [200] * 16, skew=2.0)
    n = 1820
    sym = _draw_symbols(rng, n, tabs, b)
    states, words = oracle.tile_encode(sym, tabs, b)
    ideal = _ideal_bits(sym, tabs, b)
    # information held in the 32 terminal states beyond the initial 2^15
    held = np.log2(states.astype(float) / (1 << 15)).sum()
    coded = 16 * len(words) + held
    assert abs(coded - ideal) < 0.002 * ideal + 64, (coded, ideal)


def test_single_symbol_tables_move_no_words():
    b = 15
    tabs = [np.array([1 << 15, 0], np.uint16)] + [np.array([1 << 15], np.uint16)] * 16
    # coset-1 tables unused -> give them zero alphabets
    for c1 in range(2, 17, 2):
        tabs[c1] = np.zeros(0, np.uint16)
    sym = np.zeros((100, 9), np.int32)
    states, words = oracle.tile_encode(sym, tabs, b)
    assert len(words) == 0 and np.all(states == 1 << 15)
    rc, dec = oracle.tile_decode(100, states, words, tabs, b)
    assert rc == oracle.TILE_OK and np.array_equal(dec, sym)


def test_full_alphabet_uniform_table():
    b = 9
    M = 1 << b
    uni = np.ones(M, np.uint16)
    tabs = [np.array([M // 2, M // 2], np.uint16)] + [uni] * 16
    rng = np.random.default_rng(2)
    n = 64
    sym = rng.integers(0, M, size=(n, 9)).astype(np.int32)
    sym[:, 0] = rng.integers(0, 2, size=n)
    states, words = oracle.tile_encode(sym, tabs, b)
    # 1 bit for c + 9 bits for each of 8 fields per vector, less what the states hold
    held = np.log2(states.astype(float) / (1 << 15)).sum()
    assert abs(16 * len(words) + held - n * (1 + 8 * 9)) < 0.002 * n * 73 + 4
    rc, dec = oracle.tile_decode(n, states, words, tabs, b)
    assert rc == oracle.TILE_OK and np.array_equal(dec, sym)


def test_decoder_flags_corruption():
    rng = np.random.default_rng(4)
    b = 11
    tabs = _random_tables(rng, b, [2] + [40] * 16)
    n = 300
    sym = _draw_symbols(rng, n, tabs, b)
    states, words = oracle.tile_encode(sym, tabs, b)
    # truncated payload: the decoder runs out of words or ends in a wrong state
    rc, _ = oracle.tile_decode(n, states, words[:-3], tabs, b)
    assert rc in (oracle.TILE_OVERRUN, oracle.TILE_BAD_STATE, oracle.TILE_BAD_LENGTH)
    # extra words are reported as a length mismatch
    rc, _ = oracle.tile_decode(n, states, np.concatenate([words, words[:2]]), tabs, b)
    assert rc != oracle.TILE_OK
    # flipped payload bits / corrupted states are caught by the terminal-state check
    for trial in range(20):
        w2 = words.copy()
        i = rng.integers(0, len(w2))
        w2[i] ^= np.uint16(1 << int(rng.integers(0, 16)))
        rc, _ = oracle.tile_decode(n, states, w2, tabs, b)
        assert rc != oracle.TILE_OK
        s2 = states.copy()
        s2[rng.integers(0, 32)] ^= np.uint32(1 << int(rng.integers(0, 15)))
        rc, _ = oracle.tile_decode(n, s2, words, tabs, b)
        assert rc != oracle.TILE_OK
