"""GPU parity: the HIP decoder against the CPU oracle, through the C ABI.

Inputs are seeded synthetic tensors compressed by the oracle's encoder; the
GPU decodes the same arrays.  Lattice coordinates, FP8 and INT8 codes and BF16
bit patterns must match bit for bit (BF16 follows the oracle's fp32 operation
order y = fp32(x * fp32(s * r_row)), so no tolerance is needed).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _gpu_out_numpy(t: torch.Tensor, kind: str) -> np.ndarray:
    # bit patterns (signed zeros and infinities compare exactly)
    if kind in ("bf16", "fp16"):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if kind == "fp8":
        return t.view(torch.uint8).cpu().numpy()
    if kind == "fp32":
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def _ref_bits(ref: np.ndarray, kind: str) -> np.ndarray:
    return ref.view(np.uint32) if kind == "fp32" else ref


def _max_coordinate_freq(ct) -> int:
    return max(int(ct.freqs[ct.freq_base[k]:ct.freq_base[k] + ct.alphabet[k]].max())
               for k in range(1, 17) if ct.alphabet[k])


def _check_parity(ct, kinds=("bf16", "lattice2x"), label=""):
    p = ep.PackedTensor.from_arrays(ct)
    for kind in kinds:
        ref, rst = oracle.decode(ct, kind)
        out, st = ep.decode_tensor(p, kind, with_status=True)
        torch.cuda.synchronize()
        got = _gpu_out_numpy(out, kind)
        ref = _ref_bits(ref, kind)
        assert np.all(st.cpu().numpy()[: ct.T] == 0), f"{label} {kind}: tile status"
        assert np.all(rst == 0)
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            raise AssertionError(f"{label} {kind}: {len(bad)} mismatches, first at {bad[:5].tolist()}")


def test_library_exports_and_version():
    L = ep.lib()
    for name in ep.EXPORTS:
        assert hasattr(L, name)
    assert L.ep_abi_version() == 3


@pytest.mark.parametrize("V", [512, 455])
def test_w256x512_4bpp_bit_exact(V):
    spec = synthgen.workload("w256x512_4bpp_fp32" if V == 512 else "w256x512_4bpp_fp32_s4096")[0]
    W = spec.weights().numpy()
    ct = oracle.encode(W, spec.target_bpp, V=spec.vectors_per_tile, b=spec.prob_bits)
    assert ct.b == 12 and ct.V == V
    _check_parity(ct, label=f"V={V}")


@pytest.mark.parametrize("b", list(range(9, 16)))
def test_every_precision(b):
    # scale picked so the alphabets fit 2^b; ragged shapes, V not a multiple of 32
    rng = np.random.default_rng(b)
    rows, cols = int(rng.integers(3, 70)), 8 * int(rng.integers(1, 90))
    W = synthgen.student_t_weights(rows, cols, 100 + b).numpy()
    s = {9: 0.5, 10: 0.25, 11: 0.1, 12: 0.05, 13: 0.02, 14: 0.01, 15: 0.004}[b]
    ct = oracle.encode_fixed_scale(W, s, V=int(rng.integers(32, 200)), b=b)
    _check_parity(ct, kinds=("bf16", "lattice2x", "fp16", "fp32"), label=f"b={b} {rows}x{cols} V={ct.V}")


def test_routes_fp8_and_int8_codes():
    W = synthgen.student_t_weights(96, 1024, 42).numpy()
    ct8 = oracle.encode(W, 5.0, route="fp8")
    _check_parity(ct8, kinds=("fp8", "lattice2x", "bf16"), label="fp8 route")
    cti = oracle.encode(W, 8.0, route="int8")
    _check_parity(cti, kinds=("int8", "uint8", "lattice2x"), label="int8 route 8bpp")
    cti2 = oracle.encode(W, 2.0, route="int8")
    _check_parity(cti2, kinds=("int8",), label="int8 route 2bpp")


def test_int8_and_fp8_saturation_paths():
    # decoding a direct-route tensor into INT8 / FP8 exercises clamping and subnormals
    W = (synthgen.student_t_weights(64, 512, 7).numpy() * 4000.0).astype(np.float32)
    ct = oracle.encode(W, 6.0)
    _check_parity(ct, kinds=("int8", "uint8", "fp8"), label="saturation")
    Ws = (synthgen.student_t_weights(64, 512, 8).numpy() * 1e-2).astype(np.float32)
    cts = oracle.encode(Ws, 6.0)
    _check_parity(cts, kinds=("fp8",), label="fp8 subnormals")


def test_fp16_overflow_and_subnormal_paths():
    # products above 65520 become infinities, products below 2^-14 FP16 subnormals
    Wb = (synthgen.student_t_weights(64, 512, 17).numpy() * 3e6).astype(np.float32)
    ctb = oracle.encode(Wb, 6.0)
    ref, _ = oracle.decode(ctb, "fp16")
    assert np.any((ref & 0x7FFF) == 0x7C00)
    _check_parity(ctb, kinds=("fp16", "fp32"), label="fp16 overflow")
    Wt = (synthgen.student_t_weights(64, 512, 18).numpy() * 1e-4).astype(np.float32)
    ctt = oracle.encode(Wt, 6.0)
    ref, _ = oracle.decode(ctt, "fp16")
    assert np.any(((ref & 0x7C00) == 0) & ((ref & 0x3FF) != 0))
    _check_parity(ctt, kinds=("fp16", "fp32"), label="fp16 subnormals")


def test_single_symbol_and_empty_coset_tables():
    # all-zero rows quantise to the origin: coset 1 never occurs (its tables are
    # empty) and every coordinate table holds one symbol (f = M, no renormalisation)
    W = np.zeros((16, 256), np.float32)
    ct = oracle.encode_fixed_scale(W, 1.0, V=40, b=11)
    assert ct.alphabet[2] == 0 and ct.alphabet[1] == 1
    _check_parity(ct, label="degenerate tables")


def test_batch_mixed_tensors_one_call():
    rng = np.random.default_rng(3)
    cts, kinds = [], []
    for i in range(7):
        rows, cols = int(rng.integers(1, 200)), 8 * int(rng.integers(1, 300))
        W = synthgen.student_t_weights(rows, cols, 500 + i).numpy()
        tgt = float(rng.choice([2.0, 4.0, 8.0]))
        route = ["direct", "fp8", "int8"][i % 3]
        cts.append(oracle.encode(W, tgt, V=int(rng.integers(32, 500)), route=route))
        kinds.append({"direct": ["bf16", "fp16", "fp32"][i % 9 // 3], "fp8": "fp8",
                      "int8": ["int8", "uint8"][i // 3 % 2]}[route])
    # an empty tensor in the middle of the batch
    cts.insert(3, oracle.encode(np.zeros((0, 64), np.float32), 4.0))
    kinds.insert(3, "bf16")
    packed = [ep.PackedTensor.from_arrays(c) for c in cts]
    outs, sts = ep.decode_batch(packed, kinds, with_status=True)
    torch.cuda.synchronize()
    for i, (ct, kind) in enumerate(zip(cts, kinds)):
        ref, _ = oracle.decode(ct, kind)
        assert np.array_equal(_gpu_out_numpy(outs[i], kind), _ref_bits(ref, kind)), f"tensor {i}"
        assert np.all(sts[i].cpu().numpy()[: ct.T] == 0)


def test_deterministic_repeat_and_workspace_reuse():
    W = synthgen.student_t_weights(300, 768, 9).numpy()
    ct = oracle.encode(W, 4.0, V=100)
    p = ep.PackedTensor.from_arrays(ct)
    ws = torch.empty(ep.workspace_size([p]), dtype=torch.uint8, device="cuda")
    a, _ = ep.decode_tensor(p, "bf16", workspace=ws)
    b, _ = ep.decode_tensor(p, "bf16", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("target, b, outliers, rows, cols, seed, V", [
    (4.0, 11, 0.0, 64, 512, 11, 64),        # packed tables
    (4.0, 12, 0.0, 64, 512, 11, 64),        # narrow tables
    (8.0, 12, 0.002, 96, 2048, 11, 64),     # hybrid tables (A > 256 at b = 12)
    (7.0, 11, 0.002, 192, 2048, 101, 0),    # hybrid at b = 11 with per-slot entries (A > 1024, f < 128)
    (8.0, 13, 0.002, 96, 2048, 11, 64),     # global tables
])
def test_corrupt_streams_flagged_like_oracle(target, b, outliers, rows, cols, seed, V):
    W = synthgen.student_t_weights(rows, cols, seed, outlier_frac=outliers).numpy()
    ct = oracle.encode(W, target, V=V, b=b)
    print(f"[corrupt] b={ct.b} A={ct.alphabet[1:].max()} T={ct.T}", flush=True)
    if b == 11 and V == 0:
        assert ct.alphabet[1:].max() > 1024 and _max_coordinate_freq(ct) < 128
    rng = np.random.default_rng(0)
    pl = ct.payload.copy()
    stt = ct.states.copy()
    off = ct.offsets.copy()
    bad_tiles = set()
    for t in (1, 4, 9):
        pl[ct.offsets[t] + int(rng.integers(0, ct.offsets[t + 1] - ct.offsets[t]))] ^= np.uint16(0x0210)
        bad_tiles.add(t)
    stt[32 * 6 + 17] ^= np.uint32(0x100)
    bad_tiles.add(6)
    off[12] += 1          # tile 11 one word longer, tile 12 one word shorter
    bad_tiles.update({11, 12})
    ct2 = dataclasses.replace(ct, payload=pl, states=stt, offsets=off)
    _, rst = oracle.decode(ct2, "bf16")
    p = ep.PackedTensor.from_arrays(ct2)
    _, st = ep.decode_tensor(p, "bf16", with_status=True)
    gst = st.cpu().numpy()[: ct.T]
    assert set(np.nonzero(rst)[0].tolist()) == bad_tiles
    assert np.array_equal(gst != 0, rst != 0)
    # good tiles still decode exactly
    ref, _ = oracle.decode(ct2, "bf16")
    out, _ = ep.decode_tensor(p, "bf16")
    got = _gpu_out_numpy(out, "bf16").reshape(-1)
    for t in range(ct.T):
        if t in bad_tiles:
            continue
        lo, hi = t * ct.V * 8, min((t + 1) * ct.V * 8, got.size)
        assert np.array_equal(got[lo:hi], ref.reshape(-1)[lo:hi])


def test_offsets_beyond_payload_are_contained():
    W = synthgen.student_t_weights(32, 256, 12).numpy()
    ct = oracle.encode(W, 4.0, V=32)
    off = ct.offsets.copy()
    off[-1] += 5000       # the last tile claims words that do not exist
    ct2 = dataclasses.replace(ct, offsets=off)
    p = ep.PackedTensor.from_arrays(ct2)
    # the buffer really ends at the true payload end (padded to 8 words as the ABI asks)
    nw = int(ct.offsets[-1])
    p = dataclasses.replace(p, payload=p.payload[: (nw + 7) // 8 * 8].clone(), nwords=nw)
    _, st = ep.decode_tensor(p, "bf16", with_status=True)
    gst = st.cpu().numpy()[: ct.T]
    assert gst[-1] != 0 and np.all(gst[:-1] == 0)


def test_invalid_arguments_rejected():
    W = synthgen.student_t_weights(8, 64, 1).numpy()
    ct = oracle.encode(W, 4.0, V=32)
    p = ep.PackedTensor.from_arrays(ct)
    with pytest.raises(ep.EpError) as ei:
        ep.decode_batch([dataclasses.replace(p, T=p.T + 1)], "bf16")
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    with pytest.raises(ep.EpError):
        ep.decode_batch([dataclasses.replace(p, b=16)], "bf16")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ep.EpError) as ei:
        ep.decode_batch([p], "bf16", workspace=small)
    assert ei.value.status == ep.EP_ERR_WORKSPACE


@pytest.mark.parametrize("b, s, lo, hi", [(10, 0.07, 513, 1024), (11, 0.07, 513, 1024), (11, 0.05, 1025, 2048)])
def test_wide_alphabets(b, s, lo, hi):
    # alphabets above 512 symbols: the wide packed layout (up to 1024 symbols at
    # b = 10, 11), and the cached global-table layout beyond it
    W = synthgen.student_t_weights(64, 1024, 11 + b, outlier_frac=0.002).numpy()
    ct = oracle.encode_fixed_scale(W, s, V=96, b=b)
    assert lo <= int(ct.alphabet[1:].max()) <= hi
    _check_parity(ct, kinds=("bf16", "lattice2x", "fp8", "int8", "uint8"), label=f"b={b} A={ct.alphabet[1:].max()}")


@pytest.mark.parametrize("rows, cols, V", [
    (40, 8, 32),        # one vector per row: every round wraps 32 rows
    (33, 16, 33),       # two vectors per row, V not a multiple of 32
    (7, 248, 61),       # 31 vectors per row
    (1, 4096, 7200),    # V at its maximum, one row, one partial tile
    (300, 64, 7200),    # several rows per tile at the maximum V
])
def test_row_wrap_and_tile_size_limits(rows, cols, V):
    W = synthgen.student_t_weights(rows, cols, rows * 1000 + cols).numpy()
    ct = oracle.encode_fixed_scale(W, 0.1, V=V, b=11)
    assert ct.V == V and ct.alphabet[1:].max() > 8
    _check_parity(ct, kinds=("bf16", "lattice2x", "int8"), label=f"{rows}x{cols} V={V}")


def test_tensor_smaller_than_one_round():
    # fewer vectors than lanes in a half-wave: a single partial round
    W = synthgen.student_t_weights(2, 64, 77).numpy()
    ct = oracle.encode_fixed_scale(W, 0.1, V=32, b=11)
    assert ct.T == 1 and ct.rows * ct.cols // 8 < 32
    _check_parity(ct, kinds=("bf16", "lattice2x", "fp32"), label="16 vectors")


@pytest.mark.parametrize("coding", ["pooled", "direct_z8"])
@pytest.mark.parametrize("target, b", [(4.0, 11), (4.0, 9), (4.0, 10), (7.0, 11), (4.0, 12), (8.0, 13)])
def test_table4_coding_variants(coding, target, b):
    # the two ablations of the paper's Table 4 through every table layout: pooled
    # tables share one frequency table per field between the cosets; direct z8
    # sets the descriptor's field8 flag
    W = synthgen.student_t_weights(160, 1024, 70 + b, bf16=True).numpy()
    ct = oracle.encode(W, target, b=b, coding=coding)
    print(f"[table4] {coding} target={target} b={ct.b} A={ct.alphabet[1:].max()}", flush=True)
    _check_parity(ct, kinds=("lattice2x", "bf16", "int8"), label=f"{coding} b={ct.b}")
    std = oracle.encode(W, target, b=b)
    assert np.array_equal(oracle.decode(std, "lattice2x")[0], oracle.decode(ct, "lattice2x")[0])


def _rounding_probe_values() -> np.ndarray:
    # every exponent of 2^-30 .. 2^16 (FP8 and FP16 subnormals to FP16 overflow) with
    # all 128 patterns of the top 7 mantissa bits and low bits at the BF16 (bit 15),
    # FP16 (bit 12) and FP8 (bit 19, inside the top bits) ties and next to them
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x3000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    exps = np.arange(127 - 30, 127 + 17, dtype=np.uint32)
    hi = np.arange(128, dtype=np.uint32) << 16
    bits = (exps[:, None, None] << 23) | hi[None, :, None] | lows[None, None, :]
    bits = bits.reshape(-1)
    vals = np.concatenate([bits, bits | 0x80000000]).view(np.float32)
    halves = np.arange(-261, 262, dtype=np.float32) * np.float32(0.5)          # INT8 ties and limits
    near = np.concatenate([np.nextafter(halves, np.float32(np.inf)), np.nextafter(halves, np.float32(-np.inf))])
    special = np.float32([0.0, -0.0, 448.0, -448.0, 464.0, -464.0, 480.0, 1e30, -1e30, 65504.0, 65520.0,
                          -65520.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 1e-45, -1e-45, 1.17549435e-38])
    rng = np.random.default_rng(17)
    uni = rng.uniform(-500, 500, 1 << 20).astype(np.float32)
    rb = (rng.integers(90, 150, 1 << 18, dtype=np.uint32) << 23) | rng.integers(0, 1 << 23, 1 << 18, dtype=np.uint32)
    rb |= rng.integers(0, 2, 1 << 18, dtype=np.uint32) << 31
    v = np.concatenate([vals, halves, near, special, uni, rb.view(np.float32)])
    pad = (-v.size) % 4
    return np.concatenate([v, np.zeros(pad, np.float32)])


def test_container_rounding_matches_oracle_at_every_boundary():
    # ep_convert_f32 runs the decode kernel's own conversion code (FP8 through the
    # hardware v_cvt_pk_fp8_f32 after a v_med3 clamp)
    v = _rounding_probe_values()
    y = torch.from_numpy(v).cuda()
    refs = {"bf16": oracle.f32_to_bf16(v), "fp16": oracle.f32_to_fp16(v), "fp8": oracle.f32_to_fp8(v),
            "int8": oracle.f32_to_int8(v), "uint8": oracle.f32_to_uint8(v)}
    for kind, ref in refs.items():
        got = _gpu_out_numpy(ep.convert_f32(y, kind), kind)
        torch.cuda.synchronize()
        ref = np.asarray(ref).view(got.dtype)
        if not np.array_equal(got, ref):
            bad = np.flatnonzero(got != ref)
            i = bad[0]
            raise AssertionError(f"{kind}: {bad.size} of {v.size} differ; first y={v[i]!r} "
                                 f"(bits {v[i:i+1].view(np.uint32)[0]:#010x}) gpu={got[i]} oracle={ref[i]}")


@pytest.mark.parametrize("target, b, outliers, seed, split", [
    (7.0, 11, 0.002, 101, True),      # every f < 128: per-slot entries and values in LDS
    (6.0, 11, 0.01, 108, False),      # some f >= 128: u16 slot maps in LDS, entries from the workspace
    (8.0, 12, 0.0, 102, False),       # b = 12: always the slot maps
    (7.0, 12, 0.0, 102, False),
])
def test_hybrid_layout_large_alphabets(target, b, outliers, seed, split):
    # b = 11 with alphabets above 1024 and b = 12 above 256.  At b = 11 the table
    # build keeps per-slot entries when every frequency is below 128; otherwise
    # the decoder reads the u16 slot maps and the per-symbol entries.
    W = synthgen.student_t_weights(192, 2048, seed, bf16=True, outlier_frac=outliers).numpy()
    ct = oracle.encode(W, target, b=b)
    amax, fmax = int(ct.alphabet[1:].max()), _max_coordinate_freq(ct)
    print(f"[hybrid] target={target} b={ct.b} A={amax} max f={fmax}", flush=True)
    assert ct.b == b and amax > (1024 if b == 11 else 256)
    assert (b == 11 and fmax < 128) == split
    _check_parity(ct, kinds=("lattice2x", "bf16", "fp8", "uint8"), label=f"hybrid b={b} A={amax} f<={fmax}")


def test_rows_whose_half_multiplier_is_inexact():
    # g = fp32(s * r) subnormal with an odd last bit: g/2 is not exact, so the tensor
    # takes the (z + c/2) * g product; decoded in one batch beside an ordinary tensor
    W = synthgen.student_t_weights(48, 512, 33).numpy()
    ct = oracle.encode(W, 4.0, V=64)
    rs = ct.row_scales.copy()
    rs[3] = np.float32(3e-39)
    rs[10] = np.float32(-7.3e-40)
    g = (np.float32(ct.s) * rs[[3, 10]]).astype(np.float32)
    half = (g * np.float32(0.5)).astype(np.float32)
    assert np.any((half * np.float32(2.0)).astype(np.float32) != g)      # the slow case is hit
    slow = dataclasses.replace(ct, row_scales=rs)
    plain = oracle.encode(synthgen.student_t_weights(32, 256, 34).numpy(), 4.0, V=32)
    for kind in ("fp32", "bf16", "fp16", "lattice2x"):
        packed = [ep.PackedTensor.from_arrays(c) for c in (slow, plain)]
        outs, sts = ep.decode_batch(packed, kind, with_status=True)
        torch.cuda.synchronize()
        for c, o, s_ in zip((slow, plain), outs, sts):
            ref, _ = oracle.decode(c, kind)
            assert np.all(s_.cpu().numpy()[: c.T] == 0)
            assert np.array_equal(_gpu_out_numpy(o, kind), _ref_bits(ref, kind)), kind


def test_large_batch_runs_and_work_counter():
    """Enough small tiles to fill every resident block with full chunks.

    12 tensors of 807 tiles (V = 32; the last chunk of each tensor partial)
    make blocks whose chunk ranges straddle tensor boundaries, so blocks
    decode several runs and take tile pairs beyond their first from the work
    counter.  Every output is compared whole against the oracle.
    """
    cts = [oracle.encode(synthgen.student_t_weights(200, 1032, 700 + i).numpy(), 4.0, V=32) for i in range(12)]
    assert all(ct.b == 11 and ct.T == 807 for ct in cts)
    kinds = ["bf16"] * 12
    packed = [ep.PackedTensor.from_arrays(c) for c in cts]
    for rep in range(2):
        outs, sts = ep.decode_batch(packed, kinds, with_status=True)
        torch.cuda.synchronize()
        for i, ct in enumerate(cts):
            ref, _ = oracle.decode(ct, "bf16")
            assert np.array_equal(_gpu_out_numpy(outs[i], "bf16"), ref), f"rep {rep} tensor {i}"
            assert np.all(sts[i].cpu().numpy()[: ct.T] == 0)


@pytest.mark.parametrize("s", [8.0, 12.0])
def test_packed_direct_and_symbol_entries(s):
    """b = 11 packed tables in both entry forms on the same data: at s = 8 every
    table has several symbols (direct-value entries); at s = 12 some coordinate
    tables hold one symbol (f = 2^11 needs 12 bits, so the symbol form is used)."""
    W = synthgen.student_t_weights(128, 512, 61).numpy()
    ct = oracle.encode_fixed_scale(W, s, V=64, b=11)
    assert ct.b == 11
    assert (1 in ct.alphabet[1:].tolist()) == (s == 12.0)
    _check_parity(ct, kinds=("bf16", "lattice2x", "fp8", "int8"), label=f"s={s}")


def test_decode_on_a_side_stream_keeps_its_buffers():
    # decode_tensor / decode_batch allocate their workspace (and any outputs and
    # statuses) on the launch stream.  Work queued at once on the caller's current
    # stream, allocating blocks of the workspace's size and writing them, must not
    # get that memory while the decode still reads it.
    W = synthgen.student_t_weights(3072, 2048, 13, bf16=True).numpy()
    ct = oracle.encode(W, 4.0)
    p = ep.PackedTensor.from_arrays(ct)
    ref, _ = oracle.decode(ct, "bf16")
    nws = ep.workspace_size([p])
    side = torch.cuda.Stream()                 # default priority
    torch.cuda.synchronize()
    for _ in range(3):
        out, st = ep.decode_tensor(p, "bf16", with_status=True, stream=side)
        outs, sts = ep.decode_batch([p, p], "bf16", with_status=True, stream=side)
        junk = [torch.full((nws,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(16)]
        junk += [torch.full((max(p.T, 1),), 7, dtype=torch.int32, device="cuda") for _ in range(16)]
        side.synchronize()
        torch.cuda.synchronize()
        for o, s in [(out, st)] + list(zip(outs, sts)):
            assert np.all(s.cpu().numpy()[: ct.T] == 0)
            assert np.array_equal(_gpu_out_numpy(o, "bf16"), ref)
        del junk
