"""Which decode form a tensor takes, read back from the workspace, with parity against the oracle.

The decoder chooses a table layout per tensor and, inside some layouts, entry
forms that the table build drops when a frequency is too large: the per-slot
entries of the hybrid layout at b = 11 (every f < 128, every value in 16 bits),
the fp16 byte entries of fields 1..7 (direct packed tensors) and the i16 byte
entries of all tables (other packed and wide tensors), both needing every
f < 256.  The decoded weights are identical whichever form runs, so parity
alone cannot show which one did.  These tests read the descriptor the library
wrote to the workspace after ep_batch_prepare (its field offsets are pinned by
static_asserts in the decoder source): the host's choice, and the table build's
flags, which hold the call's number when a frequency rules a form out.  They
check the expected form, then compare the decode with the oracle.

Inputs are oracle-encoded seeded weights; some containers get a table's
min_offset shifted, which keeps the coded symbols valid and moves the decoded
values (both decoders follow the shifted offsets), to reach the branches the
encoder's own containers do not: non-direct packed tables and values beyond
16 bits.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")

DEVTENSOR_BYTES = 576
FIELD_OFFSET = {"variant": 36, "call": 56, "direct": 72, "split": 76, "byte_cand": 80, "bytev": 84,
                "bad_split": 556, "bad_bytes": 560}
P11, W11, H11 = 2, 4, 6          # decode-table placements (the library's Variant numbering)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _max_f(ct, tables):
    return max(int(ct.table(k).max()) for k in tables if ct.alphabet[k])


def _shift(ct, k, delta):
    mv = ct.minval.copy()
    mv[k] += delta
    return dataclasses.replace(ct, minval=mv)


def _read_flags(ct):
    p = ep.PackedTensor.from_arrays(ct, device="cuda")
    outs = ep.alloc_outputs([p], ["bf16"], "cuda")
    ws = torch.empty(ep.workspace_size([p]), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    batch = ep.BatchArgs([p], ["bf16"], outs, None, ws)
    batch.prepare(ep.C.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    rec = ws[:DEVTENSOR_BYTES].cpu().numpy().view(np.uint32)
    raw = {name: int(rec[off // 4]) for name, off in FIELD_OFFSET.items()}
    assert raw["call"] != 0
    # the form the decoder runs: the host's choice unless the build ruled it out
    raw["split"] = int(raw["split"] != 0 and raw["bad_split"] != raw["call"])
    raw["bytev"] = int(raw["bytev"] != 0 and raw["bad_bytes"] != raw["call"])
    return raw


def _parity(ct, kinds, label):
    p = ep.PackedTensor.from_arrays(ct, device="cuda")
    for kind in kinds:
        ref, rst = oracle.decode(ct, kind)
        out, st = ep.decode_tensor(p, kind, with_status=True)
        torch.cuda.synchronize()
        assert np.all(rst == 0) and np.all(st.cpu().numpy()[: ct.T] == 0), f"{label} {kind}: tile status"
        got = out.view(torch.int16).cpu().numpy().view(np.uint16) if kind == "bf16" else out.cpu().numpy()
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            raise AssertionError(f"{label} {kind}: {len(bad)} mismatches, first at {bad[:4].tolist()}")


def _encode(rows, cols, target, coding="standard", outliers=0.0):
    W = synthgen.student_t_weights(rows, cols, 81, bf16=True, outlier_frac=outliers).numpy()
    return oracle.encode(W, target, b=11, coding=coding)


def _run(ct, expect, label, kinds=("bf16", "int8", "lattice2x")):
    flags = _read_flags(ct)
    got = {k: flags[k] for k in expect}
    assert got == expect, f"{label}: decoder chose {got}, expected {expect}"
    _parity(ct, kinds, label)


def test_fp16_byte_entries_kept_on_a_direct_packed_tensor():
    ct = _encode(256, 4096, 4.3)
    assert int(ct.alphabet[1:].max()) <= 512 and _max_f(ct, range(1, 15)) <= 255
    _run(ct, {"variant": P11, "direct": 1, "byte_cand": 1, "bytev": 1}, "fp16 byte entries")


def test_fp16_byte_entries_dropped_when_a_frequency_exceeds_255():
    ct = _encode(256, 4096, 2.0)
    assert _max_f(ct, range(1, 15)) > 255
    _run(ct, {"variant": P11, "direct": 1, "byte_cand": 1, "bytev": 0}, "fp16 byte entries dropped")


def test_i16_byte_entries_kept_on_a_wide_tensor():
    ct = _encode(512, 4096, 5.0, outliers=0.002)
    assert 512 < int(ct.alphabet[1:].max()) <= 1024 and _max_f(ct, range(1, 17)) <= 255
    _run(ct, {"variant": W11, "byte_cand": 2, "bytev": 1}, "i16 byte entries, wide")


def test_i16_byte_entries_dropped_on_a_wide_tensor_when_a_frequency_exceeds_255():
    ct = _encode(512, 4096, 4.5, outliers=0.002)
    assert 512 < int(ct.alphabet[1:].max()) <= 1024 and _max_f(ct, range(1, 17)) > 255
    _run(ct, {"variant": W11, "byte_cand": 2, "bytev": 0}, "i16 byte entries dropped, wide")


def test_i16_byte_entries_on_a_packed_tensor_that_is_not_direct():
    # coset 0 of field 1 moved 600 below coset 1: the field spans too much for direct entries
    ct = _shift(_encode(1024, 4096, 5.0), 1, -600)
    assert int(ct.alphabet[1:].max()) <= 512 and _max_f(ct, range(1, 17)) <= 255
    _run(ct, {"variant": P11, "direct": 0, "byte_cand": 2, "bytev": 1}, "i16 byte entries, packed")


def test_no_byte_entries_when_values_leave_16_bits():
    ct = _shift(_encode(512, 4096, 5.0, outliers=0.002), 3, 20000)
    _run(ct, {"variant": W11, "byte_cand": 0, "bytev": 0}, "values beyond 16 bits, wide")


@pytest.mark.parametrize("coding, target, outliers", [("standard", 6.2, 0.002), ("pooled", 6.0, 0.002),
                                                      ("direct_z8", 6.0, 0.002)])
def test_hybrid_b11_per_slot_entries(coding, target, outliers):
    ct = _encode(512, 4096, target, coding=coding, outliers=outliers)
    assert ct.b == 11 and int(ct.alphabet[1:].max()) > 1024 and _max_f(ct, range(1, 17)) < 128
    _run(ct, {"variant": H11, "split": 1}, f"hybrid b=11 per-slot entries, {coding}")


def test_hybrid_b11_per_slot_entries_dropped_when_a_frequency_reaches_128():
    ct = _encode(512, 4096, 5.0, outliers=0.01)
    assert ct.b == 11 and int(ct.alphabet[1:].max()) > 1024 and _max_f(ct, range(1, 17)) >= 128
    _run(ct, {"variant": H11, "split": 0}, "hybrid b=11, f >= 128")


@pytest.mark.parametrize("coding", ["standard", "direct_z8"])
def test_hybrid_b11_falls_back_when_values_leave_16_bits(coding):
    # every f < 128, but table 3's values moved past 2^15: the slot maps and
    # per-symbol entries decode it instead of the per-slot entries
    base = _encode(512, 4096, 6.2 if coding == "standard" else 6.0, coding=coding, outliers=0.002)
    assert _max_f(base, range(1, 17)) < 128
    ct = _shift(base, 3, 17000)
    _run(ct, {"variant": H11, "split": 0}, f"hybrid b=11 i16 fallback, {coding}")


def _read_batch_variants(cts):
    ps = [ep.PackedTensor.from_arrays(ct, device="cuda") for ct in cts]
    outs = ep.alloc_outputs(ps, ["bf16"] * len(ps), "cuda")
    ws = torch.empty(ep.workspace_size(ps), dtype=torch.uint8, device="cuda")
    batch = ep.BatchArgs(ps, ["bf16"] * len(ps), outs, None, ws)
    batch.prepare(ep.C.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    rec = ws[: DEVTENSOR_BYTES * len(ps)].cpu().numpy().view(np.uint32)
    return [int(rec[(i * DEVTENSOR_BYTES + FIELD_OFFSET["variant"]) // 4]) for i in range(len(ps))]


def test_packed_tensors_join_the_wide_launch_of_their_batch():
    # a packed-size tensor decodes in the wide layout when its batch has a wide
    # tensor at the same b (one launch instead of two), except with a one-symbol
    # table, whose f = 2^11 the wide entries cannot hold; alone it stays packed
    packed = _encode(256, 4096, 4.3)
    wide = _encode(512, 4096, 5.0, outliers=0.002)
    single = oracle.encode(np.zeros((16, 256), np.float32), 4.0, b=11)
    assert int(packed.alphabet[1:].max()) <= 512 and 512 < int(wide.alphabet[1:].max()) <= 1024
    assert single.b == 11 and any(single.alphabet[k] == 1 for k in range(1, 17))
    assert _read_batch_variants([packed]) == [P11]
    assert _read_batch_variants([packed, wide, single]) == [W11, W11, P11]
    cts = [packed, wide, single]
    for kind in ("bf16", "int8", "lattice2x"):
        outs, sts = ep.decode_batch([ep.PackedTensor.from_arrays(ct, device="cuda") for ct in cts], [kind] * 3,
                                    with_status=True)
        torch.cuda.synchronize()
        for i, ct in enumerate(cts):
            ref, rst = oracle.decode(ct, kind)
            out = outs[i]
            got = out.view(torch.int16).cpu().numpy().view(np.uint16) if kind == "bf16" else out.cpu().numpy()
            assert np.all(rst == 0) and np.all(sts[i].cpu().numpy()[: ct.T] == 0), f"tensor {i} {kind}: status"
            assert np.array_equal(got, ref), f"tensor {i} {kind}: {int(np.sum(got != ref))} mismatches"
