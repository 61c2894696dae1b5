"""GPU parity at the workloads' full sizes, in the benchmark's launch configuration.

Inputs are the benchmark's seeded tensors at their real shapes, compressed by
the host encoder (pinned byte-identical to the oracle's encoder by
test_host_encoder.py).  Every tensor of a set is decoded by one
ep_decode_batch call, as bench.py does, and every tensor is compared whole,
byte for byte, against the oracle's decode of the same container (the oracle
runs on host threads, one tensor per thread).
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")
from dit_weight_compression_amd import encoder  # noqa: E402

THREADS = min(16, os.cpu_count() or 1)
NP_VIEW = {"bf16": (torch.int16, np.uint16), "fp8": (torch.uint8, np.uint8),
           "int8": (torch.int8, np.int8)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _log(msg):
    print(msg, flush=True)


def _encode(specs):
    """Host-encode every spec; a few tensors at a time, each on a share of the threads."""
    par = 4 if len(specs) >= 8 else 1
    per = max(1, THREADS // par)

    def one(s):
        W = s.weights(device="cuda").cpu().numpy()
        return encoder.encode(W, s.target_bpp, V=s.vectors_per_tile or 0, b=s.prob_bits or 0,
                              route=s.route, threads=per)

    t0 = time.time()
    with ThreadPoolExecutor(par) as pool:
        cts = list(pool.map(one, specs))
    _log(f"[fullsize] host-encoded {len(cts)} tensors in {time.time() - t0:.0f}s")
    return cts


def _decode_batch(cts, kinds):
    packed = [ep.PackedTensor.from_arrays(ct, device="cuda") for ct in cts]
    outs, sts = ep.decode_batch(packed, kinds, with_status=True)
    torch.cuda.synchronize()
    for ct, st in zip(cts, sts):
        s = st.cpu().numpy()[: ct.T]
        assert np.all(s == 0), f"{ct.rows}x{ct.cols}: tile status {np.unique(s)}"
    return outs


def _compare_whole(cts, kinds, outs):
    """Every tensor against the oracle, byte for byte; oracle decodes on host threads."""
    def ref(i):
        r, st = oracle.decode(cts[i], kinds[i])
        return r, st

    t0 = time.time()
    weights = 0
    with ThreadPoolExecutor(THREADS) as pool:
        for lo in range(0, len(cts), 2 * THREADS):          # bounded number of references in flight
            idx = list(range(lo, min(len(cts), lo + 2 * THREADS)))
            for i, (r, st) in zip(idx, pool.map(ref, idx)):
                ct, kind = cts[i], kinds[i]
                assert np.all(st == 0), f"tensor {i}: oracle tile status {np.unique(st)}"
                tv, nv = NP_VIEW[kind]
                got = outs[i].view(tv).cpu().numpy().view(nv).reshape(ct.rows, ct.cols)
                if not np.array_equal(got, r):
                    bad = np.flatnonzero(got.reshape(-1) != r.reshape(-1))
                    raise AssertionError(f"tensor {i} ({ct.rows}x{ct.cols}, b={ct.b}, {kind}): "
                                         f"{bad.size} mismatches, first at weight {bad[0]} "
                                         f"(tile {bad[0] // (8 * ct.V)})")
                weights += ct.rows * ct.cols
    _log(f"[fullsize] {len(cts)} tensors, {weights / 1e9:.3f} G weights bit-exact "
         f"(oracle compare {time.time() - t0:.0f}s)")
    return weights


def test_w3840_every_target_whole_tensor():
    specs = [synthgen.workload(f"w3840_{t}bpp")[0] for t in (4, 5, 6, 7, 8)]
    cts = _encode(specs)
    bs = sorted({ct.b for ct in cts})
    outs = _decode_batch(cts, ["bf16"] * len(cts))
    for ct, out in zip(cts, outs):
        ref, _ = oracle.decode(ct, "bf16")
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), f"b={ct.b} bpp={ct.bpp:.3f}"
    _log(f"[fullsize] 3840x3840 at 4..8 bpp, precisions {bs}: whole tensors bit-exact")


@pytest.mark.timeout(900)
def test_dit_set_whole_batch_bit_exact():
    specs = synthgen.workload("dit_linear_set_30x5_4bpp_bf16")
    assert len(specs) == 150
    cts = _encode(specs)
    kinds = ["bf16"] * len(cts)
    outs = _decode_batch(cts, kinds)
    assert _compare_whole(cts, kinds, outs) == sum(s.rows * s.cols for s in specs)


@pytest.mark.timeout(900)
def test_llm_fp8_set_whole_batch_bit_exact():
    specs = synthgen.workload("llm_prefill_16x5_fp8route_5bpp")
    assert len(specs) == 80
    cts = _encode(specs)
    kinds = ["fp8"] * len(cts)
    outs = _decode_batch(cts, kinds)
    assert _compare_whole(cts, kinds, outs) == sum(s.rows * s.cols for s in specs)


@pytest.mark.timeout(900)
def test_mixed_int8_set_whole_batch_bit_exact():
    specs = synthgen.workload("mixed_300_int8route_2or8bpp")
    assert len(specs) == 300
    assert any(s.target_bpp == 8.0 for s in specs) and any(s.target_bpp == 2.0 for s in specs)
    cts = _encode(specs)
    assert len({c.b for c in cts}) >= 2                    # several probability precisions in one batch
    kinds = ["int8"] * len(cts)
    outs = _decode_batch(cts, kinds)
    assert _compare_whole(cts, kinds, outs) == sum(s.rows * s.cols for s in specs)
