"""GPU parity at the workloads' full sizes, in the benchmark's launch configuration.

Inputs are the benchmark's seeded tensors at their real shapes, compressed by
the host encoder (pinned byte-identical to the oracle's encoder by
test_host_encoder.py).  Every tensor of a set is decoded by one
ep_decode_batch call, as bench.py does.  Small sets are compared whole against
the oracle; for the large sets every tile status is checked and sampled tiles
(first, last and random ones) are decoded by the oracle one by one and
compared byte for byte.
"""
import os
import time

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
    cts = []
    t0 = time.time()
    for i, s in enumerate(specs):
        W = s.weights(device="cuda").cpu().numpy()
        cts.append(encoder.encode(W, s.target_bpp, V=s.vectors_per_tile or 0, b=s.prob_bits or 0,
                                  route=s.route, threads=THREADS))
        del W
        if (i + 1) % 25 == 0:
            _log(f"[fullsize] encoded {i + 1}/{len(specs)} ({time.time() - t0:.0f}s)")
    return cts


def _decode_batch(cts, kinds):
    packed = [ep.PackedTensor.from_arrays(ct, device="cuda") for ct in cts]
    outs, sts = ep.decode_batch(packed, kinds, with_status=True)
    torch.cuda.synchronize()
    for ct, st in zip(cts, sts):
        s = st.cpu().numpy()[: ct.T]
        assert np.all(s == 0), f"{ct.rows}x{ct.cols}: tile status {np.unique(s)}"
    return outs


def _flat(out, kind):
    tv, nv = NP_VIEW[kind]
    return out.view(tv).reshape(-1), nv


def _check_sampled(cts, kinds, outs, per_tensor, rng):
    bufs = {}
    checked = 0
    for ct, kind, out in zip(cts, kinds, outs):
        if ct.T == 0:
            continue
        flat, nv = _flat(out, kind)
        key = (ct.rows, ct.cols, kind)
        if key not in bufs:
            bufs[key] = np.zeros((ct.rows, ct.cols), nv)
        ref = bufs[key]
        picks = {0, ct.T - 1} | set(rng.integers(0, ct.T, size=per_tensor).tolist())
        nvec = ct.rows * ct.cols // 8
        for t in sorted(picks):
            _, st = oracle.decode(ct, kind, t, t + 1, out=ref)
            assert st[t] == 0
            a, b = 8 * t * ct.V, 8 * min((t + 1) * ct.V, nvec)
            got = flat[a:b].cpu().numpy().view(nv)
            exp = ref.reshape(-1)[a:b]
            if not np.array_equal(got, exp):
                bad = np.flatnonzero(got != exp)
                raise AssertionError(f"{ct.rows}x{ct.cols} {kind} tile {t}: {bad.size} mismatches, "
                                     f"first at weight {a + bad[0]}")
            checked += 1
    return checked


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


@pytest.mark.timeout(600)
def test_dit_set_full_batch_sampled_tiles():
    specs = synthgen.workload("dit_linear_set_30x5_4bpp_bf16")
    cts = _encode(specs)
    outs = _decode_batch(cts, ["bf16"] * len(cts))
    n = _check_sampled(cts, ["bf16"] * len(cts), outs, 3, np.random.default_rng(3))
    _log(f"[fullsize] DiT set: {len(cts)} tensors, all tile statuses ok, {n} sampled tiles bit-exact")


@pytest.mark.timeout(300)
def test_llm_fp8_route_two_layers_sampled_tiles():
    specs = synthgen.workload("llm_prefill_16x5_fp8route_5bpp")[:10]
    cts = _encode(specs)
    outs = _decode_batch(cts, ["fp8"] * len(cts))
    n = _check_sampled(cts, ["fp8"] * len(cts), outs, 6, np.random.default_rng(4))
    _log(f"[fullsize] LLM FP8 route: {len(cts)} tensors, {n} sampled tiles bit-exact")


@pytest.mark.timeout(300)
def test_mixed_int8_route_subset_sampled_tiles():
    specs = synthgen.workload("mixed_300_int8route_2or8bpp")[:60]
    assert any(s.target_bpp == 8.0 for s in specs) and any(s.target_bpp == 2.0 for s in specs)
    cts = _encode(specs)
    outs = _decode_batch(cts, ["int8"] * len(cts))
    n = _check_sampled(cts, ["int8"] * len(cts), outs, 4, np.random.default_rng(5))
    _log(f"[fullsize] mixed INT8 route: {len(cts)} tensors (b {sorted({c.b for c in cts})}), "
         f"{n} sampled tiles bit-exact")
