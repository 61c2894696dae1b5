"""GPU parity of the device compressor (ep_encode_device) against the oracle.

The device compressor must produce the oracle's container byte for byte:
scale, probability precision, tables, row scales, route scales, terminal
states, tile offsets and payload.  Small cases compare against the CPU
oracle's encoder directly; the full-size layer compares against the host
compressor, which tests/test_host_encoder.py pins to the oracle on the same
algorithm.  Every container is also decoded by the GPU decoder with all tile
statuses OK.
"""
import numpy as np
import pytest
import torch

import oracle
import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")
from dit_weight_compression_amd import encoder  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _host_arrays(d):
    """The device container's arrays as numpy, in the oracle's dtypes."""
    p = d.packed
    torch.cuda.synchronize()
    R, T = p.rows, p.T
    out = dict(
        row_scales=p.row_scales.cpu().numpy()[:R],
        states=p.states.cpu().numpy().view(np.uint32)[: 32 * T],
        offsets=p.offsets.cpu().numpy().view(np.uint32)[: T + 1],
        payload=p.payload.cpu().numpy().view(np.uint16)[: p.nwords],
        freqs=p.freqs.cpu().numpy().view(np.uint16)[: d.num_freqs],
        alphabet=p.alphabet, minval=p.minval, freq_base=p.freq_base,
    )
    if d.route != "direct":
        out["route_scales"] = d.route_scales.cpu().numpy()[:R]
    return out


def _assert_same_container(ref, d, label):
    p = d.packed
    for f in ("rows", "cols", "V", "T", "b"):
        assert getattr(ref, f) == getattr(p, f), f"{label}: {f}"
    assert np.float32(ref.s).tobytes() == np.float32(p.s).tobytes(), f"{label}: scale"
    got = _host_arrays(d)
    names = ["row_scales", "states", "offsets", "payload", "freqs", "alphabet", "minval", "freq_base"]
    if d.route != "direct":
        names.append("route_scales")
    for f in names:
        a = np.asarray(getattr(ref, f))
        b = got[f]
        assert a.shape == b.shape, f"{label}: {f} shape {a.shape} vs {b.shape}"
        if a.tobytes() != b.tobytes():
            bad = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
            raise AssertionError(f"{label}: {f} differs at {len(bad)} positions, first {bad[:5].tolist()}")
    assert ref.stored_bytes == p.stored_bytes, f"{label}: stored bytes"


def _decode_ok(d, kind="bf16"):
    p = d.packed
    if p.T == 0:
        return None
    out, st = ep.decode_tensor(p, kind, with_status=True)
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy()[: p.T] == 0)
    return out


CASES = [
    ("w256x512 4bpp b12 V512", lambda: synthgen.workload("w256x512_4bpp_fp32")[0].weights().numpy(),
     4.0, 512, 12, "direct"),
    ("w256x512 4bpp S4096", lambda: synthgen.workload("w256x512_4bpp_fp32")[0].weights().numpy(),
     4.0, 455, 12, "direct"),
    ("300x1024 outliers 8bpp", lambda: synthgen.student_t_weights(300, 1024, 5, outlier_frac=0.001).numpy(),
     8.0, 0, 0, "direct"),
    ("200x768 fp8 route 5bpp", lambda: synthgen.student_t_weights(200, 768, 6).numpy(), 5.0, 0, 0, "fp8"),
    ("200x768 int8 route 2bpp", lambda: synthgen.student_t_weights(200, 768, 7).numpy(), 2.0, 0, 0, "int8"),
    ("37x264 ragged 3bpp", lambda: synthgen.student_t_weights(37, 264, 8).numpy(), 3.0, 0, 0, "direct"),
    ("33x64 V50 ragged tail", lambda: synthgen.student_t_weights(33, 64, 7).numpy(), 4.0, 50, 0, "direct"),
    ("1x8 single vector", lambda: synthgen.student_t_weights(1, 8, 12).numpy(), 4.0, 0, 0, "direct"),
    ("64x256 6bpp b9", lambda: synthgen.student_t_weights(64, 256, 13).numpy(), 6.0, 0, 9, "direct"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_device_encoder_matches_oracle(case):
    label, make, target, V, b, route = case
    W = make()
    print(f"[device encoder] {label} shape={W.shape}", flush=True)
    ref = oracle.encode(W, target, V=V, b=b, route=route)
    d = ep.encode_device(torch.from_numpy(W).cuda(), target, V=V, b=b, route=route)
    _assert_same_container(ref, d, label)
    assert d.est_bpp == pytest.approx(ref.est_bpp, rel=1e-12)
    _decode_ok(d)


def test_device_encoder_zero_row_and_empty_tensor():
    W = synthgen.student_t_weights(16, 128, 8).numpy()
    W[3] = 0.0
    ref = oracle.encode(W, 4.0, V=32)
    d = ep.encode_device(torch.from_numpy(W).cuda(), 4.0, V=32)
    _assert_same_container(ref, d, "zero row")
    out = _decode_ok(d)
    assert torch.all(out[3] == 0)
    E = np.zeros((0, 64), np.float32)
    ref = oracle.encode(E, 4.0)
    d = ep.encode_device(torch.zeros((0, 64), dtype=torch.float32, device="cuda"), 4.0)
    assert d.packed.T == 0 and d.packed.nwords == 0
    _assert_same_container(ref, d, "empty")


def test_device_encoder_precision_escalation():
    # 0.1% outliers x20 at 8 bpp: the alphabet outgrows 2^12 and b is raised
    W = synthgen.workload("w3840_8bpp")[0].weights().numpy()[:960]
    print("[device encoder] escalation 960x3840", flush=True)
    ref = oracle.encode(W, 8.0)
    d = ep.encode_device(torch.from_numpy(W).cuda(), 8.0)
    assert ref.b > 12
    _assert_same_container(ref, d, "escalation")
    _decode_ok(d)


def test_device_encoder_scale_coarsening():
    # a lone outlier needs more than 2^15 symbols at the scale a 13 bpp target asks for
    W = synthgen.student_t_weights(512, 4096, 6).numpy()
    W[0, 0] = 1e4
    print("[device encoder] coarsening 512x4096", flush=True)
    ref = oracle.encode(W, 13.0)
    d = ep.encode_device(torch.from_numpy(W).cuda(), 13.0)
    assert ref.b == 15
    _assert_same_container(ref, d, "coarsening")
    _decode_ok(d)


def test_device_encoder_workspace_reuse():
    # two calls in a row on one workspace, the second smaller
    W1 = synthgen.student_t_weights(96, 512, 21).numpy()
    W2 = synthgen.student_t_weights(40, 256, 22).numpy()
    ws = torch.empty(ep.encode_device_workspace_size(96, 512, 4.0), dtype=torch.uint8, device="cuda")
    for W in (W1, W2):
        ref = oracle.encode(W, 4.0)
        d = ep.encode_device(torch.from_numpy(W).cuda(), 4.0, workspace=ws)
        _assert_same_container(ref, d, f"reuse {W.shape}")


@pytest.mark.parametrize("route", ["direct", "fp8"])
def test_device_encoder_full_reference_layer(route):
    # the reference layer shape (10240 x 3840, BF16-rounded weights) at 4 bpp
    w = synthgen.workload("ref_layer_10240x3840_4bpp_bf16")[0]
    W = w.weights().numpy()
    print(f"[device encoder] reference layer {W.shape} route={route}", flush=True)
    ref = encoder.encode(W, 4.0, route=route, threads=0)
    d = ep.encode_device(torch.from_numpy(W).cuda(), 4.0, route=route)
    _assert_same_container(ref, d, f"reference layer {route}")
    assert d.est_bpp == ref.est_bpp
    _decode_ok(d, "bf16" if route == "direct" else "fp8")


@pytest.mark.parametrize("coding", ["pooled", "direct_z8"])
@pytest.mark.parametrize("target", [2.0, 4.0, 8.0])
def test_device_encoder_table4_codings(coding, target):
    # the two ablations of the paper's Table 4: same points and scales, other tables
    W = synthgen.student_t_weights(256, 1024, 31, bf16=True).numpy()
    print(f"[device encoder] {coding} target={target}", flush=True)
    ref = oracle.encode(W, target, coding=coding)
    d = ep.encode_device(torch.from_numpy(W).cuda(), target, coding=coding)
    _assert_same_container(ref, d, f"{coding} {target}")
    assert d.packed.field8 == (1 if coding == "direct_z8" else 0)
    out = _decode_ok(d, "lattice2x")
    std = oracle.encode(W, target)
    assert np.array_equal(out.cpu().numpy(), oracle.decode(std, "lattice2x")[0])


RDO_CASES = [
    # (label, rows, cols, seed, target, K, sweeps, route)
    ("3bpp K5 one sweep", 256, 512, 3, 3.0, 5, 1, "direct"),
    ("3bpp K9 two sweeps", 192, 768, 51, 3.0, 9, 2, "direct"),
    ("4bpp K3 three sweeps, ragged rows", 77, 264, 52, 4.0, 3, 3, "direct"),
    ("2bpp K5 fp8 route", 128, 512, 53, 2.0, 5, 1, "fp8"),
    ("6bpp K4 int8 route", 96, 384, 54, 6.0, 4, 2, "int8"),
    ("K1 is the baseline", 64, 256, 55, 3.0, 1, 1, "direct"),
    ("no sweep is the baseline", 64, 256, 56, 3.0, 5, 0, "direct"),
    ("layer-width rows 1024 x 3840, 3bpp K5", 1024, 3840, 57, 3.0, 5, 1, "direct"),
]


@pytest.mark.parametrize("label, rows, cols, seed, target, K, sweeps, route", RDO_CASES)
def test_device_refinement_matches_oracle(label, rows, cols, seed, target, K, sweeps, route):
    W = synthgen.student_t_weights(rows, cols, seed).numpy()
    print(f"[rdo] {label}", flush=True)
    ref = oracle.encode_rdo(W, target, K=K, sweeps=sweeps, route=route)
    d = ep.encode_device(torch.from_numpy(W).cuda(), target, route=route, candidates=K, sweeps=sweeps)
    _assert_same_container(ref, d, label)
    out = _decode_ok(d, "bf16" if route == "direct" else route)
    ref_out, _ = oracle.decode(ref, "bf16" if route == "direct" else route)
    view = {"direct": torch.int16, "fp8": torch.uint8, "int8": torch.int8}[route]
    got = out.view(view).cpu().numpy()
    assert np.array_equal(got.view(ref_out.dtype), ref_out), label
    if K == 1 or sweeps == 0:
        _assert_same_container(oracle.encode(W, target, route=route), d, label + " (baseline)")


@pytest.mark.timeout(300)
def test_device_refinement_full_reference_layer():
    # the reference layer shape at the paper's refinement setting (3 bpp, K = 5, one sweep),
    # against the CPU oracle's refinement
    w = synthgen.workload("ref_layer_10240x3840_4bpp_bf16")[0]
    W = w.weights().numpy()
    print(f"[rdo] reference layer {W.shape}", flush=True)
    ref = oracle.encode_rdo(W, 3.0, K=5, sweeps=1)
    d = ep.encode_device(torch.from_numpy(W).cuda(), 3.0, candidates=5, sweeps=1)
    _assert_same_container(ref, d, "reference layer, refinement")
    _decode_ok(d)
