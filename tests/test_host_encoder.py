"""The host encoder library against the CPU oracle's encoder.

The benchmark and the full-size GPU tests compress their inputs with the
multithreaded host encoder (dit_weight_compression_amd/csrc/ep_encode.cpp).
These tests pin it to the oracle: on the same input it must produce the same
container byte for byte (scale, precision, tables, row scales, states,
offsets, payload), so a container from either side is the oracle's container.
"""
import numpy as np
import pytest

import oracle
import synthgen
from dit_weight_compression_amd import encoder

ARRAYS = ("row_scales", "states", "offsets", "payload", "freqs", "alphabet", "minval", "freq_base")


def _assert_identical(o, e):
    for f in ("rows", "cols", "V", "T", "b", "route"):
        assert getattr(o, f) == getattr(e, f), f
    assert np.float32(o.s).tobytes() == np.float32(e.s).tobytes()
    for f in ARRAYS:
        a, b = np.asarray(getattr(o, f)), np.asarray(getattr(e, f))
        assert a.shape == b.shape and a.tobytes() == b.tobytes(), f
    if o.route != "direct":
        assert np.asarray(o.route_scales).tobytes() == np.asarray(e.route_scales).tobytes()
    assert o.stored_bytes == e.stored_bytes


@pytest.mark.parametrize("case", [
    ("w256x512 4bpp b12 V512", lambda: synthgen.workload("w256x512_4bpp_fp32")[0].weights().numpy(),
     4.0, 512, 12, "direct"),
    ("300x1024 outliers 8bpp", lambda: synthgen.student_t_weights(300, 1024, 5, outlier_frac=0.001).numpy(),
     8.0, 0, 0, "direct"),
    ("200x768 fp8 route 5bpp", lambda: synthgen.student_t_weights(200, 768, 6).numpy(), 5.0, 0, 0, "fp8"),
    ("200x768 int8 route 2bpp", lambda: synthgen.student_t_weights(200, 768, 7).numpy(), 2.0, 0, 0, "int8"),
    ("37x264 ragged 3bpp", lambda: synthgen.student_t_weights(37, 264, 8).numpy(), 3.0, 0, 0, "direct"),
], ids=lambda c: c[0])
def test_host_encoder_matches_oracle(case):
    _, make, target, V, b, route = case
    W = make()
    o = oracle.encode(W, target, V=V, b=b, route=route)
    e = encoder.encode(W, target, V=V, b=b, route=route, threads=4)
    _assert_identical(o, e)


def test_host_encoder_matches_oracle_with_precision_escalation():
    # 0.1% outliers x20 at 8 bpp: the alphabet outgrows 2^12 and b is raised
    W = synthgen.workload("w3840_8bpp")[0].weights().numpy()[:960]
    o = oracle.encode(W, 8.0)
    e = encoder.encode(W, 8.0, threads=8)
    _assert_identical(o, e)
    assert o.b > 12


def test_host_encoder_thread_count_does_not_change_output():
    W = synthgen.student_t_weights(128, 1024, 9).numpy()
    a = encoder.encode(W, 4.0, threads=1)
    b = encoder.encode(W, 4.0, threads=7)
    _assert_identical(a, b)
