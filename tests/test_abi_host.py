"""Host-side checks of the C ABI (no GPU needed).

The HIP library and the host encoder library must load, export every function
their headers declare, and reject malformed descriptors before touching the
device (argument errors are returned synchronously, before any launch).
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import dit_weight_compression_amd as ep
from dit_weight_compression_amd import encoder

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(ep_\w+)\s*\(", text, flags=re.M)))


def test_decoder_library_exports_every_declared_function():
    names = _declared_functions("entropack.h")
    assert set(names) == set(ep.EXPORTS), names
    L = ep.lib()
    for n in names:
        assert hasattr(L, n), n


def test_encoder_library_exports_every_declared_function():
    names = _declared_functions("entropack_encode.h")
    assert set(names) == set(encoder.EXPORTS), names
    L = encoder.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = ep.lib()
    text = open(os.path.join(ROOT, "include", "entropack.h")).read()
    version = int(re.search(r"#define EP_ABI_VERSION (\d+)", text).group(1))
    assert L.ep_abi_version() == version
    assert L.ep_status_string(ep.EP_OK) == b"EP_OK"
    assert L.ep_status_string(ep.EP_ERR_INVALID_ARG) == b"EP_ERR_INVALID_ARG"
    assert L.ep_status_string(ep.EP_ERR_WORKSPACE) == b"EP_ERR_WORKSPACE"
    assert L.ep_status_string(12345) == b"EP_UNKNOWN_STATUS"


def _desc(rows=64, cols=256, V=64, b=11, fake_ptr=0x1000):
    d = ep.EpTensorDesc()
    d.rows, d.cols, d.vectors_per_tile, d.prob_bits = rows, cols, V, b
    nvec = rows * cols // 8
    d.num_tiles = (nvec + V - 1) // V
    d.scale = 0.5
    for f in ("row_scales", "tile_states", "tile_offsets", "payload", "freqs"):
        setattr(d, f, fake_ptr)
    d.payload_words = 100
    d.alphabet[0] = 2
    for k in range(1, 17):
        d.alphabet[k] = 8
        d.min_offset[k] = -4
        d.freq_base[k] = 2 + 8 * (k - 1)
    return d


def _ws_status(d, n=1):
    L = ep.lib()
    size = C.c_size_t(0)
    arr = (ep.EpTensorDesc * n)(*([d] * n))
    rc = L.ep_workspace_size(C.cast(arr, C.c_void_p), n, C.byref(size))
    return rc, size.value, L.ep_last_error().decode()


def test_workspace_size_of_valid_descriptors():
    rc, size, _ = _ws_status(_desc())
    assert rc == ep.EP_OK and size > 0 and size % 256 == 0
    rc2, size2, _ = _ws_status(_desc(), n=3)
    assert rc2 == ep.EP_OK and size2 > size
    L = ep.lib()
    zero = C.c_size_t(7)
    assert L.ep_workspace_size(None, 0, C.byref(zero)) == ep.EP_OK and zero.value >= 0


@pytest.mark.parametrize("mutate, needle", [
    (lambda d: setattr(d, "cols", 12), "cols"),
    (lambda d: setattr(d, "rows", -1), "rows"),
    (lambda d: setattr(d, "vectors_per_tile", 16), "vectors_per_tile"),
    (lambda d: setattr(d, "vectors_per_tile", 8000), "vectors_per_tile"),
    (lambda d: setattr(d, "prob_bits", 8), "prob_bits"),
    (lambda d: setattr(d, "prob_bits", 16), "prob_bits"),
    (lambda d: setattr(d, "num_tiles", 3), "num_tiles"),
    (lambda d: d.alphabet.__setitem__(0, 3), "coset bit"),
    (lambda d: d.alphabet.__setitem__(5, 4096), "alphabet"),
    (lambda d: d.min_offset.__setitem__(3, -(1 << 20)), "2^19"),
    (lambda d: setattr(d, "payload", 0x1002), "aligned"),
    (lambda d: setattr(d, "freqs", None), "NULL"),
    (lambda d: setattr(d, "field8", 2), "field8"),
])
def test_malformed_descriptors_are_rejected(mutate, needle):
    d = _desc()
    mutate(d)
    rc, _, msg = _ws_status(d)
    assert rc == ep.EP_ERR_INVALID_ARG, (rc, msg)
    assert needle in msg, msg


def test_prepare_rejects_missing_plan_and_small_workspace():
    L = ep.lib()
    d = _desc()
    arr = (ep.EpTensorDesc * 1)(d)
    dt = (C.c_int * 1)(0)
    outs = (C.c_void_p * 1)(0x2000)
    vp = C.c_void_p
    assert L.ep_batch_prepare(C.cast(arr, vp), C.cast(dt, vp), C.cast(outs, vp), None, 1,
                              None, 0, None, None) == ep.EP_ERR_INVALID_ARG
    plan = ep.EpBatchPlan()
    rc = L.ep_batch_prepare(C.cast(arr, vp), C.cast(dt, vp), C.cast(outs, vp), None, 1,
                            None, 0, None, C.byref(plan))
    assert rc == ep.EP_ERR_WORKSPACE
    bad = (C.c_int * 1)(7)
    rc = L.ep_batch_prepare(C.cast(arr, vp), C.cast(bad, vp), C.cast(outs, vp), None, 1,
                            None, 0, None, C.byref(plan))
    assert rc == ep.EP_ERR_INVALID_ARG and b"dtype" in L.ep_last_error()
    # a plan that prepare did not fill is refused by launch
    assert L.ep_batch_launch(C.byref(ep.EpBatchPlan()), None) == ep.EP_ERR_INVALID_ARG


def test_noalloc_entry_point_rejects_batches_beyond_its_scratch():
    # the checks run on the host before any HIP call: no GPU needed
    L = ep.lib()
    vp = C.c_void_p
    d = _desc(rows=4096, cols=4096, V=32)
    rc, one, _ = _ws_status(d)
    assert rc == ep.EP_OK
    n = ep.NOALLOC_SCRATCH_BYTES // one + 1
    rc, total, _ = _ws_status(d, n)
    assert rc == ep.EP_OK and total > ep.NOALLOC_SCRATCH_BYTES
    arr = (ep.EpTensorDesc * n)(*([d] * n))
    dt = (C.c_int * n)(*([0] * n))
    outs = (C.c_void_p * n)(*([0x2000] * n))
    rc = L.ep_decode_batch_noalloc(C.cast(arr, vp), C.cast(dt, vp), C.cast(outs, vp), None, n, None)
    msg = L.ep_last_error().decode()
    assert rc == ep.EP_ERR_WORKSPACE, (rc, msg)
    assert str(total) in msg and str(ep.NOALLOC_SCRATCH_BYTES) in msg
    # malformed arguments are refused the same way as by ep_decode_batch
    assert L.ep_decode_batch_noalloc(C.cast(arr, vp), None, C.cast(outs, vp), None, 1, None) == ep.EP_ERR_INVALID_ARG
    bad = _desc()
    bad.cols = 12
    arr1 = (ep.EpTensorDesc * 1)(bad)
    assert L.ep_decode_batch_noalloc(C.cast(arr1, vp), C.cast(dt, vp), C.cast(outs, vp), None, 1,
                                     None) == ep.EP_ERR_INVALID_ARG
    text = open(os.path.join(ROOT, "include", "entropack.h")).read()
    assert int(re.search(r"#define EP_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(1)) << 20 \
        == ep.NOALLOC_SCRATCH_BYTES


def test_python_binding_has_no_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(ep, "_lib", None)
    monkeypatch.setattr(ep, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        ep.lib()


def test_device_encoder_exports_every_declared_function():
    names = _declared_functions("entropack_device_encode.h")
    assert set(names) == set(ep.DEVICE_ENCODE_EXPORTS), names
    L = ep.lib()
    for n in names:
        assert hasattr(L, n), n


def test_device_encoder_workspace_size_and_argument_errors():
    import ctypes as C
    from dit_weight_compression_amd import encoder as enc
    L = ep.lib()
    n = C.c_size_t()
    bad = [(-1, 64, 4.0, 0, 0), (4, 60, 4.0, 0, 0), (4, 0, 4.0, 0, 0), (4, 64, 4.0, 31, 0),
           (4, 64, 4.0, 0, 3), (4, 64, 0.0, 0, 0), (4, 64, float("nan"), 0, 0)]
    for rows, cols, tgt, V, route in bad:
        assert L.ep_encode_device_workspace_size(rows, cols, tgt, V, route, C.byref(n)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device_workspace_size(4, 64, 4.0, 0, 0, None) == ep.EP_ERR_INVALID_ARG
    # the per-weight arrays dominate: 36 B of fields per vector, 18 B of word scratch per tiled vector
    sizes = {}
    for rows, route in ((1000, 0), (2000, 0), (2000, 1)):
        assert L.ep_encode_device_workspace_size(rows, 1024, 4.0, 0, route, C.byref(n)) == ep.EP_OK
        sizes[rows, route] = n.value
        nvec = rows * 1024 // 8
        V = 16384 // 9
        T = -(-nvec // V)
        assert n.value >= 36 * nvec + 18 * T * V + (4 * rows * 1024 if route else 0)
    assert sizes[2000, 0] > sizes[1000, 0] and sizes[2000, 1] > sizes[2000, 0]
    # argument checks happen on the host, before any device call
    info = enc.EncodedInfo()
    fake = C.c_void_p(1 << 40)
    ws_need = ep.encode_device_workspace_size(8, 64, 4.0)
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 0, 0, 0, fake, ws_need, None, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device(None, 8, 64, 4.0, 0, 0, 0, 0, fake, ws_need, None, C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device(C.c_void_p((1 << 40) + 4), 8, 64, 4.0, 0, 0, 0, 0, fake, ws_need, None,
                              C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 8, 0, 0, fake, ws_need, None, C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 16, 0, 0, fake, ws_need, None, C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 0, 0, 0, fake, ws_need - 1, None,
                              C.byref(info)) == ep.EP_ERR_WORKSPACE
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 0, 0, 0, None, ws_need, None, C.byref(info)) == ep.EP_ERR_WORKSPACE
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 0, 0, 0, C.c_void_p((1 << 40) + 128), ws_need, None,
                              C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert b"aligned" in L.ep_last_error()
    assert L.ep_encode_device(fake, 8, 64, 4.0, 0, 0, 0, 3, fake, ws_need, None,
                              C.byref(info)) == ep.EP_ERR_INVALID_ARG
    # emit rejects a header that does not describe an encoded tensor
    info.rows, info.cols, info.vectors_per_tile, info.num_tiles = 8, 64, 32, 99
    assert L.ep_encode_device_emit(fake, C.byref(info), None, None, None, None, None, None,
                                   None) == ep.EP_ERR_INVALID_ARG


def test_convert_argument_errors():
    import ctypes as C
    L = ep.lib()
    fake = C.c_void_p(1 << 40)
    assert L.ep_convert_f32(fake, fake, 6, 0, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_convert_f32(None, fake, 8, 0, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_convert_f32(C.c_void_p((1 << 40) + 8), fake, 8, 0, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_convert_f32(fake, C.c_void_p((1 << 40) + 4), 8, 0, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_convert_f32(fake, fake, 8, 100, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_convert_f32(fake, fake, 8, 4, None) == ep.EP_ERR_INVALID_ARG   # FP32 needs no rounding
    assert L.ep_convert_f32(fake, fake, 0, 0, None) == ep.EP_OK


def test_device_refinement_workspace_size_and_argument_errors():
    import ctypes as C
    from dit_weight_compression_amd import encoder as enc
    L = ep.lib()
    n = C.c_size_t()
    for K in (0, 33):
        assert L.ep_encode_device_rdo_workspace_size(64, 256, 3.0, 0, 0, K, C.byref(n)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device_rdo_workspace_size(64, 60, 3.0, 0, 0, 5, C.byref(n)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device_rdo_workspace_size(64, 256, 3.0, 0, 0, 5, None) == ep.EP_ERR_INVALID_ARG
    base = ep.encode_device_workspace_size(1000, 1024, 3.0)
    sizes = [ep.encode_device_rdo_workspace_size(1000, 1024, 3.0, candidates=K) for K in (1, 5, 9)]
    nvec = 1000 * 1024 // 8
    # every candidate keeps its own fields (36 B per vector)
    assert sizes[0] >= base + 36 * nvec and sizes[1] - sizes[0] >= 4 * 36 * nvec and sizes[2] > sizes[1]
    info = enc.EncodedInfo()
    fake = C.c_void_p(1 << 40)
    need = ep.encode_device_rdo_workspace_size(8, 64, 3.0, candidates=5)
    for K in (0, 33):
        assert L.ep_encode_device_rdo(fake, 8, 64, 3.0, 0, 0, 0, K, 1, fake, need, None,
                                      C.byref(info)) == ep.EP_ERR_INVALID_ARG
    assert L.ep_encode_device_rdo(fake, 8, 64, 3.0, 0, 0, 0, 5, 1, fake, need - 1, None,
                                  C.byref(info)) == ep.EP_ERR_WORKSPACE
    assert L.ep_encode_device_rdo(fake, 8, 64, 3.0, 0, 0, 0, 5, 1, fake, need, None, None) == ep.EP_ERR_INVALID_ARG
