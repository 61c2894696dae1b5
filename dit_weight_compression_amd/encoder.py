"""ctypes binding of the host compressor (include/entropack_encode.h).

Produces the arrays the GPU decoder consumes; see PackedTensor.from_arrays.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ENC_LIB_PATH = os.path.join(HERE, "libentropack_encode.so")
ROUTES = {"direct": 0, "fp8": 1, "int8": 2}
EXPORTS = ["ep_encode_host", "ep_encoded_get_info", "ep_encoded_copy", "ep_encoded_free"]


class EncodedInfo(C.Structure):
    _fields_ = [
        ("rows", C.c_int64), ("cols", C.c_int64),
        ("vectors_per_tile", C.c_uint32), ("num_tiles", C.c_uint32), ("prob_bits", C.c_uint32),
        ("scale", C.c_float), ("route", C.c_int32), ("estimated_bpp", C.c_double),
        ("payload_words", C.c_uint64), ("num_freqs", C.c_uint32), ("stored_bytes", C.c_uint64),
        ("alphabet", C.c_uint32 * 17), ("min_offset", C.c_int32 * 17), ("freq_base", C.c_uint32 * 17),
        ("coding", C.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(ENC_LIB_PATH):
            raise ImportError(f"{ENC_LIB_PATH} is missing: run __graft_entry__.build()")
        L = C.CDLL(ENC_LIB_PATH)
        vp = C.c_void_p
        L.ep_encode_host.argtypes = [vp, C.c_int64, C.c_int64, C.c_double, C.c_uint32, C.c_uint32,
                                     C.c_int, C.c_int, C.POINTER(vp)]
        L.ep_encode_host.restype = C.c_int
        L.ep_encoded_get_info.argtypes = [vp, C.POINTER(EncodedInfo)]
        L.ep_encoded_get_info.restype = C.c_int
        L.ep_encoded_copy.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.ep_encoded_copy.restype = C.c_int
        L.ep_encoded_free.argtypes = [vp]
        _lib = L
    return _lib


@dataclasses.dataclass
class HostContainer:
    rows: int
    cols: int
    V: int
    T: int
    b: int
    s: float
    route: str
    est_bpp: float
    stored_bytes: int
    row_scales: np.ndarray
    route_scales: Optional[np.ndarray]
    states: np.ndarray
    offsets: np.ndarray
    payload: np.ndarray
    freqs: np.ndarray
    alphabet: np.ndarray
    minval: np.ndarray
    freq_base: np.ndarray

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def bpp(self) -> float:
        return 8.0 * self.stored_bytes / self.numel if self.numel else 0.0


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def encode(W, target_bpp: float, V: int = 0, b: int = 0, route: str = "direct",
           threads: int = 0) -> HostContainer:
    """Compress a float32 [rows, cols] host matrix at a target rate."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    R, Cc = W.shape
    h = C.c_void_p()
    L = lib()
    rc = L.ep_encode_host(_ptr(W) if W.size else None, R, Cc, float(target_bpp), V, b,
                          ROUTES[route], threads, C.byref(h))
    if rc != 0:
        raise ValueError(f"ep_encode_host failed with status {rc}")
    try:
        I = EncodedInfo()
        L.ep_encoded_get_info(h, C.byref(I))
        T, nw, nf = I.num_tiles, I.payload_words, I.num_freqs
        rs = np.zeros(max(R, 1), np.float32)
        qs = np.zeros(max(R, 1), np.float32) if route != "direct" else None
        st = np.zeros(max(32 * T, 1), np.uint32)
        off = np.zeros(T + 1, np.uint32)
        pl = np.zeros(max(nw, 1), np.uint16)
        fr = np.zeros(max(nf, 1), np.uint16)
        L.ep_encoded_copy(h, _ptr(rs), None if qs is None else _ptr(qs), _ptr(st), _ptr(off),
                          _ptr(pl), _ptr(fr))
        return HostContainer(R, Cc, I.vectors_per_tile, T, I.prob_bits, float(I.scale), route,
                             I.estimated_bpp, int(I.stored_bytes), rs[:R],
                             None if qs is None else qs[:R], st[: 32 * T], off, pl[:nw], fr[:nf],
                             np.array(I.alphabet, np.uint32), np.array(I.min_offset, np.int32),
                             np.array(I.freq_base, np.uint32))
    finally:
        L.ep_encoded_free(h)
