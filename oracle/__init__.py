"""EntroPack CPU oracle -- TEST INFRASTRUCTURE ONLY.

ctypes binding of the plain C oracle in this directory (see epo.h for what it
follows).  Only ``tests/``, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the GPU library never links or calls it.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libepo_oracle.so")
SOURCES = ["epo_lattice.c", "epo_rans.c", "epo_codec.c", "epo_convert.c"]

ROUTES = {"direct": 0, "fp8": 1, "int8": 2}
# field codings: the method's, and the two ablations of the paper's Table 4
CODINGS = {"standard": 0, "pooled": 1, "direct_z8": 2}
OUT_KINDS = {"bf16": 0, "fp8": 1, "int8": 2, "fp16": 3, "uint8": 4, "fp32": 101, "lattice2x": 100, "f32": 101,
             "fields": 102}
OUT_NUMPY = {"bf16": np.uint16, "fp8": np.uint8, "int8": np.int8, "fp16": np.uint16, "uint8": np.uint8,
             "fp32": np.float32,
             "lattice2x": np.int32, "f32": np.float32}
TILE_OK, TILE_BAD_STATE, TILE_BAD_LENGTH, TILE_OVERRUN, TILE_EMPTY_TABLE = 0, 1, 2, 3, 4
NTABLES = 17
LANES = 32


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into libepo_oracle.so (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", LIB_PATH + ".tmp"]
    cmd += [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def _p(t):
    return C.POINTER(t)


def _declare(L):
    i64, u32, i32, u64, f64, f32 = C.c_int64, C.c_uint32, C.c_int32, C.c_uint64, C.c_double, C.c_float
    vp = C.c_void_p
    L.epo_round_half_even.argtypes = [vp, i64, vp]
    L.epo_d8_nearest.argtypes = [vp, vp]
    L.epo_e8_nearest_batch.argtypes = [vp, i64, vp, vp]
    L.epo_point_to_fields_batch.argtypes = [vp, i64, vp]
    L.epo_fields_to_point_batch.argtypes = [vp, i64, vp]
    L.epo_row_rms.argtypes = [vp, i64, i64, vp]
    L.epo_normalize_freqs.argtypes = [vp, u32, u32, vp]
    L.epo_normalize_freqs.restype = C.c_int
    L.epo_tile_encode.argtypes = [u32, vp, vp, vp, vp, u32, vp, vp, u32, vp]
    L.epo_tile_encode.restype = C.c_int
    L.epo_tile_decode.argtypes = [u32, vp, vp, u32, vp, vp, u32, vp, vp]
    L.epo_tile_decode.restype = C.c_int
    L.epo_default_vectors_per_tile.argtypes = [f64]
    L.epo_default_vectors_per_tile.restype = u32
    L.epo_default_prob_bits.argtypes = [f64]
    L.epo_default_prob_bits.restype = u32
    L.epo_num_tiles.argtypes = [i64, i64, u32]
    L.epo_num_tiles.restype = u64
    L.epo_stored_bytes.argtypes = [i64, u32, u64, vp, C.c_int]
    L.epo_stored_bytes.restype = u64
    L.epo_sample_rows.argtypes = [i64, i64, vp, vp]
    L.epo_estimate_bpp.argtypes = [vp, i64, i64, vp, vp, i64, f64, u32, u32, C.c_int]
    L.epo_estimate_bpp.restype = f64
    L.epo_encode.argtypes = [vp, i64, i64, f64, u32, u32, C.c_int, _p(vp)]
    L.epo_encode.restype = C.c_int
    L.epo_encode_fixed_scale.argtypes = [vp, i64, i64, f32, u32, u32, C.c_int, _p(vp)]
    L.epo_encode_fixed_scale.restype = C.c_int
    L.epo_tensor_free.argtypes = [vp]
    L.epo_tensor_info.argtypes = [vp, _p(i64), _p(i64), _p(u32), _p(u32), _p(u32), _p(f32),
                                  _p(u64), _p(u32), _p(C.c_int), _p(f64)]
    L.epo_tensor_tables.argtypes = [vp, vp, vp, vp]
    L.epo_tensor_copy.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.epo_decode.argtypes = [i64, i64, u32, u32, u32, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                             C.c_int, vp, vp, u32, u32]
    L.epo_decode.restype = C.c_int
    L.epo_encode_coded.argtypes = [vp, i64, i64, f64, u32, u32, C.c_int, C.c_int, _p(vp)]
    L.epo_encode_coded.restype = C.c_int
    L.epo_tensor_coding.argtypes = [vp]
    L.epo_tensor_coding.restype = C.c_int
    L.epo_stored_bytes_coded.argtypes = [i64, u32, u64, vp, C.c_int, C.c_int]
    L.epo_stored_bytes_coded.restype = u64
    L.epo_decode_coded.argtypes = [i64, i64, u32, u32, u32, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                                   C.c_int, C.c_int, vp, vp, u32, u32]
    L.epo_decode_coded.restype = C.c_int
    L.epo_f32_to_bf16_batch.argtypes = [vp, i64, vp]
    L.epo_f32_to_f16_batch.argtypes = [vp, i64, vp]
    L.epo_f32_to_fp8e4m3_batch.argtypes = [vp, i64, vp]
    L.epo_f32_to_int8_batch.argtypes = [vp, i64, vp]
    L.epo_f32_to_uint8_batch.argtypes = [vp, i64, vp]
    L.epo_fp8e4m3_value.argtypes = [C.c_uint8]
    L.epo_fp8e4m3_value.restype = f64
    L.epo_route_precast.argtypes = [vp, i64, i64, C.c_int, vp, vp]
    L.epo_bpp.argtypes = [vp, vp, C.c_int]
    L.epo_bpp.restype = f64
    L.epo_rel_l2.argtypes = [vp, vp, i64]
    L.epo_rel_l2.restype = f64
    L.epo_rdo_ratios.argtypes = [u32, vp]
    L.epo_encode_rdo.argtypes = [vp, i64, i64, f64, u32, u32, C.c_int, u32, u32, _p(vp)]
    L.epo_encode_rdo.restype = C.c_int
    L.epo_rdo_trace.argtypes = [vp, i64, i64, f64, u32, u32, C.c_int, u32, vp, vp, vp, _p(i64),
                                _p(f64), vp, _p(f32), _p(u32)]
    L.epo_rdo_trace.restype = C.c_int


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- lattice
def round_half_even(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().epo_round_half_even(_ptr(x), x.size, _ptr(out))
    return out


def d8_nearest(v) -> np.ndarray:
    v = _c(v, np.float64).reshape(-1, 8)
    out = np.empty_like(v)
    for i in range(v.shape[0]):
        lib().epo_d8_nearest(_ptr(v[i]), out[i].ctypes.data_as(C.c_void_p))
    return out


def e8_nearest(v):
    """Nearest E8 points of the rows of v ([n, 8]); returns (points, coset bits)."""
    v = _c(v, np.float64).reshape(-1, 8)
    x = np.empty_like(v)
    c = np.empty(v.shape[0], np.int32)
    lib().epo_e8_nearest_batch(_ptr(v), v.shape[0], _ptr(x), _ptr(c))
    return x, c


def point_to_fields(x) -> np.ndarray:
    x = _c(x, np.float64).reshape(-1, 8)
    f = np.empty((x.shape[0], 9), np.int32)
    lib().epo_point_to_fields_batch(_ptr(x), x.shape[0], _ptr(f))
    return f


def fields_to_point(f) -> np.ndarray:
    f = _c(f, np.int32).reshape(-1, 9)
    x = np.empty((f.shape[0], 8), np.float64)
    lib().epo_fields_to_point_batch(_ptr(f), f.shape[0], _ptr(x))
    return x


def row_rms(W) -> np.ndarray:
    W = _c(W, np.float32)
    out = np.empty(W.shape[0], np.float64)
    lib().epo_row_rms(_ptr(W), W.shape[0], W.shape[1], _ptr(out))
    return out


# ----------------------------------------------------------------- rANS
def normalize_freqs(counts, b: int) -> Optional[np.ndarray]:
    counts = _c(counts, np.uint64)
    f = np.zeros(max(counts.size, 1), np.uint16)
    rc = lib().epo_normalize_freqs(_ptr(counts), counts.size, b, _ptr(f))
    return None if rc != 0 else f[: counts.size]


def _table_ptrs(freqs: Sequence[np.ndarray]):
    arrs = [_c(f, np.uint16) if len(f) else np.zeros(1, np.uint16) for f in freqs]
    ptrs = (C.c_void_p * NTABLES)(*[a.ctypes.data for a in arrs])
    alpha = np.array([len(f) for f in freqs], np.uint32)
    return arrs, ptrs, alpha


def tile_encode(sym, freqs: Sequence[np.ndarray], b: int):
    """Encode one tile of zero-based symbols sym [n, 9] (sym[:, 0] = coset bit)."""
    sym = _c(sym, np.int32).reshape(-1, 9)
    n = sym.shape[0]
    keep, ptrs, alpha = _table_ptrs(freqs)
    states = np.zeros(LANES, np.uint32)
    cap = 9 * n
    words = np.zeros(max(cap, 1), np.uint16)
    nw = C.c_uint32(0)
    rc = lib().epo_tile_encode(n, _ptr(sym), None, ptrs, _ptr(alpha), b, _ptr(states),
                               _ptr(words), cap, C.byref(nw))
    if rc != 0:
        raise ValueError(f"tile_encode failed: {rc}")
    return states, words[: nw.value].copy()


def tile_decode(n: int, states, words, freqs: Sequence[np.ndarray], b: int):
    states = _c(states, np.uint32)
    nw = len(words)
    words = _c(words, np.uint16) if nw else np.zeros(1, np.uint16)
    keep, ptrs, alpha = _table_ptrs(freqs)
    sym = np.zeros((max(n, 1), 9), np.int32)
    rc = lib().epo_tile_decode(n, _ptr(states), _ptr(words), nw, ptrs, _ptr(alpha), b,
                               _ptr(sym), None)
    return rc, sym[:n]


# ----------------------------------------------------------------- tensor codec
def default_vectors_per_tile(target_bpp: float) -> int:
    return int(lib().epo_default_vectors_per_tile(float(target_bpp)))


def default_prob_bits(target_bpp: float) -> int:
    return int(lib().epo_default_prob_bits(float(target_bpp)))


def num_tiles(rows: int, cols: int, V: int) -> int:
    return int(lib().epo_num_tiles(rows, cols, V))


def stored_bytes(rows: int, T: int, nwords: int, alphabet, route: str = "direct",
                 coding: str = "standard") -> int:
    a = _c(alphabet, np.uint32)
    return int(lib().epo_stored_bytes_coded(rows, T, nwords, _ptr(a), ROUTES[route], CODINGS[coding]))


def sample_rows(rows: int, cols: int) -> np.ndarray:
    out = np.zeros(max(rows, 1), np.int64)
    n = C.c_int64(0)
    lib().epo_sample_rows(rows, cols, _ptr(out), C.byref(n))
    return out[: n.value]


def estimate_bpp(W, s: float, b: int, V: int, route: str = "direct") -> float:
    W = _c(W, np.float32)
    R, Cc = W.shape
    norms = row_rms(W)
    samp = sample_rows(R, Cc)
    return float(lib().epo_estimate_bpp(_ptr(W), R, Cc, _ptr(norms), _ptr(samp), samp.size,
                                        float(s), b, V, ROUTES[route]))


@dataclasses.dataclass
class Container:
    """One compressed tensor as plain arrays (the stored representation)."""
    rows: int
    cols: int
    V: int
    T: int
    b: int
    s: float
    route: str
    est_bpp: float
    row_scales: np.ndarray      # float32 [rows]
    route_scales: Optional[np.ndarray]  # float32 [rows] (fp8/int8 routes)
    states: np.ndarray          # uint32 [T*32]
    offsets: np.ndarray         # uint32 [T+1]
    payload: np.ndarray         # uint16 [offsets[T]]
    freqs: np.ndarray           # uint16, 17 tables concatenated
    alphabet: np.ndarray        # uint32 [17]
    minval: np.ndarray          # int32 [17]
    freq_base: np.ndarray       # uint32 [17]
    coding: str = "standard"    # "pooled": coset slots share tables; "direct_z8": field 8 is z8

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def nwords(self) -> int:
        return int(self.offsets[-1]) if self.T > 0 else 0

    @property
    def stored_bytes(self) -> int:
        return stored_bytes(self.rows, self.T, self.nwords, self.alphabet, self.route, self.coding)

    @property
    def bpp(self) -> float:
        return 8.0 * self.stored_bytes / self.numel if self.numel else 0.0

    def table(self, k: int) -> np.ndarray:
        return self.freqs[self.freq_base[k]: self.freq_base[k] + self.alphabet[k]]


def _from_handle(h) -> Container:
    L = lib()
    rows, cols = C.c_int64(), C.c_int64()
    V, T, b, nf = C.c_uint32(), C.c_uint32(), C.c_uint32(), C.c_uint32()
    s = C.c_float()
    nw = C.c_uint64()
    route = C.c_int()
    est = C.c_double()
    L.epo_tensor_info(h, C.byref(rows), C.byref(cols), C.byref(V), C.byref(T), C.byref(b),
                      C.byref(s), C.byref(nw), C.byref(nf), C.byref(route), C.byref(est))
    alpha = np.zeros(NTABLES, np.uint32)
    minv = np.zeros(NTABLES, np.int32)
    fb = np.zeros(NTABLES, np.uint32)
    L.epo_tensor_tables(h, _ptr(alpha), _ptr(minv), _ptr(fb))
    rs = np.zeros(max(rows.value, 1), np.float32)
    qs = np.zeros(max(rows.value, 1), np.float32) if route.value else None
    st = np.zeros(max(LANES * T.value, 1), np.uint32)
    off = np.zeros(T.value + 1, np.uint32)
    pl = np.zeros(max(nw.value, 1), np.uint16)
    fr = np.zeros(max(nf.value, 1), np.uint16)
    L.epo_tensor_copy(h, _ptr(rs), _ptr(qs), _ptr(st), _ptr(off), _ptr(pl), _ptr(fr))
    rname = {v: k for k, v in ROUTES.items()}[route.value]
    cname = {v: k for k, v in CODINGS.items()}[L.epo_tensor_coding(h)]
    return Container(rows.value, cols.value, V.value, T.value, b.value, float(s.value), rname,
                     est.value, rs[: rows.value], None if qs is None else qs[: rows.value],
                     st[: LANES * T.value], off, pl[: nw.value], fr[: nf.value], alpha, minv, fb, cname)


def encode(W, target_bpp: float, V: int = 0, b: int = 0, route: str = "direct",
           coding: str = "standard") -> Container:
    """Compress a float32 [rows, cols] matrix at a target rate (scale search).

    coding selects the field coding (the method's, or a Table 4 ablation on the
    same quantised points and row scales)."""
    W = _c(W, np.float32)
    R, Cc = W.shape
    h = C.c_void_p()
    rc = lib().epo_encode_coded(_ptr(W), R, Cc, float(target_bpp), V, b, ROUTES[route],
                                CODINGS[coding], C.byref(h))
    if rc != 0:
        raise ValueError(f"oracle encode failed: {rc}")
    try:
        return _from_handle(h)
    finally:
        lib().epo_tensor_free(h)


def encode_fixed_scale(W, s: float, V: int, b: int, route: str = "direct") -> Container:
    W = _c(W, np.float32)
    R, Cc = W.shape
    h = C.c_void_p()
    rc = lib().epo_encode_fixed_scale(_ptr(W), R, Cc, float(s), V, b, ROUTES[route], C.byref(h))
    if rc != 0:
        raise ValueError(f"oracle encode_fixed_scale failed: {rc}")
    try:
        return _from_handle(h)
    finally:
        lib().epo_tensor_free(h)


def rdo_ratios(K: int) -> np.ndarray:
    """The K nested candidate ratios of the per-row refinement (rho_1 = 1 first)."""
    out = np.zeros(max(K, 1), np.float64)
    lib().epo_rdo_ratios(K, _ptr(out))
    return out[:K]


def encode_rdo(W, target_bpp: float, V: int = 0, b: int = 0, route: str = "direct", K: int = 5,
               sweeps: int = 1) -> Container:
    """encode() followed by the per-row rate-distortion refinement (K candidate
    resolutions per row, `sweeps` model-update and selection sweeps)."""
    W = _c(W, np.float32)
    R, Cc = W.shape
    h = C.c_void_p()
    rc = lib().epo_encode_rdo(_ptr(W), R, Cc, float(target_bpp), V, b, ROUTES[route], K, sweeps, C.byref(h))
    if rc != 0:
        raise ValueError(f"oracle encode_rdo failed: {rc}")
    try:
        return _from_handle(h)
    finally:
        lib().epo_tensor_free(h)


def rdo_trace(W, target_bpp: float, V: int = 0, b: int = 0, route: str = "direct", K: int = 5) -> dict:
    """The refinement's first sweep: distortions D [rows, K], rates R [rows, K]
    (units of 2^-16 bit), candidate row scales, the budget, lambda and the
    selection; s and b of the baseline."""
    W = _c(W, np.float32)
    R, Cc = W.shape
    D = np.zeros((R, K), np.float64)
    Rt = np.zeros((R, K), np.int64)
    rs = np.zeros((R, K), np.float32)
    sel = np.zeros(R, np.int32)
    budget, lam, s, bb = C.c_int64(), C.c_double(), C.c_float(), C.c_uint32()
    rc = lib().epo_rdo_trace(_ptr(W), R, Cc, float(target_bpp), V, b, ROUTES[route], K, _ptr(D), _ptr(Rt),
                             _ptr(rs), C.byref(budget), C.byref(lam), _ptr(sel), C.byref(s), C.byref(bb))
    if rc != 0:
        raise ValueError(f"oracle rdo_trace failed: {rc}")
    return {"D": D, "R": Rt, "row_scales": rs, "budget": budget.value, "lambda": lam.value, "sel": sel,
            "s": s.value, "b": bb.value}


def decode(ct: Container, kind: str = "bf16", tile_begin: int = 0, tile_end: Optional[int] = None,
           out: Optional[np.ndarray] = None):
    """Decode tiles [tile_begin, tile_end) of a container; returns (out, tile_status)."""
    if tile_end is None:
        tile_end = ct.T
    if kind == "fields":
        shape = (ct.rows * ct.cols // 8, 9)
        dt = np.int32
    else:
        shape = (ct.rows, ct.cols)
        dt = OUT_NUMPY[kind]
    if out is None:
        out = np.zeros(shape, dt)
    status = np.full(max(ct.T, 1), -1, np.int32)
    pl = ct.payload if ct.payload.size else np.zeros(1, np.uint16)
    fr = ct.freqs if ct.freqs.size else np.zeros(1, np.uint16)
    rs = ct.row_scales if ct.row_scales.size else np.zeros(1, np.float32)
    st = ct.states if ct.states.size else np.zeros(1, np.uint32)
    coding = CODINGS[getattr(ct, "coding", "standard")]
    rc = lib().epo_decode_coded(ct.rows, ct.cols, ct.V, ct.T, ct.b, ct.s, _ptr(_c(rs, np.float32)),
                                _ptr(_c(st, np.uint32)), _ptr(_c(ct.offsets, np.uint32)),
                                _ptr(_c(pl, np.uint16)), _ptr(_c(fr, np.uint16)),
                                _ptr(_c(ct.freq_base, np.uint32)), _ptr(_c(ct.alphabet, np.uint32)),
                                _ptr(_c(ct.minval, np.int32)), coding, OUT_KINDS[kind], _ptr(out),
                                _ptr(status), tile_begin, tile_end)
    if rc != 0:
        raise ValueError(f"oracle decode rejected its arguments: {rc}")
    return out, status[: ct.T]


# ----------------------------------------------------------------- conversions and metrics
def f32_to_bf16(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint16)
    lib().epo_f32_to_bf16_batch(_ptr(y), y.size, _ptr(out))
    return out


def f32_to_fp16(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint16)
    lib().epo_f32_to_f16_batch(_ptr(y), y.size, _ptr(out))
    return out


def f32_to_fp8(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().epo_f32_to_fp8e4m3_batch(_ptr(y), y.size, _ptr(out))
    return out


def f32_to_uint8(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().epo_f32_to_uint8_batch(_ptr(y), y.size, _ptr(out))
    return out


def f32_to_int8(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.int8)
    lib().epo_f32_to_int8_batch(_ptr(y), y.size, _ptr(out))
    return out


def fp8_value(code: int) -> float:
    return float(lib().epo_fp8e4m3_value(code))


def route_precast(W, route: str):
    W = _c(W, np.float32)
    R, Cc = W.shape
    Wq = np.empty_like(W)
    q = np.empty(R, np.float32)
    lib().epo_route_precast(_ptr(W), R, Cc, ROUTES[route], _ptr(Wq), _ptr(q))
    return Wq, q


def bpp(stored: Sequence[int], numel: Sequence[int]) -> float:
    a = np.array(stored, np.uint64)
    b = np.array(numel, np.uint64)
    return float(lib().epo_bpp(_ptr(a), _ptr(b), len(a)))


def rel_l2(Wq, W) -> float:
    Wq = _c(Wq, np.float32)
    W = _c(W, np.float32)
    return float(lib().epo_rel_l2(_ptr(Wq), _ptr(W), W.size))


def bf16_to_f32(u16) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (plain bit shift)."""
    u = np.asarray(u16, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)
