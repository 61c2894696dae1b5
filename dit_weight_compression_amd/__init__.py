"""MI355X EntroPack decoder: thin Python binding of the C ABI in include/entropack.h.

Every step of the decode runs in the HIP library (libentropack_mi355x.so);
this module only marshals arguments.  PyTorch supplies device memory and the
current HIP stream.  There is no CPU fallback: if the library is missing the
import of the decode functions fails loudly.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libentropack_mi355x.so")
NTABLES = 17

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_WORKSPACE, EP_ERR_HIP = 0, -1, -2, -3, -4
DTYPES = {"bf16": 0, "fp8": 1, "int8": 2, "fp16": 3, "fp32": 4, "uint8": 5, "lattice2x": 100}
TILE_OK, TILE_BAD_STATE, TILE_BAD_LENGTH, TILE_OVERRUN, TILE_EMPTY_TABLE = 0, 1, 2, 3, 4

# every symbol include/entropack.h declares
EXPORTS = ["ep_status_string", "ep_last_error", "ep_abi_version", "ep_workspace_size",
           "ep_decode_batch", "ep_decode_tensor", "ep_batch_prepare", "ep_batch_launch",
           "ep_convert_f32", "ep_decode_batch_noalloc"]
NOALLOC_SCRATCH_BYTES = 64 << 20      # EP_NOALLOC_SCRATCH_BYTES
# every symbol include/entropack_device_encode.h declares (same library)
DEVICE_ENCODE_EXPORTS = ["ep_encode_device_workspace_size", "ep_encode_device",
                         "ep_encode_device_emit", "ep_encode_device_rdo_workspace_size",
                         "ep_encode_device_rdo"]
ROUTES = {"direct": 0, "fp8": 1, "int8": 2}
CODINGS = {"standard": 0, "pooled": 1, "direct_z8": 2}   # ep_coding


class EpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class EpTensorDesc(C.Structure):
    _fields_ = [
        ("rows", C.c_int64),
        ("cols", C.c_int64),
        ("vectors_per_tile", C.c_uint32),
        ("num_tiles", C.c_uint32),
        ("prob_bits", C.c_uint32),
        ("scale", C.c_float),
        ("row_scales", C.c_void_p),
        ("tile_states", C.c_void_p),
        ("tile_offsets", C.c_void_p),
        ("payload", C.c_void_p),
        ("payload_words", C.c_uint64),
        ("freqs", C.c_void_p),
        ("freq_base", C.c_uint32 * NTABLES),
        ("alphabet", C.c_uint32 * NTABLES),
        ("min_offset", C.c_int32 * NTABLES),
        ("field8", C.c_uint32),
    ]


class EpBatchPlan(C.Structure):
    _fields_ = [("opaque", C.c_uint64 * 256)]


_lib = None


def lib():
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no CPU fallback for the decoder)")
        # torch first: it loads the HIP runtime it was built with, and the
        # library then binds to that same runtime (the two share a soname;
        # whichever loads first serves the process)
        import torch  # noqa: F401

        L = C.CDLL(LIB_PATH)
        vp = C.c_void_p
        L.ep_status_string.argtypes = [C.c_int]
        L.ep_status_string.restype = C.c_char_p
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = C.c_char_p
        L.ep_abi_version.restype = C.c_int
        L.ep_workspace_size.argtypes = [vp, C.c_int, C.POINTER(C.c_size_t)]
        L.ep_workspace_size.restype = C.c_int
        L.ep_decode_batch.argtypes = [vp, vp, vp, vp, C.c_int, vp, C.c_size_t, vp]
        L.ep_decode_batch.restype = C.c_int
        L.ep_decode_tensor.argtypes = [vp, C.c_int, vp, vp, vp, C.c_size_t, vp]
        L.ep_decode_tensor.restype = C.c_int
        L.ep_batch_prepare.argtypes = [vp, vp, vp, vp, C.c_int, vp, C.c_size_t, vp, vp]
        L.ep_batch_prepare.restype = C.c_int
        L.ep_batch_launch.argtypes = [vp, vp]
        L.ep_batch_launch.restype = C.c_int
        L.ep_convert_f32.argtypes = [vp, vp, C.c_uint64, C.c_int, vp]
        L.ep_convert_f32.restype = C.c_int
        L.ep_decode_batch_noalloc.argtypes = [vp, vp, vp, vp, C.c_int, vp]
        L.ep_decode_batch_noalloc.restype = C.c_int
        L.ep_encode_device_workspace_size.argtypes = [C.c_int64, C.c_int64, C.c_double, C.c_uint32,
                                                      C.c_int, C.POINTER(C.c_size_t)]
        L.ep_encode_device_workspace_size.restype = C.c_int
        L.ep_encode_device.argtypes = [vp, C.c_int64, C.c_int64, C.c_double, C.c_uint32, C.c_uint32,
                                       C.c_int, C.c_int, vp, C.c_size_t, vp, vp]
        L.ep_encode_device.restype = C.c_int
        L.ep_encode_device_emit.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.ep_encode_device_emit.restype = C.c_int
        L.ep_encode_device_rdo_workspace_size.argtypes = [C.c_int64, C.c_int64, C.c_double, C.c_uint32,
                                                          C.c_int, C.c_uint32, C.POINTER(C.c_size_t)]
        L.ep_encode_device_rdo_workspace_size.restype = C.c_int
        L.ep_encode_device_rdo.argtypes = [vp, C.c_int64, C.c_int64, C.c_double, C.c_uint32, C.c_uint32,
                                           C.c_int, C.c_uint32, C.c_uint32, vp, C.c_size_t, vp, vp]
        L.ep_encode_device_rdo.restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != EP_OK:
        L = lib()
        raise EpError(rc, f"{L.ep_status_string(rc).decode()}: {L.ep_last_error().decode()}")


def _torch():
    import torch
    return torch


@dataclasses.dataclass
class PackedTensor:
    """A compressed tensor resident in device memory (the decoder's input)."""
    rows: int
    cols: int
    V: int
    T: int
    b: int
    s: float
    alphabet: np.ndarray
    minval: np.ndarray
    freq_base: np.ndarray
    row_scales: "object"    # torch float32 [rows]
    states: "object"        # torch int32 [T*32] (u32 bits)
    offsets: "object"       # torch int32 [T+1] (u32 bits)
    payload: "object"       # torch int16 [words] (u16 bits)
    freqs: "object"         # torch int16 (u16 bits)
    stored_bytes: int = 0

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    nwords: int = 0         # payload words (the device buffer is padded to a multiple of 8)
    field8: int = 0         # 1: field 8 holds z8 (the direct-z8 coding), 0: m

    @classmethod
    def from_arrays(cls, ct, device="cuda", stored_bytes: int = 0) -> "PackedTensor":
        """Upload a container given as numpy arrays (fields as in oracle.Container)."""
        torch = _torch()

        def up(a, np_dt, t_dt):
            a = np.ascontiguousarray(a, dtype=np_dt)
            if a.size == 0:
                a = np.zeros(1, np_dt)
            return torch.from_numpy(a.view(t_dt)).to(device)

        # words actually present (a corrupt final offset must not extend the buffer)
        nw = min(int(ct.offsets[-1]), int(np.asarray(ct.payload).size)) if ct.T > 0 else 0
        # the decoder reads whole 16-byte groups: pad the payload to a multiple of 8 words
        padded = np.zeros(max((nw + 7) // 8 * 8, 8), np.uint16)
        padded[:nw] = np.asarray(ct.payload)[:nw]
        payload = up(padded, np.uint16, np.int16)
        return cls(int(ct.rows), int(ct.cols), int(ct.V), int(ct.T), int(ct.b), float(ct.s),
                   np.asarray(ct.alphabet, np.uint32).copy(), np.asarray(ct.minval, np.int32).copy(),
                   np.asarray(ct.freq_base, np.uint32).copy(),
                   up(ct.row_scales, np.float32, np.float32), up(ct.states, np.uint32, np.int32),
                   up(ct.offsets, np.uint32, np.int32), payload, up(ct.freqs, np.uint16, np.int16),
                   stored_bytes, nw, 1 if getattr(ct, "coding", "standard") == "direct_z8" else 0)

    def desc(self) -> EpTensorDesc:
        d = EpTensorDesc()
        d.rows, d.cols = self.rows, self.cols
        d.vectors_per_tile, d.num_tiles, d.prob_bits = self.V, self.T, self.b
        d.scale = self.s
        d.row_scales = self.row_scales.data_ptr()
        d.tile_states = self.states.data_ptr()
        d.tile_offsets = self.offsets.data_ptr()
        d.payload = self.payload.data_ptr()
        d.payload_words = self.nwords if self.T > 0 else 0
        d.freqs = self.freqs.data_ptr()
        for k in range(NTABLES):
            d.freq_base[k] = int(self.freq_base[k])
            d.alphabet[k] = int(self.alphabet[k])
            d.min_offset[k] = int(self.minval[k])
        d.field8 = int(self.field8)
        return d


def torch_dtype(name: str):
    torch = _torch()
    return {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "int8": torch.int8,
            "fp16": torch.float16, "fp32": torch.float32, "uint8": torch.uint8,
            "lattice2x": torch.int32}[name]


def workspace_size(packed: Sequence[PackedTensor]) -> int:
    n = len(packed)
    descs = (EpTensorDesc * max(n, 1))(*[p.desc() for p in packed])
    out = C.c_size_t(0)
    _check(lib().ep_workspace_size(C.cast(descs, C.c_void_p), n, C.byref(out)))
    return int(out.value)


class BatchArgs:
    """Marshalled arguments of one ep_decode_batch call (kept alive by this object)."""

    def __init__(self, packed, dtypes, outs, statuses, workspace):
        n = len(packed)
        self.n = n
        self.descs = (EpTensorDesc * max(n, 1))(*[p.desc() for p in packed])
        self.dt = (C.c_int * max(n, 1))(*[DTYPES[d] for d in dtypes])
        self.outp = (C.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
        self.stp = None
        if statuses is not None:
            self.stp = (C.c_void_p * max(n, 1))(*[s.data_ptr() if s is not None else None
                                                  for s in statuses])
        self.ws = workspace
        self.keep = (packed, outs, statuses)

    def call(self, stream_ptr):
        _check(lib().ep_decode_batch(C.cast(self.descs, C.c_void_p), C.cast(self.dt, C.c_void_p),
                                     C.cast(self.outp, C.c_void_p),
                                     None if self.stp is None else C.cast(self.stp, C.c_void_p),
                                     self.n, self.ws.data_ptr(), self.ws.numel(), stream_ptr))

    def prepare(self, stream_ptr) -> EpBatchPlan:
        plan = EpBatchPlan()
        _check(lib().ep_batch_prepare(C.cast(self.descs, C.c_void_p), C.cast(self.dt, C.c_void_p),
                                      C.cast(self.outp, C.c_void_p),
                                      None if self.stp is None else C.cast(self.stp, C.c_void_p),
                                      self.n, self.ws.data_ptr(), self.ws.numel(), stream_ptr,
                                      C.byref(plan)))
        return plan

    @staticmethod
    def launch(plan: EpBatchPlan, stream_ptr):
        _check(lib().ep_batch_launch(C.byref(plan), stream_ptr))


def alloc_outputs(packed: Sequence[PackedTensor], dtypes: Sequence[str], device="cuda"):
    torch = _torch()
    return [torch.empty((p.rows, p.cols), dtype=torch_dtype(d), device=device)
            for p, d in zip(packed, dtypes)]


def decode_batch(packed: Sequence[PackedTensor], dtypes, outs=None, with_status: bool = False,
                 workspace=None, stream=None):
    """Decode tensors with one ep_decode_batch call; returns (outs, statuses)."""
    torch = _torch()
    if isinstance(dtypes, str):
        dtypes = [dtypes] * len(packed)
    dev = packed[0].payload.device if packed else torch.device("cuda")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    # Buffers made here are allocated on the launch stream: the caching
    # allocator then hands their memory only to later work on that stream,
    # which runs after the decode even when the caller's current stream differs.
    with torch.cuda.stream(stream):
        if outs is None:
            outs = alloc_outputs(packed, dtypes, dev)
        statuses = None
        if with_status:
            statuses = [torch.full((max(p.T, 1),), -1, dtype=torch.int32, device=dev) for p in packed]
        if workspace is None:
            workspace = torch.empty(workspace_size(packed), dtype=torch.uint8, device=dev)
    args = BatchArgs(packed, dtypes, outs, statuses, workspace)
    args.call(C.c_void_p(stream.cuda_stream))
    return outs, statuses


def decode_batch_noalloc(packed: Sequence[PackedTensor], dtypes, outs, statuses=None, stream=None):
    """Decode into caller-made outputs with ep_decode_batch_noalloc (the library's static scratch).

    statuses: None or one int32 device tensor of at least max(T, 1) entries per tensor.
    """
    torch = _torch()
    if isinstance(dtypes, str):
        dtypes = [dtypes] * len(packed)
    dev = packed[0].payload.device if packed else torch.device("cuda")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    n = len(packed)
    descs = (EpTensorDesc * max(n, 1))(*[p.desc() for p in packed])
    dt = (C.c_int * max(n, 1))(*[DTYPES[d] for d in dtypes])
    outp = (C.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    stp = None
    if statuses is not None:
        stp = (C.c_void_p * max(n, 1))(*[s.data_ptr() if s is not None else None for s in statuses])
    _check(lib().ep_decode_batch_noalloc(C.cast(descs, C.c_void_p), C.cast(dt, C.c_void_p),
                                         C.cast(outp, C.c_void_p),
                                         None if stp is None else C.cast(stp, C.c_void_p), n,
                                         C.c_void_p(stream.cuda_stream)))
    return outs, statuses


def decode_tensor(p: PackedTensor, dtype: str = "bf16", out=None, with_status: bool = False,
                  workspace=None, stream=None):
    """Decode one tensor with ep_decode_tensor; returns (out, status)."""
    torch = _torch()
    dev = p.payload.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.stream(stream):      # see decode_batch: allocations on the launch stream
        if out is None:
            out = alloc_outputs([p], [dtype], dev)[0]
        status = torch.full((max(p.T, 1),), -1, dtype=torch.int32, device=dev) if with_status else None
        if workspace is None:
            workspace = torch.empty(workspace_size([p]), dtype=torch.uint8, device=dev)
    d = p.desc()
    _check(lib().ep_decode_tensor(C.byref(d), DTYPES[dtype], out.data_ptr(),
                                  None if status is None else status.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(),
                                  C.c_void_p(stream.cuda_stream)))
    return out, status


# the C ABI names
ep_decode_tensor = decode_tensor
ep_decode_batch = decode_batch
ep_decode_batch_noalloc = decode_batch_noalloc
ep_workspace_size = workspace_size


# ---------------------------------------------------------------- device compressor
def encode_device_workspace_size(rows: int, cols: int, target_bpp: float, V: int = 0,
                                 route: str = "direct") -> int:
    n = C.c_size_t()
    _check(lib().ep_encode_device_workspace_size(rows, cols, float(target_bpp), V, ROUTES[route],
                                                 C.byref(n)))
    return n.value


@dataclasses.dataclass
class DeviceEncoded:
    """Result of encode_device: the container on the device plus its header."""
    packed: PackedTensor
    route: str
    route_scales: "object"   # torch float32 [rows] (FP8 / INT8 routes), else None
    est_bpp: float
    num_freqs: int
    coding: str = "standard"


def encode_device_rdo_workspace_size(rows: int, cols: int, target_bpp: float, V: int = 0,
                                     route: str = "direct", candidates: int = 5) -> int:
    n = C.c_size_t()
    _check(lib().ep_encode_device_rdo_workspace_size(rows, cols, float(target_bpp), V, ROUTES[route],
                                                     candidates, C.byref(n)))
    return n.value


def encode_device(W, target_bpp: float, V: int = 0, b: int = 0, route: str = "direct",
                  workspace=None, stream=None, coding: str = "standard", candidates: int = 0,
                  sweeps: int = 0) -> DeviceEncoded:
    """Compress a float32 device tensor [rows, cols] with ep_encode_device.

    The container matches the host compressor's byte for byte; its arrays are
    left on W's device, ready for decode_tensor / decode_batch.  coding selects
    a Table 4 ablation ("pooled", "direct_z8") on the same points and scales.
    candidates > 0 runs ep_encode_device_rdo instead (the per-row
    rate-distortion refinement with that many resolutions per row and
    `sweeps` sweeps; standard coding only).
    """
    from .encoder import EncodedInfo
    torch = _torch()
    if W.dtype != torch.float32 or W.dim() != 2 or not W.is_cuda:
        raise ValueError("W must be a 2-D float32 device tensor")
    if candidates and coding != "standard":
        raise ValueError("the refinement uses the standard coding")
    W = W.contiguous()
    R, Cc = W.shape
    dev = W.device
    if workspace is None:
        n = (encode_device_rdo_workspace_size(R, Cc, target_bpp, V, route, candidates) if candidates
             else encode_device_workspace_size(R, Cc, target_bpp, V, route))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    sp = C.c_void_p(stream.cuda_stream)
    info = EncodedInfo()
    wp = W.data_ptr() if W.numel() else None
    if candidates:
        _check(lib().ep_encode_device_rdo(wp, R, Cc, float(target_bpp), V, b, ROUTES[route], candidates, sweeps,
                                          workspace.data_ptr(), workspace.numel(), sp, C.byref(info)))
    else:
        _check(lib().ep_encode_device(wp, R, Cc, float(target_bpp), V, b, ROUTES[route], CODINGS[coding],
                                      workspace.data_ptr(), workspace.numel(), sp, C.byref(info)))
    T, nw, nf = info.num_tiles, int(info.payload_words), info.num_freqs
    rs = torch.empty(max(R, 1), dtype=torch.float32, device=dev)
    qs = torch.empty(max(R, 1), dtype=torch.float32, device=dev) if route != "direct" else None
    st = torch.empty(max(32 * T, 1), dtype=torch.int32, device=dev)
    off = torch.empty(T + 1, dtype=torch.int32, device=dev)
    # the decoder reads whole 16-byte groups: pad to a multiple of 8 words
    pl = torch.zeros(max((nw + 7) // 8 * 8, 8), dtype=torch.int16, device=dev)
    fr = torch.zeros(max(nf, 1), dtype=torch.int16, device=dev)
    _check(lib().ep_encode_device_emit(workspace.data_ptr(), C.byref(info), rs.data_ptr(),
                                       None if qs is None else qs.data_ptr(), st.data_ptr(),
                                       off.data_ptr(), pl.data_ptr(), fr.data_ptr(), sp))
    p = PackedTensor(R, Cc, info.vectors_per_tile, T, info.prob_bits, float(info.scale),
                     np.array(info.alphabet, np.uint32), np.array(info.min_offset, np.int32),
                     np.array(info.freq_base, np.uint32), rs, st, off, pl, fr,
                     int(info.stored_bytes), nw, 1 if coding == "direct_z8" else 0)
    return DeviceEncoded(p, route, qs, float(info.estimated_bpp), nf, coding)


ep_encode_device = encode_device
ep_encode_device_workspace_size = encode_device_workspace_size
ep_encode_device_rdo_workspace_size = encode_device_rdo_workspace_size


def convert_f32(y, dtype: str, stream=None):
    """Container rounding of a float32 device tensor (ep_convert_f32); returns the codes."""
    torch = _torch()
    y = y.contiguous()
    if y.dtype != torch.float32 or not y.is_cuda or y.numel() % 4:
        raise ValueError("y must be a float32 device tensor with a multiple of 4 elements")
    out = torch.empty(y.shape, dtype=torch_dtype(dtype), device=y.device)
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    _check(lib().ep_convert_f32(y.data_ptr(), out.data_ptr(), y.numel(), DTYPES[dtype],
                                C.c_void_p(stream.cuda_stream)))
    return out


ep_convert_f32 = convert_f32
