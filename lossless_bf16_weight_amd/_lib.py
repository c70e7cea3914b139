"""ctypes binding of libdf11.so (C ABI in include/df11.h).

Argument marshalling only: validation, table building, encoding and every
decode step run inside the library (host C++ and the HIP kernel).  There is
no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdf11.so")

OK, E_ARG, E_FORMAT, E_UNSUPPORTED, E_HIP, E_CORRUPT, E_NOMEM = range(7)
FLAG_SHA256 = 1
MAX_BATCH = 64
# DF11_ABI_VERSION of include/df11.h that these argument lists follow
ABI_VERSION = 2


class DF11Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class TensorInfo(ctypes.Structure):
    _fields_ = [
        ("n_elems", ctypes.c_uint64),
        ("ndim", ctypes.c_uint32),
        ("n_chunks", ctypes.c_uint32),
        ("dims", ctypes.c_uint64 * 8),
        ("total_bits", ctypes.c_uint64),
        ("container_bytes", ctypes.c_uint64),
        ("meta_bytes", ctypes.c_uint64),
        ("bytes_read_per_decode", ctypes.c_uint64),
        ("code_len", ctypes.c_uint8 * 256),
        ("flags", ctypes.c_uint32),
        ("sha256", ctypes.c_uint8 * 32),
    ]

    def as_dict(self) -> dict:
        return {
            "n_elems": self.n_elems, "ndim": self.ndim, "n_chunks": self.n_chunks,
            "dims": [self.dims[i] for i in range(self.ndim)], "total_bits": self.total_bits,
            "container_bytes": self.container_bytes, "meta_bytes": self.meta_bytes,
            "bytes_read_per_decode": self.bytes_read_per_decode,
            "code_len": np.array(self.code_len[:], np.uint8),
            "flags": self.flags, "sha256": bytes(self.sha256),
        }


_lib = None

EXPORTS = [
    "df11_validate", "df11_container_bound", "df11_encode", "df11_encode_ex", "df11_encode_device", "df11_encode_device_batch",
    "df11_encode_device_batch_noalloc", "df11_sha256",
    "df11_verify_words", "df11_plan", "df11_plan_destroy", "df11_plan_set_wgs_per_cu",
    "df11_plan_info", "df11_decode", "df11_decode_batch", "df11_check", "df11_last_error",
    "df11_status_str", "df11_abi_version", "df11_bw_control",
    "df11_nf12_bound", "df11_nf12_encode", "df11_nf12_validate", "df11_nf12_decode",
    "df11_nf12_decode_batch",
]


def lib():
    """Load libdf11.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
                          "or lossless_bf16_weight_amd._build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, u64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64
    L.df11_validate.argtypes = [vp, sz, ctypes.POINTER(TensorInfo)]
    L.df11_validate.restype = ctypes.c_int
    L.df11_container_bound.argtypes = [u64]
    L.df11_container_bound.restype = u64
    L.df11_encode.argtypes = [vp, u64, ctypes.c_int, ctypes.POINTER(u64), vp, u64,
                              ctypes.POINTER(u64), ctypes.c_int]
    L.df11_encode.restype = ctypes.c_int
    L.df11_encode_ex.argtypes = [vp, u64, ctypes.c_int, ctypes.POINTER(u64), ctypes.c_uint32, vp, u64,
                                 ctypes.POINTER(u64), ctypes.c_int]
    L.df11_encode_ex.restype = ctypes.c_int
    L.df11_encode_device.argtypes = [vp, u64, ctypes.c_int, ctypes.POINTER(u64), vp, u64, ctypes.POINTER(u64),
                                     ctypes.c_int, vp]
    L.df11_encode_device.restype = ctypes.c_int
    L.df11_encode_device_batch.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(u64),
                                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(u64), ctypes.POINTER(vp),
                                           ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.c_int, vp]
    L.df11_encode_device_batch.restype = ctypes.c_int
    L.df11_encode_device_batch_noalloc.argtypes = L.df11_encode_device_batch.argtypes
    L.df11_encode_device_batch_noalloc.restype = ctypes.c_int
    L.df11_sha256.argtypes = [vp, u64, vp]
    L.df11_sha256.restype = None
    L.df11_verify_words.argtypes = [vp, sz, vp, u64]
    L.df11_verify_words.restype = ctypes.c_int
    L.df11_plan.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(sz), ctypes.c_int, ctypes.c_int,
                            ctypes.c_uint32, ctypes.POINTER(vp)]
    L.df11_plan.restype = ctypes.c_int
    L.df11_plan_destroy.argtypes = [vp]
    L.df11_plan_destroy.restype = None
    L.df11_plan_set_wgs_per_cu.argtypes = [vp, ctypes.c_int]
    L.df11_plan_set_wgs_per_cu.restype = ctypes.c_int
    L.df11_plan_info.argtypes = [vp, ctypes.c_int, ctypes.POINTER(TensorInfo)]
    L.df11_plan_info.restype = ctypes.c_int
    L.df11_decode.argtypes = [vp, ctypes.c_int, vp, vp, vp]
    L.df11_decode.restype = ctypes.c_int
    L.df11_decode_batch.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]
    L.df11_decode_batch.restype = ctypes.c_int
    L.df11_check.argtypes = [vp, vp]
    L.df11_check.restype = ctypes.c_int
    L.df11_last_error.argtypes = []
    L.df11_last_error.restype = ctypes.c_char_p
    L.df11_status_str.argtypes = [ctypes.c_int]
    L.df11_status_str.restype = ctypes.c_char_p
    L.df11_abi_version.argtypes = []
    L.df11_abi_version.restype = ctypes.c_int
    L.df11_bw_control.argtypes = [vp, u64, vp, u64, ctypes.c_int, vp]
    L.df11_bw_control.restype = ctypes.c_int
    L.df11_nf12_bound.argtypes = [u64]
    L.df11_nf12_bound.restype = u64
    L.df11_nf12_encode.argtypes = [vp, u64, vp, u64, ctypes.POINTER(u64), ctypes.c_int]
    L.df11_nf12_encode.restype = ctypes.c_int
    L.df11_nf12_validate.argtypes = [vp, sz, ctypes.POINTER(u64)]
    L.df11_nf12_validate.restype = ctypes.c_int
    L.df11_nf12_decode.argtypes = [vp, vp, vp, ctypes.c_int, vp]
    L.df11_nf12_decode.restype = ctypes.c_int
    L.df11_nf12_decode_batch.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         ctypes.c_int, ctypes.c_int, vp]
    L.df11_nf12_decode_batch.restype = ctypes.c_int
    _lib = L
    return L


def _raise(st: int):
    if st != OK:
        raise DF11Error(st, lib().df11_last_error().decode())


def _host_u8(buf) -> np.ndarray:
    a = np.asarray(buf)
    if a.dtype != np.uint8:
        a = a.view(np.uint8)
    return np.ascontiguousarray(a.reshape(-1))


# ----------------------------------------------------------------- host --

def container_bound(n: int) -> int:
    return int(lib().df11_container_bound(n))


def encode(words, shape=None, threads: int = 0, sha256: bool = False) -> np.ndarray:
    """Encode BF16 bit patterns (uint16/int16 numpy array, host) into a
    version-4 container (uint8 numpy array); with sha256, the header holds
    the SHA-256 of the source words."""
    w = np.ascontiguousarray(np.asarray(words).view(np.uint16).reshape(-1))
    shape = tuple(np.asarray(words).shape) if shape is None else tuple(shape)
    dims = (ctypes.c_uint64 * max(1, len(shape)))(*shape)
    cap = container_bound(w.size)
    out = np.empty(cap, np.uint8)
    nbytes = ctypes.c_uint64(0)
    st = lib().df11_encode_ex(w.ctypes.data, w.size, len(shape), dims, FLAG_SHA256 if sha256 else 0,
                              out.ctypes.data, cap, ctypes.byref(nbytes), threads)
    if st != OK:
        raise DF11Error(st, f"df11_encode_ex: status {st}")
    return out[: nbytes.value]


def _cuda_words(x, what: str):
    """A device tensor of 16-bit words (the library reads it on the GPU: a
    host tensor's pointer must never reach it)."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{what}: a CUDA tensor is needed")
    if x.element_size() != 2:
        raise ValueError(f"{what}: a 16-bit dtype is needed, not {x.dtype}")
    return x.contiguous().view(torch.int16)


def encode_device(words, shape=None, stream=None):
    """Encode a 16-bit device tensor (BF16 bit patterns, on a GPU) into a
    version-4 container on the same device (uint8 tensor): the bytes
    encode() writes for the same words, computed by the GPU kernels."""
    import torch
    w = _cuda_words(words, "words").reshape(-1)
    shape = tuple(words.shape) if shape is None else tuple(shape)
    dims = (ctypes.c_uint64 * max(1, len(shape)))(*shape)
    out = torch.empty(container_bound(w.numel()), dtype=torch.uint8, device=w.device)
    nbytes = ctypes.c_uint64(0)
    _raise(lib().df11_encode_device(w.data_ptr() if w.numel() else None, w.numel(), len(shape), dims,
                                    out.data_ptr(), out.numel(), ctypes.byref(nbytes), w.device.index or 0,
                                    _stream_handle(stream)))
    return out[: nbytes.value]


def encode_device_batch(tensors, stream=None, outs=None, noalloc=False):
    """encode_device() for several device tensors (one device) sharing one
    wait on the stream; returns their containers (uint8 device tensors).
    outs: the caller's output buffers (uint8 device tensors of at least
    container_bound bytes each), else new ones.  noalloc: call
    df11_encode_device_batch_noalloc (at most 64 tensors), which allocates
    nothing for its histograms."""
    import torch
    ws = [_cuda_words(t, f"tensor {i}") for i, t in enumerate(tensors)]
    k = len(ws)
    if k == 0:
        return []
    dev = ws[0].device
    for i, w in enumerate(ws):
        if w.device != dev:
            raise ValueError(f"tensor {i}: on {w.device}, tensor 0 on {dev}")
        if w.dim() > 8:
            raise ValueError(f"tensor {i}: {w.dim()} dimensions, at most 8")
    if outs is None:
        outs = [torch.empty(container_bound(w.numel()), dtype=torch.uint8, device=dev) for w in ws]
    elif len(outs) != k:
        raise ValueError("one output buffer per tensor")
    else:
        for i, o in enumerate(outs):
            _check_device_tensor(o, f"output {i}", 0, dev.index or 0)
    dims = (ctypes.c_uint64 * (8 * k))()
    for t, w in enumerate(ws):
        for i, d in enumerate(w.shape):
            dims[8 * t + i] = d
    nbytes = (ctypes.c_uint64 * k)()
    fn = lib().df11_encode_device_batch_noalloc if noalloc else lib().df11_encode_device_batch
    _raise(fn(
        k, (ctypes.c_void_p * k)(*[w.data_ptr() if w.numel() else None for w in ws]),
        (ctypes.c_uint64 * k)(*[w.numel() for w in ws]), (ctypes.c_int * k)(*[w.dim() for w in ws]), dims,
        (ctypes.c_void_p * k)(*[o.data_ptr() for o in outs]),
        (ctypes.c_uint64 * k)(*[o.numel() * o.element_size() for o in outs]),
        nbytes, dev.index or 0, _stream_handle(stream)))
    return [o.view(torch.uint8)[: nbytes[t]] for t, o in enumerate(outs)]


def sha256(data) -> bytes:
    """SHA-256 digest of a host buffer (bytes or a numpy array's bytes)."""
    a = np.ascontiguousarray(np.frombuffer(data, np.uint8) if isinstance(data, (bytes, bytearray))
                             else np.asarray(data)).view(np.uint8).reshape(-1)
    out = np.zeros(32, np.uint8)
    lib().df11_sha256(a.ctypes.data if a.size else None, a.size, out.ctypes.data)
    return out.tobytes()


def verify_status(container, words) -> int:
    """df11_verify_words status: OK when the SHA-256 of `words` (host,
    16-bit) equals the one in the container's header, E_CORRUPT when it
    differs, E_UNSUPPORTED when the header holds none."""
    c = _host_u8(container)
    w = np.ascontiguousarray(np.asarray(words).view(np.uint16).reshape(-1))
    return int(lib().df11_verify_words(c.ctypes.data, c.size, w.ctypes.data if w.size else None, w.size))


def verify(container, words) -> bool:
    """True when the words' SHA-256 equals the header's, False when it
    differs; raises DF11Error when the container cannot be checked."""
    st = verify_status(container, words)
    if st == E_CORRUPT:
        return False
    _raise(st)
    return True


def verify_decoded(container, out, stream=None) -> bool:
    """verify() of a decoded device tensor: waits for `stream`, copies the
    words to host memory and checks their hash against the header's."""
    import torch
    (stream or torch.cuda.current_stream()).synchronize()
    return verify(container, out.view(torch.int16).cpu().numpy())


def validate(container) -> dict:
    c = _host_u8(container)
    info = TensorInfo()
    _raise(lib().df11_validate(c.ctypes.data, c.size, ctypes.byref(info)))
    return info.as_dict()


def validate_status(container) -> int:
    c = _host_u8(container)
    return int(lib().df11_validate(c.ctypes.data, c.size, None))


# ----------------------------------------------------------------- plan --

def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Plan:
    """Decode plan for a list of containers (host copies of at least their
    metadata prefix)."""

    def __init__(self, host_containers: Sequence, device: int = 0):
        metas = [_host_u8(c) for c in host_containers]
        n = len(metas)
        ptrs = (ctypes.c_void_p * n)(*[m.ctypes.data for m in metas])
        sizes = (ctypes.c_size_t * n)(*[m.size for m in metas])
        h = ctypes.c_void_p()
        _raise(lib().df11_plan(ptrs, sizes, n, device, 0, ctypes.byref(h)))
        self._h = h
        self.n_tensors = n
        self.device = device
        self.infos = [self.info(t) for t in range(n)]

    @property
    def handle(self):
        return self._h

    def info(self, t: int) -> dict:
        info = TensorInfo()
        _raise(lib().df11_plan_info(self._h, t, ctypes.byref(info)))
        return info.as_dict()

    def set_wgs_per_cu(self, n: int) -> None:
        """Decode workgroups per compute unit for this plan's later
        launches: 0 for as many as fit, else a cap (df11_plan_set_wgs_per_cu)."""
        _raise(lib().df11_plan_set_wgs_per_cu(self._h, int(n)))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().df11_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _check_device_tensor(x, what: str, min_bytes: int, device: int, words16: bool = False):
    """What the C ABI cannot check for a device pointer: a contiguous CUDA
    tensor on the plan's device, at least min_bytes long (and of a 16-bit
    dtype for decoded words).  Alignment is checked by the library."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{what}: a CUDA tensor is needed")
    if (x.device.index or 0) != device:
        raise ValueError(f"{what}: on cuda:{x.device.index}, the decode runs on cuda:{device}")
    if not x.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    if words16 and x.element_size() != 2:
        raise ValueError(f"{what}: a 16-bit dtype is needed, not {x.dtype}")
    if x.numel() * x.element_size() < min_bytes:
        raise ValueError(f"{what}: {x.numel() * x.element_size()} bytes, at least {min_bytes} needed")


def _check_decode_args(plan: "Plan", t: int, container, out):
    if 0 <= t < plan.n_tensors:   # (another tensor number: the library reports it)
        info = plan.infos[t]
        _check_device_tensor(container, f"tensor {t}'s container", info["container_bytes"], plan.device)
        _check_device_tensor(out, f"tensor {t}'s output", 2 * info["n_elems"], plan.device, words16=True)


def decode(plan: Plan, t: int, container, out, stream=None):
    """Enqueue the decode of tensor t: container (uint8, device) -> out
    (16-bit dtype, device, n_elems)."""
    _check_decode_args(plan, t, container, out)
    _raise(lib().df11_decode(plan.handle, t, container.data_ptr(), out.data_ptr(),
                             _stream_handle(stream)))


def decode_batch(plan: Plan, containers: List, outs: List, stream=None):
    n = plan.n_tensors
    if len(containers) != n or len(outs) != n:
        raise ValueError("one container and one output per planned tensor")
    for t in range(n):
        _check_decode_args(plan, t, containers[t], outs[t])
    cp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in containers])
    op = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    _raise(lib().df11_decode_batch(plan.handle, cp, op, _stream_handle(stream)))


def bw_control(src, dst, device: int = 0, stream=None):
    """Enqueue the bandwidth-control kernel: read all of `src`, write all of
    `dst` (device tensors, sizes multiples of 16 bytes, `src` no larger than
    `dst`), no decoding."""
    _check_device_tensor(src, "src", 0, device)
    _check_device_tensor(dst, "dst", 0, device)
    _raise(lib().df11_bw_control(src.data_ptr(), src.numel() * src.element_size(), dst.data_ptr(),
                                 dst.numel() * dst.element_size(), device, _stream_handle(stream)))


def check(plan: Plan, stream=None):
    """Synchronize the stream and raise DF11Error(E_CORRUPT) if a decode found
    a stream inconsistent with its index."""
    _raise(lib().df11_check(plan.handle, _stream_handle(stream)))


# ---- NF12: the fixed-rate 12-bit format (layout in include/df11.h) --------

NF12_HEADER = 256


def nf12_encode(words, threads: int = 0) -> np.ndarray:
    """NF12 container (uint8 numpy array, host) of BF16 bit patterns."""
    w = np.ascontiguousarray(np.asarray(words).view(np.uint16).reshape(-1))
    cap = int(lib().df11_nf12_bound(w.size))
    out = np.empty(max(cap, 1), np.uint8)
    nbytes = ctypes.c_uint64(0)
    _raise(lib().df11_nf12_encode(w.ctypes.data, w.size, out.ctypes.data, cap, ctypes.byref(nbytes), threads))
    return out[: nbytes.value]


def nf12_validate(container) -> int:
    """Element count of a valid NF12 container (host); raises DF11Error."""
    c = _host_u8(container)
    n = ctypes.c_uint64(0)
    _raise(lib().df11_nf12_validate(c.ctypes.data, c.size, ctypes.byref(n)))
    return int(n.value)


def _check_nf12_args(h: np.ndarray, container, out, device: int):
    """The header validated (the library's error for a bad one), then the
    device tensors against its element count and total size."""
    _raise(lib().df11_nf12_validate(h.ctypes.data, NF12_HEADER, None))
    n = int(h[16:24].view(np.uint64)[0])
    total = int(h[72:80].view(np.uint64)[0])
    _check_device_tensor(container, "NF12 container", total, device)
    _check_device_tensor(out, "NF12 output", 2 * n, device, words16=True)


def nf12_decode(host_header, container, out, device: int = 0, stream=None):
    """Enqueue the decode of an NF12 container: host_header = host copy of
    (at least) its first 256 bytes, container = the device copy (uint8),
    out = device tensor of n_elems 16-bit words."""
    h = _host_u8(host_header)
    if h.size < NF12_HEADER:
        raise ValueError("the NF12 header is 256 bytes")
    _check_nf12_args(h, container, out, device)
    _raise(lib().df11_nf12_decode(h.ctypes.data, container.data_ptr(), out.data_ptr(), device,
                                  _stream_handle(stream)))


def nf12_decode_batch(host_headers: List, containers: List, outs: List, device: int = 0, stream=None):
    """Enqueue the decode of several NF12 containers (host header copies,
    device containers, device outputs), in as few launches as possible."""
    n = len(host_headers)
    if len(containers) != n or len(outs) != n:
        raise ValueError("one header, one container and one output per tensor")
    hs = [_host_u8(h) for h in host_headers]
    if any(h.size < NF12_HEADER for h in hs):
        raise ValueError("the NF12 header is 256 bytes")
    for h, c, o in zip(hs, containers, outs):
        _check_nf12_args(h, c, o, device)
    hp = (ctypes.c_void_p * n)(*[h.ctypes.data for h in hs])
    cp = (ctypes.c_void_p * n)(*[c.data_ptr() for c in containers])
    op = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    _raise(lib().df11_nf12_decode_batch(hp, cp, op, n, device, _stream_handle(stream)))
