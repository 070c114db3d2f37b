"""ctypes binding of libiq.so (include/iq.h), argument marshalling only.

Functions carry the C names.  Device buffers are torch tensors (PyTorch is used
for device memory and streams only); every step of the computation runs in the
library's HIP kernels.  If the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libiq.so")

IQ_OK = 0
IQ_FULL, IQ_FAST, IQ_PLANAR = 0, 1, 2
IQ_F32, IQ_F16 = 0, 1

_LIB = None


class IQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"iq status {status}: {message}")
        self.status = status


class IQConfigC(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("quats", ctypes.c_void_p),
        ("centroids", ctypes.POINTER(ctypes.c_float)),
    ]


class IQCacheC(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("capacity", ctypes.c_int64),
    ]


def lib() -> ctypes.CDLL:
    """Load libiq.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise IQError(-5, f"{LIB_PATH} is not built (python -m compressed_space_attention_isoquant_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.iq_codebook.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_float)]
        L.iq_codebook.restype = ctypes.c_int
        L.iq_quantize_append.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32, P,
                                         ctypes.POINTER(IQCacheC), P]
        L.iq_quantize_append.restype = ctypes.c_int
        L.iq_quantize_append_many.argtypes = [ctypes.POINTER(IQConfigC), i32, ctypes.POINTER(ctypes.c_void_p), i32,
                                              i32, i32, P, ctypes.POINTER(IQCacheC), P]
        L.iq_quantize_append_many.restype = ctypes.c_int
        L.iq_quantize_append_rope.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32, i32, P,
                                              ctypes.POINTER(IQCacheC), P, P]
        L.iq_quantize_append_rope.restype = ctypes.c_int
        L.iq_decode_attention_rope.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32,
                                               ctypes.POINTER(IQCacheC), P, i32, ctypes.POINTER(IQCacheC), P,
                                               i64, ctypes.c_float, P, i32, P, P, P, ctypes.c_size_t, P]
        L.iq_decode_attention_rope.restype = ctypes.c_int
        L.iq_dequantize.argtypes = [ctypes.POINTER(IQConfigC), ctypes.POINTER(IQCacheC), i32, P, i32,
                                    P, i32, P]
        L.iq_dequantize.restype = ctypes.c_int
        L.iq_decode_workspace_bytes.argtypes = [ctypes.POINTER(IQConfigC), i32, i32, i64]
        L.iq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.iq_decode_attention.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32,
                                          ctypes.POINTER(IQCacheC), ctypes.POINTER(IQCacheC), P, i64,
                                          ctypes.c_float, P, i32, P, P, P, ctypes.c_size_t, P]
        L.iq_decode_attention.restype = ctypes.c_int
        L.iq_decode_attention_partial.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32,
                                                  ctypes.POINTER(IQCacheC), ctypes.POINTER(IQCacheC), P,
                                                  i64, ctypes.c_float, i32, P, ctypes.c_size_t, P]
        L.iq_decode_attention_partial.restype = ctypes.c_int
        L.iq_decode_attention_merge.argtypes = [ctypes.POINTER(IQConfigC), i32, i32, i64, P, i32, P, P,
                                                P, ctypes.c_size_t, P]
        L.iq_decode_attention_merge.restype = ctypes.c_int
        L.iq_decode_attention_noalloc.argtypes = [ctypes.POINTER(IQConfigC), P, i32, i32, i32,
                                                  ctypes.POINTER(IQCacheC), ctypes.POINTER(IQCacheC), P, i64,
                                                  ctypes.c_float, P, i32, P, P, P]
        L.iq_decode_attention_noalloc.restype = ctypes.c_int
        L.iq_probe_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
        L.iq_probe_stream_read.restype = ctypes.c_int
        L.iq_status_string.argtypes = [ctypes.c_int]
        L.iq_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != IQ_OK:
        raise IQError(status, iq_status_string(status))


def iq_status_string(status: int) -> str:
    return lib().iq_status_string(int(status)).decode()


def iq_codebook(bits: int, head_dim: int) -> np.ndarray:
    """Host fp32 Lloyd-Max codebook (ascending) from the library."""
    out = np.empty(1 << bits, dtype=np.float32)
    _check(lib().iq_codebook(bits, head_dim, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


@dataclass
class Config:
    """Mirror of iq_config.  ``quats``: device fp32 tensor of block-rotation
    parameters, (H_kv, d/4, 2, 4) quaternion pairs for Full and Fast or
    (H_kv, d/2, 2) pair rotations for Planar; ``centroids``: host fp32 array
    of 2**bits values."""

    head_dim: int
    bits: int
    variant: int
    num_kv_heads: int
    quats: object
    centroids: np.ndarray
    _c: IQConfigC = field(default=None, repr=False)

    def c(self) -> IQConfigC:
        self.centroids = np.ascontiguousarray(self.centroids, dtype=np.float32)
        self._c = IQConfigC(self.head_dim, self.bits, self.variant, self.num_kv_heads,
                            _ptr(self.quats),
                            self.centroids.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        return self._c


@dataclass
class PackedCache:
    """Mirror of iq_cache: ``codes`` uint8 (B, H_kv, cap, d*b/8) and ``norms``
    int16 holding fp16 bit patterns (B, H_kv, cap), both device tensors."""

    codes: object
    norms: object

    @property
    def capacity(self) -> int:
        return int(self.codes.shape[2])

    def c(self) -> IQCacheC:
        return IQCacheC(_ptr(self.codes), _ptr(self.norms), self.capacity)


def new_cache(batch: int, num_kv_heads: int, capacity: int, head_dim: int, bits: int, device) -> PackedCache:
    import torch

    codes = torch.zeros((batch, num_kv_heads, capacity, head_dim * bits // 8), dtype=torch.uint8, device=device)
    norms = torch.zeros((batch, num_kv_heads, capacity), dtype=torch.int16, device=device)
    return PackedCache(codes, norms)


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return IQ_F32
    if t.dtype == torch.float16:
        return IQ_F16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def iq_quantize_append(cfg: Config, x, start_pos, out: PackedCache, stream=None) -> None:
    """x: (B, n_new, H_kv, d) fp32/fp16; start_pos: int32 (B,) device tensor."""
    batch, n_new = int(x.shape[0]), int(x.shape[1])
    cc, oc = cfg.c(), out.c()
    _check(lib().iq_quantize_append(ctypes.byref(cc), _ptr(x), _dtype_code(x), batch, n_new,
                                    _ptr(start_pos), ctypes.byref(oc), _stream(stream)))


def prepare_append_many(cfgs, xs, outs):
    """Marshal the arguments of iq_quantize_append_many once: returns
    f(start_pos, stream=None) that enqueues the call (the tensors must stay
    alive and in place).  Tensor i: xs[i] (B, n_new, H_kv, d), quantised with
    cfgs[i] into outs[i]; all of one shape, dtype and codebook."""
    n = len(xs)
    if not (len(cfgs) == n == len(outs)) or n == 0:
        raise ValueError("cfgs, xs and outs must be non-empty lists of one length")
    batch, n_new = int(xs[0].shape[0]), int(xs[0].shape[1])
    for x in xs:
        if tuple(x.shape) != tuple(xs[0].shape) or x.dtype != xs[0].dtype:
            raise ValueError("every input must have the first one's shape and dtype")
    keep = [c.c() for c in cfgs]
    cc = (IQConfigC * n)(*keep)
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    oc = (IQCacheC * n)(*[o.c() for o in outs])
    dt = _dtype_code(xs[0])
    L = lib()

    def call(start_pos, stream=None):
        _check(L.iq_quantize_append_many(cc, n, xp, dt, batch, n_new, _ptr(start_pos), oc, _stream(stream)))

    call.keep = (keep, cfgs, xs, outs)
    return call


def iq_quantize_append_many(cfgs, xs, start_pos, outs, stream=None) -> None:
    """Tensor i: xs[i] (B, n_new, H_kv, d), quantised with cfgs[i] into outs[i];
    all of one shape, dtype and codebook; start_pos int32 (B,) device tensor."""
    prepare_append_many(cfgs, xs, outs)(start_pos, stream)


def iq_quantize_append_rope(cfg: Config, x, rope_dim: int, start_pos, out: PackedCache, rope_out,
                            stream=None) -> None:
    """x: (B, n_new, H_kv, d + rope_dim) fp32/fp16, RoPE coordinates last;
    rope_out: int16 (B, H_kv, capacity, rope_dim) device tensor (fp16 bits)."""
    batch, n_new = int(x.shape[0]), int(x.shape[1])
    cc, oc = cfg.c(), out.c()
    _check(lib().iq_quantize_append_rope(ctypes.byref(cc), _ptr(x), _dtype_code(x), batch, n_new, int(rope_dim),
                                         _ptr(start_pos), ctypes.byref(oc), _ptr(rope_out), _stream(stream)))


def iq_dequantize(cfg: Config, cache: PackedCache, start_pos, n: int, out, stream=None) -> None:
    """out: (B, n, H_kv, d) fp32/fp16 device tensor."""
    batch = int(out.shape[0])
    cc, ic = cfg.c(), cache.c()
    _check(lib().iq_dequantize(ctypes.byref(cc), ctypes.byref(ic), batch, _ptr(start_pos), int(n),
                               _ptr(out), _dtype_code(out), _stream(stream)))


def iq_decode_workspace_bytes(cfg: Config, batch: int, num_q_heads: int, max_kv_len: int) -> int:
    cc = cfg.c()
    return int(lib().iq_decode_workspace_bytes(ctypes.byref(cc), batch, num_q_heads, int(max_kv_len)))


def iq_decode_attention(cfg: Config, q, k: PackedCache, v: PackedCache, kv_len, max_kv_len: int,
                        softmax_scale: float, out, lse=None, argmax=None, workspace=None,
                        stream=None) -> None:
    """q/out: (B, Hq, d); kv_len int32 (B,) device; lse fp32 (B, Hq), argmax
    int32 (B, Hq) optional; workspace uint8 device tensor of at least
    iq_decode_workspace_bytes bytes."""
    batch, hq = int(q.shape[0]), int(q.shape[1])
    cc, kc, vc = cfg.c(), k.c(), v.c()
    if workspace is None:
        raise ValueError("workspace tensor required (size from iq_decode_workspace_bytes)")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().iq_decode_attention(ctypes.byref(cc), _ptr(q), _dtype_code(q), batch, hq,
                                     ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), int(max_kv_len),
                                     float(softmax_scale), _ptr(out), _dtype_code(out),
                                     _ptr(lse), _ptr(argmax), _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def iq_decode_attention_rope(cfg: Config, q, k: PackedCache, k_rope, v: PackedCache, kv_len, max_kv_len: int,
                             softmax_scale: float, out, lse=None, argmax=None, workspace=None,
                             stream=None) -> None:
    """As iq_decode_attention with a RoPE sub-block: q (B, Hq, d + r), k_rope
    int16 (B, H_kv, capacity, r) fp16 bits; out (B, Hq, d)."""
    batch, hq = int(q.shape[0]), int(q.shape[1])
    rope_dim = int(k_rope.shape[-1])
    cc, kc, vc = cfg.c(), k.c(), v.c()
    if workspace is None:
        raise ValueError("workspace tensor required (size from iq_decode_workspace_bytes)")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().iq_decode_attention_rope(ctypes.byref(cc), _ptr(q), _dtype_code(q), batch, hq,
                                          ctypes.byref(kc), _ptr(k_rope), rope_dim, ctypes.byref(vc),
                                          _ptr(kv_len), int(max_kv_len), float(softmax_scale), _ptr(out),
                                          _dtype_code(out), _ptr(lse), _ptr(argmax), _ptr(workspace), ws_bytes,
                                          _stream(stream)))


def iq_decode_attention_partial(cfg: Config, q, k: PackedCache, v: PackedCache, kv_len, max_kv_len: int,
                                softmax_scale: float, workspace, track_argmax: bool = True,
                                stream=None) -> None:
    """Split phase of iq_decode_attention (partial softmax states into workspace)."""
    batch, hq = int(q.shape[0]), int(q.shape[1])
    cc, kc, vc = cfg.c(), k.c(), v.c()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().iq_decode_attention_partial(ctypes.byref(cc), _ptr(q), _dtype_code(q), batch, hq,
                                             ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len),
                                             int(max_kv_len), float(softmax_scale), int(bool(track_argmax)),
                                             _ptr(workspace), ws_bytes, _stream(stream)))


def iq_decode_attention_merge(cfg: Config, batch: int, num_q_heads: int, max_kv_len: int, out,
                              lse=None, argmax=None, workspace=None, stream=None) -> None:
    """Merge phase of iq_decode_attention (combine, normalise, one R^T)."""
    cc = cfg.c()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().iq_decode_attention_merge(ctypes.byref(cc), int(batch), int(num_q_heads), int(max_kv_len),
                                           _ptr(out), _dtype_code(out), _ptr(lse), _ptr(argmax),
                                           _ptr(workspace), ws_bytes, _stream(stream)))


def iq_decode_attention_noalloc(cfg: Config, q, k: PackedCache, v: PackedCache, kv_len, max_kv_len: int,
                                softmax_scale: float, out, lse=None, argmax=None, stream=None) -> None:
    """iq_decode_attention with the library's own fixed workspace (no
    workspace argument, nothing allocated)."""
    batch, hq = int(q.shape[0]), int(q.shape[1])
    cc, kc, vc = cfg.c(), k.c(), v.c()
    _check(lib().iq_decode_attention_noalloc(ctypes.byref(cc), _ptr(q), _dtype_code(q), batch, hq,
                                             ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), int(max_kv_len),
                                             float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(lse),
                                             _ptr(argmax), _stream(stream)))


def iq_probe_stream_read(buf, sink, stream=None) -> None:
    """Measurement helper (include/iq_probe.h): reads the device tensor
    ``buf`` (16-byte aligned, size a multiple of 16 bytes) once; ``sink`` is a
    device tensor of at least 4 bytes."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().iq_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
