"""The C-ABI library loads, exports every symbol the headers under include/ declare, and
validates arguments on the host before anything is enqueued (CPU only: no
compute is launched here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from compressed_space_attention_isoquant_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Every function the headers under include/ declare."""
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(iq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"iq_quantize_append", "iq_dequantize", "iq_decode_attention",
                          "iq_decode_workspace_bytes", "iq_status_string", "iq_codebook",
                          "iq_decode_attention_partial", "iq_decode_attention_merge",
                          "iq_quantize_append_rope", "iq_decode_attention_rope", "iq_quantize_append_many",
                          "iq_probe_stream_read"}
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert B.iq_status_string(s)
    assert B.iq_status_string(123) == "unknown status"


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_library_codebook_equals_oracle(bits, d):
    # independent implementations of the Lloyd iteration reach the same
    # fixed point and the same fp32 rounding
    assert np.array_equal(B.iq_codebook(bits, d), O.codebook(bits, d))


def test_codebook_errors():
    L = B.lib()
    assert L.iq_codebook(3, 128, None) == -1
    buf = (ctypes.c_float * 64)()
    assert L.iq_codebook(5, 128, buf) == -2
    assert L.iq_codebook(0, 128, buf) == -2


class FakeTensor:
    """Stand-in carrying only a device address: every call below must fail in
    host validation, before any HIP call."""

    def __init__(self, addr, shape=(1, 1, 1, 1), dtype="float32"):
        self.addr = addr
        self.shape = shape
        import torch
        self.dtype = getattr(torch, dtype)

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self.addr

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return 1


def cfg(d=128, bits=3, variant=0, hkv=4, quats=0x1000, centroids=None):
    c = B.Config(d, bits, variant, hkv, FakeTensor(quats),
                 O.codebook(bits, d) if centroids is None else centroids)
    return c


def call_quant(c, x=0x2000, xdt=0, batch=1, n=1, sp=0x3000, codes=0x4000, norms=0x5000, cap=8):
    L = B.lib()
    cc = c.c()
    cache = B.IQCacheC(codes, norms, cap)
    return L.iq_quantize_append(ctypes.byref(cc), x, xdt, batch, n, sp, ctypes.byref(cache), None)


def test_quantize_validation():
    assert call_quant(cfg(d=96)) == -2
    assert call_quant(cfg(bits=5)) == -2
    assert call_quant(cfg(variant=3)) == -1      # Full, Fast and Planar are 0, 1, 2
    assert call_quant(cfg(variant=-1)) == -1
    assert call_quant(cfg(hkv=0)) == -1
    assert call_quant(cfg(quats=0x1004)) == -3
    assert call_quant(cfg(), x=0) == -1
    assert call_quant(cfg(), x=0x2008) == -3
    assert call_quant(cfg(), xdt=7) == -2
    assert call_quant(cfg(), batch=0) == -1
    assert call_quant(cfg(), n=9, cap=8) == -1
    assert call_quant(cfg(), sp=0) == -1
    assert call_quant(cfg(), codes=0) == -1
    assert call_quant(cfg(), norms=0x5002) == -3
    assert call_quant(cfg(), cap=0) == -1
    # batch * n_new must fit the kernels' 32-bit vector indices
    assert call_quant(cfg(), batch=1 << 16, n=1 << 15, cap=1 << 15) == -1
    bad = O.codebook(3, 128).copy()
    bad[3], bad[4] = bad[4], bad[3]
    assert call_quant(cfg(centroids=bad)) == -1
    nan = O.codebook(3, 128).copy()
    nan[0] = np.nan
    assert call_quant(cfg(centroids=nan)) == -1
    # quantize takes any finite, ascending fp32 codebook: a level with more
    # than 11 significant bits passes the configuration check (the call then
    # stops at the dtype, the next check)
    fine = O.codebook(3, 128).copy()
    fine[5] = np.nextafter(fine[5], np.float32(1))
    assert call_quant(cfg(centroids=fine), xdt=7) == -2


def call_decode(c, hq=32, batch=1, max_len=16, cap=16, ws_bytes=None, q=0x2000, out=0x6000,
                ws=0x7000, lse=None, arg=None, qdt=1, odt=0, kv=0x8000, scale=0.088):
    L = B.lib()
    cc = c.c()
    k = B.IQCacheC(0x4000, 0x5000, cap)
    v = B.IQCacheC(0x4000, 0x5000, cap)
    if ws_bytes is None:
        ws_bytes = L.iq_decode_workspace_bytes(ctypes.byref(cc), batch, hq, max_len)
    return L.iq_decode_attention(ctypes.byref(cc), q, qdt, batch, hq, ctypes.byref(k), ctypes.byref(v),
                                 kv, max_len, scale, out, odt, lse, arg, ws, ws_bytes, None)


def test_decode_validation():
    L = B.lib()
    c = cfg()
    cc = c.c()
    need = L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 32, 16)
    assert need > 0
    # workspace is O(pieces x d) per query head, never O(T x d)
    big = L.iq_decode_workspace_bytes(ctypes.byref(cc), 64, 32, 32768)
    assert big < 64 * 4 * 32768 * 128 * 2 // 16
    assert L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 30, 16) == 0
    assert call_decode(c, hq=30) == -1                      # Hq % H_kv != 0
    assert call_decode(c, hq=64) == -2                      # group 16 not built
    assert call_decode(c, ws_bytes=need - 1) == -4
    assert call_decode(c, max_len=17, cap=16) == -1
    assert call_decode(c, q=0x2004) == -3
    assert call_decode(c, lse=0x9004) == -3
    assert call_decode(c, qdt=3) == -2
    assert call_decode(c, kv=0) == -1
    assert call_decode(c, scale=float("inf")) == -1
    assert call_decode(c, batch=0) == -1
    assert call_decode(c, batch=65536) == -2                # grid limit
    assert L.iq_decode_workspace_bytes(ctypes.byref(cc), 65536, 32, 16) == 0
    assert call_decode(cfg(d=64)) == -2


def ratio_codebook(smallest):
    """Eight ascending levels with largest magnitude 1 and ``smallest`` the
    smallest positive one."""
    return np.array([-1.0, -0.5, -0.25, -0.125, smallest, 0.25, 0.5, 1.0], np.float32)


def test_decode_codebook_exactness():
    """Decode multiplies the levels (times the power of two that brings the
    largest into [1, 2)) on fp16 matrix cores, so it takes a codebook only if
    every scaled level is an fp16 number exactly: 11 significant bits over a
    max/min magnitude ratio below 2^14 always; the first 11-bit level past
    that is rejected (IQ_ERR_UNSUPPORTED, workspace size 0), while quantize
    still takes it.  Exact fp16 subnormals are accepted."""
    L = B.lib()
    ok_edge = 2.0 ** -14 * (1 + 2.0 ** -10)          # ratio just below 2^14: normal fp16
    first_bad = 2.0 ** -15 * (1 + 2.0 ** -10)        # ratio just below 2^15: not on the subnormal grid
    for smallest, fits in ((ok_edge, True), (first_bad, False), (2.0 ** -15, True), (3 * 2.0 ** -24, True),
                           (2.0 ** -25, False)):
        c = cfg(centroids=ratio_codebook(smallest))
        cc = c.c()
        need = L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 32, 16)
        assert (need > 0) == fits, smallest
        # an accepted codebook reaches the workspace check, a rejected one stops before
        assert call_decode(c, ws_bytes=0) == (-4 if fits else -2), smallest
        assert call_quant(c, xdt=7) == -2                    # quantize: past the codebook, stops at the dtype
    # the library's own codebooks always fit
    for bits in (2, 3, 4):
        for d in (128, 256, 512):
            cc = cfg(d=d, bits=bits).c()
            assert L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 32, 16) > 0
    # more than 11 significant bits: quantize yes, decode no
    fine = O.codebook(3, 128).copy()
    fine[5] = np.nextafter(fine[5], np.float32(1))
    assert call_decode(cfg(centroids=fine)) == -2


def test_dequantize_validation():
    L = B.lib()
    c = cfg()
    cc = c.c()
    cache = B.IQCacheC(0x4000, 0x5000, 8)
    assert L.iq_dequantize(ctypes.byref(cc), ctypes.byref(cache), 1, 0x3000, 9, 0x6000, 0, None) == -1
    assert L.iq_dequantize(ctypes.byref(cc), ctypes.byref(cache), 1, 0x3000, 4, 0x6002, 0, None) == -3
    assert L.iq_dequantize(ctypes.byref(cc), ctypes.byref(cache), 1, 0x3000, 4, 0x6000, 9, None) == -2
    assert L.iq_dequantize(ctypes.byref(cc), None, 1, 0x3000, 4, 0x6000, 0, None) == -1
    huge = B.IQCacheC(0x4000, 0x5000, 1 << 15)
    assert L.iq_dequantize(ctypes.byref(cc), ctypes.byref(huge), 1 << 16, 0x3000, 1 << 15, 0x6000, 0, None) == -1


def test_partial_and_merge_validation():
    L = B.lib()
    c = cfg()
    cc = c.c()
    need = L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 32, 16)
    k = B.IQCacheC(0x4000, 0x5000, 16)
    # partial: misaligned q, small workspace, bad group
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2004, 1, 1, 32, ctypes.byref(k), ctypes.byref(k),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -3
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 32, ctypes.byref(k), ctypes.byref(k),
                                         0x8000, 16, 0.1, 1, 0x7000, need - 16, None) == -4
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 64, ctypes.byref(k), ctypes.byref(k),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -2
    # a (sequence, head) region of 2^30 bytes or more is beyond 32-bit in-region offsets
    rows = (1 << 30) // 48
    huge = B.IQCacheC(0x4000, 0x5000, rows + 1)
    fine = B.IQCacheC(0x4000, 0x5000, rows)
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 32, ctypes.byref(huge), ctypes.byref(k),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -2
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 32, ctypes.byref(k), ctypes.byref(huge),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -2
    assert (1 << 30) - rows * 48 <= 48 and fine.capacity * 48 < (1 << 30)
    # an odd capacity: the last row's norm would straddle the region's end
    odd = B.IQCacheC(0x4000, 0x5000, 17)
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 32, ctypes.byref(odd), ctypes.byref(k),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -2
    assert L.iq_decode_attention_partial(ctypes.byref(cc), 0x2000, 1, 1, 32, ctypes.byref(k), ctypes.byref(odd),
                                         0x8000, 16, 0.1, 1, 0x7000, need, None) == -2
    # merge: null out, bad dtype, misaligned argmax
    assert L.iq_decode_attention_merge(ctypes.byref(cc), 1, 32, 16, None, 0, None, None, 0x7000, need, None) == -1
    assert L.iq_decode_attention_merge(ctypes.byref(cc), 1, 32, 16, 0x6000, 5, None, None, 0x7000, need, None) == -2
    assert L.iq_decode_attention_merge(ctypes.byref(cc), 1, 32, 16, 0x6000, 0, None, 0x9002, 0x7000, need, None) == -3
    assert L.iq_decode_attention_merge(ctypes.byref(cc), 1, 32, 16, 0x6000, 0, None, None, 0x7000, need - 4, None) == -4


def expected_workspace(batch, hq, hkv, d, max_len):
    """Workspace bytes from the documented layout, each part rounded up to
    256 bytes: the plan (a 16-byte header, 4096 per-wave shares of four
    int32 and batch + 1 int32 segment bases), the rotated queries (2 fp16 rows of
    d + 64 coordinates per query head), their scales (one float per query
    head), then the records: d + 4 floats per query head of a group for each
    of batch x H_kv + 4096 pieces.  No term grows with max_len."""
    up = lambda x: -(-x // 256) * 256
    group = hq // hkv
    plan = up(16 + 16 * 4096 + 4 * (batch + 1))
    qrot = up(batch * hq * 2 * (d + 64) * 2)
    qscale = up(batch * hq * 4)
    records = (batch * hkv + 4096) * group * (d + 4) * 4
    return plan + qrot + qscale + records


@pytest.mark.parametrize("batch,hq,hkv,d,max_len", [
    (64, 16, 8, 256, 32768), (64, 32, 4, 128, 32768), (1, 32, 4, 128, 8192), (1, 8, 8, 128, 131072),
    (1, 32, 4, 128, 32768), (16, 32, 4, 128, 32768),
    (4200, 2, 1, 128, 40), (3, 8, 2, 512, 1), (256, 8, 8, 256, 32768), (2, 4, 4, 128, 0)])
def test_decode_workspace_geometry(batch, hq, hkv, d, max_len):
    """The workspace layout, observed through its size."""
    L = B.lib()
    c = cfg(d=d, hkv=hkv)
    cc = c.c()
    got = L.iq_decode_workspace_bytes(ctypes.byref(cc), batch, hq, max_len)
    assert got == expected_workspace(batch, hq, hkv, d, max_len)



def test_rope_validation():
    """The RoPE entry points check their extra arguments before launching."""
    L = B.lib()
    c = cfg()
    cc = c.c()
    cache = B.IQCacheC(0x4000, 0x5000, 16)

    def append(rope_dim, rope_out=0x9000, x=0x2000):
        return L.iq_quantize_append_rope(ctypes.byref(cc), x, 1, 1, 4, rope_dim, 0x3000, ctypes.byref(cache),
                                         rope_out, None)

    assert append(0) == -1                      # use iq_quantize_append without RoPE coordinates
    assert append(12) == -2                     # not a multiple of 8
    assert append(520) == -2                    # above 512
    assert append(64, rope_out=None) == -1
    assert append(64, rope_out=0x9008) == -3

    need = L.iq_decode_workspace_bytes(ctypes.byref(cc), 1, 32, 16)

    def decode(rope_dim, k_rope=0x9000, conf=c, ws_bytes=need):
        ccx = conf.c()
        return L.iq_decode_attention_rope(ctypes.byref(ccx), 0x2000, 1, 1, 32, ctypes.byref(cache), k_rope,
                                          rope_dim, ctypes.byref(cache), 0x8000, 16, 0.1, 0x6000, 0, None, None,
                                          0x7000, ws_bytes, None)

    assert decode(0) == -1
    assert decode(32) == -2                     # the kernels take 64
    assert decode(64, k_rope=None) == -1
    assert decode(64, k_rope=0x9004) == -3
    # head_dim 512 at 4 bits: two stages with RoPE rows do not fit in LDS
    big = cfg(d=512, bits=4)
    assert decode(64, conf=big, ws_bytes=L.iq_decode_workspace_bytes(ctypes.byref(big.c()), 1, 32, 16)) == -2
    assert decode(64, ws_bytes=need - 1) == -4


def test_append_many_validation():
    """Several tensors per call: the configs must agree in shape and codebook."""
    L = B.lib()
    n = 3
    base = [cfg() for _ in range(n)]

    def call(cfgs, count=n, xs=(0x2000, 0x2100, 0x2200), cap=8):
        cc = (B.IQConfigC * len(cfgs))(*[c.c() for c in cfgs])
        xp = (ctypes.c_void_p * len(xs))(*xs)
        outs = (B.IQCacheC * len(cfgs))(*[B.IQCacheC(0x4000, 0x5000, cap) for _ in cfgs])
        return L.iq_quantize_append_many(cc, count, xp, 1, 1, 4, 0x3000, outs, None)

    assert call(base, count=0) == -1
    assert call(base[:2] + [cfg(bits=2)]) == -1                 # another bit width
    assert call(base[:2] + [cfg(hkv=2)]) == -1                  # another head count
    other = cfg()
    other.centroids = other.centroids.copy()
    other.centroids[0] *= 2.0                                  # still a valid codebook
    assert call(base[:2] + [other]) == -1                       # another codebook
    assert call(base, xs=(0x2000, 0x2108, 0x2200)) == -3        # misaligned input
    assert call(base, xs=(0x2000, 0, 0x2200)) == -1
    assert call(base, cap=2) == -1                              # n_new above a capacity
    assert call(base[:2] + [cfg(d=96)]) == -2


def test_probe_validation():
    """The read-bandwidth probe rejects bad arguments on the host, before any
    GPU call (the pointers below are never dereferenced)."""
    L = B.lib()
    S = ctypes.c_size_t
    assert L.iq_probe_stream_read(None, S(1024), ctypes.c_void_p(4096), None) == -1
    assert L.iq_probe_stream_read(ctypes.c_void_p(4096), S(1024), None, None) == -1
    assert L.iq_probe_stream_read(ctypes.c_void_p(4096), S(0), ctypes.c_void_p(4096), None) == -1
    assert L.iq_probe_stream_read(ctypes.c_void_p(4096), S(1000), ctypes.c_void_p(4096), None) == -1
    assert L.iq_probe_stream_read(ctypes.c_void_p(4100), S(1024), ctypes.c_void_p(4096), None) == -3
