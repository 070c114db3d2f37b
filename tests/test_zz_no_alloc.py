"""GPU check of iq_decode_attention_noalloc (the decode entry point that
allocates nothing and keeps its workspace in a fixed array of the library):
two calls in a row, the second smaller, each against iq_decode_attention on
the same inputs with a workspace of the caller's."""

import numpy as np
import pytest

import oracle as O
from compressed_space_attention_isoquant_amd import binding as B
from tests.gpu_helpers import DEV, make_config, quantize_rows, say, scale_for, torch

pytestmark = pytest.mark.gpu


def both_calls(cfg, q, kc, vc, lens, out_dtype, with_lse):
    t = torch()
    batch, hq, d = q.shape
    qd = t.from_numpy(np.ascontiguousarray(q)).to(DEV)
    kv = t.from_numpy(np.asarray(lens, np.int32)).to(DEV)
    max_len = int(max(lens))
    res = []
    for noalloc in (False, True):
        out = t.empty((batch, hq, d), dtype=out_dtype, device=DEV)
        lse = t.empty((batch, hq), dtype=t.float32, device=DEV) if with_lse else None
        arg = t.empty((batch, hq), dtype=t.int32, device=DEV) if with_lse else None
        if noalloc:
            B.iq_decode_attention_noalloc(cfg, qd, kc, vc, kv, max_len, scale_for(d), out, lse, arg)
        else:
            ws = t.empty((B.iq_decode_workspace_bytes(cfg, batch, hq, max_len),), dtype=t.uint8, device=DEV)
            ws.fill_(0x5A)
            B.iq_decode_attention(cfg, qd, kc, vc, kv, max_len, scale_for(d), out, lse, arg, ws)
        t.cuda.synchronize()
        res.append([x.cpu().numpy() for x in (out, lse, arg) if x is not None])
    return res


def test_noalloc_equals_workspace_entry_point_twice():
    """A call on 4 ragged sequences (one empty) with fp32 output, lse and
    argmax, then a smaller call (2 sequences, fp16 output, no lse/argmax) on
    the same fixed workspace: each bit for bit equal to iq_decode_attention
    with a caller workspace (same kernels, same work split)."""
    t = torch()
    d, bits, hq, hkv = 128, 3, 32, 4
    rng = np.random.default_rng(90)
    cfg, _ = make_config(d, bits, O.FULL, hkv)
    cap = 3000
    k = (rng.standard_normal((4, cap, hkv, d)) * 2).astype(np.float16)
    v = (rng.standard_normal((4, cap, hkv, d)) * 2).astype(np.float16)
    kc, vc = quantize_rows(cfg, k), quantize_rows(cfg, v)
    q = rng.standard_normal((4, hq, d)).astype(np.float16)
    ref, got = both_calls(cfg, q, kc, vc, [3000, 17, 2500, 0], t.float32, True)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    assert np.all(got[0][3] == 0) and np.all(got[2][3] == -1)
    say("noalloc call 1 (4 sequences up to 3000 tokens): equal to the workspace entry point")
    # second, smaller call: two sequences, another KV layout
    hq2, hkv2 = 8, 2
    cfg2, _ = make_config(d, bits, O.FAST, hkv2)
    k2 = (rng.standard_normal((2, 900, hkv2, d)) * 2).astype(np.float16)
    v2 = (rng.standard_normal((2, 900, hkv2, d)) * 2).astype(np.float16)
    kc2, vc2 = quantize_rows(cfg2, k2), quantize_rows(cfg2, v2)
    q2 = rng.standard_normal((2, hq2, d)).astype(np.float16)
    ref2, got2 = both_calls(cfg2, q2, kc2, vc2, [900, 5], t.float16, False)
    assert np.array_equal(ref2[0], got2[0])
    say("noalloc call 2 (2 sequences up to 900 tokens): equal to the workspace entry point")


def test_noalloc_rejects_sizes_past_its_array():
    """A size whose workspace exceeds the fixed array (head_dim 512, 8 query
    heads per KV head) is rejected with IQ_ERR_WORKSPACE before anything
    runs."""
    t = torch()
    cfg, _ = make_config(512, 3, O.FULL, 1)
    kc = B.new_cache(1, 1, 16, 512, 3, DEV)
    vc = B.new_cache(1, 1, 16, 512, 3, DEV)
    q = t.zeros((1, 8, 512), dtype=t.float16, device=DEV)
    out = t.empty((1, 8, 512), dtype=t.float32, device=DEV)
    kv = t.full((1,), 16, dtype=t.int32, device=DEV)
    assert B.iq_decode_workspace_bytes(cfg, 1, 8, 16) > 64 << 20
    with pytest.raises(B.IQError) as e:
        B.iq_decode_attention_noalloc(cfg, q, kc, vc, kv, 16, 0.05, out)
    assert e.value.status == -4
