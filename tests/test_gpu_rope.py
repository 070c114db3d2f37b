"""GPU parity of the RoPE sub-block split (keys whose last coordinates are
RoPE coordinates, neither rotated nor quantised) against the oracle.

Bars as for the plain path: content codes bit-exact outside the 1e-6
boundary band, norms bit-exact outside the fp16 midpoint band, the fp16 RoPE
coordinates bit-exact, attention outputs within max-abs 2e-3 on the fp32
output for fp16 queries and 1e-5 for fp32 queries, lse within 1e-4, argmax
equal.
"""

import numpy as np
import pytest

import oracle as O
from compressed_space_attention_isoquant_amd import binding as B
from tests.gpu_helpers import DEV, host_cache, make_config, reconcile_codes, reconcile_norms, say, scale_for, torch
from tests.test_gpu_decode import check_outputs

pytestmark = pytest.mark.gpu

R = 64


def append_keys(cfg, k, cap, start):
    """k: host (B, n, H_kv, d + R); returns (PackedCache, rope int16 tensor)."""
    t = torch()
    batch, n, hkv, _ = k.shape
    cache = B.new_cache(batch, hkv, cap, cfg.head_dim, cfg.bits, DEV)
    rope = t.zeros((batch, hkv, cap, R), dtype=t.int16, device=DEV)
    sp = t.from_numpy(np.asarray(start, np.int32)).to(DEV)
    B.iq_quantize_append_rope(cfg, t.from_numpy(np.ascontiguousarray(k)).to(DEV), R, sp, cache, rope)
    return cache, rope


@pytest.mark.parametrize("d,dt", [(128, np.float16), (128, np.float32), (256, np.float16), (512, np.float32)])
def test_rope_append(d, dt):
    bits, batch, n, hkv, cap = 3, 2, 37, 2, 50
    start = [3, 0]
    rng = np.random.default_rng(60 + d)
    cfg, quats = make_config(d, bits, O.FULL, hkv)
    k = (rng.standard_normal((batch, n, hkv, d + R)) * 3).astype(dt)
    cache, rope = append_keys(cfg, k, cap, start)
    codes, norms = host_cache(cache)
    rp = rope.cpu().numpy().view(np.uint16)
    cb = O.codebook(bits, d)
    for b in range(batch):
        rows = slice(start[b], start[b] + n)
        for h in range(hkv):
            ref = O.quantize_rope(k[b, :, h], quats[h], cb, O.FULL, R)
            _, nf, nm = reconcile_codes(codes[b, h, rows], ref["codes"], ref["flags"], bits, d)
            reconcile_norms(norms[b, h, rows], ref["norm16"], ref["norm_flags"])
            assert np.array_equal(rp[b, h, rows], ref["rope16"])
            untouched = np.ones(cap, bool)
            untouched[rows] = False
            assert not rp[b, h, untouched].any() and not codes[b, h, untouched].any()
    say(f"rope append d={d} {np.dtype(dt).name}: content codes and norms as the oracle's, RoPE rows bit-exact")


def oracle_rope_decode(q, k, v, quats, cfg, lens, kc, rope, vc):
    """The oracle's attention over its own quantisation of k (content) and v,
    boundary-band ties resolved to the GPU's validated choice, RoPE rows from
    the oracle (checked equal to the GPU's)."""
    t_codes, t_norms = host_cache(kc)
    v_codes, v_norms = host_cache(vc)
    rp = rope.cpu().numpy().view(np.uint16)
    d, bits, hkv = cfg.head_dim, cfg.bits, cfg.num_kv_heads
    cb = O.codebook(bits, d)
    outs, lses, args = [], [], []
    for b in range(q.shape[0]):
        T = int(lens[b])
        kr = np.zeros((hkv, T, d * bits // 8), np.uint8)
        kn = np.zeros((hkv, T), np.uint16)
        kp = np.zeros((hkv, T, R), np.uint16)
        vr, vn = np.zeros_like(kr), np.zeros_like(kn)
        for g in range(hkv):
            if T == 0:
                continue
            rk = O.quantize_rope(k[b, :T, g], quats[g], cb, cfg.variant, R)
            ck, _, _ = reconcile_codes(t_codes[b, g, :T], rk["codes"], rk["flags"], bits, d)
            nk, _, _ = reconcile_norms(t_norms[b, g, :T], rk["norm16"], rk["norm_flags"])
            assert np.array_equal(rp[b, g, :T], rk["rope16"])
            kr[g], kn[g], kp[g] = O.pack(ck, bits), nk, rk["rope16"]
            rv = O.quantize(v[b, :T, g], quats[g], cb, cfg.variant)
            cv, _, _ = reconcile_codes(v_codes[b, g, :T], rv["codes"], rv["flags"], bits, d)
            nv, _, _ = reconcile_norms(v_norms[b, g, :T], rv["norm16"], rv["norm_flags"])
            vr[g], vn[g] = O.pack(cv, bits), nv
        o, l, a = O.attend_rope(q[b], kr, kn, kp, vr, vn, quats, cb, bits, cfg.variant, scale_for(d))
        outs.append(o)
        lses.append(l)
        args.append(a)
    return np.stack(outs), np.stack(lses), np.stack(args)


def run_rope_decode(cfg, q, kc, rope, vc, lens, max_len):
    t = torch()
    batch, hq, _ = q.shape
    d = cfg.head_dim
    out = t.empty((batch, hq, d), dtype=t.float32, device=DEV)
    lse = t.empty((batch, hq), dtype=t.float32, device=DEV)
    arg = t.empty((batch, hq), dtype=t.int32, device=DEV)
    ws = t.empty((B.iq_decode_workspace_bytes(cfg, batch, hq, max_len),), dtype=t.uint8, device=DEV)
    B.iq_decode_attention_rope(cfg, t.from_numpy(np.ascontiguousarray(q)).to(DEV), kc, rope, vc,
                               t.from_numpy(np.asarray(lens, np.int32)).to(DEV), max_len, scale_for(d), out, lse,
                               arg, ws)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy(), arg.cpu().numpy()


@pytest.mark.parametrize("d,bits,hq,hkv,variant,qdt", [
    (128, 3, 8, 8, O.FULL, np.float16), (128, 2, 16, 4, O.FAST, np.float16), (128, 4, 8, 2, O.PLANAR, np.float16),
    (128, 3, 32, 4, O.FAST, np.float16), (128, 3, 16, 8, O.FULL, np.float32),
    (256, 3, 16, 8, O.FAST, np.float16), (256, 4, 8, 1, O.FULL, np.float32), (256, 2, 4, 4, O.PLANAR, np.float16),
    (512, 3, 8, 2, O.FULL, np.float16), (512, 2, 16, 2, O.FAST, np.float32)])
def test_rope_decode_ragged(d, bits, hq, hkv, variant, qdt):
    """Three sequences (one empty, one a single token, one of 651 tokens)."""
    cap, lens = 700, [0, 1, 651]
    batch = len(lens)
    rng = np.random.default_rng(61 + bits + hq + d - 128)
    cfg, quats = make_config(d, bits, variant, hkv)
    k = (rng.standard_normal((batch, cap, hkv, d + R)) * 2).astype(np.float16)
    v = (rng.standard_normal((batch, cap, hkv, d)) * 2).astype(np.float16)
    q = rng.standard_normal((batch, hq, d + R)).astype(qdt)
    kc, rope = append_keys(cfg, k, cap, [0] * batch)
    vc = B.new_cache(batch, hkv, cap, d, bits, DEV)
    t = torch()
    B.iq_quantize_append(cfg, t.from_numpy(v).to(DEV), t.zeros((batch,), dtype=t.int32, device=DEV), vc)
    got, lse, arg = run_rope_decode(cfg, q, kc, rope, vc, lens, max(lens))
    ref, rlse, rarg = oracle_rope_decode(q, k, v, quats, cfg, lens, kc, rope, vc)
    # fp32 queries and outputs: the fp32 I/O bar (the fp16 RoPE rows are
    # exact inputs on both sides, so they set no looser bound)
    tol = 1e-5 if qdt == np.float32 else 2e-3
    check_outputs(f"rope decode d={d} b={bits} G={hq // hkv} v={variant} q={np.dtype(qdt).name}", got, lse, arg,
                  ref, rlse, rarg, tol, check_arg=True)
    assert np.all(got[0] == 0) and np.all(arg[0] == -1)


def test_rope_decode_8k_positional_needles():
    """One 8K context, 32 query / 4 KV heads: for each KV head one token's
    RoPE key is planted along a query head's RoPE part, with content keys
    random, so that only the RoPE term can make it the argmax."""
    d, bits, hq, hkv, T = 128, 3, 32, 4, 8192
    rng = np.random.default_rng(62)
    cfg, quats = make_config(d, bits, O.FULL, hkv)
    k = rng.standard_normal((1, T, hkv, d + R))
    v = rng.standard_normal((1, T, hkv, d))
    q = rng.standard_normal((1, hq, d + R))
    planted = []
    for g in range(hkv):
        h = g * (hq // hkv) + g % (hq // hkv)
        p = int(rng.integers(0, T))
        qr = q[0, h, d:]
        k[0, p, g, d:] = 40.0 * qr / np.linalg.norm(qr)
        planted.append((h, p))
    k, v, q = k.astype(np.float16), v.astype(np.float16), q.astype(np.float16)
    kc, rope = append_keys(cfg, k, T, [0])
    vc = B.new_cache(1, hkv, T, d, bits, DEV)
    t = torch()
    B.iq_quantize_append(cfg, t.from_numpy(v).to(DEV), t.zeros((1,), dtype=t.int32, device=DEV), vc)
    got, lse, arg = run_rope_decode(cfg, q, kc, rope, vc, [T], T)
    ref, rlse, rarg = oracle_rope_decode(q, k, v, quats, cfg, [T], kc, rope, vc)
    check_outputs("rope decode 8K", got, lse, arg, ref, rlse, rarg, 2e-3, check_arg=True)
    for h, p in planted:
        assert arg[0, h] == p and rarg[0, h] == p
    say(f"rope decode 8K: planted RoPE keys are the argmax of their heads {planted}")
