"""GPU parity of the stage-1 path (quantize -> dequantize) against the oracle.

Bars (from the method's tolerance statement): packed codes bit-exact except
elements within 1e-6 of a decision threshold (counted and reported); fp16
norms bit-exact except norms within 1e-6 of an fp16 rounding midpoint;
dequantized vectors within max-abs 1e-5 (fp32 output) or 2e-3 (fp16 output)
of the oracle's dequantization of its own codes and norms (inside the bands,
where both neighbours are correct, with the GPU's validated choice).
"""

import math

import numpy as np
import pytest

import oracle as O
from compressed_space_attention_isoquant_amd import binding as B
from compressed_space_attention_isoquant_amd import inputs
from tests.gpu_helpers import (DEV, host_cache, make_config, quantize_rows, reconcile_codes,
                               reconcile_norms, say, torch)
from tests.test_oracle_quantizer import quant_mse_closed_form

pytestmark = pytest.mark.gpu

TOL = {np.float32: 1e-5, np.float16: 2e-3}
SETTINGS = [(v, d, b, dt) for v in (O.FULL, O.FAST) for d in (128, 256, 512) for b in (2, 3, 4)
            for dt in (np.float16, np.float32)]
# the 2-D special case: every width and bit count on ragged counts, full size at b = 3
PLANAR_SETTINGS = [(O.PLANAR, d, b, dt) for d in (128, 256, 512) for b in (2, 3, 4)
                   for dt in (np.float16, np.float32)]
PLANAR_FULL_SIZE = [s for s in PLANAR_SETTINGS if s[2] == 3]


def dequantize_gpu(cfg, cache, batch, n, hkv, d, out_dtype, start=0):
    t = torch()
    out = t.empty((batch, n, hkv, d), dtype=t.float16 if out_dtype == np.float16 else t.float32, device=DEV)
    sp = t.full((batch,), start, dtype=t.int32, device=DEV)
    B.iq_dequantize(cfg, cache, sp, n, out)
    t.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check_stage1(x, variant, d, bits, out_dtype, label):
    """x: (n, d) host vectors, one head.  Full element-by-element comparison."""
    n = x.shape[0]
    cfg, quats = make_config(d, bits, variant, 1)
    cache = quantize_rows(cfg, x[None, :, None, :])
    codes, norms = host_cache(cache)
    ref = O.quantize(x, quats[0], O.codebook(bits, d), variant)
    rc, nf, nfm = reconcile_codes(codes[0, 0], ref["codes"], ref["flags"], bits, d)
    rn, nnf, nnm = reconcile_norms(norms[0, 0], ref["norm16"], ref["norm_flags"])
    got = dequantize_gpu(cfg, cache, 1, n, 1, d, out_dtype)[0, :, 0]
    # the oracle dequantizes its own codes (boundary-band ties as the GPU chose)
    want = O.dequantize_codes(rc, rn, quats[0], O.codebook(bits, d), variant)
    err = float(np.max(np.abs(got - want)))
    say(f"{label}: n={n} flagged={nf} flagged_mismatch={nfm} norm_flagged={nnf} "
        f"norm_mismatch={nnm} dequant_maxabs={err:.3g}")
    assert err <= TOL[out_dtype], err
    return codes, norms, got


def test_c1_full_d128_b3_fp32():
    """4,096 unit vectors, d = 128, fp32, 3-bit, Full, quaternions from seed 0."""
    d, bits = 128, 3
    x = inputs.unit_vectors(4096, d, np.float32, seed=1)
    codes, norms, xr = check_stage1(x, O.FULL, d, bits, np.float32, "C1")
    err = np.sum((x.astype(np.float64) - xr) ** 2, axis=-1)
    expect = quant_mse_closed_form(d, O.codebook(bits, d))
    se = np.std(err) / math.sqrt(len(err))
    say(f"C1 MSE={np.mean(err):.6f} closed-form={expect:.6f} (+-4se {4 * se:.2g})")
    assert abs(np.mean(err) - expect) < 4 * se


@pytest.mark.parametrize("variant,d,bits,dt", SETTINGS + PLANAR_SETTINGS)
def test_stage1_settings_ragged(variant, d, bits, dt):
    # a count that is not a multiple of the per-workgroup vector count
    x = inputs.unit_vectors(1037, d, dt, seed=7 + d + bits)
    check_stage1(x, variant, d, bits, dt, f"ragged v={variant} d={d} b={bits} {np.dtype(dt).name}")


def test_edge_vectors():
    d, bits = 128, 3
    x = np.zeros((5, d), np.float32)
    x[1, 7] = 1.0                                  # a basis vector
    x[2] = 1e-20                                   # tiny
    x[3] = np.linspace(-3, 3, d)                   # large, non-unit
    x[4, :] = 0.5                                  # constant (WHT concentrates it)
    check_stage1(x, O.FULL, d, bits, np.float32, "edge")
    one = inputs.unit_vectors(1, 256, np.float16, seed=3)
    check_stage1(one, O.FAST, 256, 2, np.float16, "single")


def check_custom_codebook(cent, variant, d, dt, label):
    """Quantize with caller-supplied centroids; codes and norms against the
    oracle run on the same centroids."""
    t = torch()
    bits = int(np.log2(len(cent)))
    cent = np.asarray(cent, np.float32)
    quats = inputs.rotation_params(1, d, variant, seed=inputs.QUATERNION_SEED)
    cfg = B.Config(d, bits, variant, 1, t.from_numpy(quats).to(DEV), cent)
    x = inputs.unit_vectors(777, d, dt, seed=11 + bits)
    cache = quantize_rows(cfg, x[None, :, None, :])
    codes, norms = host_cache(cache)
    ref = O.quantize(x, quats[0], cent.astype(np.float64), variant)
    rc, nf, nfm = reconcile_codes(codes[0, 0], ref["codes"], ref["flags"], bits, d)
    rn, _, _ = reconcile_norms(norms[0, 0], ref["norm16"], ref["norm_flags"])
    got = dequantize_gpu(cfg, cache, 1, len(x), 1, d, np.float32)[0, :, 0]
    want = O.dequantize_codes(rc, rn, quats[0], cent.astype(np.float64), variant)
    err = float(np.max(np.abs(got - want)))
    hist = np.bincount(rc.ravel(), minlength=len(cent))
    say(f"{label}: flagged={nf} flagged_mismatch={nfm} dequant_maxabs={err:.3g} levels used={hist.tolist()}")
    assert err <= 1e-5
    return hist


def test_custom_codebook_with_close_thresholds():
    """Two decision thresholds 1e-6 apart (centroids 0, 2^-20, 2^-19): no
    cell of the code-lookup table can separate them, so the kernel counts
    thresholds directly; codes must still match."""
    cent = [-0.25, -0.125, -0.0625, 0.0, 2.0 ** -20, 2.0 ** -19, 0.125, 0.25]
    check_custom_codebook(cent, O.FULL, 128, np.float32, "close thresholds")


def test_custom_codebook_asymmetric():
    """An asymmetric 16-level codebook (fp16-exact levels) narrower than the
    data: values beyond the outer thresholds land in the clamped end cells."""
    k = np.arange(16) / 15.0
    cent = np.float16(-0.09 + 0.15 * k ** 1.3).astype(np.float32)
    hist = check_custom_codebook(cent, O.FAST, 256, np.float16, "asymmetric")
    assert hist[0] > 0 and hist[-1] > 0


@pytest.mark.parametrize("bits,d,variant,dt", [(3, 128, O.FULL, np.float32), (2, 256, O.FAST, np.float16),
                                                (4, 512, O.PLANAR, np.float32)])
def test_full_precision_fp32_codebook(bits, d, variant, dt):
    """Stage 1 takes a caller's codebook at full fp32 precision (the Lloyd-Max
    levels for N(0, 1/d) cast to fp32, not held to 11 significant bits): codes
    and dequantized vectors against the oracle on the same levels."""
    cent = (O.lloyd_max_gaussian(bits) / np.sqrt(d)).astype(np.float32)
    assert not np.array_equal(cent, O.codebook(bits, d))          # really beyond fp16 precision
    check_custom_codebook(cent, variant, d, dt, f"fp32 codebook b={bits} d={d}")


def test_append_offsets_batches_and_heads():
    """batch 3, 4 KV heads, rows appended at different start positions."""
    t = torch()
    d, bits, hkv, batch, n, cap = 256, 3, 4, 3, 40, 100
    cfg, quats = make_config(d, bits, O.FAST, hkv)
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((batch, n, hkv, d)) * 5).astype(np.float16)
    starts = np.array([0, 17, 60], np.int32)
    cache = B.new_cache(batch, hkv, cap, d, bits, DEV)
    B.iq_quantize_append(cfg, t.from_numpy(x).to(DEV), t.from_numpy(starts).to(DEV), cache)
    codes, norms = host_cache(cache)
    cb = O.codebook(bits, d)
    own = {}
    for b in range(batch):
        for h in range(hkv):
            ref = O.quantize(x[b, :, h], quats[h], cb, O.FAST)
            rows = codes[b, h, starts[b]:starts[b] + n]
            rc, _, _ = reconcile_codes(rows, ref["codes"], ref["flags"], bits, d)
            rn, _, _ = reconcile_norms(norms[b, h, starts[b]:starts[b] + n], ref["norm16"], ref["norm_flags"])
            own[b, h] = (rc, rn)
            # rows outside the appended range stay untouched (zero)
            untouched = np.ones(cap, bool)
            untouched[starts[b]:starts[b] + n] = False
            assert not codes[b, h, untouched].any() and not norms[b, h, untouched].any()
    out = t.empty((batch, n, hkv, d), dtype=t.float32, device=DEV)
    B.iq_dequantize(cfg, cache, t.from_numpy(starts).to(DEV), n, out)
    got = out.cpu().numpy()
    for b in range(batch):
        for h in range(hkv):
            want = O.dequantize_codes(own[b, h][0], own[b, h][1], quats[h], cb, O.FAST)
            assert np.max(np.abs(got[b, :, h] - want)) <= 1e-5 * max(1.0, np.max(np.abs(want)))


def test_prefill_bulk_compression():
    """Deferred-prefill compression ([RQ] Appendix C): two sequences' 2,048
    prefill tokens x 8 KV heads appended in one call each (n_new = 2048) at
    different start rows; sampled (sequence, head) pairs against the oracle,
    rows outside the appended ranges untouched."""
    t = torch()
    d, bits, hkv, batch, n, cap = 128, 3, 8, 2, 2048, 2100
    cfg, quats = make_config(d, bits, O.FULL, hkv)
    rng = np.random.default_rng(17)
    ch = inputs.outlier_channels(rng, hkv, d)
    scale = np.ones((hkv, d))
    for h in range(hkv):
        scale[h, ch[h]] = inputs.OUTLIER_SCALE
    x = (rng.standard_normal((batch, n, hkv, d)) * scale).astype(np.float16)
    starts = np.array([0, 52], np.int32)
    cache = B.new_cache(batch, hkv, cap, d, bits, DEV)
    B.iq_quantize_append(cfg, t.from_numpy(x).to(DEV), t.from_numpy(starts).to(DEV), cache)
    codes, norms = host_cache(cache)
    cb = O.codebook(bits, d)
    for b, h in ((0, 0), (0, 7), (1, 3), (1, 6)):
        ref = O.quantize(x[b, :, h], quats[h], cb, O.FULL)
        rows = slice(starts[b], starts[b] + n)
        _, nf, nfm = reconcile_codes(codes[b, h, rows], ref["codes"], ref["flags"], bits, d)
        reconcile_norms(norms[b, h, rows], ref["norm16"], ref["norm_flags"])
        untouched = np.ones(cap, bool)
        untouched[rows] = False
        assert not codes[b, h, untouched].any() and not norms[b, h, untouched].any()
        say(f"prefill (b={b}, h={h}): flagged={nf} flagged_mismatch={nfm}")


@pytest.mark.parametrize("idx,setting", list(enumerate(SETTINGS)) +
                         [(100 + i, s) for i, s in enumerate(PLANAR_FULL_SIZE)])
def test_c2_full_size_sampled(idx, setting):
    """2^20 unit vectors per setting quantized and dequantized on the GPU; the
    oracle checks 2,048 sampled vectors (the last ones included) element by
    element, and the mean reconstruction error over all 2^20 vectors matches
    the closed form."""
    t = torch()
    variant, d, bits, dt = setting
    n = 1 << 20
    tdt = t.float16 if dt == np.float16 else t.float32
    cfg, quats = make_config(d, bits, variant, 1)
    x = inputs.device_unit_vectors(2 + idx, n, d, DEV, tdt)
    cache = B.new_cache(1, 1, n, d, bits, DEV)
    sp = t.zeros((1,), dtype=t.int32, device=DEV)
    B.iq_quantize_append(cfg, x.view(1, n, 1, d), sp, cache)
    out = t.empty((1, n, 1, d), dtype=tdt, device=DEV)
    B.iq_dequantize(cfg, cache, sp, n, out)
    mse_all = float(((x.float() - out.float().view(n, d)) ** 2).sum(dim=-1).double().mean())
    rng = np.random.default_rng(idx)
    sample = np.unique(np.concatenate([rng.choice(n, 2000, replace=False), np.arange(n - 48, n)]))
    sidx = t.from_numpy(sample).to(DEV)
    xs = x[sidx].cpu().numpy()
    rows = cache.codes[0, 0][sidx].cpu().numpy()
    norms = cache.norms[0, 0][sidx].cpu().numpy().view(np.uint16)
    got = out.view(n, d)[sidx].float().cpu().numpy().astype(np.float64)
    cb = O.codebook(bits, d)
    ref = O.quantize(xs, quats[0], cb, variant)
    rc, nf, nfm = reconcile_codes(rows, ref["codes"], ref["flags"], bits, d)
    rn, _, _ = reconcile_norms(norms, ref["norm16"], ref["norm_flags"])
    want = O.dequantize_codes(rc, rn, quats[0], cb, variant)
    err = float(np.max(np.abs(got - want)))
    expect = quant_mse_closed_form(d, cb)
    say(f"C2[{idx}] v={variant} d={d} b={bits} {np.dtype(dt).name}: flagged={nf}/{nfm} "
        f"dequant_maxabs={err:.3g} mse={mse_all:.6f} closed={expect:.6f}")
    assert err <= TOL[dt]
    # fp16 inputs are unit vectors only to fp16 precision: allow 0.5% slack
    assert abs(mse_all - expect) < (0.002 if dt == np.float32 else 0.005) * expect + 2e-5


def test_append_many_equals_single_appends():
    """20 tensors (two launches of up to 16) with their own rotations appended
    in one call: every cache equals what a separate iq_quantize_append call
    writes; one tensor is also checked against the oracle."""
    t = torch()
    d, bits, hkv, batch, n, cap, count = 128, 3, 4, 2, 300, 320, 20
    rng = np.random.default_rng(70)
    cfgs, quats = [], []
    for i in range(count):
        q = inputs.quaternions(hkv, d, seed=100 + i)
        quats.append(q)
        cfgs.append(B.Config(d, bits, O.FULL, hkv, t.from_numpy(q).to(DEV), B.iq_codebook(bits, d)))
    xs = [t.from_numpy((rng.standard_normal((batch, n, hkv, d)) * 3).astype(np.float16)).to(DEV)
          for _ in range(count)]
    sp = t.from_numpy(np.array([7, 0], np.int32)).to(DEV)
    many = [B.new_cache(batch, hkv, cap, d, bits, DEV) for _ in range(count)]
    B.iq_quantize_append_many(cfgs, xs, sp, many)
    for i in range(count):
        one = B.new_cache(batch, hkv, cap, d, bits, DEV)
        B.iq_quantize_append(cfgs[i], xs[i], sp, one)
        t.cuda.synchronize()
        assert t.equal(one.codes, many[i].codes) and t.equal(one.norms, many[i].norms), i
    codes, norms = host_cache(many[13])
    x = xs[13].cpu().numpy()
    for b, s0 in ((0, 7), (1, 0)):
        for h in range(hkv):
            ref = O.quantize(x[b, :, h], quats[13][h], O.codebook(bits, d), O.FULL)
            reconcile_codes(codes[b, h, s0:s0 + n], ref["codes"], ref["flags"], bits, d)
            reconcile_norms(norms[b, h, s0:s0 + n], ref["norm16"], ref["norm_flags"])
    say(f"append many: {count} tensors equal to single appends; tensor 13 as the oracle's")
