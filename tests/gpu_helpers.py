"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and bring its results back to the host for comparison with the oracle."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O
from compressed_space_attention_isoquant_amd import binding as B
from compressed_space_attention_isoquant_amd import inputs

DEV = "cuda:0"


def torch():
    import torch as _t

    return _t


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_config(d, bits, variant, hkv, quat_seed=inputs.QUATERNION_SEED):
    t = torch()
    quats = inputs.rotation_params(hkv, d, variant, seed=quat_seed)
    qdev = t.from_numpy(quats).to(DEV)
    cfg = B.Config(d, bits, variant, hkv, qdev, B.iq_codebook(bits, d))
    return cfg, quats


def quantize_rows(cfg, x_host, capacity=None, start=0):
    """x_host (B, n, H_kv, d) numpy fp32/fp16 -> PackedCache on the GPU."""
    t = torch()
    batch, n, hkv, d = x_host.shape
    cap = n + start if capacity is None else capacity
    cache = B.new_cache(batch, hkv, cap, d, cfg.bits, DEV)
    x = t.from_numpy(np.ascontiguousarray(x_host)).to(DEV)
    sp = t.full((batch,), start, dtype=t.int32, device=DEV)
    B.iq_quantize_append(cfg, x, sp, cache)
    return cache


def host_cache(cache):
    """(codes uint8 (B,H,cap,row), norms uint16 (B,H,cap)) on the host."""
    torch().cuda.synchronize()
    codes = cache.codes.cpu().numpy()
    norms = cache.norms.cpu().numpy().view(np.uint16)
    return codes, norms


def reconcile_codes(gpu_rows, ref_codes, ref_flags, bits, d):
    """Validate GPU rows against the oracle's codes and return the codes the
    oracle uses next: its own, except inside the boundary band where both
    neighbouring codes are correct and the GPU's choice is kept after checking
    it is one of them.  Raises on any unflagged mismatch.
    Returns (codes, n_flagged, n_flagged_mismatched)."""
    got = O.unpack(gpu_rows, bits, d)
    mism = got != ref_codes
    bad = mism & ~ref_flags
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} unflagged code mismatches, first at {idx.tolist()}")
    far = mism & (np.abs(got - ref_codes) != 1)
    if far.any():
        raise AssertionError(f"{int(far.sum())} flagged codes are not a neighbouring level")
    return np.where(ref_flags, got, ref_codes), int(ref_flags.sum()), int(mism.sum())


def reconcile_norms(gpu_norms, ref_norm16, ref_flags):
    """fp16 norms: bit-exact outside the rounding-midpoint band, one fp16 step
    apart inside it.  Returns (norms, n_flagged, n_mismatched)."""
    gpu_norms = np.asarray(gpu_norms, np.uint16)
    ref_norm16 = np.asarray(ref_norm16, np.uint16)
    mism = gpu_norms != ref_norm16
    bad = mism & ~ref_flags
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} unflagged norm mismatches, first at {idx.tolist()}")
    step = np.abs(gpu_norms.astype(np.int64) - ref_norm16.astype(np.int64))
    if (mism & (step != 1)).any():
        raise AssertionError("flagged norms more than one fp16 step apart")
    return np.where(ref_flags, gpu_norms, ref_norm16), int(ref_flags.sum()), int(mism.sum())


def compare_codes(gpu_rows, ref_codes, ref_flags, bits, d):
    _, nf, nm = reconcile_codes(gpu_rows, ref_codes, ref_flags, bits, d)
    return nf, nm


def compare_norms(gpu_norms, ref_norm16, ref_flags):
    _, nf, nm = reconcile_norms(gpu_norms, ref_norm16, ref_flags)
    return nf, nm


def oracle_cache(x_tokens, quats, cb, variant, bits, gpu_rows, gpu_norms):
    """The oracle's own packed cache for inputs x_tokens (T, H_kv, d): its
    quantization of every head, with boundary-band ties resolved to the GPU's
    validated choice.  gpu_rows (H_kv, T, row), gpu_norms (H_kv, T).
    Returns (rows (H_kv, T, row) uint8, norms (H_kv, T) uint16, stats)."""
    T, hkv, d = x_tokens.shape
    rows = np.empty((hkv, T, d * bits // 8), np.uint8)
    norms = np.empty((hkv, T), np.uint16)
    stats = [0, 0, 0]
    for g in range(hkv):
        ref = O.quantize(x_tokens[:, g], quats[g], cb, variant)
        codes, nf, nm = reconcile_codes(gpu_rows[g], ref["codes"], ref["flags"], bits, d)
        nrm, _, nn = reconcile_norms(gpu_norms[g], ref["norm16"], ref["norm_flags"])
        rows[g] = O.pack(codes, bits)
        norms[g] = nrm
        stats[0] += nf
        stats[1] += nm
        stats[2] += nn
    return rows, norms, stats


def scale_for(d):
    return 1.0 / math.sqrt(d)
