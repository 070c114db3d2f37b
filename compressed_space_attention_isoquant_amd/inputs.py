"""Seeded synthetic inputs for the IsoQuant packed-KV path.

This module is the one piece shared by the oracle side (tests) and the device
side (tests, bench): it produces *inputs only* and holds none of the method's
arithmetic (no rotation, quantiser, codebook, packing or attention).

Recipes (host generators use ``numpy.random.default_rng(seed)`` (PCG64) in
FP64 and cast with round-to-nearest-even):

* quaternions: seed 0 for every workload; q = g / ||g|| with g ~ N(0, I_4)
  drawn as an array of shape (H_kv, d/4, 2, 4), cast to fp32 (uniform on S^3).
* planar pair rotations: seed 0; z = g / |g| with g ~ N(0, I_2) drawn as an
  array of shape (H_kv, d/2, 2), cast to fp32 (uniform angle).
* stage-1 vectors: entries N(0, 1), each vector L2-normalised in FP64, cast
  to the I/O dtype.
* decode K/V: entries N(0, 1) with, per KV head, 4 channels drawn without
  replacement (independently for K and V) scaled by 10 before the fp16 cast;
  the same channels for every token.  Queries N(0, 1) fp16.
* needles: 16 needles in one context, needle n in KV head g = n mod 4, aligned
  to query head 8 g + n // 4, at distinct seeded positions; its key is
  m_g (0.9 q^ + sqrt(0.19) u^) where m_g is the median key norm of that head,
  q^ the unit query direction and u^ a seeded unit vector orthogonal to q^.
* large batched workloads are drawn on the device with ``torch.Generator``
  seeded per sequence (same distributions; values differ from NumPy's).
"""

from __future__ import annotations

import numpy as np

OUTLIER_CHANNELS = 4
OUTLIER_SCALE = 10.0
QUATERNION_SEED = 0


def quaternions(num_kv_heads: int, head_dim: int, seed: int = QUATERNION_SEED) -> np.ndarray:
    """(H_kv, d/4, 2, 4) fp32 unit quaternions (q_L, q_R) per block, (w,x,y,z)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((num_kv_heads, head_dim // 4, 2, 4))
    q = g / np.linalg.norm(g, axis=-1, keepdims=True)
    return q.astype(np.float32)


def planar_rotations(num_kv_heads: int, head_dim: int, seed: int = QUATERNION_SEED) -> np.ndarray:
    """(H_kv, d/2, 2) fp32 unit complex numbers (cos, sin), one per pair of
    coordinates: z = g / |g| with g ~ N(0, I_2), i.e. a uniform angle."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((num_kv_heads, head_dim // 2, 2))
    z = g / np.linalg.norm(g, axis=-1, keepdims=True)
    return z.astype(np.float32)


PLANAR = 2


def rotation_params(num_kv_heads: int, head_dim: int, variant: int, seed: int = QUATERNION_SEED) -> np.ndarray:
    """The block-rotation parameters a variant reads: quaternion pairs for
    Full (0) and Fast (1), pair rotations for Planar (2)."""
    if variant == PLANAR:
        return planar_rotations(num_kv_heads, head_dim, seed)
    return quaternions(num_kv_heads, head_dim, seed)


def unit_vectors(n: int, head_dim: int, dtype, seed: int) -> np.ndarray:
    """(n, d) vectors with i.i.d. N(0,1) entries, L2-normalised, cast to dtype."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, head_dim))
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(dtype)


def outlier_channels(rng: np.random.Generator, num_kv_heads: int, head_dim: int) -> np.ndarray:
    """(H_kv, 4) channel indices per KV head, drawn without replacement."""
    return np.stack([rng.choice(head_dim, OUTLIER_CHANNELS, replace=False)
                     for _ in range(num_kv_heads)])


def kv_tokens(rng: np.random.Generator, n_tokens: int, channels: np.ndarray, head_dim: int) -> np.ndarray:
    """(n_tokens, H_kv, d) fp16 K or V rows with channel-wise outliers."""
    hkv = channels.shape[0]
    x = rng.standard_normal((n_tokens, hkv, head_dim))
    for h in range(hkv):
        x[:, h, channels[h]] *= OUTLIER_SCALE
    return x.astype(np.float16)


def decode_case(seed: int, kv_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                needles: int = 0) -> dict:
    """One sequence for decode attention: q (Hq, d), k/v (T, H_kv, d), fp16.

    With ``needles`` > 0, plants that many needles as described in the module
    docstring and returns their (query head, kv head, position) triples.
    """
    rng = np.random.default_rng(seed)
    ch_k = outlier_channels(rng, num_kv_heads, head_dim)
    ch_v = outlier_channels(rng, num_kv_heads, head_dim)
    k = kv_tokens(rng, kv_len, ch_k, head_dim)
    v = kv_tokens(rng, kv_len, ch_v, head_dim)
    q = rng.standard_normal((num_q_heads, head_dim)).astype(np.float16)
    planted = []
    if needles:
        group = num_q_heads // num_kv_heads
        pos = rng.choice(kv_len, needles, replace=False)
        med = np.median(np.linalg.norm(k.astype(np.float64), axis=-1), axis=0)   # (H_kv,)
        for n in range(needles):
            g = n % num_kv_heads
            h = group * g + n // num_kv_heads
            qh = q[h].astype(np.float64)
            qhat = qh / np.linalg.norm(qh)
            u = rng.standard_normal(head_dim)
            u -= (u @ qhat) * qhat
            u /= np.linalg.norm(u)
            key = med[g] * (0.9 * qhat + np.sqrt(0.19) * u)
            k[pos[n], g] = key.astype(np.float16)
            planted.append((int(h), int(g), int(pos[n])))
    return {"q": q, "k": k, "v": v, "channels_k": ch_k, "channels_v": ch_v,
            "needles": planted}


def batch_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int64)


# ---------------------------------------------------------------------------
# Device-side draws for workloads too large to build on the host.
# ---------------------------------------------------------------------------

def device_kv(seed: int, index: int, n_tokens: int, channels: np.ndarray, head_dim: int, device):
    """(n_tokens, H_kv, d) fp16 torch tensor on ``device`` with channel-wise
    outliers; stream ``(seed, index)`` selects an independent draw."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + int(index))
    hkv = channels.shape[0]
    x = torch.randn((n_tokens, hkv, head_dim), generator=gen, device=device, dtype=torch.float32)
    scale = torch.ones((hkv, head_dim), device=device, dtype=torch.float32)
    for h in range(hkv):
        scale[h, torch.as_tensor(channels[h], device=device)] = OUTLIER_SCALE
    return (x * scale).to(torch.float16)


def device_normal(seed: int, index: int, shape, device, dtype):
    """N(0,1) torch tensor of ``shape`` cast to ``dtype`` on ``device``."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + int(index))
    return torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32).to(dtype)


def device_unit_vectors(seed: int, n: int, head_dim: int, device, dtype):
    """(n, d) unit vectors drawn on ``device`` (N(0,1) entries, L2-normalised
    in fp32, cast to dtype)."""
    import torch

    x = device_normal(seed, 0, (n, head_dim), device, torch.float32)
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(dtype)
