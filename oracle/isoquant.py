"""Plain FP64 reference of the IsoQuant packed-KV path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It is slow on purpose: every step is written the
way the pages state it, vectorised over vectors/tokens with NumPy but with no
blocking, fusion or reordering beyond that.

Conventions (readings of points the pages leave open, each listed in the
design notes of the repository):

* WHT: Sylvester (natural) order, H[i, j] = (-1)^popcount(i & j) / sqrt(d), no
  random sign diagonal.
* SO(4) blocks: 0-based contiguous blocks x[4i : 4i+4]; a block is the
  quaternion w + x i + y j + z k (scalar first) with Hamilton's rule i j = k.
  Stored quaternions are ``quats[h, i, 0, :] = q_L`` and ``quats[h, i, 1, :] =
  q_R`` in (w, x, y, z) order.  Full: v -> q_L v conj(q_R); Fast keeps the left
  isoclinic factor only: v -> q_L v.  The FP32 quaternions given as input are
  re-normalised in FP64 here.
* Planar (the 2-D special case): 0-based contiguous pairs x[2i : 2i+2], each
  read as the complex number x[2i] + x[2i+1] i and multiplied by the unit
  complex number stored at ``params[h, i] = (cos, sin)`` (re-normalised in
  FP64).  In two dimensions the left and right factors commute, so one
  rotation per pair is all there is; the WHT comes first as for SO(4).
* Quantiser: thresholds t_k = (c_k + c_{k+1}) / 2 computed in FP64 from the
  FP32 centroids; code = number of thresholds strictly below the value (a tie
  takes the lower code).  Elements within 1e-6 of a threshold are flagged.
* Norm: s = ||x||_2 in FP64, stored as IEEE fp16 rounded to nearest even.
  A zero vector has s = 0 and rotates the zero vector.
* BitPack_b: bit r of code i is bit (b*i + r) of the row, bytes little-endian
  (LSB-first bitstream), d*b/8 bytes per vector.
* Zero-length attention (kv_len = 0): output 0, lse = -inf, argmax = -1.
* RoPE sub-block split (for MLA-style keys, which the pages name as a
  limitation): a key is (content, positional) with the r positional (RoPE)
  coordinates last.  Only the content part goes through Algorithm 1 (its
  own norm, rotation, codes); the positional part is neither rotated nor
  quantised and is kept in fp16 (round to nearest even).  Scores add the
  positional dot product, unscaled by the content norm; values carry no
  positional part.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "FULL",
    "FAST",
    "PLANAR",
    "BOUNDARY_BAND",
    "lloyd_max_gaussian",
    "codebook",
    "round_significand",
    "thresholds",
    "wht",
    "qmul",
    "qconj",
    "unit_quaternions",
    "so4_forward",
    "so4_inverse",
    "planar_forward",
    "planar_inverse",
    "rotate",
    "rotate_inverse",
    "rotate_scalar",
    "quantize",
    "norm_fp16",
    "pack",
    "unpack",
    "row_bytes",
    "dequantize",
    "dequantize_codes",
    "attend",
    "attend_rotated",
    "attend_dense",
    "quantize_rope",
    "attend_rope",
]

FULL = 0
FAST = 1
PLANAR = 2

# Width of the decision-boundary band: an element whose rotated value lies
# closer than this to a threshold may legitimately take either neighbouring
# code in a different (fp32) evaluation order.
BOUNDARY_BAND = 1e-6


# ---------------------------------------------------------------------------
# Codebook: Lloyd-Max scalar quantiser (RotaryQuant §3.2, Step 3: codebooks
# minimising expected distortion under the post-rotation marginal; the
# marginal taken is N(0, 1/d)).
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    """Standard normal density; 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _mass(a: float, b: float) -> float:
    """P(a < X <= b) for X ~ N(0, 1), evaluated on the side that avoids
    cancellation."""
    if a >= 0.0:
        # upper tail: Q(a) - Q(b), Q(x) = P(X > x)
        qa = 0.5 * math.erfc(a / math.sqrt(2.0))
        qb = 0.0 if math.isinf(b) else 0.5 * math.erfc(b / math.sqrt(2.0))
        return qa - qb
    pb = 1.0 if math.isinf(b) else 0.5 * math.erfc(-b / math.sqrt(2.0))
    pa = 0.0 if math.isinf(a) else 0.5 * math.erfc(-a / math.sqrt(2.0))
    return pb - pa


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 200000) -> np.ndarray:
    """Lloyd iteration for the 2**bits-level minimum-MSE quantiser of N(0, 1).

    Alternates the two optimality conditions: every threshold is the midpoint
    of its two neighbouring centroids, and every centroid is the conditional
    mean of its cell, E[X | t_{k-1} < X <= t_k] = (phi(t_{k-1}) - phi(t_k)) /
    (Phi(t_k) - Phi(t_{k-1})).  Stops when no centroid moves by more than
    ``tol``.  Returns FP64 centroids in ascending order.
    """
    n = 1 << bits
    # start from evenly spaced points over +-2 sigma
    c = np.linspace(-2.0, 2.0, n)
    for _ in range(max_iter):
        t = np.concatenate(([-math.inf], 0.5 * (c[:-1] + c[1:]), [math.inf]))
        new = np.empty(n)
        for k in range(n):
            a, b = t[k], t[k + 1]
            new[k] = (_phi(a) - _phi(b)) / _mass(a, b)
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    return c


def round_significand(x: np.ndarray, digits: int = 11) -> np.ndarray:
    """Round FP64 values to ``digits`` significant bits, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 2.0 ** digits), e - digits)


def codebook(bits: int, head_dim: int) -> np.ndarray:
    """Codebook for coordinates of a rotated unit vector, N(0, 1/d).

    The Gaussian Lloyd-Max centroids scaled by 1/sqrt(d) and held at fp16
    precision: each value rounded (ties to even) to 11 significant bits, so
    that a power-of-two multiple of it is an exact fp16 number.  Returned as
    FP32 (exact); this array is what both the oracle and the device path
    consume.
    """
    return round_significand(lloyd_max_gaussian(bits) / math.sqrt(head_dim)).astype(np.float32)


def thresholds(centroids: np.ndarray) -> np.ndarray:
    """Decision thresholds t_k = (c_k + c_{k+1}) / 2 in FP64 from FP32 c."""
    c = np.asarray(centroids, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


# ---------------------------------------------------------------------------
# Rotation R = R_SO(4) o H_d (RotaryQuant §3.2 eq. (2), Algorithm 1).
# ---------------------------------------------------------------------------

def wht(x: np.ndarray) -> np.ndarray:
    """Normalised Walsh-Hadamard transform along the last axis (FP64).

    Butterfly form: for h = 1, 2, 4, ..., d/2 every pair (i, i+h) with
    (i & h) == 0 becomes (a+b, a-b); the result is scaled by 1/sqrt(d).
    H_d is symmetric and orthogonal, so it is its own inverse.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    assert d >= 1 and (d & (d - 1)) == 0, "WHT length must be a power of two"
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        y = np.stack((a + b, a - b), axis=-2).reshape(lead + (d,))
        h *= 2
    return y / math.sqrt(d)


def qmul(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Hamilton product p q of quaternions stored (w, x, y, z) on the last axis."""
    pw, px, py, pz = (p[..., k] for k in range(4))
    qw, qx, qy, qz = (q[..., k] for k in range(4))
    return np.stack(
        (
            pw * qw - px * qx - py * qy - pz * qz,
            pw * qx + px * qw + py * qz - pz * qy,
            pw * qy - px * qz + py * qw + pz * qx,
            pw * qz + px * qy - py * qx + pz * qw,
        ),
        axis=-1,
    )


def qconj(q: np.ndarray) -> np.ndarray:
    """Quaternion conjugate (w, -x, -y, -z)."""
    q = np.asarray(q, dtype=np.float64)
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def unit_quaternions(quats: np.ndarray) -> np.ndarray:
    """Promote stored quaternions to FP64 and re-normalise each to unit length."""
    q = np.asarray(quats, dtype=np.float64)
    return q / np.linalg.norm(q, axis=-1, keepdims=True)


def so4_forward(y: np.ndarray, quats: np.ndarray, variant: int) -> np.ndarray:
    """Block-diagonal SO(4) rotation of the last axis.

    ``quats`` has shape (d/4, 2, 4) (one head) and broadcasts over leading
    axes of ``y``.  Full: v -> q_L v conj(q_R).  Fast: v -> q_L v.
    """
    q = unit_quaternions(quats)
    d = y.shape[-1]
    v = np.asarray(y, dtype=np.float64).reshape(y.shape[:-1] + (d // 4, 4))
    qL = q[..., 0, :]
    qR = q[..., 1, :]
    out = qmul(qL, v)
    if variant == FULL:
        out = qmul(out, qconj(qR))
    elif variant != FAST:
        raise ValueError("variant must be FULL or FAST")
    return out.reshape(y.shape)


def so4_inverse(w: np.ndarray, quats: np.ndarray, variant: int) -> np.ndarray:
    """Inverse (= transpose) of :func:`so4_forward`.

    Full: w -> conj(q_L) w q_R.  Fast: w -> conj(q_L) w.
    """
    q = unit_quaternions(quats)
    d = w.shape[-1]
    v = np.asarray(w, dtype=np.float64).reshape(w.shape[:-1] + (d // 4, 4))
    qL = q[..., 0, :]
    qR = q[..., 1, :]
    out = qmul(qconj(qL), v)
    if variant == FULL:
        out = qmul(out, qR)
    elif variant != FAST:
        raise ValueError("variant must be FULL or FAST")
    return out.reshape(w.shape)


def _unit_complex(params: np.ndarray) -> np.ndarray:
    """Stored (cos, sin) pairs promoted to FP64 unit complex numbers."""
    p = np.asarray(params, dtype=np.float64)
    z = p[..., 0] + 1j * p[..., 1]
    return z / np.abs(z)


def planar_forward(y: np.ndarray, params: np.ndarray) -> np.ndarray:
    """Block-diagonal SO(2) rotation of the last axis (the 2-D special case
    of the IsoQuant framework, IsoQuant abstract): pair i, read as the
    complex number y[2i] + y[2i+1] i, is multiplied by z_i.

    ``params`` has shape (d/2, 2) (one head) and broadcasts over leading axes.
    """
    z = _unit_complex(params)
    y = np.asarray(y, dtype=np.float64)
    v = y[..., 0::2] + 1j * y[..., 1::2]
    w = z * v
    out = np.empty(y.shape, dtype=np.float64)
    out[..., 0::2] = w.real
    out[..., 1::2] = w.imag
    return out


def planar_inverse(w: np.ndarray, params: np.ndarray) -> np.ndarray:
    """Inverse of :func:`planar_forward`: multiplication by conj(z_i)."""
    z = _unit_complex(params)
    w = np.asarray(w, dtype=np.float64)
    v = w[..., 0::2] + 1j * w[..., 1::2]
    u = np.conj(z) * v
    out = np.empty(w.shape, dtype=np.float64)
    out[..., 0::2] = u.real
    out[..., 1::2] = u.imag
    return out


def rotate(x: np.ndarray, quats: np.ndarray, variant: int) -> np.ndarray:
    """R x = R_blocks(H_d x) (RotaryQuant eq. (2)); the block rotation is
    SO(4) (Full, Fast; ``quats`` (d/4, 2, 4)) or planar (``quats`` holding
    the (d/2, 2) pair rotations)."""
    if variant == PLANAR:
        return planar_forward(wht(x), quats)
    return so4_forward(wht(x), quats, variant)


def rotate_inverse(x: np.ndarray, quats: np.ndarray, variant: int) -> np.ndarray:
    """R^T x = H_d (R_blocks^T x): the same butterfly plus the block transpose
    (RotaryQuant §3.4)."""
    if variant == PLANAR:
        return wht(planar_inverse(x, quats))
    return wht(so4_inverse(x, quats, variant))


def rotate_scalar(x, quats, variant):
    """Scalar, operation-counting evaluation of R x for one vector.

    Counts one operation per addition/subtraction in the WHT butterflies, the
    1/sqrt(d) scalings separately, and one per real multiplication in the
    quaternion products of the SO(4) stage (in the 2x2 rotations, Planar).  Returns (Rx as FP64 array,
    counts dict).  Used to pin the per-vector cost figures the pages print.
    """
    counts = {"wht_addsub": 0, "wht_scale_mul": 0, "so4_mul": 0, "so4_addsub": 0}
    y = [float(v) for v in x]
    d = len(y)
    h = 1
    while h < d:
        for i in range(d):
            if (i & h) == 0:
                a, b = y[i], y[i + h]
                y[i] = a + b
                y[i + h] = a - b
                counts["wht_addsub"] += 2
        h *= 2
    inv = 1.0 / math.sqrt(d)
    for i in range(d):
        y[i] *= inv
        counts["wht_scale_mul"] += 1

    def hamilton(p, q):
        # 16 real products, 12 additions/subtractions
        products = [[p[a] * q[b] for b in range(4)] for a in range(4)]
        counts["so4_mul"] += 16
        counts["so4_addsub"] += 12
        w = products[0][0] - products[1][1] - products[2][2] - products[3][3]
        i = products[0][1] + products[1][0] + products[2][3] - products[3][2]
        j = products[0][2] - products[1][3] + products[2][0] + products[3][1]
        k = products[0][3] + products[1][2] - products[2][1] + products[3][0]
        return [w, i, j, k]

    if variant == PLANAR:
        z = _unit_complex(quats)
        out = []
        for i in range(d // 2):
            a, b = float(z[i].real), float(z[i].imag)
            x0, x1 = y[2 * i], y[2 * i + 1]
            out.extend([a * x0 - b * x1, b * x0 + a * x1])
            counts["so4_mul"] += 4
            counts["so4_addsub"] += 2
        return np.array(out), counts

    q = unit_quaternions(quats)
    out = []
    for blk in range(d // 4):
        v = y[4 * blk: 4 * blk + 4]
        qL = [float(t) for t in q[blk, 0]]
        qR = [float(t) for t in q[blk, 1]]
        r = hamilton(qL, v)
        if variant == FULL:
            r = hamilton(r, [qR[0], -qR[1], -qR[2], -qR[3]])
        out.extend(r)
    return np.array(out), counts


# ---------------------------------------------------------------------------
# Algorithm 1: normalise -> rotate -> Lloyd-Max -> BitPack.
# ---------------------------------------------------------------------------

def norm_fp16(s: np.ndarray):
    """fp16 (round-to-nearest-even) of the FP64 norm, plus a flag marking norms
    within 1e-6 (relative) of an fp16 rounding midpoint, where a different
    (fp32) evaluation order may legitimately round the other way."""
    s = np.asarray(s, dtype=np.float64)
    s16 = s.astype(np.float16)
    with np.errstate(over="ignore"):
        up = np.nextafter(s16, np.float16(np.inf)).astype(np.float64)
        dn = np.nextafter(s16, np.float16(-np.inf)).astype(np.float64)
    base = s16.astype(np.float64)
    mid_up = 0.5 * (base + up)
    mid_dn = 0.5 * (base + dn)
    near = np.minimum(np.abs(s - mid_up), np.abs(s - mid_dn)) < 1e-6 * np.maximum(s, 1e-300)
    return s16.view(np.uint16), near


def quantize(x, quats, centroids, variant):
    """Algorithm 1 (RotaryQuant §3.2) on vectors along the last axis.

    ``x``: (..., d) fp16/fp32/FP64 input, promoted exactly to FP64.
    ``quats``: the block-rotation parameters of the head these vectors
    belong to: (d/4, 2, 4) quaternion pairs (Full, Fast) or (d/2, 2) pair
    rotations (Planar).
    ``centroids``: FP32 codebook (2**b values, ascending).

    Returns a dict with ``codes`` (int64, (..., d)), ``norm16`` (uint16 fp16
    bit patterns), ``s`` (FP64 norms), ``rotated`` (FP64 R x / s),
    ``flags`` (elements within the boundary band) and ``norm_flags``.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(s > 0.0, s, 1.0)
    xhat = np.where((s > 0.0)[..., None], x / safe[..., None], 0.0)
    xt = rotate(xhat, quats, variant)
    t = thresholds(centroids)
    codes = np.zeros(xt.shape, dtype=np.int64)
    for tk in t:
        codes += (xt > tk).astype(np.int64)
    margin = np.min(np.abs(xt[..., None] - t), axis=-1)
    norm16, norm_flags = norm_fp16(s)
    return {
        "codes": codes,
        "norm16": norm16,
        "s": s,
        "rotated": xt,
        "flags": margin < BOUNDARY_BAND,
        "norm_flags": norm_flags,
    }


def row_bytes(head_dim: int, bits: int) -> int:
    """Packed row size d*b/8 (48 bytes at d=128, b=3: RotaryQuant §3.2 Step 4)."""
    return head_dim * bits // 8


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """BitPack_b: LSB-first bitstream, d*b/8 bytes per vector (uint8)."""
    codes = np.asarray(codes, dtype=np.int64)
    d = codes.shape[-1]
    assert (d * bits) % 8 == 0
    planes = (codes[..., :, None] >> np.arange(bits)) & 1          # (..., d, b)
    stream = planes.reshape(codes.shape[:-1] + (d * bits,)).astype(np.uint8)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(rows: np.ndarray, bits: int, head_dim: int) -> np.ndarray:
    """Inverse of :func:`pack`."""
    rows = np.asarray(rows, dtype=np.uint8)
    stream = np.unpackbits(rows, axis=-1, bitorder="little")[..., : head_dim * bits]
    planes = stream.reshape(rows.shape[:-1] + (head_dim, bits)).astype(np.int64)
    return np.sum(planes << np.arange(bits), axis=-1)


def dequantize_codes(codes, norm16, quats, centroids, variant):
    """x' = fp16(s) * R^T c[codes] for codes already unpacked."""
    c = np.asarray(centroids, dtype=np.float64)
    s = np.asarray(norm16, dtype=np.uint16).view(np.float16).astype(np.float64)
    y = rotate_inverse(c[np.asarray(codes)], quats, variant)
    return y * s[..., None]


def dequantize(rows, norm16, quats, centroids, bits, variant, head_dim):
    """Stage-1 return path: unpack -> centroid -> SO(4)^T -> WHT -> x fp16(s)."""
    return dequantize_codes(unpack(rows, bits, head_dim), norm16, quats, centroids, variant)


# ---------------------------------------------------------------------------
# Decode attention.  The reconstruct-then-compute form (RotaryQuant §1,
# Figure 1 top) is the definition; the rotated-space form is Appendix A.
# ---------------------------------------------------------------------------

def _softmax_stats(scores: np.ndarray):
    """alpha, lse and first argmax of one row of FP64 scores."""
    m = np.max(scores)
    e = np.exp(scores - m)
    den = np.sum(e)
    return e / den, m + math.log(den), int(np.argmax(scores))


def attend(q, k_rows, k_norm16, v_rows, v_norm16, quats, centroids, bits, variant,
           softmax_scale, kv_len=None):
    """Dequantize-then-attend for one sequence (FP64).

    ``q``: (Hq, d).  ``k_rows``/``v_rows``: (H_kv, T, d*b/8) uint8.
    ``k_norm16``/``v_norm16``: (H_kv, T) uint16 fp16 bits.
    ``quats``: (H_kv, d/4, 2, 4).  Query head h reads KV head h // (Hq/H_kv).
    Attends over rows [0, kv_len).

    Returns (out (Hq, d), lse (Hq,) natural-log units, argmax (Hq,) int64).
    """
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_rows.shape[0]
    group = hq // hkv
    T = k_rows.shape[1] if kv_len is None else int(kv_len)
    out = np.zeros((hq, d))
    lse = np.full(hq, -np.inf)
    arg = np.full(hq, -1, dtype=np.int64)
    if T == 0:
        return out, lse, arg
    for g in range(hkv):
        kp = dequantize(k_rows[g, :T], k_norm16[g, :T], quats[g], centroids, bits, variant, d)
        vp = dequantize(v_rows[g, :T], v_norm16[g, :T], quats[g], centroids, bits, variant, d)
        for h in range(g * group, (g + 1) * group):
            # row-wise sums: identical rows give bit-identical scores (ties)
            scores = softmax_scale * np.sum(kp * q[h], axis=-1)
            alpha, lse[h], arg[h] = _softmax_stats(scores)
            out[h] = alpha @ vp
    return out, lse, arg


def attend_rotated(q, k_rows, k_norm16, v_rows, v_norm16, quats, centroids, bits,
                   variant, softmax_scale, kv_len=None):
    """Compressed-space evaluation (RotaryQuant Appendix A): q~ = R q, scores
    s_j * (q~ . c[codes_j]), aggregate in rotated space, one R^T at the end.
    Must equal :func:`attend` up to FP64 rounding."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_rows.shape[0]
    group = hq // hkv
    T = k_rows.shape[1] if kv_len is None else int(kv_len)
    c = np.asarray(centroids, dtype=np.float64)
    out = np.zeros((hq, d))
    lse = np.full(hq, -np.inf)
    arg = np.full(hq, -1, dtype=np.int64)
    if T == 0:
        return out, lse, arg
    for g in range(hkv):
        ck = c[unpack(k_rows[g, :T], bits, d)]
        cv = c[unpack(v_rows[g, :T], bits, d)]
        sk = np.asarray(k_norm16[g, :T], dtype=np.uint16).view(np.float16).astype(np.float64)
        sv = np.asarray(v_norm16[g, :T], dtype=np.uint16).view(np.float16).astype(np.float64)
        for h in range(g * group, (g + 1) * group):
            qt = rotate(q[h], quats[g], variant)
            scores = softmax_scale * sk * np.sum(ck * qt, axis=-1)
            alpha, lse[h], arg[h] = _softmax_stats(scores)
            ot = (alpha * sv) @ cv
            out[h] = rotate_inverse(ot, quats[g], variant)
    return out, lse, arg


def attend_dense(q, k, v, softmax_scale):
    """Plain FP64 attention over unquantised K/V (T, d) for one head; used
    only for fidelity reports (cosine similarity), never for parity."""
    q = np.asarray(q, dtype=np.float64)
    scores = softmax_scale * np.sum(np.asarray(k, dtype=np.float64) * q, axis=-1)
    alpha, _, _ = _softmax_stats(scores)
    return alpha @ np.asarray(v, dtype=np.float64)


# ---------------------------------------------------------------------------
# RoPE sub-block split (RotaryQuant §5, the MLA/RoPE limitation: positional
# coordinates must be neither rotated nor quantised).
# ---------------------------------------------------------------------------

def quantize_rope(x, quats, centroids, variant, rope_dim):
    """Keys (..., d + r) with the r RoPE coordinates last: the content part
    (..., d) is quantised as in :func:`quantize`; the RoPE part is returned
    as fp16 bits (round to nearest even), untouched otherwise
    (``rope16``, uint16 (..., r))."""
    x = np.asarray(x)
    r = quantize(x[..., :-rope_dim], quats, centroids, variant)
    r["rope16"] = np.asarray(x[..., -rope_dim:], dtype=np.float64).astype(np.float16).view(np.uint16)
    return r


def attend_rope(q, k_rows, k_norm16, k_rope16, v_rows, v_norm16, quats, centroids, bits, variant,
                softmax_scale, kv_len=None):
    """Dequantize-then-attend with a RoPE sub-block (FP64), one sequence.

    ``q``: (Hq, d + r), RoPE coordinates last.  ``k_rope16``: (H_kv, T, r)
    fp16 bits of the keys' RoPE coordinates.  Score of token j for head h:
    softmax_scale * (q_content . k'_j + q_rope . k_rope_j), with k'_j the
    dequantised content key; the output is the weighted sum of the
    dequantised values (d coordinates).  Other arguments as :func:`attend`.
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    rope_dim = k_rope16.shape[-1]
    d = q.shape[1] - rope_dim
    hkv = k_rows.shape[0]
    group = hq // hkv
    T = k_rows.shape[1] if kv_len is None else int(kv_len)
    out = np.zeros((hq, d))
    lse = np.full(hq, -np.inf)
    arg = np.full(hq, -1, dtype=np.int64)
    if T == 0:
        return out, lse, arg
    for g in range(hkv):
        kp = dequantize(k_rows[g, :T], k_norm16[g, :T], quats[g], centroids, bits, variant, d)
        kr = np.asarray(k_rope16[g, :T], dtype=np.uint16).view(np.float16).astype(np.float64)
        vp = dequantize(v_rows[g, :T], v_norm16[g, :T], quats[g], centroids, bits, variant, d)
        for h in range(g * group, (g + 1) * group):
            scores = softmax_scale * (np.sum(kp * q[h, :d], axis=-1) + np.sum(kr * q[h, d:], axis=-1))
            alpha, lse[h], arg[h] = _softmax_stats(scores)
            out[h] = alpha @ vp
    return out, lse, arg
