"""Pins for the oracle's decode attention (CPU only).

* brute force on tiny inputs: dense rotation matrix built from the explicit
  Hadamard and quaternion multiplication matrices, scalar softmax loops;
* special cases: one token, identical keys, one dominant key, empty context;
* RotaryQuant Appendix A on real data: the rotated-space evaluation equals the
  dequantize-then-attend evaluation;
* skipping the final inverse rotation breaks the output (RotaryQuant §5,
  "Inverse rotation is mandatory");
* the inverse rotation's share of decode work (RotaryQuant §3.3, eq. 5);
* planted needles are the argmax (synthetic stand-in for the NIAH check of
  RotaryQuant Appendix F).
"""

import math

import numpy as np
import pytest

import oracle as O
from compressed_space_attention_isoquant_amd import inputs


def dense_rotation(quats_head, variant):
    if variant == O.PLANAR:
        d = quats_head.shape[0] * 2
        H = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)]) / math.sqrt(d)
        z = quats_head.astype(np.float64)
        z = z / np.linalg.norm(z, axis=-1, keepdims=True)
        B = np.zeros((d, d))
        for i in range(d // 2):
            B[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[z[i, 0], -z[i, 1]], [z[i, 1], z[i, 0]]]
        return B @ H
    d = quats_head.shape[0] * 4
    H = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)]) / math.sqrt(d)
    q = quats_head.astype(np.float64)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    B = np.zeros((d, d))
    for i in range(d // 4):
        a, b, c, e = q[i, 0]
        L = np.array([[a, -b, -c, -e], [b, a, -e, c], [c, e, a, -b], [e, -c, b, a]])
        if variant == O.FULL:
            a, b, c, e = q[i, 1] * np.array([1, -1, -1, -1])
            Rm = np.array([[a, -b, -c, -e], [b, a, e, -c], [c, -e, a, b], [e, c, -b, a]])
            L = L @ Rm
        B[4 * i:4 * i + 4, 4 * i:4 * i + 4] = L
    return B @ H


def make_case(seed, T, hq, hkv, d, bits, variant, scale_kv=1.0):
    rng = np.random.default_rng(seed)
    quats = inputs.rotation_params(hkv, d, variant, seed=seed)
    cb = O.codebook(bits, d)
    k = (rng.standard_normal((hkv, T, d)) * scale_kv).astype(np.float16)
    v = (rng.standard_normal((hkv, T, d)) * scale_kv).astype(np.float16)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    kr = np.empty((hkv, T, d * bits // 8), np.uint8)
    vr = np.empty_like(kr)
    kn = np.empty((hkv, T), np.uint16)
    vn = np.empty_like(kn)
    for g in range(hkv):
        rk = O.quantize(k[g], quats[g], cb, variant)
        rv = O.quantize(v[g], quats[g], cb, variant)
        kr[g], kn[g] = O.pack(rk["codes"], bits), rk["norm16"]
        vr[g], vn[g] = O.pack(rv["codes"], bits), rv["norm16"]
    return dict(q=q, kr=kr, kn=kn, vr=vr, vn=vn, quats=quats, cb=cb, bits=bits,
                variant=variant, d=d, k=k, v=v)


def run(case, fn=O.attend, kv_len=None, scale=None):
    d = case["d"]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return fn(case["q"], case["kr"], case["kn"], case["vr"], case["vn"], case["quats"],
              case["cb"], case["bits"], case["variant"], scale, kv_len)


@pytest.mark.parametrize("variant", [O.FULL, O.FAST, O.PLANAR])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_tiny(variant, T):
    d, hq, hkv, bits = 32, 4, 2, 3
    c = make_case(T, T, hq, hkv, d, bits, variant)
    out, lse, arg = run(c)
    scale = 1.0 / math.sqrt(d)
    cb = c["cb"].astype(np.float64)
    for h in range(hq):
        g = h // (hq // hkv)
        R = dense_rotation(c["quats"][g], variant)
        keys, vals = [], []
        for j in range(T):
            codes_k = O.unpack(c["kr"][g, j], bits, d)
            codes_v = O.unpack(c["vr"][g, j], bits, d)
            sk = float(np.array([c["kn"][g, j]], np.uint16).view(np.float16)[0])
            sv = float(np.array([c["vn"][g, j]], np.uint16).view(np.float16)[0])
            keys.append(sk * (R.T @ cb[codes_k]))
            vals.append(sv * (R.T @ cb[codes_v]))
        qh = c["q"][h].astype(np.float64)
        scores = [scale * sum(qh[i] * keys[j][i] for i in range(d)) for j in range(T)]
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        den = sum(w)
        ref = sum((w[j] / den) * vals[j] for j in range(T))
        assert np.max(np.abs(out[h] - ref)) < 1e-12
        assert abs(lse[h] - (m + math.log(den))) < 1e-12
        assert arg[h] == scores.index(m)


@pytest.mark.parametrize("T", [1, 2, 5])
def test_attend_dense_brute_force(T):
    """The fidelity reference (unquantised attention) against scalar loops:
    softmax of scale * q.k over the tokens, written out term by term, then
    the weighted sum of the values; plus its closed cases (one token gives its
    value, equal keys give the mean of the values)."""
    rng = np.random.default_rng(90 + T)
    d = 4
    q = rng.standard_normal(d)
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    scale = 0.7
    s = [scale * sum(q[i] * k[t][i] for i in range(d)) for t in range(T)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = sum(w)
    want = [sum(w[t] * v[t][i] for t in range(T)) / z for i in range(d)]
    np.testing.assert_allclose(O.attend_dense(q, k, v, scale), want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.attend_dense(q, k[:1], v[:1], scale), v[0], rtol=0, atol=1e-15)
    same = np.repeat(k[:1], T, axis=0)
    np.testing.assert_allclose(O.attend_dense(q, same, v, scale), v.mean(axis=0), rtol=0, atol=1e-13)


def test_single_token_returns_its_value():
    c = make_case(1, 1, 8, 2, 128, 3, O.FULL)
    out, lse, arg = run(c)
    for h in range(8):
        g = h // 4
        vp = O.dequantize(c["vr"][g], c["vn"][g], c["quats"][g], c["cb"], 3, O.FULL, 128)[0]
        assert np.max(np.abs(out[h] - vp)) < 1e-12
        assert arg[h] == 0


def test_identical_keys_average_values():
    c = make_case(2, 6, 4, 1, 128, 3, O.FAST)
    c["kr"][:] = c["kr"][:, :1]
    c["kn"][:] = c["kn"][:, :1]
    out, lse, arg = run(c)
    vp = O.dequantize(c["vr"][0], c["vn"][0], c["quats"][0], c["cb"], 3, O.FAST, 128)
    for h in range(4):
        assert np.max(np.abs(out[h] - vp.mean(axis=0))) < 1e-12
        assert arg[h] == 0                      # ties resolve to the lowest position
        kp = O.dequantize(c["kr"][0, :1], c["kn"][0, :1], c["quats"][0], c["cb"], 3, O.FAST, 128)[0]
        score = (1 / math.sqrt(128)) * float(kp @ c["q"][h].astype(np.float64))
        assert abs(lse[h] - (score + math.log(6))) < 1e-12


def test_dominant_key_selects_its_value():
    c = make_case(3, 16, 2, 1, 128, 3, O.FULL)
    out, lse, arg = run(c, scale=1e4)         # sharpen: softmax -> one-hot
    kp = O.dequantize(c["kr"][0], c["kn"][0], c["quats"][0], c["cb"], 3, O.FULL, 128)
    vp = O.dequantize(c["vr"][0], c["vn"][0], c["quats"][0], c["cb"], 3, O.FULL, 128)
    for h in range(2):
        j = int(np.argmax(kp @ c["q"][h].astype(np.float64)))
        assert arg[h] == j
        assert np.max(np.abs(out[h] - vp[j])) < 1e-6


def test_empty_context_and_prefix_length():
    c = make_case(4, 12, 4, 2, 128, 3, O.FULL)
    out, lse, arg = run(c, kv_len=0)
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(arg == -1)
    full = run(c, kv_len=7)
    trimmed = dict(c)
    for key in ("kr", "kn", "vr", "vn"):
        trimmed[key] = c[key][:, :7]
    ref = run(trimmed)
    for a, b in zip(full, ref):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("variant", [O.FULL, O.FAST, O.PLANAR])
@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 4), (256, 16, 8)])
def test_rotated_space_equals_reconstruct_then_compute(variant, d, hq, hkv):
    c = make_case(5 + d, 300, hq, hkv, d, 3, variant, scale_kv=4.0)
    out, lse, arg = run(c)
    out2, lse2, arg2 = run(c, fn=O.attend_rotated)
    assert np.max(np.abs(out - out2)) <= 1e-12 * max(1.0, np.max(np.abs(out)))
    assert np.max(np.abs(lse - lse2)) < 1e-11
    assert np.array_equal(arg, arg2)


def test_skipping_inverse_rotation_breaks_output():
    c = make_case(6, 200, 8, 2, 128, 3, O.FULL, scale_kv=3.0)
    out, _, _ = run(c)
    bad = np.empty_like(out)
    for h in range(8):
        g = h // 4
        bad[h] = O.rotate(out[h], c["quats"][g], O.FULL)     # = the rotated-space aggregate
    rel = np.linalg.norm(bad - out) / np.linalg.norm(out)
    assert rel > 0.5


def test_inverse_rotation_share(golden):
    g = golden("pages_closed_forms.json")["inverse_share_bound"]
    T, d = g["T"], g["d"]
    x = np.random.default_rng(0).standard_normal(d)
    _, counts = O.rotate_scalar(x, inputs.quaternions(1, d)[0], O.FAST)
    inverse_ops = counts["wht_addsub"] + 16 * (d // 4)       # 1,408 at d = 128
    decode_fmas = 2 * T * d                                  # QK and PV per query head
    share = inverse_ops / decode_fmas
    assert share < g["value"]
    assert abs(share - 0.0027) < 1e-4


def test_needles_are_argmax_and_cosine_report():
    d, hq, hkv, T = 128, 32, 4, 4096
    case = inputs.decode_case(seed=4, kv_len=T, num_q_heads=hq, num_kv_heads=hkv,
                              head_dim=d, needles=16)
    quats = inputs.quaternions(hkv, d)
    cb = O.codebook(3, d)
    kr = np.empty((hkv, T, 48), np.uint8)
    vr = np.empty_like(kr)
    kn = np.empty((hkv, T), np.uint16)
    vn = np.empty_like(kn)
    for g in range(hkv):
        rk = O.quantize(case["k"][:, g], quats[g], cb, O.FULL)
        rv = O.quantize(case["v"][:, g], quats[g], cb, O.FULL)
        kr[g], kn[g], vr[g], vn[g] = O.pack(rk["codes"], 3), rk["norm16"], O.pack(rv["codes"], 3), rv["norm16"]
    out, lse, arg = O.attend(case["q"], kr, kn, vr, vn, quats, cb, 3, O.FULL, 1 / math.sqrt(d))
    assert len(case["needles"]) == 16
    for h, g, p in case["needles"]:
        assert arg[h] == p
        ref = O.attend_dense(case["q"][h], case["k"][:, g], case["v"][:, g], 1 / math.sqrt(d))
        cos = out[h] @ ref / (np.linalg.norm(out[h]) * np.linalg.norm(ref))
        assert cos > 0.95


# ---- RoPE sub-block split -------------------------------------------------

def make_rope_case(seed, T, hq, hkv, d, r, bits, variant):
    rng = np.random.default_rng(seed)
    quats = inputs.rotation_params(hkv, d, variant, seed=seed)
    cb = O.codebook(bits, d)
    k = (rng.standard_normal((hkv, T, d + r)) * 2).astype(np.float16)
    v = (rng.standard_normal((hkv, T, d)) * 2).astype(np.float16)
    q = rng.standard_normal((hq, d + r)).astype(np.float16)
    kr = np.empty((hkv, T, d * bits // 8), np.uint8)
    vr = np.empty_like(kr)
    kn = np.empty((hkv, T), np.uint16)
    vn = np.empty_like(kn)
    kp = np.empty((hkv, T, r), np.uint16)
    for g in range(hkv):
        rk = O.quantize_rope(k[g], quats[g], cb, variant, r)
        rv = O.quantize(v[g], quats[g], cb, variant)
        kr[g], kn[g], kp[g] = O.pack(rk["codes"], bits), rk["norm16"], rk["rope16"]
        vr[g], vn[g] = O.pack(rv["codes"], bits), rv["norm16"]
    return dict(q=q, kr=kr, kn=kn, kp=kp, vr=vr, vn=vn, quats=quats, cb=cb, bits=bits, variant=variant,
                d=d, r=r, k=k, v=v)


def run_rope(c, q=None, kp=None, scale=0.125):
    return O.attend_rope(c["q"] if q is None else q, c["kr"], c["kn"], c["kp"] if kp is None else kp, c["vr"],
                         c["vn"], c["quats"], c["cb"], c["bits"], c["variant"], scale)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_rope_brute_force_tiny(T):
    """Scores written out term by term: content keys through the dense
    rotation matrix, RoPE keys as stored fp16, both dotted with the query."""
    d, r, hq, hkv, bits = 32, 8, 4, 2, 3
    c = make_rope_case(40 + T, T, hq, hkv, d, r, bits, O.FULL)
    out, lse, arg = run_rope(c)
    cb = c["cb"].astype(np.float64)
    for h in range(hq):
        g = h // (hq // hkv)
        R = dense_rotation(c["quats"][g], O.FULL)
        qh = c["q"][h].astype(np.float64)
        scores, vals = [], []
        for j in range(T):
            sk = float(np.array([c["kn"][g, j]], np.uint16).view(np.float16)[0])
            sv = float(np.array([c["vn"][g, j]], np.uint16).view(np.float16)[0])
            key = sk * (R.T @ cb[O.unpack(c["kr"][g, j], bits, d)])
            rope = c["kp"][g, j].view(np.float16).astype(np.float64)
            s = sum(qh[i] * key[i] for i in range(d)) + sum(qh[d + i] * rope[i] for i in range(r))
            scores.append(0.125 * s)
            vals.append(sv * (R.T @ cb[O.unpack(c["vr"][g, j], bits, d)]))
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        ref = sum((w[j] / sum(w)) * vals[j] for j in range(T))
        assert np.max(np.abs(out[h] - ref)) < 1e-12
        assert abs(lse[h] - (m + math.log(sum(w)))) < 1e-12
        assert arg[h] == scores.index(m)


def test_rope_reduces_to_plain_attention():
    """A zero RoPE query part gives plain attention over the content; a RoPE
    key that is the same for every token shifts every score by one constant:
    same output and argmax, lse larger by that constant."""
    d, r, hq, hkv = 128, 64, 8, 2
    c = make_rope_case(50, 200, hq, hkv, d, r, 3, O.FAST)
    plain = O.attend(c["q"][:, :d], c["kr"], c["kn"], c["vr"], c["vn"], c["quats"], c["cb"], 3, O.FAST, 0.125)
    q0 = c["q"].copy()
    q0[:, d:] = 0
    o0, l0, a0 = run_rope(c, q=q0)
    assert np.max(np.abs(o0 - plain[0])) < 1e-12 and np.max(np.abs(l0 - plain[1])) < 1e-12
    assert np.array_equal(a0, plain[2])
    const = np.broadcast_to(c["kp"][:, :1], c["kp"].shape).copy()
    o1, l1, a1 = run_rope(c, kp=const)
    kr0 = const[:, 0].view(np.float16).astype(np.float64)            # (hkv, r)
    shift = np.array([0.125 * np.dot(c["q"][h, d:].astype(np.float64), kr0[h // (hq // hkv)]) for h in range(hq)])
    assert np.max(np.abs(o1 - plain[0])) < 1e-12
    assert np.max(np.abs(l1 - (plain[1] + shift))) < 1e-11
    assert np.array_equal(a1, plain[2])


def test_rope_only_scores():
    """A zero content query: the weights are the softmax of the RoPE dot
    products alone (content norms and codes play no part)."""
    d, r, hq, hkv = 128, 64, 4, 1
    c = make_rope_case(51, 64, hq, hkv, d, r, 3, O.FULL)
    q = c["q"].copy()
    q[:, :d] = 0
    out, lse, arg = run_rope(c, q=q)
    kr = c["kp"][0].view(np.float16).astype(np.float64)
    vp = O.dequantize(c["vr"][0], c["vn"][0], c["quats"][0], c["cb"], 3, O.FULL, d)
    for h in range(hq):
        s = 0.125 * (kr @ q[h, d:].astype(np.float64))
        w = np.exp(s - s.max())
        assert np.max(np.abs(out[h] - (w / w.sum()) @ vp)) < 1e-12
        assert arg[h] == int(np.argmax(s))


def test_rope_split_keeps_positional_coordinates():
    """The content part is quantised on its own (its norm, its codes); the
    RoPE part is only rounded to fp16, to nearest with ties to even."""
    d, r = 128, 8
    quats = inputs.quaternions(1, d)[0]
    cb = O.codebook(3, d)
    rng = np.random.default_rng(52)
    x = rng.standard_normal((5, d + r))
    x[0, d:d + 5] = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -1 - 2.0 ** -11, 0.1, 65504.0 + 1.0]
    a = O.quantize_rope(x, quats, cb, O.FULL, r)
    b = O.quantize(x[:, :d], quats, cb, O.FULL)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["norm16"], b["norm16"])
    x2 = x.copy()
    x2[:, d:] *= 0.5
    assert np.array_equal(O.quantize_rope(x2, quats, cb, O.FULL, r)["norm16"], b["norm16"])
    # ties to even: 1 + 2^-11 -> 1 (0x3C00), 1 + 3 * 2^-11 -> 1 + 2^-9 (0x3C02), -(1 + 2^-11) -> -1 (0xBC00);
    # 0.1 -> 0x2E66; 65505 -> 65504 (0x7BFF)
    assert a["rope16"][0, :5].tolist() == [0x3C00, 0x3C02, 0xBC00, 0x2E66, 0x7BFF]
