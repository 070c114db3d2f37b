"""The seeded input generators: shapes, dtypes, determinism and the stated
distributions (CPU only)."""

import numpy as np

from compressed_space_attention_isoquant_amd import inputs


def test_quaternions_unit_and_deterministic():
    a = inputs.quaternions(4, 128)
    b = inputs.quaternions(4, 128)
    assert a.shape == (4, 32, 2, 4) and a.dtype == np.float32
    assert np.array_equal(a, b)
    assert np.max(np.abs(np.linalg.norm(a.astype(np.float64), axis=-1) - 1.0)) < 3e-7


def test_unit_vectors():
    x = inputs.unit_vectors(100, 256, np.float16, seed=3)
    assert x.shape == (100, 256) and x.dtype == np.float16
    assert np.max(np.abs(np.linalg.norm(x.astype(np.float64), axis=-1) - 1.0)) < 2e-3


def test_decode_case_outliers_and_needles():
    c = inputs.decode_case(seed=7, kv_len=2048, num_q_heads=32, num_kv_heads=4, head_dim=128, needles=16)
    assert c["k"].shape == (2048, 4, 128) and c["k"].dtype == np.float16
    assert c["q"].shape == (32, 128)
    k = c["k"].astype(np.float64)
    for g in range(4):
        std = k[:, g].std(axis=0)
        big = np.argsort(std)[-4:]
        assert set(big) == set(c["channels_k"][g])
        assert np.all(std[big] > 8)
    pos = [p for _, _, p in c["needles"]]
    assert len(set(pos)) == 16
    for h, g, p in c["needles"]:
        key = k[p, g]
        qh = c["q"][h].astype(np.float64)
        cos = key @ qh / np.linalg.norm(key) / np.linalg.norm(qh)
        assert abs(cos - 0.9) < 5e-3


def test_batch_lengths_range():
    L = inputs.batch_lengths(5, 64, 1024, 32768)
    assert L.shape == (64,) and L.min() >= 1024 and L.max() <= 32768
