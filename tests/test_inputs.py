"""The seeded generators: deterministic, in range, bf16 rounding as torch."""
import numpy as np
import torch

from deepseek_sparse_attention_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.5e-39, 3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.f32_to_bf16_bits(x), ref)


def test_workload_deterministic_and_in_range():
    a = I.make_workload("t", 99, I.GEOM_TOKEN, 2, 3000, [0, 1, 1], [3000, 2500, 100])
    b = I.make_workload("t", 99, I.GEOM_TOKEN, 2, 3000, [0, 1, 1], [3000, 2500, 100])
    for f in ("cache", "idx_k", "q", "idx_q", "idx_w"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    k = I.bf16_bits_to_f32(a.idx_k[0])
    assert k.min() == -8 and k.max() == 8 and np.all(k == np.round(k))
    assert set(np.unique(a.idx_w).tolist()) <= {1.0, 2.0, 3.0, 4.0}
    # rows past every query's visible range of sequence 1 are poisoned
    assert np.all(a.cache[1, 2500:] == I.BF16_NAN) and not np.any(a.cache[1, :2500] == I.BF16_NAN)
    c = I.bf16_bits_to_f32(a.cache[0]).astype(np.float64)
    assert abs(c.mean()) < 0.01 and abs(c.std() - 1) < 0.01


def test_offset_and_tie_storm_keys():
    w = I.make_workload("t", 98, I.GEOM_TOKEN, 1, 20000, [0], [20000],
                        key_range=(-4, 4), offset_std=0.5)
    k = I.bf16_bits_to_f32(w.idx_k[0])
    assert k.min() == -4 and k.max() == 4
    c = I.bf16_bits_to_f32(w.cache[0]).astype(np.float64)
    col_means = c.mean(axis=0)     # the shared per-sequence offset, std 0.5
    assert 0.35 < col_means.std() < 0.65


def test_kpool_geometry():
    w = I.make_workload("t", 97, I.GEOM_KPOOL, 1, 4096, [0], [4095])
    assert w.cache.shape == (1, 4096, 512) and w.idx_k.shape == (1, 1024, 128)
    assert np.all(w.idx_k[0, 1023] == I.BF16_NAN)      # the unfilled pool
    assert np.all(w.cache[0, 4095] == I.BF16_NAN)
