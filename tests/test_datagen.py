"""The seeded input generators: determinism, exact ignore counts, encodings."""
import math

import numpy as np
import pytest

import datagen

II = datagen.IGNORE_INDEX


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6: the even one (1 + 2^-6) wins.
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0],
                 dtype=np.float32)
    back = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x))
    assert back.tolist() == [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5, 0.0]


def test_bf16_error_bound():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    back = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x))
    assert np.max(np.abs(back - x) / np.abs(x)) <= 2.0 ** -8


def test_workload_table():
    w = datagen.WORKLOADS
    assert (w[0].N, w[0].H, w[0].V, w[0].dtype, w[0].chunk_tokens) == (512, 128, 256, "f32", 128)
    assert (w[1].N, w[1].H, w[1].V, w[1].chunk_tokens) == (8192, 4096, 128256, 1024)
    assert (w[2].N, w[2].H, w[2].V, w[2].chunk_tokens) == (16384, 3584, 152064, 2048)
    assert (w[3].N, w[3].H, w[3].V) == (16384, 4096, 128256)
    assert (w[4].N, w[4].H, w[4].V) == (8192, 2304, 256000)


def test_tiny_workload_deterministic_and_counts():
    a, b = datagen.make(0), datagen.make(0)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.W, b.W)
    assert np.array_equal(a.labels, b.labels)
    assert a.X.dtype == np.float32 and a.X.shape == (512, 128) and a.W.shape == (256, 128)
    assert int((a.labels == II).sum()) == 51
    v = a.labels[a.labels != II]
    assert v.min() >= 0 and v.max() < 256
    assert abs(float(a.W.std()) - 0.02) < 0.002


def test_w_blocks_independent_of_threads():
    a = datagen.make_custom(10, 16, 3 * datagen.W_BLOCK_ROWS + 5, "bf16", seed=3)
    old = datagen._THREADS
    try:
        datagen._THREADS = 1
        b = datagen.make_custom(10, 16, 3 * datagen.W_BLOCK_ROWS + 5, "bf16", seed=3)
    finally:
        datagen._THREADS = old
    assert a.W.dtype == np.uint16 and np.array_equal(a.W, b.W)


def test_prefix_ignore_and_rmsnorm_and_zipf():
    inp = datagen.make_custom(400, 64, 1000, "bf16", seed=5, x_dist="rmsnorm",
                              label_dist="zipf", ignore_mode="prefix", ignore_frac=0.25)
    assert np.all(inp.labels[:100] == II) and np.all(inp.labels[100:] != II)
    x = inp.X_f64()
    assert np.allclose(np.sqrt((x * x).mean(axis=1)), 1.0, atol=1e-2)
    p = datagen.zipf_probs(1000, 1.1)
    assert abs(p[0] / p[1] - 2 ** 1.1) < 1e-12
    # id 0 is the most frequent label
    counts = np.bincount(inp.labels[100:], minlength=1000)
    assert counts.argmax() == 0


def test_zipf_fractions_of_qwen_vocab():
    p = datagen.zipf_probs(152064, 1.1)
    assert abs(p[0] - 0.132) < 0.002 and abs(p[:10].sum() - 0.355) < 0.003


def test_sample_rows():
    s = datagen.sample_rows(1000, 10, 1, must=(0, 999))
    assert len(s) == 10 and s[0] == 0 and s[-1] == 999 and len(set(s)) == 10
