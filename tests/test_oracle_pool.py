"""Pins of the oracle's bit-plane layout and byte counts, and the pages' memory arithmetic."""

import os

import numpy as np
import pytest

from oracle import analytic_pool_bytes, codebook_fp32, compress_pool, pack_v_planes, unpack_v_planes
from oracle.pool import fp16_kv_bytes
from workloads import CONFIGS


def test_pack_hand_example():
    codes = np.zeros((35, 4), dtype=np.uint8)
    codes[0, 0] = 5      # 0b101
    codes[1, 0] = 2      # 0b010
    codes[31, 3] = 7
    codes[32, 1] = 4     # second group, j = 0
    codes[34, 2] = 3
    w = pack_v_planes(codes)
    assert w.shape == (2, 3, 4) and w.dtype == np.uint32
    assert w[0, 0, 0] == 0b01 and w[0, 1, 0] == 0b10 and w[0, 2, 0] == 0b01
    assert w[0, 0, 3] == w[0, 1, 3] == w[0, 2, 3] == 1 << 31
    assert w[1, 2, 1] == 1 and w[1, 0, 1] == 0 and w[1, 1, 1] == 0
    assert w[1, 0, 2] == 1 << 2 and w[1, 1, 2] == 1 << 2 and w[1, 2, 2] == 0
    assert np.count_nonzero(w) == 9


@pytest.mark.parametrize("T", [1, 31, 32, 33, 600, 1851])
def test_pack_round_trip_and_zero_padding(T):
    codes = np.random.default_rng(T).integers(0, 8, size=(2, T, 64)).astype(np.uint8)
    w = pack_v_planes(codes)
    assert w.shape == (2, (T + 31) // 32, 3, 64)
    assert np.array_equal(unpack_v_planes(w, T), codes)
    tail = T % 32
    if tail:
        assert np.all(w[:, -1] >> np.uint32(tail) == 0)


def test_analytic_bytes_equals_array_payload():
    _, b32 = codebook_fp32()
    for d, T in [(128, 40), (64, 33)]:
        rng = np.random.default_rng(d)
        k = rng.standard_normal((2, 3, T, d)).astype(np.float16)
        v = rng.standard_normal((2, 3, T, d)).astype(np.float16)
        p = compress_pool(k, v, b32)
        payload = p["k_codes"].nbytes + p["k_scales"].nbytes + p["v_norms"].nbytes + (3 * p["v_codes"].size) // 8
        assert analytic_pool_bytes(2, 3, T, d) == payload


def test_compression_ratios():
    for d, want in [(128, 512 / 186), (64, 256 / 94)]:
        ratio = fp16_kv_bytes(1, 1, 1, d) / analytic_pool_bytes(1, 1, 1, d)
        assert ratio == pytest.approx(want, rel=1e-15)
    # code-only ratio: 16+16 bits against 8+3 bits per (key, value) element
    assert 32 / 11 == pytest.approx(2.91, abs=5e-3)


def test_config_pool_bytes():
    want = [223_200, 43_315_200, 88_137_216, 195_035_136, 342_549_504]
    for cfg, w in zip(CONFIGS, want):
        assert analytic_pool_bytes(cfg.n_layers, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim) == w


def test_pages_memory_arithmetic(golden_dir):
    g = {}
    for line in open(os.path.join(golden_dir, "polykv_abstract_figures.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            g[k] = v
    ratio, agents = float(g["compression_ratio"]), int(g["agents"])
    before, after = float(g["kv_gb_before"]), float(g["kv_gb_after"])
    # 0.45 GB is 19.8 GB shared once across 15 agents at 2.91x, and 97.7% is 1 - that share
    assert before / (agents * ratio) == pytest.approx(after, abs=5e-3)
    assert 100 * (1 - 1 / (agents * ratio)) == pytest.approx(float(g["reduction_pct"]), abs=0.05)
    # the 4K Llama-3-8B headline workload here: 15 private fp16 caches against one pool
    c3 = CONFIGS[3]
    fp16_private = agents * fp16_kv_bytes(c3.n_layers, c3.n_kv_heads, c3.n_tokens, c3.head_dim)
    shared = analytic_pool_bytes(c3.n_layers, c3.n_kv_heads, c3.n_tokens, c3.head_dim)
    assert 1 - shared / fp16_private == pytest.approx(0.9758, abs=1e-4)
