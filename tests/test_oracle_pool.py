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


def test_dequant_fp16_rounds_the_double_once():
    """The fp16 step is one round-to-nearest-even of the fp64 value. Key values: with the
    fp16 scale s = 1 + 2^-10, code 127 gives 127 + 127 * 2^-10, which lies between the
    fp16 neighbours 127.0 and 127.125 (spacing 2^-4) and nearer the upper one. The
    conversion itself is checked at a tie and just above it, where a float32 detour would
    round twice and go the wrong way."""
    from oracle import dequant_fp16
    # one token-head, d = 32: code 127 * s with s = fp16(1 + 2^-10) is 127 + 127 * 2^-10,
    # exact in fp64 and in fp32; fp16 spacing at 127 is 2^-4, so it rounds to 127.125
    s = np.float16(1 + 2.0 ** -10)
    codes = np.zeros((1, 1, 1, 32), dtype=np.int8)
    codes[..., 0] = 127
    codes[..., 1] = -127
    codes[..., 2] = 1
    pool = {"k_codes": codes, "k_scales": np.full((1, 1, 1, 1), s, dtype=np.float16),
            "v_codes": np.full((1, 1, 1, 32), 3, dtype=np.uint8),
            "v_norms": np.zeros((1, 1, 1), dtype=np.float16)}
    c32, _ = codebook_fp32()
    k16, v16 = dequant_fp16(pool, c32)
    exact = 127 * (1 + 2.0 ** -10)
    assert float(k16[0, 0, 0, 0]) == 127.125 and abs(exact - 127.125) < 2.0 ** -5
    assert float(k16[0, 0, 0, 1]) == -127.125
    assert float(k16[0, 0, 0, 2]) == float(s)
    assert np.all(v16 == 0)
    # the conversion itself: 1 + 2^-11 is a tie (to even: 1), 1 + 2^-11 + 2^-40 is above
    # it (up), although a float32 detour would land on the tie first and go down
    x = np.array([1 + 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -40, 1 + 3 * 2.0 ** -11])
    assert list(x.astype(np.float16).astype(np.float64)) == [1.0, 1 + 2.0 ** -10, 1 + 2 * 2.0 ** -10]
    assert np.float32(x[1]) == np.float32(x[0])  # the float32 detour loses the difference


def test_dequant_fp16_matches_round_trip_bounds():
    """fp16 reconstructions of a seeded pool: keys within s/2 of the input plus the fp16
    rounding of the reconstruction (the q8_0 error bound), values equal elementwise to
    the fp64 reconstruction rounded."""
    from oracle import compress_pool, dequant_fp16, dequant_pool
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 2, 40, 64)).astype(np.float16)
    v = rng.standard_normal((1, 2, 40, 64)).astype(np.float16)
    c32, b32 = codebook_fp32()
    op = compress_pool(k, v, b32)
    k16, v16 = dequant_fp16(op, c32)
    kh, vh = dequant_pool(op, c32)
    s = op["k_scales"].astype(np.float64).repeat(32, axis=-1)
    err = np.abs(k16.astype(np.float64) - k.astype(np.float64))
    assert np.all(err <= s / 2 + np.abs(kh) * 2.0 ** -11 + 1e-12)
    np.testing.assert_array_equal(v16, vh.astype(np.float16))
    assert k16.dtype == np.float16 and v16.dtype == np.float16


@pytest.mark.parametrize("order", ["forward", "shuffled"])
def test_append_in_any_order_equals_one_compress(order):
    """Chunks written one at a time, in order or not, give the one-shot pool: the codecs
    work per token (q8_0 blocks lie along head_dim, the rotation and norm are per vector)."""
    from oracle import append_pool
    rng = np.random.default_rng(12)
    L, H, T, d = 2, 2, 101, 64
    k = rng.standard_normal((L, H, T, d)).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    _, b32 = codebook_fp32()
    whole = compress_pool(k, v, b32)
    cuts = [0, 1, 32, 45, 64, 100, T]
    chunks = list(zip(cuts[:-1], cuts[1:]))
    if order == "shuffled":
        chunks = [chunks[i] for i in (3, 0, 5, 2, 4, 1)]
    # start from a pool whose every code and norm is something else
    pool = {"k_codes": np.full_like(whole["k_codes"], 77), "k_scales": np.full_like(whole["k_scales"], 3.0),
            "v_codes": np.full_like(whole["v_codes"], 5), "v_norms": np.full_like(whole["v_norms"], 9.0)}
    pool["v_planes"] = pack_v_planes(pool["v_codes"])
    for a, b in chunks:
        pool = append_pool(pool, k[..., a:b, :], v[..., a:b, :], a, b32)
    for key in ("k_codes", "k_scales", "v_codes", "v_norms", "v_planes"):
        assert np.array_equal(pool[key], whole[key]), key
    with pytest.raises(ValueError):
        append_pool(pool, k[..., :5, :], v[..., :5, :], T - 4, b32)
