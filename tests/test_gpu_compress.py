"""GPU parity of the compress kernels against the oracle (keys bit-exact, values by rule)."""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from workloads import CONFIGS, gen_k_layer, gen_v_layer

from gpu_helpers import (B32, check_norms, check_v_codes, device, layout_for, new_pool,
                         read_pool, upload_kv)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_compress_full_config(cfg):
    """Every workload at full size, compressed as the benchmark does (keys and values in
    one launch, polykv_compress_kv) and checked against the oracle on every layer; the
    two single-kind launches must give the same pool bytes."""
    _say("compress parity", cfg.name)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    pool = new_pool(lay)
    pk.polykv_compress_kv(k, v, pool, lay)
    sep = new_pool(lay)
    pk.polykv_compress_k(k, sep, lay)
    pk.polykv_compress_v(v, sep, lay)
    torch.cuda.synchronize()
    assert torch.equal(pool, sep)
    del k, v, sep
    got = read_pool(pool, lay)
    H = cfg.n_kv_heads
    mism = coords = 0
    for l in range(cfg.n_layers):
        kl, vl = gen_k_layer(cfg, l), gen_v_layer(cfg, l)
        codes, scales = oracle.q8_0_encode(kl)
        sl = slice(l * H, (l + 1) * H)
        assert np.array_equal(got["k_codes"][sl], codes), "layer %d key codes" % l
        assert np.array_equal(got["k_scales"][sl].view(np.uint16), scales.view(np.uint16)), l
        vcodes, vnorms = oracle.tq_mse_encode(vl, B32)
        m, c = check_v_codes(got["v_planes"][sl], oracle.pack_v_planes(vcodes), vl, cfg.n_tokens)
        mism, coords = mism + m, coords + c
        check_norms(got["v_norms"][sl], vnorms)
    assert mism < 1e-5 * coords
    _say("  value-code mismatches %d of %d" % (mism, coords))


def _tie_blocks():
    """q8_0 blocks holding every exact rounding tie x = (k + 1/2) s that fp16 can represent,
    for every fp16 scale s that some fp16 block maximum produces, plus the fp16 neighbours
    of each tie on both sides. Element 0 of a block is its maximum |x| (so it sets s)."""
    s_all = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    with np.errstate(over="ignore"):
        base = (s_all.astype(np.float32) * np.float32(127)).astype(np.float16)
    amax = np.full(len(s_all), np.nan, dtype=np.float32)
    with np.errstate(over="ignore"):
        for off in (0, -1, 1, -2, 2):
            cand = (base.view(np.uint16).astype(np.int32) + off).clip(1, 0x7BFF).astype(np.uint16).view(np.float16)
            ok = np.isnan(amax) & np.isfinite(base) & \
                ((cand.astype(np.float32) / np.float32(127)).astype(np.float16) == s_all)
            amax[ok] = cand[ok].astype(np.float32)
    keep = ~np.isnan(amax)
    rows = []
    kk = np.arange(127, dtype=np.float64) + 0.5
    for sv, av in zip(s_all[keep].astype(np.float64), amax[keep].astype(np.float64)):
        x = kk * sv
        xh = x.astype(np.float16)
        tie = xh[(xh.astype(np.float64) == x) & (x <= av)]
        if tie.size == 0:
            continue
        up = np.nextafter(tie, np.float16(np.inf))
        dn = np.nextafter(tie, np.float16(0))
        vals = np.concatenate([tie, up[up.astype(np.float64) <= av], dn])
        signs = np.where(np.arange(vals.size) % 2 == 0, 1, -1).astype(np.float16)
        vals = vals * signs
        for i in range(0, vals.size, 31):
            blk = np.zeros(32, dtype=np.float16)
            blk[0] = np.float16(av)
            chunk = vals[i:i + 31]
            blk[1:1 + chunk.size] = chunk
            rows.append(blk)
    return np.stack(rows)


def test_k_codes_exact_at_every_representable_tie():
    """Round-half-even of x / s at every exact tie (and next to it), bit-exact."""
    blocks = _tie_blocks()
    d = 128
    nb = d // 32
    T = (len(blocks) + nb - 1) // nb
    kx = np.zeros((T * nb, 32), dtype=np.float16)
    kx[:len(blocks)] = blocks
    kx = kx.reshape(1, 1, T, d)
    _say("tie blocks", len(blocks), "tokens", T)
    lay = pk.polykv_pool_layout(1, 1, d, T)
    pool = new_pool(lay)
    pk.polykv_compress_k(torch.from_numpy(kx).to(device()), pool, lay)
    torch.cuda.synchronize()
    got = read_pool(pool, lay)
    codes, scales = oracle.q8_0_encode(kx[0])
    assert np.array_equal(got["k_scales"][0].view(np.uint16), scales[0].view(np.uint16))
    bad = np.argwhere(got["k_codes"][0] != codes[0])
    assert bad.size == 0, (len(bad), bad[:5])


@pytest.mark.parametrize("T", [1, 31, 33, 100])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_compress_ragged_and_dims(T, d):
    rng = np.random.default_rng(T * 1000 + d)
    L, H = 2, 3
    kx = (rng.standard_normal((L, H, T, d)) * rng.lognormal(0, 1, (L, H, 1, d))).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    pool = new_pool(lay)
    pk.polykv_compress_k(torch.from_numpy(kx).to(device()), pool, lay)
    pk.polykv_compress_v(torch.from_numpy(vx).to(device()), pool, lay)
    got = read_pool(pool, lay)
    codes, scales = oracle.q8_0_encode(kx)
    assert np.array_equal(got["k_codes"], codes.reshape(L * H, T, d))
    assert np.array_equal(got["k_scales"].view(np.uint16), scales.reshape(L * H, T, d // 32).view(np.uint16))
    vcodes, vnorms = oracle.tq_mse_encode(vx, B32)
    check_v_codes(got["v_planes"], oracle.pack_v_planes(vcodes).reshape(L * H, -1, 3, d),
                  vx.reshape(L * H, T, d), T)
    check_norms(got["v_norms"], vnorms.reshape(L * H, T))


def test_compress_special_values():
    d, T = 128, 64
    kx = np.zeros((1, 1, T, d), dtype=np.float16)
    kx[0, 0, 0, 0] = 127 / 128                                   # scale 2^-7 exactly
    kx[0, 0, 0, 1:9] = [(2 * j + 1) / 256 for j in range(8)]     # ties k + 1/2
    kx[0, 0, 0, 9:17] = [-(2 * j + 1) / 256 for j in range(8)]
    kx[0, 0, 2, 0] = np.float16(178 * 2.0 ** -24)                 # subnormal scale, clamp
    kx[0, 0, 2, 1] = np.float16(-178 * 2.0 ** -24)
    kx[0, 0, 3, :] = 65504.0                                      # largest fp16
    kx[0, 0, 4, :] = -0.0
    vx = np.zeros((1, 1, T, d), dtype=np.float16)
    vx[0, 0, 1, 5] = 3.0                                          # one-hot
    vx[0, 0, 2, :] = 0.5                                          # constant
    vx[0, 0, 3, :] = -2.0
    vx[0, 0, 4, 7] = -1e-4
    vx[0, 0, 5:, :] = np.random.default_rng(1).standard_normal((T - 5, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(1, 1, d, T)
    pool = new_pool(lay)
    pk.polykv_compress_k(torch.from_numpy(kx).to(device()), pool, lay)
    pk.polykv_compress_v(torch.from_numpy(vx).to(device()), pool, lay)
    got = read_pool(pool, lay)
    codes, scales = oracle.q8_0_encode(kx)
    assert np.array_equal(got["k_codes"][0], codes[0, 0])
    assert np.array_equal(got["k_scales"][0].view(np.uint16), scales[0, 0].view(np.uint16))
    assert list(got["k_codes"][0, 0, 1:9]) == [0, 2, 2, 4, 4, 6, 6, 8]
    vcodes, vnorms = oracle.tq_mse_encode(vx, B32)
    want = oracle.pack_v_planes(vcodes).reshape(1, -1, 3, d)
    check_v_codes(got["v_planes"], want, vx.reshape(1, T, d), T)
    # tokens 0-4 are constructed (zero, one-hot, constants): their codes admit no slack,
    # including the zero coordinates of the constant vectors that sit on the middle boundary
    low5 = np.uint32(0x1F)
    assert np.array_equal(got["v_planes"][0, 0] & low5, want[0, 0] & low5)
    assert np.array_equal(got["v_norms"][0, :5].view(np.uint16), vnorms[0, 0, :5].view(np.uint16))
    check_norms(got["v_norms"], vnorms.reshape(1, T))


def test_layer_range_writes_only_its_layers():
    L, H, d, T = 3, 2, 128, 70
    lay = pk.polykv_pool_layout(L, H, d, T)
    rng = np.random.default_rng(3)
    kx = rng.standard_normal((1, H, T, d)).astype(np.float16)
    pool = new_pool(lay, fill=0x5A)
    before = pool.clone()
    pk.polykv_compress_k(torch.from_numpy(kx).to(device()), pool, lay, layer_begin=1, layer_count=1)
    pk.polykv_compress_v(torch.from_numpy(kx).to(device()), pool, lay, layer_begin=1, layer_count=1)
    got = read_pool(pool, lay)
    old = read_pool(before, lay)
    for name in got:
        for t in (0, 1, 4, 5):
            assert np.array_equal(got[name][t].view(np.uint8), old[name][t].view(np.uint8)), (name, t)
    codes, _ = oracle.q8_0_encode(kx)
    assert np.array_equal(got["k_codes"][2:4], codes[0])
    # bytes outside every payload are untouched
    flat, flat0 = pool.cpu().numpy(), before.cpu().numpy()
    mask = np.ones(lay.total_bytes, dtype=bool)
    G = (T + 31) // 32
    for off, stride, n in [(lay.k_codes_off, lay.k_codes_tile_stride, T * d),
                           (lay.k_scales_off, lay.k_scales_tile_stride, T * d // 16),
                           (lay.v_planes_off, lay.v_planes_tile_stride, G * 3 * d * 4),
                           (lay.v_norms_off, lay.v_norms_tile_stride, 2 * T)]:
        for t in range(L * H):
            mask[off + t * stride: off + t * stride + n] = False
    assert np.array_equal(flat[mask], flat0[mask])


def test_non_default_stream_and_determinism():
    cfg = CONFIGS[1]
    lay = layout_for(cfg)
    k, v = upload_kv(cfg, layers=range(cfg.n_layers))
    s = torch.cuda.Stream()
    pools = []
    for _ in range(2):
        pool = new_pool(lay)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            pk.polykv_compress_k(k, pool, lay, stream=s)
            pk.polykv_compress_v(v, pool, lay, stream=s)
        pools.append(pool)
    s.synchronize()
    assert torch.equal(pools[0], pools[1])


@pytest.mark.parametrize("cfg", [CONFIGS[1], CONFIGS[3]], ids=lambda c: c.name)
def test_concurrent_key_and_value_compress(cfg):
    """polykv_compress_k and polykv_compress_v write disjoint regions of the pool, so they may
    run at the same time: launched on two streams with no order between them (each of several
    rounds into a fresh copy of a garbage-filled pool), the pool is byte-identical to the
    one written by the two calls in sequence."""
    _say("concurrent compress", cfg.name)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    base = new_pool(lay, fill=0x77)
    seq = base.clone()
    pk.polykv_compress_k(k, seq, lay)
    pk.polykv_compress_v(v, seq, lay)
    torch.cuda.synchronize()
    sk, sv = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(3):
        pool = base.clone()
        torch.cuda.synchronize()
        # the value compress first on its stream in odd rounds, so both orders of issue occur
        order = [(sv, lambda: pk.polykv_compress_v(v, pool, lay, stream=sv)),
                 (sk, lambda: pk.polykv_compress_k(k, pool, lay, stream=sk))]
        if r % 2 == 0:
            order.reverse()
        for st, fn in order:
            with torch.cuda.stream(st):
                fn()
        sk.synchronize()
        sv.synchronize()
        assert torch.equal(pool, seq), "round %d" % r


@pytest.mark.parametrize("d", [64, 128])
def test_vector_alu_value_compress(d):
    """polykv_compress_v_path with the vector-ALU rotation at head_dim 64 and 128 (the sizes
    where the matrix-core rotation is the automatic choice): oracle parity by the value
    rule, and the same pool as the matrix-core path except at boundary coordinates."""
    L, H, T = 2, 3, 333
    rng = np.random.default_rng(d + 5)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    vx[0, 1, 7] = 0.0                      # a zero vector
    vx[1, 2, 11] = np.float16(0.5)         # a constant vector (ties at y = 0)
    lay = pk.polykv_pool_layout(L, H, d, T)
    v = torch.from_numpy(vx).to(device())
    pools = {}
    for path in (pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA):
        pool = new_pool(lay)
        pk.polykv_compress_v(v, pool, lay, path=path)
        torch.cuda.synchronize()
        pools[path] = read_pool(pool, lay)
    want_codes, want_norms = oracle.tq_mse_encode(vx, B32)
    want_planes = oracle.pack_v_planes(want_codes).reshape(L * H, -1, 3, d)
    for path, got in pools.items():
        m, c = check_v_codes(got["v_planes"], want_planes, vx.reshape(L * H, T, d), T)
        check_norms(got["v_norms"], want_norms.reshape(L * H, T))
        _say("  path %d: value-code mismatches %d of %d" % (path, m, c))
