"""GPU dequantisation (pool -> fp16 K and V) against the oracle, through the C ABI.

Rules:
- keys: bit-exact. code * s is exact in fp32, so the library's one rounding to fp16 and
  the oracle's rounding of the exact fp64 product must agree everywhere;
- values: the library runs the inverse FWHT in fp32 before its one rounding to fp16, the
  oracle rounds its fp64 value x. The fp32 result y is within E = (log2(d) * 2^-24 * S) *
  n/d + 2^-24 |x| of x (S = sum of the token's |centroids|: every stage of the butterfly
  tree rounds partial sums over disjoint coordinate sets, whose magnitudes add up to at
  most S; the scaling by n/d rounds once more). Rounding to nearest is monotone, so the
  library's fp16 value must lie between RNE16(x - E) and RNE16(x + E). Away from zero that
  allows at most the other fp16 neighbour of x, and only where x lies within E of the
  midpoint between the two; where x is (near) 0 it allows a few subnormal steps.
"""

import math

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import B32, C32, device, layout_for, pool_from_arrays, upload_kv
from workloads import CONFIGS

pytestmark = pytest.mark.gpu


def _pool(L, H, d, T, seed, k_scale=1.0, zero_v_tokens=()):
    rng = np.random.default_rng(seed)
    kx = (rng.standard_normal((L, H, T, d)) * k_scale).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    for t in zero_v_tokens:
        vx[:, :, t, :] = 0
    lay = pk.polykv_pool_layout(L, H, d, T)
    op = oracle.compress_pool(kx, vx, B32)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    return lay, torch.from_numpy(img).to(device()), op


def check_v(got16, op, n_tokens, centroids=None):
    """The value rule above; returns the number of elements that differ from the oracle.
    centroids: the codebook's (default: the built-in one)."""
    C = C32 if centroids is None else np.asarray(centroids, dtype=np.float32)
    _, v64 = oracle.dequant_pool(op, C, n_tokens)
    _, want16 = oracle.dequant_fp16(op, C, n_tokens)
    got16 = np.asarray(got16, dtype=np.float16).reshape(want16.shape)
    g = got16.astype(np.float64)
    w = want16.astype(np.float64)
    bad = g != w
    if not bad.any():
        return 0
    d = want16.shape[-1]
    codes = op["v_codes"] if "v_codes" in op else oracle.unpack_v_planes(op["v_planes"], n_tokens)
    S = np.abs(np.asarray(C, dtype=np.float64)[codes.astype(np.intp)]).sum(axis=-1, keepdims=True)
    f = op["v_norms"].astype(np.float64)[..., None] / d
    E = (math.log2(d) * 2.0 ** -24 * S) * f + 2.0 ** -24 * np.abs(v64)
    E = np.broadcast_to(E, v64.shape)
    idx = np.nonzero(bad)
    lo = (v64[idx] - E[idx] * 1.0001).astype(np.float16).astype(np.float64)
    hi = (v64[idx] + E[idx] * 1.0001).astype(np.float16).astype(np.float64)
    assert np.all((lo <= g[idx]) & (g[idx] <= hi)), "a value lies outside the fp32 error bound"
    return int(bad.sum())


@pytest.mark.parametrize("shape", [(1, 2, 128, 600), (2, 3, 64, 95), (1, 2, 256, 33), (1, 1, 128, 1),
                                   (2, 2, 64, 64), (1, 1, 64, 33), (1, 2, 64, 1)],
                         ids=lambda s: "L%dH%dd%dT%d" % s)
def test_dequant_small(shape):
    L, H, d, T = shape
    print("dequant", shape, flush=True)
    lay, pool, op = _pool(L, H, d, T, seed=T + d, zero_v_tokens=(0,) if T > 1 else ())
    k = torch.full((L, H, T, d), float("nan"), dtype=torch.float16, device=device())
    v = torch.full_like(k, float("nan"))
    pk.polykv_dequant_k(pool, lay, k)
    pk.polykv_dequant_v(pool, lay, v)
    torch.cuda.synchronize()
    k16, _ = oracle.dequant_fp16(op, C32, T)
    assert np.array_equal(k.cpu().numpy().view(np.uint16), k16.view(np.uint16))
    nbad = check_v(v.cpu().numpy(), op, T)
    assert nbad <= max(16, 2e-3 * v.numel())  # about 5e-4 of elements sit that close to a midpoint


@pytest.mark.parametrize("k_scale", [1e-5, 300.0])
def test_dequant_k_extreme_scales(k_scale):
    # tiny keys give subnormal fp16 scales and results; large keys large ones
    L, H, d, T = 1, 2, 128, 70
    lay, pool, op = _pool(L, H, d, T, seed=9, k_scale=k_scale)
    k = torch.empty((L, H, T, d), dtype=torch.float16, device=device())
    pk.polykv_dequant_k(pool, lay, k)
    torch.cuda.synchronize()
    k16, _ = oracle.dequant_fp16(op, C32, T)
    assert np.array_equal(k.cpu().numpy().view(np.uint16), k16.view(np.uint16))


def test_dequant_layer_range_writes_only_its_layers():
    L, H, d, T = 3, 2, 128, 100
    lay, pool, op = _pool(L, H, d, T, seed=4)
    k = torch.full((1, H, T, d), float("nan"), dtype=torch.float16, device=device())
    v = torch.full_like(k, float("nan"))
    pk.polykv_dequant_k(pool, lay, k, layer_begin=1, layer_count=1)
    pk.polykv_dequant_v(pool, lay, v, layer_begin=1, layer_count=1)
    torch.cuda.synchronize()
    sub = {key: val[1:2] for key, val in op.items()}
    k16, _ = oracle.dequant_fp16(sub, C32, T)
    assert np.array_equal(k.cpu().numpy().view(np.uint16), k16.view(np.uint16))
    check_v(v.cpu().numpy(), sub, T)


def test_dequant_full_size_sampled():
    """The 4K Llama-3-8B pool compressed on the GPU, dequantised on the GPU; tiles 0, a
    middle one and the last checked against the oracle's dequantisation of those tiles."""
    cfg = CONFIGS[3]
    lay = layout_for(cfg)
    kin, vin = upload_kv(cfg)
    pool = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=device())
    pk.polykv_compress_k(kin, pool, lay)
    pk.polykv_compress_v(vin, pool, lay)
    del kin, vin
    k = torch.empty((cfg.n_layers, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim), dtype=torch.float16, device=device())
    v = torch.empty_like(k)
    pk.polykv_dequant_k(pool, lay, k)
    pk.polykv_dequant_v(pool, lay, v)
    torch.cuda.synchronize()
    tiles = cfg.n_layers * cfg.n_kv_heads
    sel = [0, tiles // 2 + 3, tiles - 1]
    views = pk.pool_views(pool, lay)
    op = {"k_codes": views["k_codes"][sel].cpu().numpy(),
          "k_scales": views["k_scales"][sel].cpu().numpy(),
          "v_planes": views["v_planes"][sel].cpu().numpy().view(np.uint32),
          "v_norms": views["v_norms"][sel].cpu().numpy()}
    k16, _ = oracle.dequant_fp16(op, C32, cfg.n_tokens)
    kg = k.view(tiles, cfg.n_tokens, cfg.head_dim)[sel].cpu().numpy()
    assert np.array_equal(kg.view(np.uint16), k16.view(np.uint16))
    vg = v.view(tiles, cfg.n_tokens, cfg.head_dim)[sel].cpu().numpy()
    nbad = check_v(vg, op, cfg.n_tokens)
    assert nbad <= 1e-3 * vg.size
