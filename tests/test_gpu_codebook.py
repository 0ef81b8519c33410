"""Parity with codebooks other than the built-in one, through the C ABI's cb argument.

PolyKV, Abstract: values take 3-bit Lloyd-Max codes fitted to N(0,1); the library's entry
points also accept any other symmetric 8-level codebook (ascending centroids and
boundaries, c[k] = -c[7 - k], boundary 3 at 0). Two are used here:
- "uniform": centroids (k - 3.5) / 2, boundaries at the midpoints; every value is exact in
  fp16;
- "scaled": the built-in table times 1.37 (centroids and boundaries in fp32); its
  centroids are not fp16 numbers, so the matrix-core decode's fp16 scale lambda is chosen
  for them rather than for the built-in table.
Compress (codes by the value rule with these boundaries), dequantisation (the fp32
transform bound with these centroids) and decode on both kernels (2e-3 per row, against
the oracle's decode of the same pool with these centroids) are checked.
"""

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import (B32, C32, DECODE_REL_TOL, check_norms, check_v_codes, device, new_pool,
                         pool_from_arrays, read_pool, row_rel_err)
from test_gpu_dequant import check_v

pytestmark = pytest.mark.gpu


def _tables(name):
    if name == "uniform":
        c = ((np.arange(8, dtype=np.float64) - 3.5) / 2).astype(np.float32)
        b = ((np.arange(7, dtype=np.float64) - 3.0) / 2).astype(np.float32)
    else:
        c = (C32 * np.float32(1.37)).astype(np.float32)
        b = (B32 * np.float32(1.37)).astype(np.float32)
    assert np.all(c == -c[::-1]) and b[3] == 0.0 and np.all(np.diff(c) > 0)
    return c, b


def _cb(c, b):
    cb = pk.polykv_codebook_t()
    for i in range(8):
        cb.centroid[i] = float(c[i])
    for i in range(7):
        cb.boundary[i] = float(b[i])
    return cb


@pytest.mark.parametrize("name", ["uniform", "scaled"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_compress_and_dequant_with_codebook(name, d):
    L, H, T = 2, 3, 333
    print("codebook compress/dequant", name, d, flush=True)
    c, b = _tables(name)
    cb = _cb(c, b)
    rng = np.random.default_rng(d + len(name))
    kx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    pool = new_pool(lay)
    pk.polykv_compress_kv(torch.from_numpy(kx).to(device()), torch.from_numpy(vx).to(device()), pool, lay, cb=cb)
    got = read_pool(pool, lay)
    vcodes, vnorms = oracle.tq_mse_encode(vx, b)
    want = oracle.pack_v_planes(vcodes).reshape(L * H, -1, 3, d)
    check_v_codes(got["v_planes"], want, vx.reshape(L * H, T, d), T, boundaries=b)
    check_norms(got["v_norms"], vnorms.reshape(L * H, T))
    # dequantisation of the oracle's pool with these centroids
    op = oracle.compress_pool(kx, vx, b)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    opool = torch.from_numpy(img).to(device())
    v16 = torch.full((L, H, T, d), float("nan"), dtype=torch.float16, device=device())
    pk.polykv_dequant_v(opool, lay, v16, cb=cb)
    torch.cuda.synchronize()
    nbad = check_v(v16.cpu().numpy(), op, T, centroids=c)
    if name == "scaled":
        assert nbad <= max(16, 2e-3 * v16.numel())
    # "uniform": sums of half-integers times the stored norm and 1/sqrt(d) put a few per cent
    # of exact results on or within the fp32 bound of an fp16 midpoint (about 12% exactly on
    # one at d = 64, where 1/sqrt(d) is dyadic), so either neighbour is right there and only
    # the bound check above applies


@pytest.mark.parametrize("name", ["uniform", "scaled"])
@pytest.mark.parametrize("path", [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA], ids=["valu", "mfma"])
@pytest.mark.parametrize("shape", [(2, 2, 128, 600, 15, 4), (2, 4, 64, 333, 5, 1)],
                         ids=lambda s: "L%dH%dd%dT%dA%dG%d" % s)
def test_decode_with_codebook(name, path, shape):
    L, H, d, T, A, G = shape
    print("codebook decode", name, path, shape, flush=True)
    c, b = _tables(name)
    cb = _cb(c, b)
    rng = np.random.default_rng(T + d)
    kx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    op = oracle.compress_pool(kx, vx, b)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    pool = torch.from_numpy(img).to(device())
    qn = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    q = torch.from_numpy(qn).to(device())
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path, cb=cb)
    torch.cuda.synchronize()
    kh, vh = oracle.dequant_pool(op, c)
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    err = row_rel_err(out.cpu().numpy(), ref)
    print("  worst row relative error %.3e" % err, flush=True)
    assert err <= DECODE_REL_TOL, err
