"""Shared helpers of the GPU tests: device inputs, pool read-back and comparison rules.

The rules (tolerances and what counts as a match) live here so that every GPU test uses
the same ones:
- key codes and scales: bit-exact;
- value codes: a differing code is allowed only where the oracle's fp64 rotated coordinate
  lies within 1e-5 of a decision boundary, and such coordinates must be fewer than 1e-5 of
  all coordinates;
- value norms: within one fp16 ulp (they differ only where an fp32 and an fp64 sum round
  to different sides of an fp16 rounding midpoint);
- decode outputs: per query row, max |o - o_ref| / max |o_ref| <= 2e-3 against the fp64
  oracle.
"""

import numpy as np
import torch

import agent_q8_quant_amd as pk
import oracle
from workloads import gen_k_layer, gen_q_step, gen_v_layer

V_BOUNDARY_WINDOW = 1e-5
V_MISMATCH_FRACTION = 1e-5
DECODE_REL_TOL = 2e-3

C32, B32 = oracle.codebook_fp32()


def device():
    return torch.device("cuda", 0)


def layout_for(cfg):
    return pk.polykv_pool_layout(cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_tokens)


def new_pool(layout, fill=0xA5):
    """A pool buffer with every byte set, so that unwritten bytes are visible."""
    return torch.full((layout.total_bytes,), fill, dtype=torch.uint8, device=device())


def upload_kv(cfg, layers=None):
    layers = list(range(cfg.n_layers)) if layers is None else list(layers)
    k = torch.empty((len(layers), cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim), dtype=torch.float16, device=device())
    v = torch.empty_like(k)
    for i, l in enumerate(layers):
        k[i].copy_(torch.from_numpy(gen_k_layer(cfg, l)))
        v[i].copy_(torch.from_numpy(gen_v_layer(cfg, l)))
    return k, v


def upload_q(cfg, step):
    return torch.from_numpy(gen_q_step(cfg, step)).to(device())


def read_pool(pool, layout):
    """numpy copies of the four regions, each [tiles][...]."""
    v = pk.pool_views(pool, layout)
    return {"k_codes": v["k_codes"].cpu().numpy(),
            "k_scales": v["k_scales"].cpu().numpy(),
            "v_planes": v["v_planes"].cpu().numpy().view(np.uint32),
            "v_norms": v["v_norms"].cpu().numpy()}


def pool_from_arrays(layout, k_codes, k_scales, v_planes, v_norms):
    """A host byte image of a pool holding the given arrays ([tiles][...] each)."""
    buf = np.zeros(layout.total_bytes, dtype=np.uint8)

    def put(off, stride, arr):
        arr = np.ascontiguousarray(arr)
        tiles = arr.shape[0]
        flat = arr.reshape(tiles, -1).view(np.uint8)
        for t in range(tiles):
            buf[off + t * stride: off + t * stride + flat.shape[1]] = flat[t]

    put(layout.k_codes_off, layout.k_codes_tile_stride, k_codes)
    put(layout.k_scales_off, layout.k_scales_tile_stride, k_scales)
    put(layout.v_planes_off, layout.v_planes_tile_stride, v_planes)
    put(layout.v_norms_off, layout.v_norms_tile_stride, v_norms)
    return buf


def check_v_codes(gpu_planes, want_planes, v_fp16, n_tokens, boundaries=None):
    """Apply the value-code rule to one set of tiles.

    gpu_planes, want_planes: uint32 [tiles][G][3][d]; v_fp16: the input [tiles][T][d];
    boundaries: the codebook's (default: the built-in one).
    Returns (number of mismatched coordinates, number of coordinates).
    """
    diff = np.bitwise_xor(gpu_planes, want_planes)
    n_coords = v_fp16.shape[0] * n_tokens * v_fp16.shape[-1]
    if not diff.any():
        return 0, n_coords
    tiles, G, P, d = diff.shape
    bad = set()
    for t, g, p, i in zip(*np.nonzero(diff)):
        w = int(diff[t, g, p, i])
        for j in range(32):
            if (w >> j) & 1:
                tok = 32 * g + j
                assert tok < n_tokens, "a padding bit was set"
                bad.add((t, tok, i))
    bad = sorted(bad)
    # the oracle's fp64 rotated coordinates of the affected vectors
    b = np.asarray(B32 if boundaries is None else boundaries, dtype=np.float64)
    for (t, tok, i) in bad:
        y = oracle.rotated_coordinates(v_fp16[t, tok])[i]
        assert np.min(np.abs(y - b)) < V_BOUNDARY_WINDOW, (t, tok, i, y)
    assert len(bad) < V_MISMATCH_FRACTION * n_coords, (len(bad), n_coords)
    return len(bad), n_coords


def check_norms(gpu_norms, want_norms):
    g = gpu_norms.astype(np.float16).view(np.uint16).astype(np.int32)
    w = want_norms.astype(np.float16).view(np.uint16).astype(np.int32)
    assert np.all(np.abs(g - w) <= 1), np.max(np.abs(g - w))
    return int(np.count_nonzero(g != w))


def row_rel_err(out, ref):
    """Per-row max |o - ref| / max |ref| over the last axis; returns the worst."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / den))


def oracle_pool_on_device(L, H, d, T, seed, k_scale=1.0):
    """The oracle's pool of seeded N(0,1) K/V (K optionally scaled), uploaded as the
    library's byte image; returns (layout, device pool, k_hat, v_hat) with the oracle's
    fp64 per-token reconstructions [L][H][T][d]."""
    rng = np.random.default_rng(seed)
    kx = (rng.standard_normal((L, H, T, d)) * k_scale).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    op = oracle.compress_pool(kx, vx, B32)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    kh, vh = oracle.dequant_pool(op, C32)
    return lay, torch.from_numpy(img).to(device()), kh, vh
