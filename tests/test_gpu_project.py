"""Fused K/V projection + compression on the GPU, through the C ABI.

- The plain projection (polykv_project_kv) against the oracle's fp64 projection: the GPU
  sums exact fp16 x fp16 products in fp32, so its sum y lies within
  E = hidden * 2^-24 * sum_k |x_k w_k| of the exact x (any order of fp32 additions, with a
  little slack for the order-dependent gamma term); rounding to nearest is monotone, so the
  fp16 result lies between RNE16(x - E) and RNE16(x + E).
- The fused kernel (polykv_project_compress) writes exactly the pool bytes of the plain
  projection followed by polykv_append_k/v (the same accumulators are rounded to fp16 and
  the same codecs run on them), into a garbage-filled pool, for chunks that start at a
  multiple of 32 and have ragged lengths; every byte outside the chunk is left alone.
"""

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import device, new_pool

pytestmark = pytest.mark.gpu


def _inputs(n_tok, hidden, H, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_tok, hidden)).astype(np.float16)
    wk = (rng.standard_normal((H * d, hidden)) / np.sqrt(hidden)).astype(np.float16)
    wv = (rng.standard_normal((H * d, hidden)) / np.sqrt(hidden)).astype(np.float16)
    return x, wk, wv


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def check_projection(got16, x, w, H, d):
    exact = oracle.project_fp64(x, w, H, d)
    absum = oracle.project_fp64(np.abs(x.astype(np.float64)), np.abs(w.astype(np.float64)), H, d)
    E = x.shape[1] * 2.0 ** -24 * absum * 1.01 + 1e-30
    lo = (exact - E).astype(np.float16).astype(np.float64)
    hi = (exact + E).astype(np.float16).astype(np.float64)
    g = np.asarray(got16, dtype=np.float64).reshape(exact.shape)
    assert np.all((lo <= g) & (g <= hi)), "projection outside the fp32 summation bound"
    return int(np.sum(g != exact.astype(np.float16).astype(np.float64)))


@pytest.mark.parametrize("shape", [(100, 64, 3, 64), (300, 256, 2, 128), (128, 512, 1, 128), (33, 128, 4, 64)],
                         ids=lambda s: "n%dK%dH%dd%d" % s)
def test_plain_projection(shape):
    n, hidden, H, d = shape
    print("project", shape, flush=True)
    x, wk, wv = _inputs(n, hidden, H, d, seed=n + hidden)
    k = torch.full((H, n, d), float("nan"), dtype=torch.float16, device=device())
    v = torch.full_like(k, float("nan"))
    pk.polykv_project_kv(_dev(x), _dev(wk), _dev(wv), k, v, H, d)
    torch.cuda.synchronize()
    nk = check_projection(k.cpu().numpy(), x, wk, H, d)
    nv = check_projection(v.cpu().numpy(), x, wv, H, d)
    assert nk + nv <= 0.01 * 2 * k.numel()
    # K only
    k2 = torch.empty_like(k)
    pk.polykv_project_kv(_dev(x), _dev(wk), None, k2, None, H, d)
    torch.cuda.synchronize()
    assert torch.equal(k2, k)


@pytest.mark.parametrize("case", [(2, 3, 64, 300, 256, 0, 300, 1), (2, 2, 128, 600, 128, 64, 100, 0),
                                  (1, 1, 128, 256, 64, 128, 128, 0), (1, 2, 64, 97, 512, 32, 65, 0)],
                         ids=lambda c: "L%dH%dd%dT%dK%d_at%d_n%d_l%d" % c)
def test_fused_equals_projection_then_append(case):
    L, H, d, T, hidden, tb, n, layer = case
    print("fused", case, flush=True)
    x, wk, wv = _inputs(n, hidden, H, d, seed=T + n)
    lay = pk.polykv_pool_layout(L, H, d, T)
    rng = np.random.default_rng(7)
    img = rng.integers(0, 256, lay.total_bytes, dtype=np.uint8)
    fused = torch.from_numpy(img.copy()).to(device())
    plain = torch.from_numpy(img.copy()).to(device())
    xd, wkd, wvd = _dev(x), _dev(wk), _dev(wv)
    pk.polykv_project_compress(xd, wkd, wvd, fused, lay, layer, tb)
    k = torch.empty((H, n, d), dtype=torch.float16, device=device())
    v = torch.empty_like(k)
    pk.polykv_project_kv(xd, wkd, wvd, k, v, H, d)
    pk.polykv_append_k(k, plain, lay, tb, layer_begin=layer, layer_count=1)
    pk.polykv_append_v(v, plain, lay, tb, layer_begin=layer, layer_count=1)
    torch.cuda.synchronize()
    a, b = fused.cpu().numpy(), plain.cpu().numpy()
    assert np.array_equal(a, b), "fused pool differs from projection + append at %d bytes" % int(np.sum(a != b))
    assert not np.array_equal(a, img)


def test_fused_rejects_unaligned_chunks_and_bad_shapes():
    lay = pk.polykv_pool_layout(1, 1, 128, 128)
    pool = new_pool(lay)
    x = torch.zeros((40, 64), dtype=torch.float16, device=device())
    w = torch.zeros((128, 64), dtype=torch.float16, device=device())
    with pytest.raises(pk.PolyKVError):
        pk.polykv_project_compress(x, w, w, pool, lay, 0, 16)       # token_begin % 32 != 0
    with pytest.raises(pk.PolyKVError):
        pk.polykv_project_compress(x, w, w, pool, lay, 0, 96)       # past the capacity
    x2 = torch.zeros((40, 48), dtype=torch.float16, device=device())
    w2 = torch.zeros((128, 48), dtype=torch.float16, device=device())
    with pytest.raises(pk.PolyKVError):
        pk.polykv_project_compress(x2, w2, w2, pool, lay, 0, 0)     # hidden not a multiple of 64


def test_full_size_llama_layer():
    """One Llama-3-8B layer at 4,096 tokens (hidden 4096, 8 KV heads of 128), the shape the
    benchmark times: sampled token rows of the plain projection against the oracle, and the
    whole fused pool against projection + append."""
    n, hidden, H, d = 4096, 4096, 8, 128
    print("project full size", flush=True)
    x, wk, wv = _inputs(n, hidden, H, d, seed=3)
    lay = pk.polykv_pool_layout(1, H, d, n)
    xd, wkd, wvd = _dev(x), _dev(wk), _dev(wv)
    k = torch.empty((H, n, d), dtype=torch.float16, device=device())
    v = torch.empty_like(k)
    pk.polykv_project_kv(xd, wkd, wvd, k, v, H, d)
    fused = new_pool(lay, fill=0x5A)
    plain = new_pool(lay, fill=0x5A)
    pk.polykv_project_compress(xd, wkd, wvd, fused, lay, 0, 0)
    pk.polykv_append_k(k, plain, lay, 0)
    pk.polykv_append_v(v, plain, lay, 0)
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    rows = np.r_[0:8, 1000:1008, 2047:2056, 4088:4096]
    kg = k.cpu().numpy()[:, rows]
    vg = v.cpu().numpy()[:, rows]
    check_projection(kg, x[rows], wk, H, d)
    check_projection(vg, x[rows], wv, H, d)


# ---- the fused pool against the oracle ------------------------------------------------

def _exact_inputs(n_tok, hidden, H, d, seed):
    """Operands whose fp32 accumulation is exact in any order: x holds integers in [-8, 8]
    and the weights integers in [-64, 64] times 2^-10, so every product and every partial
    sum is a multiple of 2^-10 below 2^11 in magnitude (hidden <= 4096): at most 21
    significant bits. The GPU's fp32 sum is then the exact sum, and its one rounding to
    fp16 is the oracle's RNE16 of the fp64 product."""
    assert hidden <= 4096
    rng = np.random.default_rng(seed)
    x = rng.integers(-8, 9, (n_tok, hidden)).astype(np.float16)
    wk = (rng.integers(-64, 65, (H * d, hidden)) * 2.0 ** -10).astype(np.float16)
    wv = (rng.integers(-64, 65, (H * d, hidden)) * 2.0 ** -10).astype(np.float16)
    return x, wk, wv


def _check_chunk_against_oracle(pool, lay, layer, tb, x, wk, wv):
    """The chunk's tokens of one layer in the GPU pool against the oracle's compression of
    the oracle's fp16 projection: key codes and scales bit-exact, value codes per the
    boundary rule, norms within one fp16 ulp."""
    from gpu_helpers import B32, V_BOUNDARY_WINDOW, V_MISMATCH_FRACTION, check_norms, read_pool
    s = lay.shape
    H, d = s.n_kv_heads, s.head_dim
    n = x.shape[0]
    k16 = oracle.project_fp16(x, wk, H, d)[None]      # [1][H][n][d]
    v16 = oracle.project_fp16(x, wv, H, d)[None]
    want = oracle.compress_pool(k16, v16, B32)
    got = read_pool(pool, lay)
    tiles = slice(layer * H, (layer + 1) * H)
    toks = slice(tb, tb + n)
    assert np.array_equal(got["k_codes"][tiles][:, toks], want["k_codes"][0])
    assert np.array_equal(got["k_scales"][tiles][:, toks].view(np.uint16), want["k_scales"][0].view(np.uint16))
    codes = oracle.unpack_v_planes(got["v_planes"][tiles], s.n_tokens)[:, toks]   # [H][n][d]
    diff = np.argwhere(codes != want["v_codes"][0])
    b = B32.astype(np.float64)
    for h, t, i in diff:
        y = oracle.rotated_coordinates(v16[0, h, t])[i]
        assert np.min(np.abs(y - b)) < V_BOUNDARY_WINDOW, (h, t, i, y)
    assert len(diff) <= V_MISMATCH_FRACTION * codes.size, len(diff)
    check_norms(got["v_norms"][tiles][:, toks], want["v_norms"][0])
    return len(diff)


@pytest.mark.parametrize("case", [(2, 3, 64, 300, 256, 0, 300, 1), (2, 2, 128, 600, 128, 64, 100, 0),
                                  (1, 1, 128, 256, 64, 128, 128, 0), (1, 2, 64, 97, 512, 32, 65, 0)],
                         ids=lambda c: "L%dH%dd%dT%dK%d_at%d_n%d_l%d" % c)
def test_fused_pool_equals_oracle(case):
    """polykv_project_compress against oracle.compress_pool(oracle.project_fp16(x, w)) on
    operands whose fp16 projection is exact, in a garbage-filled pool."""
    L, H, d, T, hidden, tb, n, layer = case
    print("fused vs oracle", case, flush=True)
    x, wk, wv = _exact_inputs(n, hidden, H, d, seed=T + n + 1)
    lay = pk.polykv_pool_layout(L, H, d, T)
    img = np.random.default_rng(11).integers(0, 256, lay.total_bytes, dtype=np.uint8)
    pool = torch.from_numpy(img).to(device())
    pk.polykv_project_compress(_dev(x), _dev(wk), _dev(wv), pool, lay, layer, tb)
    torch.cuda.synchronize()
    _check_chunk_against_oracle(pool, lay, layer, tb, x, wk, wv)


def test_fused_llama_layer_against_oracle_and_decode():
    """One Llama-3-8B layer at 4,096 tokens (hidden 4096, 8 KV heads of 128) through the fused
    kernel: the pool against the oracle's projection + compression, then the 15-agent GQA-4
    decode of that pool against the oracle's attention over the same pool."""
    from gpu_helpers import C32, DECODE_REL_TOL, read_pool, row_rel_err
    n, hidden, H, d, A, G = 4096, 4096, 8, 128, 15, 4
    print("fused full size vs oracle", flush=True)
    x, wk, wv = _exact_inputs(n, hidden, H, d, seed=5)
    lay = pk.polykv_pool_layout(1, H, d, n)
    pool = new_pool(lay, fill=0x3C)
    pk.polykv_project_compress(_dev(x), _dev(wk), _dev(wv), pool, lay, 0, 0)
    torch.cuda.synchronize()
    nd = _check_chunk_against_oracle(pool, lay, 0, 0, x, wk, wv)
    print("  value codes differing from the oracle: %d" % nd, flush=True)
    got = read_pool(pool, lay)
    gp = {"k_codes": got["k_codes"].reshape(1, H, n, d), "k_scales": got["k_scales"].reshape(1, H, n, d // 32),
          "v_planes": got["v_planes"].reshape(1, H, -1, 3, d), "v_norms": got["v_norms"].reshape(1, H, n)}
    kh, vh = oracle.dequant_pool(gp, C32, n)
    qn = np.random.default_rng(6).standard_normal((1, A, H * G, d)).astype(np.float32)
    q = _dev(qn)
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared(pool, lay, q, out, A, G, d ** -0.5)
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    err = row_rel_err(out.cpu().numpy(), ref)
    print("  decode worst row error %.3e" % err, flush=True)
    assert err <= DECODE_REL_TOL
