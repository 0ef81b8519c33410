"""Chunked (append) compression and prefix decode on the GPU, through the C ABI.

- Appending the chunks of a context, in order or shuffled, into a pool full of other bytes
  gives the same payload as one compress of the whole context (bit-exact; the one-shot
  compress itself is checked against the oracle in test_gpu_compress.py), and the keys
  equal the oracle's append bit for bit.
- An append writes its own tokens only: every other byte of the pool is unchanged, except
  plane bits of tokens at or past the pool's length in the groups it touches, which are 0.
- The prefix decode over the first n_valid tokens of a partly filled pool (the rest of the
  pool filled with 0xFF bytes: NaN scales and norms) matches the oracle's decode over those
  tokens, on both decode kernels.
"""

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import B32, C32, DECODE_REL_TOL, device, new_pool, row_rel_err

pytestmark = pytest.mark.gpu
PATHS = [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA]


def _payload(pool, lay):
    v = pk.pool_views(pool, lay)
    return {k: np.ascontiguousarray(t.cpu().numpy()) for k, t in v.items()}


def _kv(L, H, T, d, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, H, T, d)).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    return k, v


def _append(pool, lay, k, v, a, b, fused=False):
    kc = torch.from_numpy(np.ascontiguousarray(k[..., a:b, :])).to(device())
    vc = torch.from_numpy(np.ascontiguousarray(v[..., a:b, :])).to(device())
    if fused:
        pk.polykv_append_kv(kc, vc, pool, lay, a)
    else:
        pk.polykv_append_k(kc, pool, lay, a)
        pk.polykv_append_v(vc, pool, lay, a)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("order", ["forward", "shuffled"])
@pytest.mark.parametrize("shape", [(2, 2, 128, 600), (1, 3, 64, 95), (1, 2, 256, 70)],
                         ids=lambda s: "L%dH%dd%dT%d" % s)
def test_append_equals_one_shot(shape, order, fused):
    """fused: the chunks go in through polykv_append_kv (keys and values in one launch)."""
    L, H, d, T = shape
    print("append", shape, order, fused, flush=True)
    k, v = _kv(L, H, T, d, seed=T)
    lay = pk.polykv_pool_layout(L, H, d, T)
    one = new_pool(lay, fill=0x00)
    pk.polykv_compress_k(torch.from_numpy(k).to(device()), one, lay)
    pk.polykv_compress_v(torch.from_numpy(v).to(device()), one, lay)
    cuts = sorted({0, 1, 31, 33, 64, T // 2, T - 1, T})
    chunks = list(zip(cuts[:-1], cuts[1:]))
    if order == "shuffled":
        chunks = chunks[::2][::-1] + chunks[1::2]
    app = new_pool(lay, fill=0xA5)
    for a, b in chunks:
        _append(app, lay, k, v, a, b, fused)
    torch.cuda.synchronize()
    got, want = _payload(app, lay), _payload(one, lay)
    for key in want:
        assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), key
    # keys against the oracle's appends
    op = {"k_codes": np.zeros((L, H, T, d), np.int8), "k_scales": np.zeros((L, H, T, d // 32), np.float16),
          "v_codes": np.zeros((L, H, T, d), np.uint8), "v_norms": np.zeros((L, H, T), np.float16)}
    op["v_planes"] = oracle.pack_v_planes(op["v_codes"])
    for a, b in chunks:
        op = oracle.append_pool(op, k[..., a:b, :], v[..., a:b, :], a, B32)
    assert np.array_equal(got["k_codes"].reshape(op["k_codes"].shape), op["k_codes"])
    assert np.array_equal(got["k_scales"].view(np.uint16).reshape(op["k_scales"].shape),
                          op["k_scales"].view(np.uint16))


@pytest.mark.parametrize("shape", [(2, 3, 128, 333), (3, 2, 64, 600), (1, 2, 256, 70), (1, 1, 128, 1),
                                   (32, 8, 128, 256)], ids=lambda s: "L%dH%dd%dT%d" % s)
def test_fused_compress_equals_separate(shape):
    """polykv_compress_kv writes the bytes of polykv_compress_k + polykv_compress_v, over
    the whole allocation (padding included), on layers [1, L) of a pool whose layer 0
    holds other bytes."""
    L, H, d, T = shape
    print("fused compress", shape, flush=True)
    k, v = _kv(L, H, T, d, seed=7 * T + d)
    k[0, 0, 0] = 0.0                                  # a zero key block and value vector
    v[0, 0, 0] = 0.0
    lay = pk.polykv_pool_layout(L, H, d, T)
    lb, lc = (1, L - 1) if L > 1 else (0, 1)
    kk = torch.from_numpy(np.ascontiguousarray(k[lb:lb + lc])).to(device())
    vv = torch.from_numpy(np.ascontiguousarray(v[lb:lb + lc])).to(device())
    sep, fus = new_pool(lay, fill=0x5A), new_pool(lay, fill=0x5A)
    pk.polykv_compress_k(kk, sep, lay, layer_begin=lb, layer_count=lc)
    pk.polykv_compress_v(vv, sep, lay, layer_begin=lb, layer_count=lc)
    pk.polykv_compress_kv(kk, vv, fus, lay, layer_begin=lb, layer_count=lc)
    torch.cuda.synchronize()
    assert torch.equal(sep, fus)


def test_append_writes_only_its_tokens():
    L, H, d, T = 1, 2, 128, 200
    k, v = _kv(L, H, T, d, seed=5)
    lay = pk.polykv_pool_layout(L, H, d, T)
    rng = np.random.default_rng(6)
    img = rng.integers(0, 256, lay.total_bytes, dtype=np.uint8)
    pool = torch.from_numpy(img.copy()).to(device())
    a, b = 45, 180                       # starts and ends inside 32-token groups
    _append(pool, lay, k, v, a, b)
    torch.cuda.synchronize()
    after = pool.cpu().numpy()
    before_views = _payload(torch.from_numpy(img).to(device()), lay)
    after_views = _payload(pool, lay)
    # codes, scales, norms: only tokens [a, b) change
    for key in ("k_codes", "k_scales", "v_norms"):
        x, y = before_views[key], after_views[key]
        keep = np.ones(x.shape[1], bool)
        keep[a:b] = False
        assert np.array_equal(np.ascontiguousarray(x[:, keep]).view(np.uint8),
                              np.ascontiguousarray(y[:, keep]).view(np.uint8)), key
    # plane words: bits of tokens outside [a, b) (all below T here) unchanged
    x = before_views["v_planes"].view(np.uint32)
    y = after_views["v_planes"].view(np.uint32)
    tok = np.arange(x.shape[1] * 32).reshape(x.shape[1], 32)
    outside = (tok < a) | (tok >= b)
    mask = np.zeros(x.shape[1], np.uint32)
    for g in range(x.shape[1]):
        for j in range(32):
            if outside[g, j]:
                mask[g] |= np.uint32(1 << j)
    m = mask[None, :, None, None]
    assert np.array_equal(x & m, y & m)
    # nothing outside the four payload regions moved
    touched = np.zeros(lay.total_bytes, bool)
    for off, stride, nbytes in ((lay.k_codes_off, lay.k_codes_tile_stride, T * d),
                                (lay.k_scales_off, lay.k_scales_tile_stride, T * d // 16),
                                (lay.v_planes_off, lay.v_planes_tile_stride, ((T + 31) // 32) * 3 * d * 4),
                                (lay.v_norms_off, lay.v_norms_tile_stride, 2 * T)):
        for t in range(L * H):
            touched[off + t * stride: off + t * stride + nbytes] = True
    assert np.array_equal(after[~touched], img[~touched])


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("n_valid", [1, 31, 32, 33, 95, 257, 300])
@pytest.mark.parametrize("shape", [(2, 2, 128, 15, 4), (2, 3, 64, 5, 1)], ids=["d128_rows60", "d64_rows5"])
def test_prefix_decode(n_valid, path, shape):
    # d = 64 with at most 16 rows runs the small-workgroup instantiation (three-deep key
    # ring, one value wave per stream)
    L, H, d, A, G = shape
    T = 300
    if path == pk.POLYKV_PATH_MFMA and A * G > 64:
        pytest.skip("rows")
    print("prefix", n_valid, path, flush=True)
    k, v = _kv(L, H, T, d, seed=n_valid)
    lay = pk.polykv_pool_layout(L, H, d, T)
    pool = new_pool(lay, fill=0xFF)      # NaN scales and norms past the prefix
    for a in range(0, n_valid, 100):
        _append(pool, lay, k, v, a, min(a + 100, n_valid))
    q = np.random.default_rng(n_valid + 1).standard_normal((L, A, H * G, d)).astype(np.float32)
    qd = torch.from_numpy(q).to(device())
    out = torch.empty_like(qd)
    lse = torch.empty((L, A, H * G), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_prefix(pool, lay, qd, out, lse, n_valid, A, G, d ** -0.5, path)
    torch.cuda.synchronize()
    op = oracle.compress_pool(k[..., :n_valid, :], v[..., :n_valid, :], B32)
    kh, vh = oracle.dequant_pool(op, C32)
    ref = oracle.shared_pool_decode(q, kh, vh, G, d ** -0.5)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert row_rel_err(got, ref) <= DECODE_REL_TOL
    want_lse = oracle.shared_pool_lse(q, kh, G, d ** -0.5)
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) <= 2e-3


def test_prefix_range_errors():
    L, H, d, T = 1, 1, 128, 40
    lay = pk.polykv_pool_layout(L, H, d, T)
    pool = new_pool(lay)
    q = torch.zeros((1, 1, 1, d), dtype=torch.float32, device=device())
    out = torch.empty_like(q)
    for bad in (0, T + 1):
        with pytest.raises(pk.PolyKVError):
            pk.polykv_attend_shared_prefix(pool, lay, q, out, None, bad, 1, 1, 0.1)


def test_append_full_size_equals_one_shot():
    """The 4K Llama-3-8B context appended as eight 512-token chunks (the benchmark's append
    figure) gives the one-shot pool byte for byte."""
    from gpu_helpers import layout_for, upload_kv
    from workloads import CONFIGS
    cfg = CONFIGS[3]
    print("append full size", flush=True)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    one = new_pool(lay, fill=0x00)
    pk.polykv_compress_k(k, one, lay)
    pk.polykv_compress_v(v, one, lay)
    app = new_pool(lay, fill=0xC3)
    for a in range(0, cfg.n_tokens, 512):
        b = min(a + 512, cfg.n_tokens)
        pk.polykv_append_k(k[:, :, a:b, :].contiguous(), app, lay, a)
        pk.polykv_append_v(v[:, :, a:b, :].contiguous(), app, lay, a)
    torch.cuda.synchronize()
    got, want = pk.pool_views(app, lay), pk.pool_views(one, lay)
    for key in want:
        assert torch.equal(got[key], want[key]), key
    # the benchmark's schedule: one-launch appends, chunks alternating over two streams
    # (512-token chunks touch disjoint 32-token groups, so they may run concurrently)
    chunks = [(a, k[:, :, a:a + 512, :].contiguous(), v[:, :, a:a + 512, :].contiguous())
              for a in range(0, cfg.n_tokens, 512)]
    s1, s2 = torch.cuda.Stream(device=device()), torch.cuda.Stream(device=device())
    torch.cuda.synchronize()
    for rnd in range(3):
        two = new_pool(lay, fill=0x3C + rnd)
        torch.cuda.synchronize()
        for n, (a, kc, vc) in enumerate(chunks):
            pk.polykv_append_kv(kc, vc, two, lay, a, stream=(s1, s2)[(n + rnd) % 2])
        s1.synchronize()
        s2.synchronize()
        got = pk.pool_views(two, lay)
        for key in want:
            assert torch.equal(got[key], want[key]), (rnd, key)
