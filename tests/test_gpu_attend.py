"""GPU parity of the shared-pool decode against the fp64 oracle."""

import functools
import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from workloads import CONFIGS, gen_k_layer, gen_q_step, gen_v_layer

from gpu_helpers import (B32, C32, DECODE_REL_TOL, device, layout_for, new_pool,
                         pool_from_arrays, read_pool, row_rel_err, upload_kv, upload_q)

pytestmark = pytest.mark.gpu

PATHS = [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sample_layers(cfg):
    return sorted({0, cfg.n_layers // 2, cfg.n_layers - 1})


def _sample_steps(cfg):
    """Steps {0, middle, last}: the first is compared over every layer, the others over
    _sample_layers."""
    return sorted({0, cfg.decode_steps // 2, cfg.decode_steps - 1})


@functools.lru_cache(maxsize=5)
def _oracle_pool(cfg):
    """The oracle's own compression of the whole workload, as [tiles][...] arrays."""
    parts = {"k_codes": [], "k_scales": [], "v_codes": [], "v_planes": [], "v_norms": []}
    for l in range(cfg.n_layers):
        p = oracle.compress_pool(gen_k_layer(cfg, l), gen_v_layer(cfg, l), B32)
        for name in parts:
            parts[name].append(p[name])
    return {n: np.concatenate(v) for n, v in parts.items()}  # first axis: tile = l * H + h


def _oracle_decode(cfg, opool, q, layers):
    H = cfg.n_kv_heads
    out = []
    for l in layers:
        sl = slice(l * H, (l + 1) * H)
        kh, vh = oracle.dequant_pool({"k_codes": opool["k_codes"][sl], "k_scales": opool["k_scales"][sl],
                                      "v_codes": opool["v_codes"][sl], "v_norms": opool["v_norms"][sl]}, C32)
        out.append(oracle.shared_pool_decode(q[l:l + 1], kh[None], vh[None], cfg.gqa, cfg.softmax_scale)[0])
    return np.stack(out)


def _supported(path, cfg):
    if path == pk.POLYKV_PATH_MFMA and not _mfma_available(cfg):
        pytest.skip("matrix-core path not available for this shape")


@functools.lru_cache(maxsize=None)
def _mfma_available(cfg):
    lay = layout_for(CONFIGS[0])
    pool = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=device())
    q = torch.zeros(1 * 1 * 2 * 128, dtype=torch.float32, device=device())
    try:
        pk.polykv_attend_shared_path(pool, lay, q, torch.empty_like(q), 1, 1, 0.1, pk.POLYKV_PATH_MFMA)
        return True
    except pk.PolyKVError:
        return False


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_decode_on_oracle_pool(cfg, path):
    """Decode alone: the GPU reads the oracle's pool, so compress differences cannot enter."""
    _supported(path, cfg)
    _say("decode parity on the oracle pool", cfg.name, "path", path)
    lay = layout_for(cfg)
    opool = _oracle_pool(cfg)
    img = pool_from_arrays(lay, opool["k_codes"], opool["k_scales"], opool["v_planes"], opool["v_norms"])
    pool = torch.from_numpy(img).to(device())
    worst = 0.0
    for step in _sample_steps(cfg):
        layers = list(range(cfg.n_layers)) if step == 0 else _sample_layers(cfg)
        qn = gen_q_step(cfg, step)
        q = torch.from_numpy(qn).to(device())
        out = torch.full_like(q, float("nan"))
        pk.polykv_attend_shared_path(pool, lay, q, out, cfg.n_agents, cfg.gqa, cfg.softmax_scale, path)
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        ref = _oracle_decode(cfg, opool, qn, layers)
        err = row_rel_err(got[layers], ref)
        worst = max(worst, err)
        _say("  step %d, %d layers: worst row relative error %.3e" % (step, len(layers), err))
        assert err <= DECODE_REL_TOL, (step, err)
    _say("  worst row relative error %.3e" % worst)


def _value_pool_differences(got, opool, T, d):
    """Per (tile, token): coordinates whose value code differs, and |norm difference|."""
    diff = np.bitwise_xor(got["v_planes"], opool["v_planes"])
    anyp = diff[:, :, 0, :] | diff[:, :, 1, :] | diff[:, :, 2, :]      # [tiles][G][d]
    bits = (anyp[..., None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)  # [tiles][G][d][32]
    nflip = bits.sum(axis=2).reshape(anyp.shape[0], -1)[:, :T]         # [tiles][T]
    dn = np.abs(got["v_norms"].astype(np.float64) - opool["v_norms"].astype(np.float64))
    return nflip, dn


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_end_to_end(cfg):
    """GPU compress then GPU decode, against the oracle's compress then decode, over every
    layer of the workload's last decode step.

    The two pools may legitimately differ (value codes of near-boundary coordinates, norms
    by one fp16 ulp). A row must meet the decode tolerance plus the largest change those
    differences can cause: for each differing token t, weight p_t (the oracle's softmax)
    times (flipped coordinates * n_t / d * widest centroid gap + |dn_t| / n_t * max |v_t|).
    Rows of tiles with identical pools get no allowance.
    """
    _say("end-to-end parity", cfg.name)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    pool = new_pool(lay)
    pk.polykv_compress_k(k, pool, lay)
    pk.polykv_compress_v(v, pool, lay)
    del k, v
    opool = _oracle_pool(cfg)
    got = read_pool(pool, lay)
    assert np.array_equal(got["k_codes"], opool["k_codes"].reshape(got["k_codes"].shape))
    nflip, dn = _value_pool_differences(got, opool, cfg.n_tokens, cfg.head_dim)
    gap = float(np.max(np.diff(C32.astype(np.float64))))
    layers = range(cfg.n_layers)
    step = cfg.decode_steps - 1
    qn = gen_q_step(cfg, step)
    q = torch.from_numpy(qn).to(device())
    out = torch.empty_like(q)
    pk.polykv_attend_shared(pool, lay, q, out, cfg.n_agents, cfg.gqa, cfg.softmax_scale)
    o = out.cpu().numpy().astype(np.float64)
    H, G, A, d = cfg.n_kv_heads, cfg.gqa, cfg.n_agents, cfg.head_dim
    worst_strict, n_allowed = 0.0, 0
    for l in layers:
        for h in range(H):
            t = l * H + h
            kh, vh = oracle.dequant_pool({"k_codes": opool["k_codes"][t], "k_scales": opool["k_scales"][t],
                                          "v_codes": opool["v_codes"][t], "v_norms": opool["v_norms"][t]}, C32)
            rows = qn[l, :, h * G:(h + 1) * G, :].reshape(A * G, d)
            w = oracle.attention_weights(rows, kh, cfg.softmax_scale)
            ref = w @ vh
            n = np.maximum(opool["v_norms"][t].astype(np.float64), got["v_norms"][t].astype(np.float64))
            per_tok = nflip[t] * n / d * gap + dn[t] / np.maximum(n, 1e-30) * np.max(np.abs(vh), axis=-1)
            allow = w @ per_tok
            err = np.max(np.abs(o[l, :, h * G:(h + 1) * G, :].reshape(A * G, d) - ref), axis=-1)
            scale = np.max(np.abs(ref), axis=-1)
            assert np.all(err <= DECODE_REL_TOL * scale + allow * 1.0001), (l, h, np.max(err / scale))
            strict = allow == 0
            n_allowed += int(np.count_nonzero(~strict))
            if np.any(strict):
                worst_strict = max(worst_strict, float(np.max(err[strict] / scale[strict])))
    _say("  rows with an allowance %d; worst error elsewhere %.3e; tokens with a differing value %d"
         % (n_allowed, worst_strict, int(np.count_nonzero(nflip) + np.count_nonzero(dn))))


def _tiny_pool(T, d=128, H=2, L=1, seed=0, v_override=None):
    """The oracle's pool of seeded inputs, uploaded as the library's byte image, so that the
    decode is compared on exactly the pool the oracle reads."""
    rng = np.random.default_rng(seed)
    kx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16) if v_override is None else v_override
    lay = pk.polykv_pool_layout(L, H, d, T)
    op = oracle.compress_pool(kx, vx, B32)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    pool = torch.from_numpy(img).to(device())
    kh, vh = oracle.dequant_pool(op, C32)
    return lay, pool, kh, vh


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 95, 600])
@pytest.mark.parametrize("rows", [(1, 1), (5, 1), (3, 4), (15, 4), (16, 4)])
def test_ragged_tokens_and_rows(T, rows, path):
    _supported(path, CONFIGS[0])
    A, G = rows
    H, d = 2, 128
    lay, pool, kh, vh = _tiny_pool(T, d=d, H=H, seed=T)
    qn = np.random.default_rng(T + 7).standard_normal((1, A, H * G, d)).astype(np.float32)
    q = torch.from_numpy(qn).to(device())
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    assert row_rel_err(out.cpu().numpy(), ref) <= DECODE_REL_TOL
    if T == 1:
        # one token: every row returns that token's reconstructed value
        for h in range(H):
            want = vh[0, h, 0]
            got = out.cpu().numpy()[0, :, h * G:(h + 1) * G, :].reshape(-1, d)
            assert np.max(np.abs(got - want)) <= DECODE_REL_TOL * np.max(np.abs(want))


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("T", [1, 32, 95, 300])
@pytest.mark.parametrize("rows", [(1, 1), (5, 1), (3, 4), (17, 1), (16, 4)])
def test_ragged_tokens_and_rows_head_dim_64(T, rows, path):
    """head_dim 64 has its own matrix-core instantiations (one, two and four 16-row blocks)."""
    _supported(path, CONFIGS[0])
    A, G = rows
    H, d = 3, 64
    lay, pool, kh, vh = _tiny_pool(T, d=d, H=H, seed=T + 64)
    qn = np.random.default_rng(T + 11).standard_normal((1, A, H * G, d)).astype(np.float32)
    q = torch.from_numpy(qn).to(device())
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    assert row_rel_err(out.cpu().numpy(), ref) <= DECODE_REL_TOL


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_head_dims(d, path):
    _supported(path, CONFIGS[0])
    if path == pk.POLYKV_PATH_MFMA and d == 256:
        pytest.skip("the matrix-core path covers head_dim 64 and 128")
    lay, pool, kh, vh = _tiny_pool(300, d=d, H=3, L=2, seed=d)
    A, G = 3, 2
    qn = np.random.default_rng(d).standard_normal((2, A, 3 * G, d)).astype(np.float32)
    q = torch.from_numpy(qn).to(device())
    out = torch.empty_like(q)
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    assert row_rel_err(out.cpu().numpy(), oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)) <= DECODE_REL_TOL


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
def test_zero_query_and_permutation(path):
    _supported(path, CONFIGS[0])
    lay, pool, kh, vh = _tiny_pool(77, seed=5)
    A, G, H, d = 4, 2, 2, 128
    qn = np.random.default_rng(2).standard_normal((1, A, H * G, d)).astype(np.float32)
    qn[0, 1] = 0.0
    q = torch.from_numpy(qn).to(device())
    out = torch.empty_like(q)
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    got = out.cpu().numpy()
    for h in range(H):
        mean = vh[0, h].mean(axis=0)
        for j in range(G):
            assert np.max(np.abs(got[0, 1, h * G + j] - mean)) <= DECODE_REL_TOL * np.max(np.abs(mean))
    perm = [3, 1, 0, 2]
    q2 = torch.from_numpy(np.ascontiguousarray(qn[:, perm])).to(device())
    out2 = torch.empty_like(q2)
    pk.polykv_attend_shared_path(pool, lay, q2, out2, A, G, d ** -0.5, path)
    assert np.array_equal(out2.cpu().numpy(), got[:, perm])


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
def test_determinism_stream_and_layer_range(path):
    cfg = CONFIGS[2]
    _supported(path, cfg)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    pool = new_pool(lay)
    pk.polykv_compress_k(k, pool, lay)
    pk.polykv_compress_v(v, pool, lay)
    q = upload_q(cfg, 3)
    outs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        with torch.cuda.stream(s):
            o = torch.empty_like(q)
            pk.polykv_attend_shared_path(pool, lay, q, o, cfg.n_agents, cfg.gqa, cfg.softmax_scale, path,
                                         stream=s)
            outs.append(o)
    s.synchronize()
    assert torch.equal(outs[0], outs[1])
    # a layer sub-range gives the same rows as the full launch
    lo = torch.empty_like(q[5:9])
    pk.polykv_attend_shared_path(pool, lay, q[5:9].contiguous(), lo, cfg.n_agents, cfg.gqa,
                                 cfg.softmax_scale, path, layer_begin=5, layer_count=4)
    assert torch.equal(lo, outs[0][5:9])


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("shape", [(128, 5, 4), (64, 5, 1)], ids=["d128_rows20", "d64_rows5"])
def test_long_context_single_tile(path, shape):
    """A 100,000-token tile (far past the pages' 7,194): offsets, chunk counts and the
    streams' merge at a length no workload reaches; the pool is compressed on the GPU and
    compared with the oracle's compress (keys bit-exact) before the decode is checked.
    d = 64 with five rows runs the small-workgroup decode (three-deep key ring)."""
    _supported(path, CONFIGS[0])
    d, A, G = shape
    L, H, T = 1, 1, 100_000
    rng = np.random.default_rng(99)
    k = rng.standard_normal((L, H, T, d)).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    pool = new_pool(lay)
    pk.polykv_compress_k(torch.from_numpy(k).to(device()), pool, lay)
    pk.polykv_compress_v(torch.from_numpy(v).to(device()), pool, lay)
    qn = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    q = torch.from_numpy(qn).to(device())
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    torch.cuda.synchronize()
    op = oracle.compress_pool(k, v, B32)
    got = read_pool(pool, lay)
    assert np.array_equal(got["k_codes"].reshape(op["k_codes"].shape), op["k_codes"])
    # decode on the GPU's own pool (its value codes may differ from the oracle's only in
    # the permitted boundary cases), reconstructed by the oracle
    gp = {"k_codes": got["k_codes"].reshape(L, H, T, d), "k_scales": got["k_scales"].reshape(L, H, T, d // 32),
          "v_planes": got["v_planes"].reshape(L, H, -1, 3, d), "v_norms": got["v_norms"].reshape(L, H, T)}
    kh, vh = oracle.dequant_pool(gp, C32, T)
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    assert row_rel_err(out.cpu().numpy(), ref) <= DECODE_REL_TOL
