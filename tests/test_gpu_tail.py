"""GPU parity of the per-row log-sum-exp export and of the private-tail merge against the
oracle (softmax attention over the union of pool and tail tokens)."""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle

from gpu_helpers import DECODE_REL_TOL, device, oracle_pool_on_device, row_rel_err

pytestmark = pytest.mark.gpu

PATHS = [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA]
# ln of the softmax normaliser: an error e changes the merge weights by a factor e^e, so
# the bar matches the output's 2e-3
LSE_ABS_TOL = 2e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _rows_supported(path, d, rows):
    return path == pk.POLYKV_PATH_VALU or (d in (64, 128) and rows <= 64)


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("shape", [(2, 2, 128, 600, 15, 4), (1, 3, 64, 95, 5, 1), (2, 1, 256, 130, 2, 3),
                                   (1, 2, 128, 33, 1, 1)], ids=lambda s: "L%dH%dd%dT%dA%dG%d" % s)
def test_lse_export(shape, path):
    L, H, d, T, A, G = shape
    if not _rows_supported(path, d, A * G):
        pytest.skip("matrix-core kernel: head_dim 64/128 only")
    _say("lse", shape, path)
    lay, pool, kh, vh = oracle_pool_on_device(L, H, d, T, seed=T + d)
    rng = np.random.default_rng(d)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    scale = d ** -0.5
    qd = torch.from_numpy(q).to(device())
    out, out_plain = torch.empty_like(qd), torch.empty_like(qd)
    lse = torch.empty((L, A, H * G), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_lse(pool, lay, qd, out, lse, A, G, scale, path)
    pk.polykv_attend_shared_path(pool, lay, qd, out_plain, A, G, scale, path)
    torch.cuda.synchronize()
    assert torch.equal(out, out_plain)  # the export changes nothing else
    want = oracle.shared_pool_lse(q, kh, G, scale)
    err = float(np.max(np.abs(lse.cpu().numpy() - want)))
    _say("  max |lse - oracle| = %.2e" % err)
    assert err <= LSE_ABS_TOL


def _tails(A, L, H, cap, d, lens, seed):
    rng = np.random.default_rng(seed)
    tk = rng.standard_normal((A, L, H, cap, d)).astype(np.float16)
    tv = rng.standard_normal((A, L, H, cap, d)).astype(np.float16)
    return tk, tv, np.asarray(lens, dtype=np.int32)


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("case", [
    # L, H, d, T, A, G, cap, tail lengths per agent
    (2, 2, 128, 600, 3, 4, 64, [0, 1, 64]),
    (1, 2, 128, 100, 2, 5, 130, [65, 130]),      # more rows than one group of four, two chunks
    (1, 3, 64, 95, 4, 1, 64, [63, 0, 7, 64]),
    (1, 1, 256, 40, 2, 2, 100, [100, 3]),
], ids=lambda c: "L%dH%dd%dT%dA%dG%dcap%d" % c[:7])
def test_tail_merge(case, path):
    L, H, d, T, A, G, cap, lens = case
    if not _rows_supported(path, d, A * G):
        pytest.skip("matrix-core kernel: head_dim 64/128 only")
    _say("tail merge", case, path)
    lay, pool, kh, vh = oracle_pool_on_device(L, H, d, T, seed=cap + d)
    rng = np.random.default_rng(T)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    scale = d ** -0.5
    tk, tv, tl = _tails(A, L, H, cap, d, lens, seed=cap)
    qd = torch.from_numpy(q).to(device())
    out = torch.empty_like(qd)
    lse = torch.empty((L, A, H * G), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_lse(pool, lay, qd, out, lse, A, G, scale, path)
    pk.polykv_attend_tail_merge(lay, qd, out, lse, torch.from_numpy(tk).to(device()),
                                torch.from_numpy(tv).to(device()), torch.from_numpy(tl).to(device()),
                                A, G, scale)
    torch.cuda.synchronize()
    want = oracle.pool_and_tail_decode(q, kh, vh, tk, tv, tl, G, scale)
    err = row_rel_err(out.cpu().numpy(), want)
    _say("  worst row error %.2e" % err)
    assert err <= DECODE_REL_TOL
    # the merged lse is the union's
    full_lse = np.zeros((L, A, H * G))
    for l in range(L):
        for a in range(A):
            for j in range(H * G):
                h = j // G
                keys = np.concatenate([kh[l, h], tk[a, l, h, :tl[a]].astype(np.float64)])
                full_lse[l, a, j] = oracle.attention_lse(q[l, a, j:j + 1], keys, scale)[0]
    assert float(np.max(np.abs(lse.cpu().numpy() - full_lse))) <= LSE_ABS_TOL


def test_tail_lengths_are_clamped_and_cap_zero_is_a_no_op():
    L, H, d, T, A, G, cap = 1, 2, 128, 64, 3, 2, 8
    lay, pool, kh, vh = oracle_pool_on_device(L, H, d, T, seed=5)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    scale = d ** -0.5
    qd = torch.from_numpy(q).to(device())
    out = torch.empty_like(qd)
    lse = torch.empty((L, A, H * G), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_lse(pool, lay, qd, out, lse, A, G, scale)
    before, lse_before = out.clone(), lse.clone()
    empty = torch.empty((A, L, H, 0, d), dtype=torch.float16, device=device())
    pk.polykv_attend_tail_merge(lay, qd, out, lse, empty, empty,
                                torch.zeros(A, dtype=torch.int32, device=device()), A, G, scale)
    torch.cuda.synchronize()
    assert torch.equal(out, before) and torch.equal(lse, lse_before)
    tk, tv, _ = _tails(A, L, H, cap, d, [0] * A, seed=9)
    tl = np.array([-5, cap + 100, 3], dtype=np.int32)  # clamped to 0, cap, 3
    pk.polykv_attend_tail_merge(lay, qd, out, lse, torch.from_numpy(tk).to(device()),
                                torch.from_numpy(tv).to(device()), torch.from_numpy(tl).to(device()),
                                A, G, scale)
    torch.cuda.synchronize()
    want = oracle.pool_and_tail_decode(q, kh, vh, tk, tv, np.array([0, cap, 3]), G, scale)
    assert row_rel_err(out.cpu().numpy(), want) <= DECODE_REL_TOL
    assert torch.equal(out[0, 0], before[0, 0])  # the agent with an empty tail is untouched


def test_tail_merge_full_size_sampled():
    """The 4K Llama-3-8B pool (compressed on the GPU) with 15 agents' private tails of up
    to 128 tokens, in the launch configuration the benchmark times: every layer is merged
    on the GPU, three layers are checked against the oracle over pool + tail tokens."""
    from gpu_helpers import C32, layout_for, read_pool, upload_kv
    from workloads import CONFIGS, gen_q_step
    cfg = CONFIGS[3]
    L, H, d, T, A, G, cap = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_tokens, cfg.n_agents, cfg.gqa, 128
    _say("tail merge full size", cfg.name)
    lay = layout_for(cfg)
    k, v = upload_kv(cfg)
    pool = torch.zeros(lay.total_bytes, dtype=torch.uint8, device=device())
    pk.polykv_compress_k(k, pool, lay)
    pk.polykv_compress_v(v, pool, lay)
    del k, v
    lens = [128, 0, 1, 31, 32, 33, 64, 65, 127, 128, 100, 7, 96, 128, 50][:A]
    rng = np.random.default_rng(2026)
    tk = rng.standard_normal((A, L, H, cap, d), dtype=np.float32).astype(np.float16)
    tv = rng.standard_normal((A, L, H, cap, d), dtype=np.float32).astype(np.float16)
    tl = np.asarray(lens, dtype=np.int32)
    qn = gen_q_step(cfg, cfg.decode_steps - 1)
    qd = torch.from_numpy(qn).to(device())
    out = torch.empty_like(qd)
    lse = torch.empty((L, A, H * G), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_lse(pool, lay, qd, out, lse, A, G, cfg.softmax_scale)
    pk.polykv_attend_tail_merge(lay, qd, out, lse, torch.from_numpy(tk).to(device()),
                                torch.from_numpy(tv).to(device()), torch.from_numpy(tl).to(device()),
                                A, G, cfg.softmax_scale)
    torch.cuda.synchronize()
    layers = [0, L // 2, L - 1]
    got = read_pool(pool, lay)
    tiles = [l * H + h for l in layers for h in range(H)]
    sub = {"k_codes": got["k_codes"][tiles].reshape(len(layers), H, T, d),
           "k_scales": got["k_scales"][tiles].reshape(len(layers), H, T, d // 32),
           "v_planes": got["v_planes"][tiles].reshape(len(layers), H, -1, 3, d),
           "v_norms": got["v_norms"][tiles].reshape(len(layers), H, T)}
    kh, vh = oracle.dequant_pool(sub, C32, T)
    want = oracle.pool_and_tail_decode(qn[layers], kh, vh, tk[:, layers], tv[:, layers], tl, G, cfg.softmax_scale)
    err = row_rel_err(out.cpu().numpy()[layers], want)
    _say("  worst row error %.2e" % err)
    assert err <= DECODE_REL_TOL
