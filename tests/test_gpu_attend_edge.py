"""GPU decode parity at the softmax-stability edge, against the fp64 oracle.

PolyKV, Abstract: keys stay at int8 so that the softmax keeps its stability. These cases
put the weights where a low-precision probability operand loses them:
- one dominant (sink) token beside thousands of identical or nearly identical keys whose
  scores lie 12 to 18 log2 units below it, so that most of a row's softmax mass sits in
  tokens with tiny individual weights;
- the same dominant token placed late, so that it raises every running maximum after most
  of the mass has been accumulated, and one spike in the last chunk of every stream;
- peaked queries (the Llama-3-8B 4K pool's queries times 4, 8 and 16).
The pool is the oracle's own compression of the inputs, so only the decode is compared.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from workloads import CONFIGS, gen_k_layer, gen_q_step, gen_v_layer

from gpu_helpers import B32, C32, DECODE_REL_TOL, device, pool_from_arrays, row_rel_err

pytestmark = pytest.mark.gpu

PATHS = [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA]
LOG2E = 1.4426950408889634
CHUNK, STREAMS = 32, 4


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _upload_oracle_pool(kx, vx):
    L, H, T, d = kx.shape
    lay = pk.polykv_pool_layout(L, H, d, T)
    op = oracle.compress_pool(kx, vx, B32)
    tiles = L * H
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    kh, vh = oracle.dequant_pool(op, C32)
    return lay, torch.from_numpy(img).to(device()), kh, vh


def _decode_and_compare(lay, pool, kh, vh, qn, A, G, path):
    d = qn.shape[-1]
    q = torch.from_numpy(np.ascontiguousarray(qn, dtype=np.float32)).to(device())
    out = torch.full_like(q, float("nan"))
    pk.polykv_attend_shared_path(pool, lay, q, out, A, G, d ** -0.5, path)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle.shared_pool_decode(qn, kh, vh, G, d ** -0.5)
    return row_rel_err(got, ref)


def _sink_case(d, A, G, T, bulk, sink_positions, seed):
    """Keys along one direction e: sink tokens at a * e, every other token at b * e (plus a
    small per-token jitter for near-identical keys). Each query row is c_r * e plus a small
    orthogonal part, with c_r chosen so that the sink's score exceeds the bulk's by
    gap_r log2 units, gap_r spread over [12, 18]."""
    rng = np.random.default_rng(seed)
    H, L = 2, 1
    R = A * G
    e = rng.standard_normal(d)
    e /= np.linalg.norm(e)
    a, b = 3.0, 0.75
    kx = np.empty((L, H, T, d))
    kx[:] = b * e
    if bulk == "near":
        kx += 0.01 * rng.standard_normal((L, H, T, d))
    for t in sink_positions:
        kx[:, :, t, :] = a * e
    kx = kx.astype(np.float16)
    vx = rng.standard_normal((L, H, T, d)).astype(np.float16)
    gaps = 12.0 + 6.0 * (np.arange(R) % 7) / 6.0
    sigma = d ** -0.5
    c = gaps / (LOG2E * sigma * (a - b))
    qn = np.empty((L, A, H * G, d), dtype=np.float32)
    for h in range(H):
        for r in range(R):
            ag, j = divmod(r, G)
            qv = c[r] * e + 0.02 * rng.standard_normal(d)
            qn[0, ag, h * G + j] = qv
    return kx, vx, qn


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [(15, 4), (5, 1)], ids=["rows60", "rows5"])
@pytest.mark.parametrize("bulk", ["identical", "near"])
def test_sink_above_identical_bulk(path, d, rows, bulk):
    """A sink at t = 0 and 4,095 identical (or near-identical) keys 12-18 log2 units below."""
    A, G = rows
    T = 4096
    kx, vx, qn = _sink_case(d, A, G, T, bulk, [0], seed=d + 7 * A)
    lay, pool, kh, vh = _upload_oracle_pool(kx, vx)
    err = _decode_and_compare(lay, pool, kh, vh, qn, A, G, path)
    _say("sink at t=0, bulk %s, d=%d, rows %d, path %d: worst row error %.3e" % (bulk, d, A * G, path, err))
    assert err <= DECODE_REL_TOL, err


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("where", ["mid", "every_stream_last"])
def test_late_spikes_raise_the_maximum(path, d, where):
    """Spikes after most of the mass has been accumulated: one sink in the middle of the
    context, or one in the last chunk of each of the four token streams (chunks of 32
    tokens dealt to the streams in turn), so that every stream raises its maximum late."""
    A, G = 15, 4
    T = 4096 - 37  # a ragged last chunk
    nc = (T + CHUNK - 1) // CHUNK
    if where == "mid":
        pos = [T // 2 + 5]
    else:
        pos = [min(T - 1, c * CHUNK + 17) for c in range(nc - STREAMS, nc)]
    kx, vx, qn = _sink_case(d, A, G, T, "near", pos, seed=d + len(pos))
    lay, pool, kh, vh = _upload_oracle_pool(kx, vx)
    err = _decode_and_compare(lay, pool, kh, vh, qn, A, G, path)
    _say("late spikes %s, d=%d, path %d: worst row error %.3e" % (where, d, path, err))
    assert err <= DECODE_REL_TOL, err


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("factor", [4.0, 8.0, 16.0])
def test_peaked_queries_on_llama_pool(path, factor):
    """The Llama-3-8B 4K workload's keys, values and step-0 queries (two of its layers),
    the queries multiplied by 4, 8 or 16: nearly one-hot softmax rows, large score ranges
    and many raises of the running maxima."""
    cfg = CONFIGS[3]
    layers = [0, 1]
    kx = np.stack([gen_k_layer(cfg, l) for l in layers])
    vx = np.stack([gen_v_layer(cfg, l) for l in layers])
    lay, pool, kh, vh = _upload_oracle_pool(kx, vx)
    qn = gen_q_step(cfg, 0)[layers] * np.float32(factor)
    err = _decode_and_compare(lay, pool, kh, vh, qn, cfg.n_agents, cfg.gqa, path)
    _say("peaked queries x%g, path %d: worst row error %.3e" % (factor, path, err))
    assert err <= DECODE_REL_TOL, err
