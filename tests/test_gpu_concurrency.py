"""Decodes that overlap each other and a writer on one pool.

PolyKV, Abstract: the pool is written once and read by several agent contexts at the same
time; when the shared context arrives in prefill chunks, each chunk is written once into its
own token range. A prefix decode over tokens [0, n_valid) only reads the 32-token groups that
hold those tokens, so it may overlap an append whose chunk starts at or past n_valid rounded
up to 32. Here two prefix decodes (one per kernel, three calls each) run on their own streams
while a third stream appends the next chunk. Every overlapped result must equal, bit for bit,
the same call made alone before the writer started, the serial results must agree with the
oracle's decode of the prefix, and the pool afterwards must hold the bytes of the chunks
appended one after another.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import B32, C32, DECODE_REL_TOL, device, new_pool, row_rel_err

pytestmark = pytest.mark.gpu

LSE_ABS_TOL = 2e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("n_valid", [512, 500], ids=["aligned", "ragged"])
def test_decodes_overlap_append(n_valid):
    L, H, d, T, A, G = 2, 2, 128, 1024, 6, 4
    _say("concurrency", dict(L=L, H=H, d=d, T=T, A=A, G=G, n_valid=n_valid))
    rng = np.random.default_rng(n_valid)
    k = rng.standard_normal((L, H, T, d)).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    kd, vd = torch.from_numpy(k).to(device()), torch.from_numpy(v).to(device())
    nxt = (n_valid + 31) // 32 * 32          # the writer's chunk starts here

    def append(pool, a, b, stream=None):
        pk.polykv_append_kv(kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), pool, lay, a, stream=stream)

    # the pool the chunks make one after another
    want_pool = new_pool(lay)
    for a, b in ((0, n_valid), (nxt, T), (n_valid, nxt)):
        if b > a:
            append(want_pool, a, b)

    pool = new_pool(lay)
    append(pool, 0, n_valid)
    scale = d ** -0.5
    qs = [torch.from_numpy(rng.standard_normal((L, A, H * G, d)).astype(np.float32)).to(device())
          for _ in range(2)]
    paths = (pk.POLYKV_PATH_MFMA, pk.POLYKV_PATH_VALU)

    def decode(q, path, stream=None):
        o = torch.full_like(q, float("nan"))
        ls = torch.full((L, A, H * G), float("nan"), dtype=torch.float32, device=device())
        return o, ls, (lambda: pk.polykv_attend_shared_prefix(pool, lay, q, o, ls, n_valid, A, G, scale,
                                                              path, stream=stream))

    # each call alone
    ref = []
    for q, path in zip(qs, paths):
        o, ls, run = decode(q, path)
        run()
        ref.append((o, ls))
    torch.cuda.synchronize()

    # the same calls overlapped, with the next chunk written meanwhile
    sw, s1, s2 = (torch.cuda.Stream(device=device()) for _ in range(3))
    jobs = []
    for q, path, st in ((qs[0], paths[0], s1), (qs[1], paths[1], s2)):
        for _ in range(3):
            o, ls, run = decode(q, path, st)
            jobs.append((path, o, ls, run))
    kc = kd[:, :, nxt:T].contiguous()
    vc = vd[:, :, nxt:T].contiguous()
    ev = torch.cuda.Event()
    ev.record()
    for st in (sw, s1, s2):
        st.wait_event(ev)
    pk.polykv_append_kv(kc, vc, pool, lay, nxt, stream=sw)
    for _, _, _, run in jobs:
        run()
    torch.cuda.synchronize()
    if nxt > n_valid:
        append(pool, n_valid, nxt)
        torch.cuda.synchronize()

    for path, o, ls, _ in jobs:
        r_o, r_ls = ref[0] if path == paths[0] else ref[1]
        assert torch.equal(o, r_o), path
        assert torch.equal(ls, r_ls), path
    assert torch.equal(pool, want_pool)

    # the serial results against the oracle's decode of the prefix
    op = oracle.compress_pool(k[..., :n_valid, :], v[..., :n_valid, :], B32)
    kh, vh = oracle.dequant_pool(op, C32)
    for q, (o, ls), path in zip(qs, ref, paths):
        qn = q.cpu().numpy()
        err = row_rel_err(o.cpu().numpy(), oracle.shared_pool_decode(qn, kh, vh, G, scale))
        lerr = float(np.max(np.abs(ls.cpu().numpy() - oracle.shared_pool_lse(qn, kh, G, scale))))
        _say("  path %d: worst row relative error %.3e, max |lse - oracle| %.2e" % (path, err, lerr))
        assert err <= DECODE_REL_TOL
        assert lerr <= LSE_ABS_TOL
