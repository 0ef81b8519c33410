"""A seeded sweep over shape combinations that the hand-picked cases do not cross.

PolyKV, Abstract: the pool is written once (q8_0 keys, 3-bit TurboQuant values) and read
by any number of agents. Each case draws layers, KV heads, head_dim, a ragged token count,
an agent count and a GQA group (rows up to 160, so some decodes take several passes), a
key magnitude and a prefix length, then checks:
- the one-launch key + value compress of the whole context against the oracle (key bytes
  exact, value codes by the value rule, norms within one fp16 ulp);
- the prefix decode with the lse export, on both kernels, against the oracle's decode of
  the same prefix of the oracle's pool.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import (B32, C32, DECODE_REL_TOL, check_norms, check_v_codes, device, new_pool,
                         pool_from_arrays, read_pool, row_rel_err)

pytestmark = pytest.mark.gpu

LSE_ABS_TOL = 2e-3


def _cases(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        T = int(rng.integers(1, 701))
        out.append(dict(L=int(rng.integers(1, 4)), H=int(rng.integers(1, 5)), d=d, T=T,
                        A=int(rng.integers(1, 21)), G=int(rng.choice([1, 2, 4, 8])),
                        n_valid=int(rng.integers(1, T + 1)), k_scale=float(rng.choice([1e-3, 1.0, 50.0])),
                        seed=int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases()


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("case", CASES, ids=["c%02d" % i for i in range(len(CASES))])
def test_sweep(case):
    L, H, d, T, A, G = (case[k] for k in ("L", "H", "d", "T", "A", "G"))
    n_valid = case["n_valid"]
    _say("sweep", case)
    rng = np.random.default_rng(case["seed"])
    k = (rng.standard_normal((L, H, T, d)) * case["k_scale"]).astype(np.float16)
    v = rng.standard_normal((L, H, T, d)).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    tiles = L * H

    # compress on the GPU against the oracle's pool
    pool = new_pool(lay)
    pk.polykv_compress_kv(torch.from_numpy(k).to(device()), torch.from_numpy(v).to(device()), pool, lay)
    torch.cuda.synchronize()
    got = read_pool(pool, lay)
    op = oracle.compress_pool(k, v, B32)
    assert np.array_equal(got["k_codes"], op["k_codes"].reshape(tiles, T, d))
    assert np.array_equal(got["k_scales"].view(np.uint16),
                          op["k_scales"].reshape(tiles, T, d // 32).astype(np.float16).view(np.uint16))
    check_v_codes(got["v_planes"], op["v_planes"].reshape(tiles, -1, 3, d), v.reshape(tiles, T, d), T)
    check_norms(got["v_norms"], op["v_norms"].reshape(tiles, T))

    # prefix decode of the oracle's own pool, both kernels
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    opool = torch.from_numpy(img).to(device())
    pre = oracle.compress_pool(k[..., :n_valid, :], v[..., :n_valid, :], B32)
    kh, vh = oracle.dequant_pool(pre, C32)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    scale = d ** -0.5
    ref = oracle.shared_pool_decode(q, kh, vh, G, scale)
    ref_lse = oracle.shared_pool_lse(q, kh, G, scale)
    qd = torch.from_numpy(q).to(device())
    for path in (pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA):
        if path == pk.POLYKV_PATH_MFMA and d == 256:
            continue  # the matrix-core kernel covers head_dim 64 and 128
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((L, A, H * G), float("nan"), dtype=torch.float32, device=device())
        pk.polykv_attend_shared_prefix(opool, lay, qd, out, lse, n_valid, A, G, scale, path)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all()
        err = row_rel_err(o, ref)
        lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
        _say("  path %d: worst row relative error %.3e, max |lse - oracle| %.2e" % (path, err, lerr))
        assert err <= DECODE_REL_TOL
        assert lerr <= LSE_ABS_TOL
