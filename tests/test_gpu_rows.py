"""Decodes with more query rows per pool tile than one launch serves.

PolyKV, Abstract: any number of agent contexts read the one pool. A tile's rows (agents x
query heads of its KV head, agent-major) are served in passes of POLYKV_ROWS_PER_PASS rows,
one launch per pass, each streaming the whole pool. Checked against the oracle row by row on
both kernels, with the lse export; the rows of each pass must also equal, bit for bit, a
call that holds only those rows (the same kernel on the same data), which pins the mapping
of a pass's rows to agents and query heads.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import DECODE_REL_TOL, device, oracle_pool_on_device, row_rel_err

pytestmark = pytest.mark.gpu

PATHS = [pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA]
LSE_ABS_TOL = 2e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("path", PATHS, ids=["valu", "mfma"])
@pytest.mark.parametrize("shape", [(1, 2, 128, 333, 17, 4),    # 68 rows: 64 + 4
                                   (2, 2, 64, 150, 33, 4),     # 132 rows: 64 + 64 + 4
                                   (1, 1, 128, 95, 1, 130),    # one agent, 130 query heads per KV head
                                   (1, 3, 64, 64, 200, 1),     # 200 agents, plain attention
                                   (1, 2, 128, 40, 16, 4)],    # exactly one full pass
                         ids=lambda s: "L%dH%dd%dT%dA%dG%d" % s)
def test_many_rows(shape, path):
    L, H, d, T, A, G = shape
    _say("rows", shape, path)
    assert pk.polykv_attend_path(pk.polykv_pool_layout(L, H, d, T), A, G) == pk.POLYKV_PATH_MFMA
    lay, pool, kh, vh = oracle_pool_on_device(L, H, d, T, seed=A * G + d)
    rng = np.random.default_rng(A + G)
    q = rng.standard_normal((L, A, H * G, d)).astype(np.float32)
    scale = d ** -0.5
    qd = torch.from_numpy(q).to(device())
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((L, A, H * G), float("nan"), dtype=torch.float32, device=device())
    pk.polykv_attend_shared_lse(pool, lay, qd, out, lse, A, G, scale, path)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any() and not torch.isnan(lse).any().item()
    err = row_rel_err(got, oracle.shared_pool_decode(q, kh, vh, G, scale))
    lerr = float(np.max(np.abs(lse.cpu().numpy() - oracle.shared_pool_lse(q, kh, G, scale))))
    _say("  worst row relative error %.3e, max |lse - oracle| %.2e" % (err, lerr))
    assert err <= DECODE_REL_TOL
    assert lerr <= LSE_ABS_TOL
    # a pass made of whole agents equals the call holding just those agents
    if G <= pk.POLYKV_ROWS_PER_PASS and pk.POLYKV_ROWS_PER_PASS % G == 0:
        per = pk.POLYKV_ROWS_PER_PASS // G
        for a0 in range(0, A, per):
            a1 = min(A, a0 + per)
            qs = qd[:, a0:a1].contiguous()
            o1 = torch.empty_like(qs)
            pk.polykv_attend_shared_path(pool, lay, qs, o1, a1 - a0, G, scale, path)
            torch.cuda.synchronize()
            assert torch.equal(o1, out[:, a0:a1]), (a0, a1)
