"""A seeded sweep over value distributions the workloads do not reach, every result against
the oracle.

PolyKV, Abstract: keys are kept at int8 (q8_0) for a stable softmax, values are TurboQuant
3-bit codes, and each agent continues on its own after the shared pool. Each case draws a
shape and then:
- keys whose 32-entry blocks span six orders of magnitude inside one token (so the block
  scales of a token differ by up to 1e6), values whose norms span six orders across tokens,
  and queries scaled by 1e-3 .. 10;
- compresses the context in random 32-aligned chunks on two streams (the pool must equal
  the oracle's bytes for the keys and follow the value rule);
- dequantises the pool to fp16 (keys exact, values within the fp32 transform bound);
- decodes on both kernels with the lse export, then merges random private tails (lengths
  0 .. cap) into that result.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
import oracle
from gpu_helpers import (B32, C32, DECODE_REL_TOL, check_norms, check_v_codes, device, new_pool,
                         pool_from_arrays, read_pool, row_rel_err)
from test_gpu_dequant import check_v

pytestmark = pytest.mark.gpu

LSE_REL_TOL = 2e-5   # lse is compared relative to max(1, |lse|)


def _cases(n=12, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(33, 600))
        out.append(dict(L=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), d=d, T=T,
                        A=int(rng.integers(1, 18)), G=int(rng.choice([1, 2, 4])),
                        q_scale=float(rng.choice([1e-3, 0.3, 1.0, 3.0, 10.0])),
                        cap=int(rng.choice([0, 1, 64, 100])), seed=int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases()


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("case", CASES, ids=["s%02d" % i for i in range(len(CASES))])
def test_stress(case):
    L, H, d, T, A, G, cap = (case[k] for k in ("L", "H", "d", "T", "A", "G", "cap"))
    _say("stress", case)
    rng = np.random.default_rng(case["seed"])
    # keys: every 32-entry block of every token gets its own magnitude in [1e-3, 1e3]
    kmag = 10.0 ** rng.uniform(-3, 3, size=(L, H, T, d // 32, 1))
    k = (rng.standard_normal((L, H, T, d // 32, 32)) * kmag).reshape(L, H, T, d).astype(np.float16)
    # values: per-token norms spread over [1e-3, 1e3]
    vmag = 10.0 ** rng.uniform(-3, 3, size=(L, H, T, 1))
    v = (rng.standard_normal((L, H, T, d)) * vmag).astype(np.float16)
    lay = pk.polykv_pool_layout(L, H, d, T)
    tiles = L * H
    op = oracle.compress_pool(k, v, B32)

    # chunked append on two streams (32-aligned boundaries)
    cuts = sorted({0, T} | {32 * int(c) for c in rng.integers(1, (T + 31) // 32, size=3)})
    pool = new_pool(lay, fill=0x5A)
    kd, vd = torch.from_numpy(k).to(device()), torch.from_numpy(v).to(device())
    s2 = torch.cuda.Stream(device=device())
    ev = torch.cuda.Event()
    ev.record()
    s2.wait_event(ev)
    for n, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        st = s2 if n % 2 else torch.cuda.current_stream()
        pk.polykv_append_kv(kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), pool, lay, a, stream=st)
    torch.cuda.synchronize()
    got = read_pool(pool, lay)
    assert np.array_equal(got["k_codes"], op["k_codes"].reshape(tiles, T, d))
    assert np.array_equal(got["k_scales"].view(np.uint16),
                          op["k_scales"].reshape(tiles, T, d // 32).astype(np.float16).view(np.uint16))
    check_v_codes(got["v_planes"], op["v_planes"].reshape(tiles, -1, 3, d), v.reshape(tiles, T, d), T)
    check_norms(got["v_norms"], op["v_norms"].reshape(tiles, T))

    # decode, dequantisation and tails on the oracle's own pool
    img = pool_from_arrays(lay, op["k_codes"].reshape(tiles, T, d), op["k_scales"].reshape(tiles, T, d // 32),
                           op["v_planes"].reshape(tiles, -1, 3, d), op["v_norms"].reshape(tiles, T))
    opool = torch.from_numpy(img).to(device())
    k16 = torch.empty((L, H, T, d), dtype=torch.float16, device=device())
    v16 = torch.empty_like(k16)
    pk.polykv_dequant_k(opool, lay, k16)
    pk.polykv_dequant_v(opool, lay, v16)
    torch.cuda.synchronize()
    want_k, _ = oracle.dequant_fp16(op, C32, T)
    assert np.array_equal(k16.cpu().numpy().view(np.uint16), want_k.view(np.uint16))
    check_v(v16.cpu().numpy(), op, T)   # every differing value within the fp32 transform bound

    kh, vh = oracle.dequant_pool(op, C32)
    q = (rng.standard_normal((L, A, H * G, d)) * case["q_scale"]).astype(np.float32)
    scale = d ** -0.5
    ref = oracle.shared_pool_decode(q, kh, vh, G, scale)
    ref_lse = oracle.shared_pool_lse(q, kh, G, scale)
    # tails drawn like the pool (per-block key magnitudes, per-token value norms), so that
    # they carry real weight in the merged softmax
    c1 = max(cap, 1)
    tkm = 10.0 ** rng.uniform(-3, 3, size=(A, L, H, c1, d // 32, 1))
    tk = (rng.standard_normal((A, L, H, c1, d // 32, 32)) * tkm).reshape(A, L, H, c1, d).astype(np.float16)[:, :, :, :cap]
    tvm = 10.0 ** rng.uniform(-3, 3, size=(A, L, H, c1, 1))
    tv = (rng.standard_normal((A, L, H, c1, d)) * tvm).astype(np.float16)[:, :, :, :cap]
    tl = rng.integers(0, cap + 1, size=A).astype(np.int32)
    tk, tv = np.ascontiguousarray(tk), np.ascontiguousarray(tv)
    want_merged = oracle.pool_and_tail_decode(q, kh, vh, tk, tv, tl, G, scale)
    # where the oracle's tails change the result, the merge must change it too
    tails_matter = tl.max() > 0 and row_rel_err(want_merged, ref) > 1e-2
    qd = torch.from_numpy(q).to(device())
    for path in (pk.POLYKV_PATH_VALU, pk.POLYKV_PATH_MFMA):
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((L, A, H * G), float("nan"), dtype=torch.float32, device=device())
        pk.polykv_attend_shared_lse(opool, lay, qd, out, lse, A, G, scale, path)
        torch.cuda.synchronize()
        o, ls = out.cpu().numpy(), lse.cpu().numpy()
        assert np.isfinite(o).all() and np.isfinite(ls).all()
        err = row_rel_err(o, ref)
        lerr = float(np.max(np.abs(ls - ref_lse) / np.maximum(1.0, np.abs(ref_lse))))
        pk.polykv_attend_tail_merge(lay, qd, out, lse, torch.from_numpy(tk).to(device()),
                                    torch.from_numpy(tv).to(device()), torch.from_numpy(tl).to(device()),
                                    A, G, scale)
        torch.cuda.synchronize()
        merged = out.cpu().numpy()
        merr = row_rel_err(merged, want_merged)
        moved = row_rel_err(merged, o) if tl.max() > 0 else 0.0
        _say("  path %d: decode %.3e, lse (relative) %.2e, after tails %.3e (tails moved rows by up to %.2e)"
             % (path, err, lerr, merr, moved))
        if tails_matter:
            assert moved > 1e-3
        assert err <= DECODE_REL_TOL
        assert lerr <= LSE_REL_TOL
        assert merr <= DECODE_REL_TOL
