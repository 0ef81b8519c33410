"""The library's calls captured in a HIP graph and replayed.

PolyKV, Abstract: the pool is written once and then read by every agent at each decode step,
so a serving loop repeats the same calls; a HIP graph replays them without host work. The
library allocates nothing and never synchronises, so its calls can be captured. Captured
here: the one-launch key + value compress, the decode with the lse export on both kernels,
a prefix decode, and the tail merge. The graph is replayed three times, with eager work and
synchronisations between the replays and every output reset before each replay; every
replay must equal the same calls made eagerly, bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

import agent_q8_quant_amd as pk
from gpu_helpers import device, new_pool

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_capture_and_replay():
    L, H, d, T, A, G, cap = 2, 2, 128, 600, 5, 4, 64
    _say("graph", dict(L=L, H=H, d=d, T=T, A=A, G=G, cap=cap))
    dev = device()
    rng = np.random.default_rng(77)
    k = torch.from_numpy(rng.standard_normal((L, H, T, d)).astype(np.float16)).to(dev)
    v = torch.from_numpy(rng.standard_normal((L, H, T, d)).astype(np.float16)).to(dev)
    q = torch.from_numpy(rng.standard_normal((L, A, H * G, d)).astype(np.float32)).to(dev)
    tk = torch.from_numpy(rng.standard_normal((A, L, H, cap, d)).astype(np.float16)).to(dev)
    tv = torch.from_numpy(rng.standard_normal((A, L, H, cap, d)).astype(np.float16)).to(dev)
    tl = torch.from_numpy(rng.integers(0, cap + 1, size=A).astype(np.int32)).to(dev)
    lay = pk.polykv_pool_layout(L, H, d, T)
    scale = d ** -0.5
    n_valid = 480

    def buffers():
        return dict(pool=new_pool(lay),
                    out=torch.empty_like(q), lse=torch.empty((L, A, H * G), dtype=torch.float32, device=dev),
                    out_v=torch.empty_like(q), lse_v=torch.empty((L, A, H * G), dtype=torch.float32, device=dev),
                    out_p=torch.empty_like(q), lse_p=torch.empty((L, A, H * G), dtype=torch.float32, device=dev))

    def reset(b):
        b["pool"].fill_(0xA5)
        for key in ("out", "lse", "out_v", "lse_v", "out_p", "lse_p"):
            b[key].fill_(float("nan"))

    def calls(b, stream):
        pk.polykv_compress_kv(k, v, b["pool"], lay, stream=stream)
        pk.polykv_attend_shared_lse(b["pool"], lay, q, b["out"], b["lse"], A, G, scale, pk.POLYKV_PATH_MFMA,
                                    stream=stream)
        pk.polykv_attend_tail_merge(lay, q, b["out"], b["lse"], tk, tv, tl, A, G, scale, stream=stream)
        pk.polykv_attend_shared_lse(b["pool"], lay, q, b["out_v"], b["lse_v"], A, G, scale, pk.POLYKV_PATH_VALU,
                                    stream=stream)
        pk.polykv_attend_shared_prefix(b["pool"], lay, q, b["out_p"], b["lse_p"], n_valid, A, G, scale,
                                       pk.POLYKV_PATH_MFMA, stream=stream)

    # the eager result
    want = buffers()
    reset(want)
    calls(want, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(want["out"]).any().item()

    got = buffers()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(got, s)   # every kernel has been launched once before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls(got, s)
    torch.cuda.synchronize()
    other = buffers()
    for r in range(3):
        reset(got)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in want:
            assert torch.equal(got[key], want[key]), (r, key)
        # eager work between the replays
        reset(other)
        calls(other, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(other["out"], want["out"])
    _say("  three replays equal the eager calls")
