"""Host-side checks of the C ABI: exports, layout, built-in codebook, argument validation.

No kernel is launched here; every call either returns before any device work or, on a
machine without a GPU, stops at the device check.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import agent_q8_quant_amd as pk
from agent_q8_quant_amd import polykv as B
from oracle import analytic_pool_bytes, codebook_fp32
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from agent_q8_quant_amd.build import build
        build()
    return pk.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "polykv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(polykv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED_SYMBOLS)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_layout(L, cfg):
    lay = pk.polykv_pool_layout(cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_tokens)
    tiles, T, d = cfg.n_layers * cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim
    G = (T + 31) // 32
    up = lambda x: (x + 255) // 256 * 256
    assert lay.k_codes_tile_stride == up(T * d)
    assert lay.k_scales_tile_stride == up(T * d // 16)
    assert lay.v_planes_tile_stride == up(G * 3 * d * 4)
    assert lay.v_norms_tile_stride == up(2 * T)
    offs = [lay.k_codes_off, lay.k_scales_off, lay.v_planes_off, lay.v_norms_off]
    strides = [lay.k_codes_tile_stride, lay.k_scales_tile_stride, lay.v_planes_tile_stride,
               lay.v_norms_tile_stride]
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs)
    for i in range(3):
        assert offs[i + 1] == offs[i] + tiles * strides[i]
    assert lay.total_bytes == offs[3] + tiles * strides[3]
    assert lay.analytic_bytes == analytic_pool_bytes(cfg.n_layers, cfg.n_kv_heads, T, d)
    # padding: at most 255 B per tile and region, plus the last token group's planes
    pad = lay.total_bytes - lay.analytic_bytes
    assert 0 <= pad <= tiles * (4 * 255 + (32 * G - T) * 3 * d // 8)


def test_default_codebook_bitwise_equals_oracle(L):
    cb = pk.polykv_codebook_default()
    c32, b32 = codebook_fp32()
    assert np.array_equal(np.array(cb.centroid[:], dtype=np.float32), c32)
    assert np.array_equal(np.array(cb.boundary[:], dtype=np.float32), b32)


def _layout(n_layers=2, H=2, d=128, T=100):
    return pk.polykv_pool_layout(n_layers, H, d, T)


def test_layout_errors(L):
    out = B.polykv_layout_t()
    for shape in [(0, 1, 128, 10), (1, 0, 128, 10), (1, 1, 128, 0), (1, 1, 32, 10), (1, 1, 96, 10)]:
        s = B.polykv_shape_t(*shape)
        assert L.polykv_pool_layout(ctypes.byref(s), ctypes.byref(out)) == -2
    assert L.polykv_pool_layout(None, ctypes.byref(out)) == -1
    with pytest.raises(pk.PolyKVError):
        pk.polykv_pool_layout(1, 1, 48, 10)


A16, A256 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)


def test_compress_validation(L):
    lay = _layout()
    lb = ctypes.byref(lay)
    assert L.polykv_compress_k(None, A256, lb, 0, 2, None) == -1
    assert L.polykv_compress_k(A16, None, lb, 0, 2, None) == -1
    assert L.polykv_compress_k(A16, A256, None, 0, 2, None) == -1
    assert L.polykv_compress_k(A16, ctypes.c_void_p(0x20010), lb, 0, 2, None) == -3
    assert L.polykv_compress_k(ctypes.c_void_p(0x10008), A256, lb, 0, 2, None) == -3
    assert L.polykv_compress_k(A16, A256, lb, 1, 2, None) == -4
    assert L.polykv_compress_k(A16, A256, lb, -1, 1, None) == -4
    assert L.polykv_compress_k(A16, A256, lb, 0, 0, None) == -4
    bad = _layout()
    bad.total_bytes -= 1
    assert L.polykv_compress_k(A16, A256, ctypes.byref(bad), 0, 2, None) == -9
    cb = pk.polykv_codebook_default()
    cb.boundary[4] += 1e-3       # no longer symmetric
    assert L.polykv_compress_v(A16, A256, lb, ctypes.byref(cb), 0, 2, None) == -8
    cb = pk.polykv_codebook_default()
    cb.centroid[0], cb.centroid[1] = cb.centroid[1], cb.centroid[0]
    assert L.polykv_compress_v(A16, A256, lb, ctypes.byref(cb), 0, 2, None) == -8
    # explicit rotation kernel: an unknown path, and the matrix cores at head_dim 256
    good = pk.polykv_codebook_default()
    assert L.polykv_compress_v_path(A16, A256, lb, ctypes.byref(good), 0, 2, None, 3) == -10
    assert L.polykv_compress_v_path(A16, A256, lb, ctypes.byref(good), 0, 2, None, -1) == -10
    lay256 = pk.polykv_pool_layout(1, 1, 256, 32)
    assert L.polykv_compress_v_path(A16, A256, ctypes.byref(lay256), None, 0, 1, None, 2) == -2


def _attend(L, lay, n_agents=2, gqa=2, scale=0.1, lb=0, lc=2, ws=None, wsb=0, path=0,
            pool=A256, q=A16, out=A16, cb=None):
    return L.polykv_attend_shared_path(pool, ctypes.byref(lay), cb, q, out, n_agents, gqa,
                                       scale, lb, lc, ws, wsb, None, path)


def test_attend_validation(L):
    lay = _layout()
    assert _attend(L, lay, pool=None) == -1
    assert _attend(L, lay, q=None) == -1
    assert _attend(L, lay, n_agents=0) == -2
    assert _attend(L, lay, q=ctypes.c_void_p(0x10004)) == -3
    assert _attend(L, lay, lb=2, lc=1) == -4
    # any row count: 68 rows pass every check (two launches); only the device is missing here
    assert _attend(L, lay, n_agents=17, gqa=4) == -6
    assert _attend(L, lay, n_agents=1 << 20, gqa=1 << 12) == -2   # rows overflow int32
    assert _attend(L, lay, scale=float("inf")) == -10
    assert _attend(L, lay, path=3) == -10
    cb = pk.polykv_codebook_default()
    cb.boundary[3] = 1e-3
    cb.boundary[2] = -1e-3
    assert _attend(L, lay, cb=ctypes.byref(cb)) == -8


def test_attend_path_choice(L):
    """The automatic choice: the matrix-core kernel wherever it applies (head_dim 64/128; it
    is faster than the vector-ALU kernel at every row count measured, 1 to 60), the
    vector-ALU kernel otherwise."""
    for d, rows, want in ((128, 60, pk.POLYKV_PATH_MFMA), (64, 17, pk.POLYKV_PATH_MFMA),
                          (128, 16, pk.POLYKV_PATH_MFMA), (128, 1, pk.POLYKV_PATH_MFMA),
                          (64, 5, pk.POLYKV_PATH_MFMA), (256, 60, pk.POLYKV_PATH_VALU),
                          (256, 1, pk.POLYKV_PATH_VALU)):
        lay = pk.polykv_pool_layout(2, 2, d, 100)
        assert pk.polykv_attend_path(lay, rows, 1) == want, (d, rows)
    lay = _layout()
    assert L.polykv_attend_path(None, 1, 1) == -1
    assert L.polykv_attend_path(ctypes.byref(lay), 0, 1) == -2
    # more rows than one launch serves: the same kernel for every pass
    assert L.polykv_attend_path(ctypes.byref(lay), 17, 4) == pk.POLYKV_PATH_MFMA
    assert pk.polykv_attend_path(pk.polykv_pool_layout(2, 2, 256, 100), 200, 1) == pk.POLYKV_PATH_VALU
    assert L.polykv_attend_path(ctypes.byref(lay), 1 << 20, 1 << 12) == -2
    bad = pk.polykv_pool_layout(2, 2, 128, 100)
    bad.k_codes_off += 16
    assert L.polykv_attend_path(ctypes.byref(bad), 1, 1) == -9


def test_tail_merge_validation(L):
    lay = _layout()
    vp = ctypes.c_void_p
    dev = vp(0x100000)
    args = dict(q=dev, out=dev, lse=dev, tk=dev, tv=dev, tl=dev, cap=8, A=2, G=2, scale=0.1, lc=2)

    def call(**kw):
        a = dict(args, **kw)
        return L.polykv_attend_tail_merge(ctypes.byref(lay), a["q"], a["out"], a["lse"], a["tk"], a["tv"],
                                          a["tl"], a["cap"], a["A"], a["G"], ctypes.c_float(a["scale"]),
                                          a["lc"], None)
    assert call(q=None) == -1
    assert call(tl=None) == -1
    assert call(tk=None) == -1          # a non-empty tail needs its buffers
    assert call(A=0) == -2
    assert call(cap=-1) == -2
    assert call(A=17, G=4) == -6        # any row count; no device here
    assert call(A=1 << 30) == -2        # layers x agents x heads workgroups overflow int32
    assert call(lc=3) == -4             # more layers than the layout holds
    assert call(scale=float("nan")) == -10
    assert call(q=vp(0x100004)) == -3
    assert call(cap=0, tk=None, tv=None) == 0   # nothing to merge: no device work at all


def test_dequant_validation(L):
    lay = _layout()
    lb = ctypes.byref(lay)
    for f in (L.polykv_dequant_k,):
        assert f(None, lb, A16, 0, 2, None) == -1
        assert f(A256, None, A16, 0, 2, None) == -1
        assert f(A256, lb, None, 0, 2, None) == -1
        assert f(ctypes.c_void_p(0x20010), lb, A16, 0, 2, None) == -3     # pool needs 256 B
        assert f(A256, lb, ctypes.c_void_p(0x10008), 0, 2, None) == -3
        assert f(A256, lb, A16, 1, 2, None) == -4
        assert f(A256, lb, A16, 0, 0, None) == -4
    assert L.polykv_dequant_v(None, lb, None, A16, 0, 2, None) == -1
    assert L.polykv_dequant_v(A256, lb, None, None, 0, 2, None) == -1
    assert L.polykv_dequant_v(ctypes.c_void_p(0x20010), lb, None, A16, 0, 2, None) == -3
    assert L.polykv_dequant_v(A256, lb, None, A16, -1, 1, None) == -4
    bad = _layout()
    bad.total_bytes -= 1
    assert L.polykv_dequant_k(A256, ctypes.byref(bad), A16, 0, 2, None) == -9
    assert L.polykv_dequant_v(A256, ctypes.byref(bad), None, A16, 0, 2, None) == -9
    cb = pk.polykv_codebook_default()
    cb.centroid[6] += 1e-3       # no longer symmetric
    assert L.polykv_dequant_v(A256, lb, ctypes.byref(cb), A16, 0, 2, None) == -8


def test_append_and_prefix_validation(L):
    lay = _layout()               # 2 layers, capacity n_tokens
    lb = ctypes.byref(lay)
    T = lay.shape.n_tokens
    for f, extra in ((L.polykv_append_k, ()), (L.polykv_append_v, (None,))):
        def call(tb, n, lbeg=0, lc=2, src=A16, pool=A256):
            return f(src, pool, lb, *extra, tb, n, lbeg, lc, None)
        assert call(0, 1, src=None) == -1
        assert call(0, 1, pool=ctypes.c_void_p(0x20010)) == -3
        assert call(-1, 2) == -4
        assert call(0, 0) == -4
        assert call(T - 3, 4) == -4         # past the capacity
        assert call(0, T, lbeg=1) == -4
    cb = pk.polykv_codebook_default()
    cb.boundary[3] = 0.1
    assert L.polykv_append_v(A16, A256, lb, ctypes.byref(cb), 0, 1, 0, 2, None) == -8
    for n_valid in (0, T + 1):
        assert L.polykv_attend_shared_prefix(A256, lb, None, A16, A16, None, n_valid, 2, 2,
                                             ctypes.c_float(0.1), 0, 2, None, 0, None, 0) == -4


def test_fused_key_value_validation(L):
    lay = _layout()
    lb = ctypes.byref(lay)
    T = lay.shape.n_tokens
    unaligned = ctypes.c_void_p(0x20010)

    def comp(k=A16, v=A16, pool=A256, lbeg=0, lc=2, cb=None):
        return L.polykv_compress_kv(k, v, pool, lb, cb, lbeg, lc, None)

    def app(tb, n, k=A16, v=A16, pool=A256, lbeg=0, lc=2, cb=None):
        return L.polykv_append_kv(k, v, pool, lb, cb, tb, n, lbeg, lc, None)

    for f in (comp, lambda **a: app(0, 1, **a)):
        assert f(k=None) == -1
        assert f(v=None) == -1
        assert f(pool=None) == -1
        assert f(pool=unaligned) == -3
        assert f(v=ctypes.c_void_p(0x10008)) == -3
        assert f(lbeg=1) == -4               # layer range past the pool
        assert f(lc=0) == -4
    assert L.polykv_compress_kv(A16, A16, A256, None, None, 0, 2, None) == -1
    assert app(-1, 2) == -4
    assert app(0, 0) == -4
    assert app(T - 3, 4) == -4
    cb = pk.polykv_codebook_default()
    cb.boundary[3] = 0.1
    assert comp(cb=ctypes.byref(cb)) == -8
    assert app(0, 1, cb=ctypes.byref(cb)) == -8
    bad = _layout()
    bad.total_bytes += 256
    assert L.polykv_compress_kv(A16, A16, A256, ctypes.byref(bad), None, 0, 2, None) == -9


def test_projection_validation(L):
    lay = _layout()
    lb = ctypes.byref(lay)
    H, d, T = lay.shape.n_kv_heads, lay.shape.head_dim, lay.shape.n_tokens

    def fused(x=A16, wk=A16, wv=A16, pool=A256, layer=0, tb=0, n=32, hidden=128, cb=None):
        return L.polykv_project_compress(x, wk, wv, pool, lb, cb, layer, tb, n, hidden, None)
    assert fused(x=None) == -1
    assert fused(wv=None) == -1
    assert fused(hidden=96) == -2          # not a multiple of 64
    assert fused(hidden=(1 << 22) + 64) == -2  # operand-tile byte offsets must fit 32 bits
    assert fused(n=0) == -2
    assert fused(x=ctypes.c_void_p(0x10008)) == -3
    assert fused(pool=ctypes.c_void_p(0x20010)) == -3
    assert fused(layer=2) == -4
    assert fused(tb=16) == -4              # chunks start at a multiple of 32
    assert fused(tb=32, n=T) == -4         # past the capacity

    def plain(x=A16, wk=A16, wv=None, k=A16, v=None, n=8, hidden=64, heads=H, hd=d):
        return L.polykv_project_kv(x, wk, wv, k, v, n, hidden, heads, hd, None)
    assert plain(k=None) == -1
    assert plain(wv=A16, v=None) == -1     # V output missing
    assert plain(hd=32) == -2
    assert plain(heads=0) == -2
    assert plain(hidden=1 << 23) == -2
    assert plain(k=ctypes.c_void_p(0x10004)) == -3


def test_strerror(L):
    for code in range(0, -11, -1):
        assert isinstance(pk.polykv_strerror(code), str) and pk.polykv_strerror(code)
    assert pk.polykv_strerror(-99) == "unknown error code"


def test_device_check_without_gpu(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lay = _layout()
    assert L.polykv_compress_k(A16, A256, ctypes.byref(lay), 0, 2, None) == -6
    assert _attend(L, lay) == -6


def test_binding_requires_device_tensors(L):
    import torch
    lay = _layout()
    with pytest.raises(TypeError):
        pk.polykv_compress_k(torch.zeros(2 * 2 * 100 * 128, dtype=torch.float16),
                             torch.zeros(lay.total_bytes, dtype=torch.uint8), lay)
