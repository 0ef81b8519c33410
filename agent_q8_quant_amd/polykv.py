"""ctypes binding of ``libpolykv.so`` (C ABI in ``include/polykv.h``).

Argument marshalling only: device buffers are torch tensors on the GPU, and every step
of the hot path runs in the library's HIP kernels. If the library is not built, loading
fails with an error; there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpolykv.so")

POLYKV_OK = 0
POLYKV_PATH_AUTO, POLYKV_PATH_VALU, POLYKV_PATH_MFMA = 0, 1, 2
POLYKV_ROWS_PER_PASS = 64  # query rows one decode launch serves per pool tile

EXPORTED_SYMBOLS = (
    "polykv_pool_layout", "polykv_codebook_default", "polykv_compress_k", "polykv_compress_v",
    "polykv_compress_v_path",
    "polykv_attend_workspace_bytes", "polykv_attend_path", "polykv_attend_shared", "polykv_attend_shared_path",
    "polykv_attend_shared_lse", "polykv_attend_shared_prefix", "polykv_attend_tail_merge",
    "polykv_append_k", "polykv_append_v", "polykv_compress_kv", "polykv_append_kv",
    "polykv_dequant_k", "polykv_dequant_v", "polykv_project_kv", "polykv_project_compress",
    "polykv_strerror",
)


class PolyKVError(RuntimeError):
    def __init__(self, code, where):
        super().__init__("%s failed: %s (%d)" % (where, polykv_strerror(code), code))
        self.code = code


class polykv_shape_t(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_tokens", ctypes.c_int32)]


class polykv_layout_t(ctypes.Structure):
    _fields_ = [("shape", polykv_shape_t),
                ("k_codes_off", ctypes.c_uint64), ("k_codes_tile_stride", ctypes.c_uint64),
                ("k_scales_off", ctypes.c_uint64), ("k_scales_tile_stride", ctypes.c_uint64),
                ("v_planes_off", ctypes.c_uint64), ("v_planes_tile_stride", ctypes.c_uint64),
                ("v_norms_off", ctypes.c_uint64), ("v_norms_tile_stride", ctypes.c_uint64),
                ("analytic_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]


class polykv_codebook_t(ctypes.Structure):
    _fields_ = [("centroid", ctypes.c_float * 8), ("boundary", ctypes.c_float * 7)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpolykv.so is not built: run `python -m agent_q8_quant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.polykv_pool_layout.argtypes = [ctypes.POINTER(polykv_shape_t), ctypes.POINTER(polykv_layout_t)]
        L.polykv_codebook_default.argtypes = [ctypes.POINTER(polykv_codebook_t)]
        L.polykv_compress_k.argtypes = [vp, vp, ctypes.POINTER(polykv_layout_t), i32, i32, vp]
        L.polykv_compress_v.argtypes = [vp, vp, ctypes.POINTER(polykv_layout_t),
                                        ctypes.POINTER(polykv_codebook_t), i32, i32, vp]
        L.polykv_compress_v_path.argtypes = [vp, vp, ctypes.POINTER(polykv_layout_t),
                                             ctypes.POINTER(polykv_codebook_t), i32, i32, vp, i32]
        L.polykv_dequant_k.argtypes = [vp, ctypes.POINTER(polykv_layout_t), vp, i32, i32, vp]
        L.polykv_project_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.polykv_project_compress.argtypes = [vp, vp, vp, vp, ctypes.POINTER(polykv_layout_t),
                                              ctypes.POINTER(polykv_codebook_t), i32, i32, i32, i32, vp]
        L.polykv_dequant_v.argtypes = [vp, ctypes.POINTER(polykv_layout_t), ctypes.POINTER(polykv_codebook_t),
                                       vp, i32, i32, vp]
        L.polykv_attend_workspace_bytes.argtypes = [ctypes.POINTER(polykv_layout_t), i32, i32, i32]
        L.polykv_attend_workspace_bytes.restype = sz
        L.polykv_attend_path.argtypes = [ctypes.POINTER(polykv_layout_t), i32, i32]
        L.polykv_attend_path.restype = ctypes.c_int
        att = [vp, ctypes.POINTER(polykv_layout_t), ctypes.POINTER(polykv_codebook_t), vp, vp,
               i32, i32, ctypes.c_float, i32, i32, vp, sz, vp]
        L.polykv_attend_shared.argtypes = att
        L.polykv_attend_shared_path.argtypes = att + [i32]
        L.polykv_attend_shared_lse.argtypes = att[:5] + [vp] + att[5:] + [i32]
        L.polykv_attend_shared_prefix.argtypes = att[:5] + [vp, i32] + att[5:] + [i32]
        L.polykv_append_k.argtypes = [vp, vp, ctypes.POINTER(polykv_layout_t), i32, i32, i32, i32, vp]
        L.polykv_append_v.argtypes = [vp, vp, ctypes.POINTER(polykv_layout_t), ctypes.POINTER(polykv_codebook_t),
                                      i32, i32, i32, i32, vp]
        L.polykv_compress_kv.argtypes = [vp, vp, vp, ctypes.POINTER(polykv_layout_t),
                                         ctypes.POINTER(polykv_codebook_t), i32, i32, vp]
        L.polykv_append_kv.argtypes = [vp, vp, vp, ctypes.POINTER(polykv_layout_t),
                                       ctypes.POINTER(polykv_codebook_t), i32, i32, i32, i32, vp]
        L.polykv_attend_tail_merge.argtypes = [ctypes.POINTER(polykv_layout_t), vp, vp, vp, vp, vp, vp,
                                               i32, i32, i32, ctypes.c_float, i32, vp]
        L.polykv_strerror.argtypes = [ctypes.c_int]
        L.polykv_strerror.restype = ctypes.c_char_p
        for name in ("polykv_pool_layout", "polykv_codebook_default", "polykv_compress_k",
                     "polykv_compress_v", "polykv_compress_v_path", "polykv_attend_shared", "polykv_attend_shared_path",
                     "polykv_attend_shared_lse", "polykv_attend_shared_prefix", "polykv_attend_tail_merge",
                     "polykv_append_k", "polykv_append_v", "polykv_compress_kv", "polykv_append_kv",
                     "polykv_dequant_k", "polykv_dequant_v", "polykv_project_kv", "polykv_project_compress"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def polykv_strerror(code: int) -> str:
    return lib().polykv_strerror(int(code)).decode()


def _check(rc, where):
    if rc != POLYKV_OK:
        raise PolyKVError(rc, where)


def polykv_pool_layout(n_layers, n_kv_heads, head_dim, n_tokens) -> polykv_layout_t:
    shape = polykv_shape_t(n_layers, n_kv_heads, head_dim, n_tokens)
    out = polykv_layout_t()
    _check(lib().polykv_pool_layout(ctypes.byref(shape), ctypes.byref(out)), "polykv_pool_layout")
    return out


def polykv_codebook_default() -> polykv_codebook_t:
    cb = polykv_codebook_t()
    _check(lib().polykv_codebook_default(ctypes.byref(cb)), "polykv_codebook_default")
    return cb


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError("%s must be contiguous %s" % (name, dtype))
    return ctypes.c_void_p(t.data_ptr())


def _layers(layout, layer_begin, layer_count):
    if layer_count is None:
        layer_count = layout.shape.n_layers - layer_begin
    return int(layer_begin), int(layer_count)


def _kv_elems(layout, layer_count):
    s = layout.shape
    return layer_count * s.n_kv_heads * s.n_tokens * s.head_dim


def polykv_compress_k(k, pool, layout, layer_begin=0, layer_count=None, stream=None):
    lb, lc = _layers(layout, layer_begin, layer_count)
    if k.numel() != _kv_elems(layout, lc) or pool.numel() < layout.total_bytes:
        raise ValueError("k or pool has the wrong size for the layout")
    rc = lib().polykv_compress_k(_dev(k, torch.float16, "k"), _dev(pool, torch.uint8, "pool"),
                                 ctypes.byref(layout), lb, lc, _stream_ptr(stream))
    _check(rc, "polykv_compress_k")


def polykv_compress_v(v, pool, layout, cb=None, layer_begin=0, layer_count=None, stream=None,
                      path=POLYKV_PATH_AUTO):
    """Compress v [layer_count][H][T][d] into the pool; path picks the rotation kernel."""
    lb, lc = _layers(layout, layer_begin, layer_count)
    if v.numel() != _kv_elems(layout, lc) or pool.numel() < layout.total_bytes:
        raise ValueError("v or pool has the wrong size for the layout")
    rc = lib().polykv_compress_v_path(_dev(v, torch.float16, "v"), _dev(pool, torch.uint8, "pool"),
                                      ctypes.byref(layout), ctypes.byref(cb) if cb is not None else None,
                                      lb, lc, _stream_ptr(stream), int(path))
    _check(rc, "polykv_compress_v_path")


def _append_size(layout, t, n_new, lc, name):
    s = layout.shape
    if t.numel() != lc * s.n_kv_heads * int(n_new) * s.head_dim:
        raise ValueError("%s has the wrong size for the chunk" % name)


def polykv_append_k(k, pool, layout, token_begin, n_new=None, layer_begin=0, layer_count=None, stream=None):
    """Compress the chunk k [layer_count][H][n_new][d] into tokens [token_begin, +n_new)."""
    lb, lc = _layers(layout, layer_begin, layer_count)
    n_new = int(k.shape[-2]) if n_new is None else int(n_new)
    _append_size(layout, k, n_new, lc, "k")
    if pool.numel() < layout.total_bytes:
        raise ValueError("pool has the wrong size for the layout")
    rc = lib().polykv_append_k(_dev(k, torch.float16, "k"), _dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                               int(token_begin), n_new, lb, lc, _stream_ptr(stream))
    _check(rc, "polykv_append_k")


def polykv_append_v(v, pool, layout, token_begin, n_new=None, cb=None, layer_begin=0, layer_count=None,
                    stream=None):
    """Compress the chunk v [layer_count][H][n_new][d] into tokens [token_begin, +n_new)."""
    lb, lc = _layers(layout, layer_begin, layer_count)
    n_new = int(v.shape[-2]) if n_new is None else int(n_new)
    _append_size(layout, v, n_new, lc, "v")
    if pool.numel() < layout.total_bytes:
        raise ValueError("pool has the wrong size for the layout")
    rc = lib().polykv_append_v(_dev(v, torch.float16, "v"), _dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                               ctypes.byref(cb) if cb is not None else None, int(token_begin), n_new, lb, lc,
                               _stream_ptr(stream))
    _check(rc, "polykv_append_v")


def polykv_compress_kv(k, v, pool, layout, cb=None, layer_begin=0, layer_count=None, stream=None):
    """Compress k and v [layer_count][H][T][d] into the pool in one call."""
    lb, lc = _layers(layout, layer_begin, layer_count)
    if k.numel() != _kv_elems(layout, lc) or v.numel() != _kv_elems(layout, lc) or pool.numel() < layout.total_bytes:
        raise ValueError("k, v or pool has the wrong size for the layout")
    rc = lib().polykv_compress_kv(_dev(k, torch.float16, "k"), _dev(v, torch.float16, "v"),
                                  _dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                                  ctypes.byref(cb) if cb is not None else None, lb, lc, _stream_ptr(stream))
    _check(rc, "polykv_compress_kv")


def polykv_append_kv(k, v, pool, layout, token_begin, n_new=None, cb=None, layer_begin=0, layer_count=None,
                     stream=None):
    """Compress the chunks k and v [layer_count][H][n_new][d] into tokens [token_begin, +n_new)."""
    lb, lc = _layers(layout, layer_begin, layer_count)
    n_new = int(k.shape[-2]) if n_new is None else int(n_new)
    _append_size(layout, k, n_new, lc, "k")
    _append_size(layout, v, n_new, lc, "v")
    if pool.numel() < layout.total_bytes:
        raise ValueError("pool has the wrong size for the layout")
    rc = lib().polykv_append_kv(_dev(k, torch.float16, "k"), _dev(v, torch.float16, "v"),
                                _dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                                ctypes.byref(cb) if cb is not None else None, int(token_begin), n_new, lb, lc,
                                _stream_ptr(stream))
    _check(rc, "polykv_append_kv")


def polykv_project_kv(x, w_k, w_v, k, v, n_heads, head_dim, stream=None):
    """fp16 K (and V) = RNE16(x W^T), head-major [n_heads][n_tok][head_dim]."""
    n_tok, hidden = int(x.shape[0]), int(x.shape[1])
    if x.dim() != 2 or w_k.shape != (n_heads * head_dim, hidden) or k.numel() != n_heads * n_tok * head_dim:
        raise ValueError("x, w_k or k has the wrong shape")
    if w_v is not None and (w_v.shape != w_k.shape or v is None or v.numel() != k.numel()):
        raise ValueError("w_v or v has the wrong shape")
    rc = lib().polykv_project_kv(_dev(x, torch.float16, "x"), _dev(w_k, torch.float16, "w_k"),
                                 _dev(w_v, torch.float16, "w_v") if w_v is not None else None,
                                 _dev(k, torch.float16, "k"), _dev(v, torch.float16, "v") if w_v is not None else None,
                                 n_tok, hidden, int(n_heads), int(head_dim), _stream_ptr(stream))
    _check(rc, "polykv_project_kv")


def polykv_project_compress(x, w_k, w_v, pool, layout, layer, token_begin, cb=None, stream=None):
    """Project x [n_tok][hidden] with w_k, w_v [H*d][hidden] and compress into the pool."""
    n_tok, hidden = int(x.shape[0]), int(x.shape[1])
    s = layout.shape
    if x.dim() != 2 or w_k.shape != (s.n_kv_heads * s.head_dim, hidden) or w_v.shape != w_k.shape:
        raise ValueError("x, w_k or w_v has the wrong shape")
    if pool.numel() < layout.total_bytes:
        raise ValueError("pool has the wrong size for the layout")
    rc = lib().polykv_project_compress(_dev(x, torch.float16, "x"), _dev(w_k, torch.float16, "w_k"),
                                       _dev(w_v, torch.float16, "w_v"), _dev(pool, torch.uint8, "pool"),
                                       ctypes.byref(layout), ctypes.byref(cb) if cb is not None else None,
                                       int(layer), int(token_begin), n_tok, hidden, _stream_ptr(stream))
    _check(rc, "polykv_project_compress")


def polykv_dequant_k(pool, layout, k, layer_begin=0, layer_count=None, stream=None):
    lb, lc = _layers(layout, layer_begin, layer_count)
    if k.numel() != _kv_elems(layout, lc) or pool.numel() < layout.total_bytes:
        raise ValueError("k or pool has the wrong size for the layout")
    rc = lib().polykv_dequant_k(_dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                                _dev(k, torch.float16, "k"), lb, lc, _stream_ptr(stream))
    _check(rc, "polykv_dequant_k")


def polykv_dequant_v(pool, layout, v, cb=None, layer_begin=0, layer_count=None, stream=None):
    lb, lc = _layers(layout, layer_begin, layer_count)
    if v.numel() != _kv_elems(layout, lc) or pool.numel() < layout.total_bytes:
        raise ValueError("v or pool has the wrong size for the layout")
    rc = lib().polykv_dequant_v(_dev(pool, torch.uint8, "pool"), ctypes.byref(layout),
                                ctypes.byref(cb) if cb is not None else None,
                                _dev(v, torch.float16, "v"), lb, lc, _stream_ptr(stream))
    _check(rc, "polykv_dequant_v")


def polykv_attend_workspace_bytes(layout, n_agents, gqa, layer_count=None) -> int:
    _, lc = _layers(layout, 0, layer_count)
    return int(lib().polykv_attend_workspace_bytes(ctypes.byref(layout), n_agents, gqa, lc))


def polykv_attend_path(layout, n_agents, gqa) -> int:
    rc = int(lib().polykv_attend_path(ctypes.byref(layout), int(n_agents), int(gqa)))
    _check(min(rc, 0), "polykv_attend_path")
    return rc


def _attend_ptrs(pool, layout, q, out, lse, n_agents, gqa, layer_begin, layer_count, cb, workspace):
    lb, lc = _layers(layout, layer_begin, layer_count)
    s = layout.shape
    n = lc * n_agents * s.n_kv_heads * gqa * s.head_dim
    if q.numel() != n or out.numel() != n or pool.numel() < layout.total_bytes:
        raise ValueError("q, out or pool has the wrong size")
    lse_ptr = None
    if lse is not None:
        if lse.numel() != n // s.head_dim:
            raise ValueError("lse has the wrong size")
        lse_ptr = _dev(lse, torch.float32, "lse")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, torch.uint8, "workspace"), workspace.numel()
    return (_dev(pool, torch.uint8, "pool"), ctypes.byref(layout), ctypes.byref(cb) if cb is not None else None,
            _dev(q, torch.float32, "q"), _dev(out, torch.float32, "out"), lse_ptr), lb, lc, ws_ptr, ws_bytes


def polykv_attend_shared_lse(pool, layout, q, out, lse, n_agents, gqa, softmax_scale,
                             path=POLYKV_PATH_AUTO, layer_begin=0, layer_count=None, cb=None,
                             workspace=None, stream=None):
    head, lb, lc, ws_ptr, ws_bytes = _attend_ptrs(pool, layout, q, out, lse, n_agents, gqa,
                                                  layer_begin, layer_count, cb, workspace)
    rc = lib().polykv_attend_shared_lse(*head, int(n_agents), int(gqa), float(softmax_scale), lb, lc,
                                        ws_ptr, ws_bytes, _stream_ptr(stream), int(path))
    _check(rc, "polykv_attend_shared_lse")


def polykv_attend_shared_prefix(pool, layout, q, out, lse, n_valid, n_agents, gqa, softmax_scale,
                                path=POLYKV_PATH_AUTO, layer_begin=0, layer_count=None, cb=None,
                                workspace=None, stream=None):
    head, lb, lc, ws_ptr, ws_bytes = _attend_ptrs(pool, layout, q, out, lse, n_agents, gqa,
                                                  layer_begin, layer_count, cb, workspace)
    rc = lib().polykv_attend_shared_prefix(*head, int(n_valid), int(n_agents), int(gqa),
                                           float(softmax_scale), lb, lc, ws_ptr, ws_bytes,
                                           _stream_ptr(stream), int(path))
    _check(rc, "polykv_attend_shared_prefix")


def polykv_attend_shared_path(pool, layout, q, out, n_agents, gqa, softmax_scale, path,
                              layer_begin=0, layer_count=None, cb=None, workspace=None,
                              stream=None):
    polykv_attend_shared_lse(pool, layout, q, out, None, n_agents, gqa, softmax_scale, path,
                             layer_begin, layer_count, cb, workspace, stream)


def polykv_attend_tail_merge(layout, q, out, lse, tail_k, tail_v, tail_len, n_agents, gqa,
                             softmax_scale, layer_count=None, stream=None):
    lc = layout.shape.n_layers if layer_count is None else int(layer_count)
    s = layout.shape
    n = lc * n_agents * s.n_kv_heads * gqa * s.head_dim
    if q.numel() != n or out.numel() != n or lse.numel() != n // s.head_dim:
        raise ValueError("q, out or lse has the wrong size")
    if tail_k.shape != tail_v.shape or tail_k.dim() != 5 or tail_k.shape[:3] != (n_agents, lc, s.n_kv_heads) \
            or tail_k.shape[4] != s.head_dim or tail_len.numel() != n_agents:
        raise ValueError("tail_k, tail_v or tail_len has the wrong shape")
    cap = int(tail_k.shape[3])
    rc = lib().polykv_attend_tail_merge(
        ctypes.byref(layout), _dev(q, torch.float32, "q"), _dev(out, torch.float32, "out"),
        _dev(lse, torch.float32, "lse"),
        _dev(tail_k, torch.float16, "tail_k") if cap else None,
        _dev(tail_v, torch.float16, "tail_v") if cap else None,
        _dev(tail_len, torch.int32, "tail_len"), cap, int(n_agents), int(gqa),
        float(softmax_scale), lc, _stream_ptr(stream))
    _check(rc, "polykv_attend_tail_merge")


def polykv_attend_shared(pool, layout, q, out, n_agents, gqa, softmax_scale, layer_begin=0,
                         layer_count=None, cb=None, workspace=None, stream=None):
    polykv_attend_shared_path(pool, layout, q, out, n_agents, gqa, softmax_scale,
                              POLYKV_PATH_AUTO, layer_begin, layer_count, cb, workspace, stream)


# ---- helpers for reading a pool back (views into a uint8 tensor; no arithmetic) --------

def pool_views(pool, layout):
    """Views of the four regions as [tiles][...] tensors (padding excluded)."""
    s = layout.shape
    tiles, T, d = s.n_layers * s.n_kv_heads, s.n_tokens, s.head_dim
    G = (T + 31) // 32

    def region(off, stride, nbytes):
        r = pool[off:off + tiles * stride].view(tiles, stride)
        return r[:, :nbytes]

    kc = region(layout.k_codes_off, layout.k_codes_tile_stride, T * d).view(torch.int8).view(tiles, T, d)
    ks = region(layout.k_scales_off, layout.k_scales_tile_stride, T * d // 16)
    vp = region(layout.v_planes_off, layout.v_planes_tile_stride, G * 3 * d * 4)
    vn = region(layout.v_norms_off, layout.v_norms_tile_stride, 2 * T)
    return {"k_codes": kc,
            "k_scales": ks.contiguous().view(torch.float16).view(tiles, T, d // 32),
            "v_planes": vp.contiguous().view(torch.int32).view(tiles, G, 3, d),
            "v_norms": vn.contiguous().view(torch.float16).view(tiles, T)}
