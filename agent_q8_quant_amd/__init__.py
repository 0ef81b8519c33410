"""PolyKV shared-pool hot path for AMD Instinct MI355X (gfx950).

The compute lives in ``libpolykv.so`` (hand-written HIP kernels behind the C ABI in
``include/polykv.h``); this package is its ctypes binding and build script.
"""

from .polykv import (  # noqa: F401
    POLYKV_ROWS_PER_PASS, POLYKV_PATH_AUTO, POLYKV_PATH_MFMA, POLYKV_PATH_VALU, PolyKVError,
    lib, polykv_attend_path, polykv_attend_shared, polykv_attend_shared_lse, polykv_attend_tail_merge, polykv_attend_shared_path, polykv_attend_workspace_bytes,
    polykv_codebook_default, polykv_codebook_t, polykv_compress_k, polykv_compress_v,
    polykv_dequant_k, polykv_dequant_v, polykv_append_k, polykv_append_v, polykv_attend_shared_prefix,
    polykv_compress_kv, polykv_append_kv,
    polykv_project_kv, polykv_project_compress,
    polykv_layout_t, polykv_pool_layout, polykv_shape_t, polykv_strerror, pool_views,
)
