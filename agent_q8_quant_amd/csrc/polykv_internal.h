// Internal interface between the host layer (host.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <atomic>

#include "polykv.h"

namespace polykv {

// Everything a kernel needs to address one pool. Offsets are in bytes from the pool base.
struct PoolGeom {
    int32_t n_kv_heads, head_dim, n_tokens, n_groups;  // n_groups = ceil(T / 32)
    uint64_t k_codes_off, k_codes_stride;
    uint64_t k_scales_off, k_scales_stride;
    uint64_t v_planes_off, v_planes_stride;
    uint64_t v_norms_off, v_norms_stride;
};

// Raise a kernel's dynamic LDS limit once per device. The attribute stays set for the
// kernel on that device, so later launches skip the call. `done` is the caller's flag word
// for that kernel (bit d: device d done); devices past 63 set it on every launch.
inline hipError_t lds_limit_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

inline PoolGeom make_geom(const polykv_layout_t& l) {
    PoolGeom g;
    g.n_kv_heads = l.shape.n_kv_heads;
    g.head_dim = l.shape.head_dim;
    g.n_tokens = l.shape.n_tokens;
    g.n_groups = (l.shape.n_tokens + 31) / 32;
    g.k_codes_off = l.k_codes_off;
    g.k_codes_stride = l.k_codes_tile_stride;
    g.k_scales_off = l.k_scales_off;
    g.k_scales_stride = l.k_scales_tile_stride;
    g.v_planes_off = l.v_planes_off;
    g.v_planes_stride = l.v_planes_tile_stride;
    g.v_norms_off = l.v_norms_off;
    g.v_norms_stride = l.v_norms_tile_stride;
    return g;
}

// Symmetric codebook as the kernels use it: the positive half only.
struct CodebookHalf {
    float centroid_pos[4];   // centroid[4..7]
    float boundary_pos[3];   // boundary[4..6]; boundary[3] is 0
    // lambda in [1, 2) for which the fp16 roundings of lambda * centroid_pos[k] have the
    // smallest worst relative error; kernels that hold centroids in fp16 store
    // lambda * c and divide the result by lambda
    float fp16_scale;
};

// Kernel launchers (defined in compress.hip / attend.hip). They return hipError_t of the
// launch. Arguments are already validated.
hipError_t launch_compress_k(const void* k_fp16, uint8_t* pool, const PoolGeom& g,
                             int32_t layer_begin, int32_t layer_count, hipStream_t s);
// The same over tokens [tok0, tok0 + n_tok) of every tile, from an input that holds that
// range only ([layer_count][H][n_tok][d]); plane bits of other tokens are kept.
hipError_t launch_compress_k_range(const void* k_fp16, uint8_t* pool, const PoolGeom& g,
                                   int32_t tok0, int32_t n_tok, int32_t layer_begin,
                                   int32_t layer_count, hipStream_t s);
// valu: the in-register butterfly kernel for every head_dim (else the matrix-core rotation
// for head_dim 64 and 128).
hipError_t launch_compress_v_range(const void* v_fp16, uint8_t* pool, const PoolGeom& g,
                                   const CodebookHalf& cb, int32_t tok0, int32_t n_tok,
                                   int32_t layer_begin, int32_t layer_count, hipStream_t s,
                                   bool valu = false);
hipError_t launch_compress_v(const void* v_fp16, uint8_t* pool, const PoolGeom& g,
                             const CodebookHalf& cb, int32_t layer_begin,
                             int32_t layer_count, hipStream_t s, bool valu = false);
// Keys and values of one token range in one launch (two launches for head_dim 256); the
// inputs hold that range only, as for the single-kind launchers.
hipError_t launch_compress_kv_range(const void* k_fp16, const void* v_fp16, uint8_t* pool,
                                    const PoolGeom& g, const CodebookHalf& cb, int32_t tok0,
                                    int32_t n_tok, int32_t layer_begin, int32_t layer_count,
                                    hipStream_t s);

struct AttendArgs {
    const uint8_t* pool;
    PoolGeom g;
    CodebookHalf cb;
    const float* q;
    float* out;
    float* lse;  // optional [layer_count][n_agents][H * gqa]: ln sum_t exp(scale q . k_t)
    int32_t n_agents, gqa, layer_begin, layer_count;
    // the launch serves rows row_begin .. row_begin + n_rows - 1 of every tile, row r being
    // agent r / gqa, query head h * gqa + r % gqa (1 <= n_rows <= 64)
    int32_t row_begin, n_rows;
    float softmax_scale;
    void* workspace;
    size_t workspace_bytes;
};

// Private-tail merge (attend_tail.hip).
struct TailArgs {
    const float* q;
    float* out;   // in: shared-pool result, out: merged result
    float* lse;   // in/out, natural log
    const void* tail_k;
    const void* tail_v;
    const int32_t* tail_len;
    int32_t tail_cap;
    int32_t n_kv_heads, head_dim, gqa, n_agents, layer_count;
    float softmax_scale;
};
hipError_t launch_attend_tail(const TailArgs& a, hipStream_t s);

// K/V projection x W^T (project.hip): fp16 [n_heads][n_tok][d] outputs (w_v may be NULL),
// or compressed straight into pool layer `layer`, tokens [tok0, tok0 + n_tok).
hipError_t launch_project(const __half* x, const __half* w_k, const __half* w_v, __half* k_out,
                          __half* v_out, int32_t n_tok, int32_t hidden, int32_t n_heads,
                          int32_t head_dim, hipStream_t s);
hipError_t launch_project_compress(const __half* x, const __half* w_k, const __half* w_v,
                                   uint8_t* pool, const PoolGeom& g, const CodebookHalf& cb,
                                   int32_t layer, int32_t tok0, int32_t n_tok, int32_t hidden,
                                   hipStream_t s);

// Pool -> fp16 K / V (dequant.hip).
hipError_t launch_dequant_k(const uint8_t* pool, void* k_fp16, const PoolGeom& g,
                            int32_t layer_begin, int32_t layer_count, hipStream_t s);
hipError_t launch_dequant_v(const uint8_t* pool, void* v_fp16, const PoolGeom& g,
                            const CodebookHalf& cb, int32_t layer_begin, int32_t layer_count,
                            hipStream_t s);

size_t attend_workspace_bytes(const PoolGeom& g, int32_t n_agents, int32_t gqa,
                              int32_t layer_count, int32_t path);
hipError_t launch_attend_valu(const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s);
bool attend_mfma_supported(const PoolGeom& g, int32_t rows);

}  // namespace polykv
