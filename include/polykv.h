/*
 * polykv.h - C ABI of the PolyKV shared-pool hot path for AMD Instinct MI355X (gfx950).
 *
 * Method source: "PolyKV: A Shared Asymmetrically-Compressed KV Cache Pool for
 * Multi-Agent LLM Inference", section "Abstract (arXiv)". Several agents share one KV
 * pool that is compressed once: keys are quantised at int8 (q8_0), values with
 * TurboQuant MSE (a Fast Walsh-Hadamard rotation followed by 3-bit Lloyd-Max codes with
 * centroids for N(0,1)); every agent then decodes against that single pool.
 *
 * Definitions of the steps the abstract leaves open (these are the library's format):
 *  - q8_0: blocks of 32 consecutive key entries along head_dim; fp16 scale
 *    s = RNE16(amax / 127) with an IEEE float32 division; code q = RNE(x / s) with the
 *    stored fp16 scale, clamped to [-127, 127]; s = 0 gives all codes 0.
 *  - TurboQuant MSE: n = ||v||_2; y = H v / n (H the +-1 Sylvester Hadamard matrix, i.e.
 *    the orthonormal FWHT of v * sqrt(d) / n); code = #{k : y > b_k} over the 7 codebook
 *    boundaries (ties go to the lower code; n = 0 gives y = 0); fp16 RNE norm stored.
 *  - Decode: out = softmax(scale * q . k_hat) . v_hat over every pool token, with
 *    k_hat = q8 code * s and v_hat = (n16 / d) * H c[code]; query head j reads KV head
 *    j / gqa.
 *
 * Conventions for every entry point:
 *  - Pointers named *_fp16, pool, q, out, workspace are DEVICE pointers; layout and
 *    codebook structs are HOST pointers. The caller allocates and owns every buffer; the
 *    library never allocates, frees or synchronises, and keeps no per-call state.
 *  - hip_stream is a hipStream_t (NULL = the null stream). All device work is
 *    asynchronous on it; buffers must stay alive until that work has completed. The
 *    device work of a call is kernel launches only (no copies or memsets), so a call
 *    may be captured into a HIP graph once every kernel it launches has been launched
 *    eagerly on the device (the first launch of a kernel sets its LDS limit).
 *  - All arguments are validated on the host before anything is launched, so an error
 *    return means nothing was enqueued. Non-finite inputs are not checked: the results
 *    for them are unspecified.
 *  - Return value: POLYKV_OK (0) or a negative POLYKV_ERR_* code.
 */
#ifndef POLYKV_H
#define POLYKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define POLYKV_OK 0
#define POLYKV_ERR_NULL (-1)       /* a required pointer is NULL                          */
#define POLYKV_ERR_SHAPE (-2)      /* head_dim not in {64,128,256}, a count < 1, or       */
                                   /* a size that overflows                               */
#define POLYKV_ERR_ALIGN (-3)      /* pool not 256-B aligned, another buffer not 16-B     */
#define POLYKV_ERR_RANGE (-4)      /* layer or token range outside the pool               */
#define POLYKV_ERR_WORKSPACE (-5)  /* workspace smaller than polykv_attend_workspace_bytes */
#define POLYKV_ERR_DEVICE (-6)     /* no HIP device, or the current device is not gfx950  */
#define POLYKV_ERR_LAUNCH (-7)     /* a kernel launch failed (hipGetLastError)             */
#define POLYKV_ERR_CODEBOOK (-8)   /* codebook not ascending, not symmetric, or b[3] != 0 */
#define POLYKV_ERR_LAYOUT (-9)     /* layout struct does not match polykv_pool_layout     */
#define POLYKV_ERR_ARG (-10)       /* another argument out of its domain                  */

#define POLYKV_ROWS_PER_PASS 64    /* query rows (agents x query heads of a KV head) one  */
                                   /* decode launch serves per pool tile; more rows take */
                                   /* further launches, each reading the pool once       */

/* Kernel choice for polykv_compress_v_path and polykv_attend_shared_path. */
#define POLYKV_PATH_AUTO 0   /* matrix cores where supported (head_dim 64/128), else VALU */
#define POLYKV_PATH_VALU 1   /* vector ALU (fp32)                                         */
#define POLYKV_PATH_MFMA 2   /* matrix cores (fp16 operands, fp32 accumulation)           */

/* Pool geometry. */
typedef struct {
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t head_dim;   /* 64, 128 or 256 */
    int32_t n_tokens;   /* >= 1 */
} polykv_shape_t;

/*
 * Byte layout of a pool. The pool is one device buffer with four regions. A "tile" is
 * one (layer, KV head) pair; tile index = layer * n_kv_heads + head. Inside a region,
 * tile k starts at region_off + k * region_tile_stride; every tile stride is its payload
 * rounded up to 256 B, and every region starts 256-B aligned.
 *  k_codes : int8   [T][d]            per tile, row-major
 *  k_scales: fp16   [T][d/32]         per tile
 *  v_planes: uint32 [ceil(T/32)][3][d] per tile; bit j of word (g, p, i) is bit p of
 *                                      the value code of token 32*g + j at coordinate i
 *                                      (bits of tokens >= T are 0)
 *  v_norms : fp16   [T]               per tile
 * analytic_bytes counts the payload exactly (1 B per key code, 2 B per scale, 3 bits per
 * value code, 2 B per norm); total_bytes is what the buffer must hold.
 */
typedef struct {
    polykv_shape_t shape;
    uint64_t k_codes_off, k_codes_tile_stride;
    uint64_t k_scales_off, k_scales_tile_stride;
    uint64_t v_planes_off, v_planes_tile_stride;
    uint64_t v_norms_off, v_norms_tile_stride;
    uint64_t analytic_bytes;
    uint64_t total_bytes;
} polykv_layout_t;

/* 3-bit codebook: centroids ascending (code 0 is the most negative) and the 7 decision
 * boundaries between them. The kernels require it symmetric about 0 with boundary[3] = 0. */
typedef struct {
    float centroid[8];
    float boundary[7];
} polykv_codebook_t;

/*
 * Fill *out with the pool layout for *shape. PolyKV, Abstract: the compressed K/V cache
 * is written a single time into one shared pool that every agent then reads; this fixes
 * where each part of that pool lives (the four regions above). Host only; touches no
 * device. Errors: NULL, SHAPE.
 */
int polykv_pool_layout(const polykv_shape_t* shape, polykv_layout_t* out);

/*
 * PolyKV, Abstract: values are quantised with 3-bit Lloyd-Max codes whose centroids are
 * fitted to the standard normal distribution (after the Hadamard rotation).
 * Fill *out with the library's Lloyd-Max codebook for N(0,1): Lloyd's iteration run in
 * fp64 to a fixed point (centroids = conditional means of their cells, boundaries =
 * midpoints), made exactly symmetric, centroids rounded to float32, boundaries = fp64
 * midpoints of the float32 centroids rounded to float32. Computed once per process,
 * thread-safe. Host only. Errors: NULL.
 */
int polykv_codebook_default(polykv_codebook_t* out);

/*
 * q8_0-compress keys into the pool. PolyKV, Abstract: keys are stored as 8-bit integers
 * in the q8_0 format, which keeps the softmax over the shared pool stable.
 *  k_fp16: device, IEEE binary16, contiguous [layer_count][n_kv_heads][n_tokens][head_dim]
 *          holding pool layers [layer_begin, layer_begin + layer_count); 16-B aligned.
 *  pool:   device, layout->total_bytes, 256-B aligned; only the k_codes and k_scales
 *          tiles of those layers are written.
 * Errors: NULL, ALIGN, RANGE, LAYOUT, DEVICE, LAUNCH.
 */
int polykv_compress_k(const void* k_fp16, void* pool, const polykv_layout_t* layout,
                      int32_t layer_begin, int32_t layer_count, void* hip_stream);

/*
 * TurboQuant-MSE-compress values into the pool (the FWHT rotation + 3-bit Lloyd-Max
 * step). v_fp16 as k_fp16 above; only the v_planes and v_norms tiles of those layers are
 * written. cb: host pointer or NULL for polykv_codebook_default; only the boundaries are
 * used. compress_k and compress_v write disjoint regions and may run concurrently.
 * Errors: NULL, ALIGN, RANGE, LAYOUT, CODEBOOK, DEVICE, LAUNCH.
 */
int polykv_compress_v(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                      const polykv_codebook_t* cb, int32_t layer_begin, int32_t layer_count,
                      void* hip_stream);

/*
 * As polykv_compress_v with an explicit kernel for the rotation (POLYKV_PATH_*):
 * POLYKV_PATH_MFMA computes y = H v on the matrix cores (head_dim 64 and 128; the
 * automatic choice there), POLYKV_PATH_VALU as an in-register butterfly on the vector ALU
 * (every head_dim; the automatic choice for 256). Both write the same pool bytes up to the
 * value-code rule at decision boundaries (codes may differ only where y lies within
 * rounding of a boundary). PolyKV, Abstract: the values are rotated by a fast
 * Walsh-Hadamard transform before their 3-bit quantisation.
 * Errors: as polykv_compress_v; SHAPE for MFMA with head_dim 256; ARG for another path.
 */
int polykv_compress_v_path(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                           const polykv_codebook_t* cb, int32_t layer_begin, int32_t layer_count,
                           void* hip_stream, int32_t path);

/*
 * Chunked (append) compression. PolyKV, Abstract: the pool is written a single time; when
 * the shared context arrives in prefill chunks, each chunk is written once, into its own
 * token range. These compress tokens [token_begin, token_begin + n_new) of every tile of
 * layers [layer_begin, layer_begin + layer_count) exactly as polykv_compress_k/v would
 * compress them within the whole context (every step is per token), so appending the
 * chunks of a context in any order gives the same pool bytes as one compress of it.
 *  k_fp16 / v_fp16: device binary16, contiguous [layer_count][n_kv_heads][n_new][head_dim]
 *          (the chunk only), 16-B aligned.
 *  pool:   device, layout->total_bytes, 256-B aligned; layout->shape.n_tokens is the
 *          capacity. Only the chunk's codes, scales, norms and plane bits are written: the
 *          plane words of a 32-token group the chunk covers in part are read, and the bits
 *          of the group's other tokens below the capacity are kept.
 *  cb (values): host pointer or NULL for polykv_codebook_default.
 * Calls whose chunks share a 32-token group must not run concurrently (stream order).
 * Errors: NULL, ALIGN, RANGE (token or layer range), LAYOUT, CODEBOOK, DEVICE, LAUNCH.
 */
int polykv_append_k(const void* k_fp16, void* pool, const polykv_layout_t* layout,
                    int32_t token_begin, int32_t n_new, int32_t layer_begin, int32_t layer_count,
                    void* hip_stream);
int polykv_append_v(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                    const polykv_codebook_t* cb, int32_t token_begin, int32_t n_new,
                    int32_t layer_begin, int32_t layer_count, void* hip_stream);

/*
 * Keys and values in one call. PolyKV, Abstract: the K and V of the shared context go into
 * the one pool that is written once; a caller that holds both compresses them together.
 * polykv_compress_kv writes exactly the bytes of polykv_compress_k followed by
 * polykv_compress_v, and polykv_append_kv those of polykv_append_k followed by
 * polykv_append_v, with the same arguments (k_fp16 and v_fp16 as described there; cb:
 * host pointer or NULL for polykv_codebook_default). For head_dim 64 and 128 one launch
 * encodes both (the value rotation on the matrix cores, as the automatic choice of
 * polykv_compress_v_path); for head_dim 256 it is the two launches in stream order.
 * Errors: NULL, ALIGN, RANGE (layer range; token range for append), LAYOUT, CODEBOOK,
 *         DEVICE, LAUNCH.
 */
int polykv_compress_kv(const void* k_fp16, const void* v_fp16, void* pool,
                       const polykv_layout_t* layout, const polykv_codebook_t* cb,
                       int32_t layer_begin, int32_t layer_count, void* hip_stream);
int polykv_append_kv(const void* k_fp16, const void* v_fp16, void* pool,
                     const polykv_layout_t* layout, const polykv_codebook_t* cb,
                     int32_t token_begin, int32_t n_new, int32_t layer_begin,
                     int32_t layer_count, void* hip_stream);

/*
 * K/V projection of one layer's prefill chunk, with the pool compression fused into its
 * epilogue. PolyKV, Abstract: the shared cache is compressed a single time, as it is
 * written; here that happens where K and V are produced, so they never reach HBM as fp16.
 *   K = RNE16(x W_k^T), V = RNE16(x W_v^T)    (fp16 operands, fp32 accumulation)
 * each rounded to fp16 as an fp16 cache would hold it, then compressed exactly as
 * polykv_append_k/v would compress those fp16 values (so the pool bytes equal those of
 * polykv_project_kv followed by polykv_append_k/v).
 *  x:        device fp16 [n_tok][hidden], row-major, 16-B aligned (the layer's input rows).
 *  w_k, w_v: device fp16 [n_kv_heads * head_dim][hidden], row-major (a linear layer's weight
 *            [out][in]); output j is dim j % head_dim of KV head j / head_dim.
 *  pool:     device, layout->total_bytes, 256-B aligned; layer `layer`, tokens
 *            [token_begin, token_begin + n_tok) are written (token_begin a multiple of 32;
 *            plane bits of later tokens below the capacity in the last group are kept).
 *  hidden:   a multiple of 64, at most 2^22; head_dim 64 or 128.
 * Errors: NULL, SHAPE, ALIGN, RANGE (layer, token range, token_begin % 32), LAYOUT,
 *         CODEBOOK, DEVICE, LAUNCH.
 */
int polykv_project_compress(const void* x, const void* w_k, const void* w_v, void* pool,
                            const polykv_layout_t* layout, const polykv_codebook_t* cb,
                            int32_t layer, int32_t token_begin, int32_t n_tok, int32_t hidden,
                            void* hip_stream);

/*
 * The same projection without the compression: k_fp16 (and v_fp16 when w_v is not NULL)
 * receive RNE16(x W^T) head-major, [n_heads][n_tok][head_dim] (16-B aligned), the input
 * layout of polykv_append_k/v for one layer. Errors: NULL, SHAPE, ALIGN, DEVICE, LAUNCH.
 */
int polykv_project_kv(const void* x, const void* w_k, const void* w_v, void* k_fp16, void* v_fp16,
                      int32_t n_tok, int32_t hidden, int32_t n_heads, int32_t head_dim,
                      void* hip_stream);

/*
 * Pool -> fp16 keys. PolyKV, Abstract: the shared pool is handed to each agent as an
 * ordinary per-layer KV cache; this reconstructs the keys of layers
 * [layer_begin, layer_begin + layer_count):
 *   k_fp16[l][h][t][i] = RNE16(code * s), s the stored fp16 scale of the 32-entry block.
 * The product is exact in fp32, so the result is the correctly rounded fp16 of the exact
 * reconstruction.
 *  pool:   device, layout->total_bytes, 256-B aligned (read only).
 *  k_fp16: device, contiguous [layer_count][n_kv_heads][n_tokens][head_dim] binary16,
 *          16-B aligned (written).
 * Errors: NULL, ALIGN, RANGE, LAYOUT, DEVICE, LAUNCH.
 */
int polykv_dequant_k(const void* pool, const polykv_layout_t* layout, void* k_fp16,
                     int32_t layer_begin, int32_t layer_count, void* hip_stream);

/*
 * Pool -> fp16 values, as polykv_dequant_k: v_fp16[l][h][t] = RNE16((n16 / d) * H c[code])
 * with n16 the stored norm, c the codebook centroids (cb: host pointer or NULL for the
 * default; only the centroids are used) and H the +-1 Sylvester matrix (inverse of the
 * compress rotation). The transform runs in fp32 before the one rounding to fp16, so an
 * element can differ from the correctly rounded value by one fp16 ulp where the exact
 * value lies within ~1e-6 relative of a rounding midpoint.
 * Errors: NULL, ALIGN, RANGE, LAYOUT, CODEBOOK, DEVICE, LAUNCH.
 */
int polykv_dequant_v(const void* pool, const polykv_layout_t* layout, const polykv_codebook_t* cb,
                     void* v_fp16, int32_t layer_begin, int32_t layer_count, void* hip_stream);


/* The decode kernel POLYKV_PATH_AUTO selects for these arguments (POLYKV_PATH_VALU or
 * POLYKV_PATH_MFMA), or a negative error code (NULL, SHAPE, LAYOUT). Host only. */
int polykv_attend_path(const polykv_layout_t* layout, int32_t n_agents, int32_t gqa);

/* Device bytes of workspace polykv_attend_shared needs for these arguments (0 if none). */
size_t polykv_attend_workspace_bytes(const polykv_layout_t* layout, int32_t n_agents,
                                     int32_t gqa, int32_t layer_count);

/*
 * One decode step of every agent against the shared pool. PolyKV, Abstract: one compressed
 * pool serves several separate agent contexts at once. The pool is only read, so any
 * number of calls may run concurrently on one pool.
 *  q:   device fp32 [layer_count][n_agents][n_kv_heads * gqa][head_dim], 16-B aligned;
 *       query head j of an agent attends KV head j / gqa.
 *  out: device fp32, same shape as q; every element is written.
 *  softmax_scale: multiplies q . k_hat before the softmax (normally 1/sqrt(head_dim)).
 *  cb: host codebook or NULL for the default; only the centroids are used.
 *  workspace: device, at least polykv_attend_workspace_bytes(...) bytes (may be NULL
 *       when that is 0).
 *  n_agents * gqa may be any count up to INT32_MAX (SHAPE above that): the rows of a tile
 *  are served in passes of POLYKV_ROWS_PER_PASS rows in agent-major order, one launch per
 *  pass, so each pass reads the whole pool once. Arguments are checked before the first
 *  launch.
 * Errors: NULL, SHAPE, ALIGN, RANGE, LAYOUT, CODEBOOK, WORKSPACE, DEVICE, LAUNCH.
 */
int polykv_attend_shared(const void* pool, const polykv_layout_t* layout,
                         const polykv_codebook_t* cb, const float* q, float* out,
                         int32_t n_agents, int32_t gqa, float softmax_scale,
                         int32_t layer_begin, int32_t layer_count,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* As polykv_attend_shared with an explicit decode kernel (POLYKV_PATH_*). */
int polykv_attend_shared_path(const void* pool, const polykv_layout_t* layout,
                              const polykv_codebook_t* cb, const float* q, float* out,
                              int32_t n_agents, int32_t gqa, float softmax_scale,
                              int32_t layer_begin, int32_t layer_count,
                              void* workspace, size_t workspace_bytes, void* hip_stream,
                              int32_t path);

/*
 * As polykv_attend_shared_path, and also the log-sum-exp of every output row:
 *  lse: device fp32 [layer_count][n_agents][n_kv_heads * gqa] (4-B aligned) or NULL;
 *       lse = ln sum_t exp(softmax_scale * q . k_hat_t) over the pool's tokens, the
 *       quantity that merges this result with attention over other tokens.
 * Errors: as polykv_attend_shared_path.
 */
int polykv_attend_shared_lse(const void* pool, const polykv_layout_t* layout,
                             const polykv_codebook_t* cb, const float* q, float* out,
                             float* lse, int32_t n_agents, int32_t gqa, float softmax_scale,
                             int32_t layer_begin, int32_t layer_count,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             int32_t path);

/*
 * As polykv_attend_shared_lse over tokens [0, n_valid) of every tile only, for a pool that
 * is filled by polykv_append_k/v up to n_valid tokens (1 <= n_valid <= n_tokens). Tokens
 * at or past n_valid are never used, whatever their bytes hold, and no byte of a token at
 * or past n_valid rounded up to a multiple of 32 is read: the call may run concurrently
 * with an append whose chunk starts there or later.
 * Errors: as polykv_attend_shared_path; RANGE also for n_valid outside [1, n_tokens].
 */
int polykv_attend_shared_prefix(const void* pool, const polykv_layout_t* layout,
                                const polykv_codebook_t* cb, const float* q, float* out,
                                float* lse, int32_t n_valid, int32_t n_agents, int32_t gqa,
                                float softmax_scale, int32_t layer_begin, int32_t layer_count,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                int32_t path);

/*
 * Private tails. PolyKV, Abstract: the one compressed pool is handed to N separate agent
 * contexts, each of which goes on by itself; the tokens an agent adds after the pool was
 * written are its own, kept uncompressed. This call attends every query row over its
 * agent's tail and merges that with the shared-pool result, so that out becomes softmax
 * attention over the union of pool and tail tokens:
 *   M = max(lse_p, lse_t), w_p = exp(lse_p - M), w_t = exp(lse_t - M),
 *   out = (w_p out_p + w_t out_t) / (w_p + w_t),  lse = M + ln(w_p + w_t).
 *  layout:  supplies n_kv_heads and head_dim (the pool itself is not read).
 *  q:       device fp32 [layer_count][n_agents][n_kv_heads * gqa][head_dim], 16-B aligned,
 *           the same queries the pool result was computed for.
 *  out, lse: device, in: the result of polykv_attend_shared_lse for q; out: the merged
 *           result (rows of an agent with an empty tail are left as they are).
 *  tail_k, tail_v: device fp16 [n_agents][layer_count][n_kv_heads][tail_cap][head_dim],
 *           16-B aligned; query head j of an agent reads KV head j / gqa of its own tail.
 *  tail_len: device int32 [n_agents]; agent a uses tail tokens [0, tail_len[a]); values
 *           outside [0, tail_cap] are clamped into it.
 *  tail_cap = 0 returns POLYKV_OK without any device work (tail_k, tail_v may be NULL).
 * Errors: NULL, SHAPE, ALIGN, RANGE, LAYOUT, ARG, DEVICE, LAUNCH.
 */
int polykv_attend_tail_merge(const polykv_layout_t* layout, const float* q, float* out,
                             float* lse, const void* tail_k, const void* tail_v,
                             const int32_t* tail_len, int32_t tail_cap, int32_t n_agents,
                             int32_t gqa, float softmax_scale, int32_t layer_count,
                             void* hip_stream);

/* Static English text for a return code. Never NULL. */
const char* polykv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* POLYKV_H */
