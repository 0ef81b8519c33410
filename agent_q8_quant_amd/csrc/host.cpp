// Host side of the C ABI: layout arithmetic, the built-in codebook, argument validation
// and kernel dispatch. Nothing here allocates device memory or synchronises.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "polykv.h"
#include "polykv_internal.h"

namespace {

constexpr uint64_t kAlign = 256;

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool shape_ok(const polykv_shape_t& s) {
    if (s.n_layers < 1 || s.n_kv_heads < 1 || s.n_tokens < 1) return false;
    if (!(s.head_dim == 64 || s.head_dim == 128 || s.head_dim == 256))
        return false;
    // keep every per-tile and whole-pool quantity comfortably inside 63 bits
    if (s.n_tokens > (1 << 26) || (int64_t)s.n_layers * s.n_kv_heads > (1 << 24)) return false;
    return true;
}

int compute_layout(const polykv_shape_t& s, polykv_layout_t* out) {
    if (!shape_ok(s)) return POLYKV_ERR_SHAPE;
    const uint64_t T = (uint64_t)s.n_tokens, d = (uint64_t)s.head_dim;
    const uint64_t tiles = (uint64_t)s.n_layers * (uint64_t)s.n_kv_heads;
    const uint64_t groups = (T + 31) / 32;
    polykv_layout_t l;
    std::memset(&l, 0, sizeof(l));
    l.shape = s;
    l.k_codes_tile_stride = round_up(T * d, kAlign);
    l.k_scales_tile_stride = round_up(T * (d / 32) * 2, kAlign);
    l.v_planes_tile_stride = round_up(groups * 3 * d * 4, kAlign);
    l.v_norms_tile_stride = round_up(T * 2, kAlign);
    uint64_t off = 0;
    l.k_codes_off = off;
    off += tiles * l.k_codes_tile_stride;
    l.k_scales_off = off;
    off += tiles * l.k_scales_tile_stride;
    l.v_planes_off = off;
    off += tiles * l.v_planes_tile_stride;
    l.v_norms_off = off;
    off += tiles * l.v_norms_tile_stride;
    l.total_bytes = off;
    l.analytic_bytes = tiles * T * (d + 2 * (d / 32) + (3 * d) / 8 + 2);
    *out = l;
    return POLYKV_OK;
}

// ---- Lloyd-Max codebook for N(0,1), fp64 ----------------------------------------------

double pdf(double x) {
    if (std::isinf(x)) return 0.0;
    return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }
double cell_mass(double a, double b) {
    if (b <= 0.0) return cell_mass(-b, -a);
    return upper_tail(a) - upper_tail(b);
}

polykv_codebook_t build_codebook() {
    // Lloyd's iteration from evenly spaced centroids; the fixed point for the Gaussian is
    // unique, so the start only changes the number of iterations.
    double c[8];
    for (int k = 0; k < 8; ++k) c[k] = -2.1 + 0.6 * k;
    for (int it = 0; it < 100000; ++it) {
        double t[9];
        t[0] = -INFINITY;
        t[8] = INFINITY;
        for (int k = 0; k < 7; ++k) t[k + 1] = 0.5 * (c[k] + c[k + 1]);
        double delta = 0.0;
        for (int k = 0; k < 8; ++k) {
            double mean = (pdf(t[k]) - pdf(t[k + 1])) / cell_mass(t[k], t[k + 1]);
            delta = std::fmax(delta, std::fabs(mean - c[k]));
            c[k] = mean;
        }
        if (delta < 1e-15) break;
    }
    polykv_codebook_t cb;
    for (int k = 0; k < 8; ++k) cb.centroid[k] = (float)((c[k] - c[7 - k]) / 2.0);
    for (int k = 0; k < 7; ++k)
        cb.boundary[k] = (float)(((double)cb.centroid[k] + (double)cb.centroid[k + 1]) / 2.0);
    return cb;
}

const polykv_codebook_t& default_codebook() {
    static const polykv_codebook_t cb = build_codebook();
    return cb;
}

bool codebook_ok(const polykv_codebook_t& cb) {
    for (int k = 0; k < 8; ++k) {
        if (!std::isfinite(cb.centroid[k]) || cb.centroid[k] != -cb.centroid[7 - k]) return false;
        if (k < 7 && !(cb.centroid[k] < cb.centroid[k + 1])) return false;
    }
    for (int k = 0; k < 7; ++k) {
        if (!std::isfinite(cb.boundary[k]) || cb.boundary[k] != -cb.boundary[6 - k]) return false;
        if (k < 6 && !(cb.boundary[k] < cb.boundary[k + 1])) return false;
    }
    return cb.boundary[3] == 0.0f;
}

// Scale lambda in [1, 2) (steps of 2^-16) minimising the worst relative fp16 rounding
// error of lambda * c over the four positive centroids.
float fp16_friendly_scale(const float* c) {
    float best_lam = 1.0f;
    double best_err = 1e30;
    for (int i = 0; i < 65536; ++i) {
        const float lam = 1.0f + (float)i / 65536.0f;
        double err = 0.0;
        for (int k = 0; k < 4; ++k) {
            const float v = lam * c[k];
            const double h = (double)(float)(_Float16)v;
            err = std::fmax(err, std::fabs(h - (double)v) / (double)v);
        }
        if (err < best_err) {
            best_err = err;
            best_lam = lam;
        }
    }
    return best_lam;
}

polykv::CodebookHalf half_of(const polykv_codebook_t& cb) {
    polykv::CodebookHalf h;
    for (int k = 0; k < 4; ++k) h.centroid_pos[k] = cb.centroid[4 + k];
    for (int k = 0; k < 3; ++k) h.boundary_pos[k] = cb.boundary[4 + k];
    // the default codebook's scale is computed once; another codebook's is cached per
    // thread for as long as the same codebook keeps being passed
    static const float default_scale = fp16_friendly_scale(&default_codebook().centroid[4]);
    if (std::memcmp(&cb, &default_codebook(), sizeof(cb)) == 0) {
        h.fp16_scale = default_scale;
    } else {
        thread_local polykv_codebook_t last_cb;
        thread_local float last_scale = 0.0f;
        if (last_scale == 0.0f || std::memcmp(&cb, &last_cb, sizeof(cb)) != 0) {
            last_scale = fp16_friendly_scale(h.centroid_pos);
            last_cb = cb;
        }
        h.fp16_scale = last_scale;
    }
    return h;
}

// ---- validation ----------------------------------------------------------------------

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_layout(const polykv_layout_t* layout) {
    if (!layout) return POLYKV_ERR_NULL;
    polykv_layout_t want;
    int rc = compute_layout(layout->shape, &want);
    if (rc != POLYKV_OK) return rc;
    if (std::memcmp(&want, layout, sizeof(want)) != 0) return POLYKV_ERR_LAYOUT;
    return POLYKV_OK;
}

int check_layers(const polykv_layout_t& l, int32_t begin, int32_t count) {
    if (count < 1 || begin < 0 || (int64_t)begin + count > l.shape.n_layers) return POLYKV_ERR_RANGE;
    return POLYKV_OK;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return POLYKV_ERR_DEVICE;
    }
    // one entry per device ordinal; computed once, read many times
    static std::mutex mu;
    static int verdict[64];  // 0 unknown, 1 ok, -1 not gfx950
    if (dev < 0 || dev >= 64) return POLYKV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (verdict[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return POLYKV_ERR_DEVICE;
        }
        verdict[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return verdict[dev] == 1 ? POLYKV_OK : POLYKV_ERR_DEVICE;
}

int launch_rc(hipError_t e) {
    if (e != hipSuccess) return POLYKV_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return POLYKV_ERR_LAUNCH;
    return POLYKV_OK;
}

}  // namespace

extern "C" {

int polykv_pool_layout(const polykv_shape_t* shape, polykv_layout_t* out) {
    if (!shape || !out) return POLYKV_ERR_NULL;
    return compute_layout(*shape, out);
}

int polykv_codebook_default(polykv_codebook_t* out) {
    if (!out) return POLYKV_ERR_NULL;
    *out = default_codebook();
    return POLYKV_OK;
}

int polykv_compress_k(const void* k_fp16, void* pool, const polykv_layout_t* layout,
                      int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!k_fp16 || !pool || !layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(k_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_compress_k(k_fp16, (uint8_t*)pool, polykv::make_geom(*layout),
                                               layer_begin, layer_count, (hipStream_t)hip_stream));
}

int polykv_compress_v(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                      const polykv_codebook_t* cb, int32_t layer_begin, int32_t layer_count,
                      void* hip_stream) {
    return polykv_compress_v_path(v_fp16, pool, layout, cb, layer_begin, layer_count, hip_stream,
                                  POLYKV_PATH_AUTO);
}

int polykv_compress_v_path(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                           const polykv_codebook_t* cb, int32_t layer_begin, int32_t layer_count,
                           void* hip_stream, int32_t path) {
    if (!v_fp16 || !pool || !layout) return POLYKV_ERR_NULL;
    if (path < POLYKV_PATH_AUTO || path > POLYKV_PATH_MFMA) return POLYKV_ERR_ARG;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(v_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    const bool mfma_ok = layout->shape.head_dim == 64 || layout->shape.head_dim == 128;
    if (path == POLYKV_PATH_MFMA && !mfma_ok) return POLYKV_ERR_SHAPE;
    const bool valu = path == POLYKV_PATH_VALU || !mfma_ok;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_compress_v(v_fp16, (uint8_t*)pool, polykv::make_geom(*layout),
                                               half_of(book), layer_begin, layer_count,
                                               (hipStream_t)hip_stream, valu));
}

static int check_tokens(const polykv_layout_t& l, int32_t token_begin, int32_t n_new) {
    if (token_begin < 0 || n_new < 1 || (int64_t)token_begin + n_new > l.shape.n_tokens)
        return POLYKV_ERR_RANGE;
    return POLYKV_OK;
}

int polykv_append_k(const void* k_fp16, void* pool, const polykv_layout_t* layout,
                    int32_t token_begin, int32_t n_new, int32_t layer_begin, int32_t layer_count,
                    void* hip_stream) {
    if (!k_fp16 || !pool || !layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(k_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((rc = check_tokens(*layout, token_begin, n_new))) return rc;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_compress_k_range(k_fp16, (uint8_t*)pool, polykv::make_geom(*layout),
                                                     token_begin, n_new, layer_begin, layer_count,
                                                     (hipStream_t)hip_stream));
}

int polykv_append_v(const void* v_fp16, void* pool, const polykv_layout_t* layout,
                    const polykv_codebook_t* cb, int32_t token_begin, int32_t n_new,
                    int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!v_fp16 || !pool || !layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(v_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((rc = check_tokens(*layout, token_begin, n_new))) return rc;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_compress_v_range(v_fp16, (uint8_t*)pool, polykv::make_geom(*layout),
                                                     half_of(book), token_begin, n_new, layer_begin,
                                                     layer_count, (hipStream_t)hip_stream));
}

static int kv_impl(const void* k_fp16, const void* v_fp16, void* pool, const polykv_layout_t* layout,
                   const polykv_codebook_t* cb, int32_t token_begin, int32_t n_new,
                   int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!k_fp16 || !v_fp16 || !pool || !layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(k_fp16, 16) || !aligned(v_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((rc = check_tokens(*layout, token_begin, n_new))) return rc;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_compress_kv_range(k_fp16, v_fp16, (uint8_t*)pool,
                                                      polykv::make_geom(*layout), half_of(book),
                                                      token_begin, n_new, layer_begin, layer_count,
                                                      (hipStream_t)hip_stream));
}

int polykv_compress_kv(const void* k_fp16, const void* v_fp16, void* pool,
                       const polykv_layout_t* layout, const polykv_codebook_t* cb,
                       int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!layout) return POLYKV_ERR_NULL;
    return kv_impl(k_fp16, v_fp16, pool, layout, cb, 0, layout->shape.n_tokens, layer_begin,
                   layer_count, hip_stream);
}

int polykv_append_kv(const void* k_fp16, const void* v_fp16, void* pool,
                     const polykv_layout_t* layout, const polykv_codebook_t* cb,
                     int32_t token_begin, int32_t n_new, int32_t layer_begin,
                     int32_t layer_count, void* hip_stream) {
    return kv_impl(k_fp16, v_fp16, pool, layout, cb, token_begin, n_new, layer_begin,
                   layer_count, hip_stream);
}

static int check_projection(int32_t n_tok, int32_t hidden, int32_t n_heads, int32_t head_dim) {
    // hidden <= 2^22 keeps every per-lane byte offset of a 256-row operand tile in 32 bits
    if (n_tok < 1 || n_heads < 1 || hidden < 64 || hidden % 64 != 0 || hidden > (1 << 22)) return POLYKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return POLYKV_ERR_SHAPE;
    return POLYKV_OK;
}

int polykv_project_kv(const void* x, const void* w_k, const void* w_v, void* k_fp16, void* v_fp16,
                      int32_t n_tok, int32_t hidden, int32_t n_heads, int32_t head_dim,
                      void* hip_stream) {
    if (!x || !w_k || !k_fp16 || (w_v && !v_fp16)) return POLYKV_ERR_NULL;
    int rc = check_projection(n_tok, hidden, n_heads, head_dim);
    if (rc) return rc;
    if (!aligned(x, 16) || !aligned(w_k, 16) || !aligned(k_fp16, 16) ||
        (w_v && (!aligned(w_v, 16) || !aligned(v_fp16, 16))))
        return POLYKV_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_project((const __half*)x, (const __half*)w_k, (const __half*)w_v,
                                            (__half*)k_fp16, (__half*)v_fp16, n_tok, hidden, n_heads,
                                            head_dim, (hipStream_t)hip_stream));
}

int polykv_project_compress(const void* x, const void* w_k, const void* w_v, void* pool,
                            const polykv_layout_t* layout, const polykv_codebook_t* cb, int32_t layer,
                            int32_t token_begin, int32_t n_tok, int32_t hidden, void* hip_stream) {
    if (!x || !w_k || !w_v || !pool || !layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if ((rc = check_projection(n_tok, hidden, layout->shape.n_kv_heads, layout->shape.head_dim))) return rc;
    if (!aligned(pool, 256) || !aligned(x, 16) || !aligned(w_k, 16) || !aligned(w_v, 16))
        return POLYKV_ERR_ALIGN;
    if (layer < 0 || layer >= layout->shape.n_layers) return POLYKV_ERR_RANGE;
    if ((rc = check_tokens(*layout, token_begin, n_tok))) return rc;
    if (token_begin % 32 != 0) return POLYKV_ERR_RANGE;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_project_compress((const __half*)x, (const __half*)w_k, (const __half*)w_v,
                                                     (uint8_t*)pool, polykv::make_geom(*layout),
                                                     half_of(book), layer, token_begin, n_tok, hidden,
                                                     (hipStream_t)hip_stream));
}

int polykv_dequant_k(const void* pool, const polykv_layout_t* layout, void* k_fp16,
                     int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!pool || !layout || !k_fp16) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(k_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_dequant_k((const uint8_t*)pool, k_fp16, polykv::make_geom(*layout),
                                              layer_begin, layer_count, (hipStream_t)hip_stream));
}

int polykv_dequant_v(const void* pool, const polykv_layout_t* layout, const polykv_codebook_t* cb,
                     void* v_fp16, int32_t layer_begin, int32_t layer_count, void* hip_stream) {
    if (!pool || !layout || !v_fp16) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (!aligned(pool, 256) || !aligned(v_fp16, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    if ((rc = check_device())) return rc;
    return launch_rc(polykv::launch_dequant_v((const uint8_t*)pool, v_fp16, polykv::make_geom(*layout),
                                              half_of(book), layer_begin, layer_count,
                                              (hipStream_t)hip_stream));
}

// Rows per tile are served in passes of at most POLYKV_ROWS_PER_PASS; every pass has at
// least one row, so the kernel choice is the same for all of them.
static int32_t first_pass_rows(int32_t n_agents, int32_t gqa) {
    return (int32_t)std::min<int64_t>((int64_t)n_agents * gqa, POLYKV_ROWS_PER_PASS);
}

static int resolve_path(const polykv::PoolGeom& g, int32_t rows, int32_t path) {
    if (path == POLYKV_PATH_AUTO)
        return polykv::attend_mfma_supported(g, rows) ? POLYKV_PATH_MFMA : POLYKV_PATH_VALU;
    return path;
}

int polykv_attend_path(const polykv_layout_t* layout, int32_t n_agents, int32_t gqa) {
    if (!layout) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (n_agents < 1 || gqa < 1) return POLYKV_ERR_SHAPE;
    if ((int64_t)n_agents * gqa > INT32_MAX) return POLYKV_ERR_SHAPE;
    polykv::PoolGeom g = polykv::make_geom(*layout);
    return resolve_path(g, first_pass_rows(n_agents, gqa), POLYKV_PATH_AUTO);
}

size_t polykv_attend_workspace_bytes(const polykv_layout_t* layout, int32_t n_agents,
                                     int32_t gqa, int32_t layer_count) {
    if (!layout || check_layout(layout) != POLYKV_OK || n_agents < 1 || gqa < 1 || layer_count < 1)
        return 0;
    if ((int64_t)n_agents * gqa > INT32_MAX) return 0;
    polykv::PoolGeom g = polykv::make_geom(*layout);
    return polykv::attend_workspace_bytes(g, n_agents, gqa, layer_count,
                                          resolve_path(g, first_pass_rows(n_agents, gqa), POLYKV_PATH_AUTO));
}

static int attend_impl(const void* pool, const polykv_layout_t* layout,
                       const polykv_codebook_t* cb, const float* q, float* out, float* lse,
                       int32_t n_valid, int32_t n_agents, int32_t gqa, float softmax_scale,
                       int32_t layer_begin, int32_t layer_count, void* workspace,
                       size_t workspace_bytes, void* hip_stream, int32_t path) {
    if (!pool || !layout || !q || !out) return POLYKV_ERR_NULL;
    if (lse && !aligned(lse, 4)) return POLYKV_ERR_ALIGN;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (n_agents < 1 || gqa < 1) return POLYKV_ERR_SHAPE;
    if (!aligned(pool, 256) || !aligned(q, 16) || !aligned(out, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_layers(*layout, layer_begin, layer_count))) return rc;
    if ((int64_t)n_agents * gqa > INT32_MAX) return POLYKV_ERR_SHAPE;
    if (!std::isfinite(softmax_scale)) return POLYKV_ERR_ARG;
    if (path < POLYKV_PATH_AUTO || path > POLYKV_PATH_MFMA) return POLYKV_ERR_ARG;
    const polykv_codebook_t& book = cb ? *cb : default_codebook();
    if (!codebook_ok(book)) return POLYKV_ERR_CODEBOOK;
    if (n_valid < 1 || n_valid > layout->shape.n_tokens) return POLYKV_ERR_RANGE;
    polykv::PoolGeom g = polykv::make_geom(*layout);
    g.n_tokens = n_valid;               // attend over tokens [0, n_valid) of every tile
    g.n_groups = (n_valid + 31) / 32;   // (strides and offsets stay those of the layout)
    const int32_t rows = n_agents * gqa;
    path = resolve_path(g, first_pass_rows(n_agents, gqa), path);
    if (path == POLYKV_PATH_MFMA && !polykv::attend_mfma_supported(g, first_pass_rows(n_agents, gqa)))
        return POLYKV_ERR_SHAPE;
    size_t need = polykv::attend_workspace_bytes(g, n_agents, gqa, layer_count, path);
    if (need > 0 && (!workspace || workspace_bytes < need)) return POLYKV_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 16)) return POLYKV_ERR_ALIGN;
    if ((rc = check_device())) return rc;
    polykv::AttendArgs a;
    a.pool = (const uint8_t*)pool;
    a.g = g;
    a.cb = half_of(book);
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.n_agents = n_agents;
    a.gqa = gqa;
    a.layer_begin = layer_begin;
    a.layer_count = layer_count;
    a.softmax_scale = softmax_scale;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    hipStream_t s = (hipStream_t)hip_stream;
    // one launch per pass of at most POLYKV_ROWS_PER_PASS rows; each streams the pool once
    for (int64_t r0 = 0; r0 < rows; r0 += POLYKV_ROWS_PER_PASS) {
        a.row_begin = (int32_t)r0;
        a.n_rows = (int32_t)std::min<int64_t>(POLYKV_ROWS_PER_PASS, rows - r0);
        rc = launch_rc(path == POLYKV_PATH_MFMA ? polykv::launch_attend_mfma(a, s)
                                                : polykv::launch_attend_valu(a, s));
        if (rc) return rc;
    }
    return POLYKV_OK;
}

int polykv_attend_shared_lse(const void* pool, const polykv_layout_t* layout,
                             const polykv_codebook_t* cb, const float* q, float* out,
                             float* lse, int32_t n_agents, int32_t gqa, float softmax_scale,
                             int32_t layer_begin, int32_t layer_count, void* workspace,
                             size_t workspace_bytes, void* hip_stream, int32_t path) {
    return attend_impl(pool, layout, cb, q, out, lse, layout ? layout->shape.n_tokens : 1,
                       n_agents, gqa, softmax_scale, layer_begin, layer_count, workspace,
                       workspace_bytes, hip_stream, path);
}

int polykv_attend_shared_prefix(const void* pool, const polykv_layout_t* layout,
                                const polykv_codebook_t* cb, const float* q, float* out,
                                float* lse, int32_t n_valid, int32_t n_agents, int32_t gqa,
                                float softmax_scale, int32_t layer_begin, int32_t layer_count,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                int32_t path) {
    return attend_impl(pool, layout, cb, q, out, lse, n_valid, n_agents, gqa, softmax_scale,
                       layer_begin, layer_count, workspace, workspace_bytes, hip_stream, path);
}

int polykv_attend_shared_path(const void* pool, const polykv_layout_t* layout,
                              const polykv_codebook_t* cb, const float* q, float* out,
                              int32_t n_agents, int32_t gqa, float softmax_scale,
                              int32_t layer_begin, int32_t layer_count, void* workspace,
                              size_t workspace_bytes, void* hip_stream, int32_t path) {
    return polykv_attend_shared_lse(pool, layout, cb, q, out, nullptr, n_agents, gqa,
                                    softmax_scale, layer_begin, layer_count, workspace,
                                    workspace_bytes, hip_stream, path);
}

int polykv_attend_tail_merge(const polykv_layout_t* layout, const float* q, float* out,
                             float* lse, const void* tail_k, const void* tail_v,
                             const int32_t* tail_len, int32_t tail_cap, int32_t n_agents,
                             int32_t gqa, float softmax_scale, int32_t layer_count,
                             void* hip_stream) {
    if (!layout || !q || !out || !lse || !tail_len) return POLYKV_ERR_NULL;
    int rc = check_layout(layout);
    if (rc) return rc;
    if (n_agents < 1 || gqa < 1 || tail_cap < 0) return POLYKV_ERR_SHAPE;
    if (layer_count < 1 || layer_count > layout->shape.n_layers) return POLYKV_ERR_RANGE;
    // one workgroup per (layer, agent, KV head)
    if ((int64_t)layer_count * n_agents * layout->shape.n_kv_heads > INT32_MAX) return POLYKV_ERR_SHAPE;
    if (!std::isfinite(softmax_scale)) return POLYKV_ERR_ARG;
    if (tail_cap > 0 && (!tail_k || !tail_v)) return POLYKV_ERR_NULL;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4) || !aligned(tail_len, 4))
        return POLYKV_ERR_ALIGN;
    if (tail_cap > 0 && (!aligned(tail_k, 16) || !aligned(tail_v, 16))) return POLYKV_ERR_ALIGN;
    if (tail_cap == 0) return POLYKV_OK;  // no tail tokens: the pool result stands
    if ((rc = check_device())) return rc;
    polykv::TailArgs a;
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.tail_k = tail_k;
    a.tail_v = tail_v;
    a.tail_len = tail_len;
    a.tail_cap = tail_cap;
    a.n_kv_heads = layout->shape.n_kv_heads;
    a.head_dim = layout->shape.head_dim;
    a.gqa = gqa;
    a.n_agents = n_agents;
    a.layer_count = layer_count;
    a.softmax_scale = softmax_scale;
    return launch_rc(polykv::launch_attend_tail(a, (hipStream_t)hip_stream));
}

int polykv_attend_shared(const void* pool, const polykv_layout_t* layout,
                         const polykv_codebook_t* cb, const float* q, float* out,
                         int32_t n_agents, int32_t gqa, float softmax_scale,
                         int32_t layer_begin, int32_t layer_count, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
    return polykv_attend_shared_path(pool, layout, cb, q, out, n_agents, gqa, softmax_scale,
                                     layer_begin, layer_count, workspace, workspace_bytes,
                                     hip_stream, POLYKV_PATH_AUTO);
}

const char* polykv_strerror(int code) {
    switch (code) {
        case POLYKV_OK: return "ok";
        case POLYKV_ERR_NULL: return "a required pointer is NULL";
        case POLYKV_ERR_SHAPE: return "unsupported shape (head_dim, counts or sizes)";
        case POLYKV_ERR_ALIGN: return "misaligned buffer (pool needs 256 B, others 16 B)";
        case POLYKV_ERR_RANGE: return "layer range or rows per tile out of range";
        case POLYKV_ERR_WORKSPACE: return "workspace missing or too small";
        case POLYKV_ERR_DEVICE: return "no HIP device or the device is not gfx950";
        case POLYKV_ERR_LAUNCH: return "kernel launch failed";
        case POLYKV_ERR_CODEBOOK: return "codebook not ascending, not symmetric, or boundary[3] != 0";
        case POLYKV_ERR_LAYOUT: return "layout does not match polykv_pool_layout for its shape";
        case POLYKV_ERR_ARG: return "argument out of its domain";
        default: return "unknown error code";
    }
}

}  // extern "C"
