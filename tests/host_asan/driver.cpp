// Drives every entry point of the host layer (host.cpp), built with the address and
// undefined-behaviour sanitizers against the stand-ins of stubs.cpp: layouts of valid and
// invalid shapes, the built-in codebook, every validation path, and the dispatch that
// follows it (which launcher runs, with which geometry and token range). Exits non-zero on
// the first unexpected result; the sanitizers abort on any memory or UB error.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "polykv.h"
#include "stubs.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static polykv_layout_t layout(int L, int H, int d, int T) {
    polykv_shape_t s = {L, H, d, T};
    polykv_layout_t l;
    const int rc = polykv_pool_layout(&s, &l);
    CHECK(rc == POLYKV_OK);
    return l;
}

static void layouts() {
    for (int d : {64, 128, 256})
        for (int T : {1, 31, 32, 33, 600, 4096, 7194}) {
            polykv_layout_t l = layout(3, 5, d, T);
            const uint64_t per = (uint64_t)d + d / 16 + 3 * d / 8 + 2;
            CHECK(l.analytic_bytes == 15ull * T * per);
            CHECK(l.total_bytes >= l.analytic_bytes && l.total_bytes % 256 == 0);
            CHECK(l.k_codes_off % 256 == 0 && l.k_scales_off % 256 == 0);
            CHECK(l.v_planes_off % 256 == 0 && l.v_norms_off % 256 == 0);
        }
    polykv_layout_t out;
    for (polykv_shape_t s : {polykv_shape_t{1, 1, 32, 10}, polykv_shape_t{1, 1, 96, 10},
                             polykv_shape_t{0, 1, 128, 10}, polykv_shape_t{1, 0, 128, 10},
                             polykv_shape_t{1, 1, 128, 0}, polykv_shape_t{1, 1, 128, -5},
                             polykv_shape_t{1 << 20, 1 << 20, 128, 1 << 20},
                             polykv_shape_t{1, 1, 128, 0x7fffffff}})
        CHECK(polykv_pool_layout(&s, &out) == POLYKV_ERR_SHAPE);
    CHECK(polykv_pool_layout(nullptr, &out) == POLYKV_ERR_NULL);
    polykv_shape_t s = {1, 1, 128, 10};
    CHECK(polykv_pool_layout(&s, nullptr) == POLYKV_ERR_NULL);
}

static void codebook() {
    polykv_codebook_t cb;
    CHECK(polykv_codebook_default(&cb) == POLYKV_OK);
    for (int k = 0; k < 8; ++k) CHECK(cb.centroid[k] == -cb.centroid[7 - k]);
    for (int k = 0; k < 7; ++k) CHECK(cb.centroid[k] < cb.boundary[k] && cb.boundary[k] < cb.centroid[k + 1]);
    CHECK(cb.boundary[3] == 0.0f);
    CHECK(std::fabs(cb.centroid[7] - 2.151946f) < 1e-5f);
    CHECK(polykv_codebook_default(nullptr) == POLYKV_ERR_NULL);
}

static void compress_and_append() {
    polykv_layout_t l = layout(4, 2, 128, 333);
    void* pool = P(0x100000);
    void* src = P(0x200000);
    polykv_codebook_t cb;
    polykv_codebook_default(&cb);

    g_stub.calls = 0;
    CHECK(polykv_compress_k(src, pool, &l, 1, 3, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "compress_k") == 0 && g_stub.a0 == 1 && g_stub.a1 == 3);
    CHECK(g_stub.geom.n_tokens == 333 && g_stub.geom.n_groups == 11 && g_stub.geom.head_dim == 128);
    CHECK(polykv_compress_v(src, pool, &l, nullptr, 0, 4, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "compress_v") == 0 && !g_stub.valu);
    CHECK(g_stub.cb.centroid_pos[3] == cb.centroid[7] && g_stub.cb.fp16_scale >= 1.0f && g_stub.cb.fp16_scale < 2.0f);
    CHECK(polykv_compress_v_path(src, pool, &l, &cb, 0, 4, nullptr, POLYKV_PATH_VALU) == POLYKV_OK && g_stub.valu);
    CHECK(polykv_compress_v_path(src, pool, &l, &cb, 0, 4, nullptr, 3) == POLYKV_ERR_ARG);
    CHECK(polykv_compress_kv(src, src, pool, &l, nullptr, 0, 4, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "compress_kv_range") == 0 && g_stub.a0 == 0 && g_stub.a1 == 333);
    CHECK(polykv_append_kv(src, src, pool, &l, nullptr, 100, 33, 2, 2, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "compress_kv_range") == 0 && g_stub.a0 == 100 && g_stub.a1 == 33);
    CHECK(polykv_append_k(src, pool, &l, 332, 1, 0, 4, nullptr) == POLYKV_OK && g_stub.a0 == 332);
    CHECK(polykv_append_v(src, pool, &l, nullptr, 0, 333, 0, 4, nullptr) == POLYKV_OK && g_stub.a1 == 333);

    // validation: nothing reaches a launcher
    const int before = g_stub.calls;
    CHECK(polykv_compress_k(nullptr, pool, &l, 0, 4, nullptr) == POLYKV_ERR_NULL);
    CHECK(polykv_compress_k(src, P(0x100010), &l, 0, 4, nullptr) == POLYKV_ERR_ALIGN);
    CHECK(polykv_compress_k(P(0x200008), pool, &l, 0, 4, nullptr) == POLYKV_ERR_ALIGN);
    CHECK(polykv_compress_k(src, pool, &l, 3, 2, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_compress_k(src, pool, &l, -1, 2, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_compress_kv(src, src, pool, &l, nullptr, 0, 0, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_append_kv(src, src, pool, &l, nullptr, 333, 1, 0, 4, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_append_kv(src, src, pool, &l, nullptr, 0x7fffffff, 0x7fffffff, 0, 4, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_append_v(src, pool, &l, nullptr, 10, 0, 0, 4, nullptr) == POLYKV_ERR_RANGE);
    polykv_codebook_t bad = cb;
    bad.centroid[2] += 1e-3f;
    CHECK(polykv_compress_v(src, pool, &l, &bad, 0, 4, nullptr) == POLYKV_ERR_CODEBOOK);
    bad = cb;
    bad.boundary[3] = 1e-6f;
    CHECK(polykv_compress_kv(src, src, pool, &l, &bad, 0, 4, nullptr) == POLYKV_ERR_CODEBOOK);
    bad = cb;
    bad.centroid[0] = NAN;
    bad.centroid[7] = NAN;
    CHECK(polykv_append_v(src, pool, &l, &bad, 0, 1, 0, 4, nullptr) == POLYKV_ERR_CODEBOOK);
    polykv_layout_t lbad = l;
    lbad.v_norms_off += 256;
    CHECK(polykv_compress_k(src, pool, &lbad, 0, 4, nullptr) == POLYKV_ERR_LAYOUT);
    lbad = l;
    lbad.shape.head_dim = 32;
    CHECK(polykv_compress_v(src, pool, &lbad, nullptr, 0, 4, nullptr) == POLYKV_ERR_SHAPE);
    CHECK(g_stub.calls == before);

    // a custom codebook (scaled copy of the default) is accepted, its fp16 scale recomputed
    polykv_codebook_t sc = cb;
    for (int k = 0; k < 8; ++k) sc.centroid[k] *= 1.5f;
    for (int k = 0; k < 7; ++k) sc.boundary[k] *= 1.5f;
    CHECK(polykv_compress_v(src, pool, &l, &sc, 0, 4, nullptr) == POLYKV_OK);
    CHECK(g_stub.cb.centroid_pos[0] == sc.centroid[4]);
    CHECK(g_stub.cb.fp16_scale >= 1.0f && g_stub.cb.fp16_scale < 2.0f);
}

static void decode() {
    polykv_layout_t l = layout(2, 4, 128, 100);
    void* pool = P(0x100000);
    const float* q = static_cast<const float*>(P(0x300000));
    float* out = static_cast<float*>(P(0x400000));
    float* lse = static_cast<float*>(P(0x500000));
    CHECK(polykv_attend_path(&l, 15, 4) == POLYKV_PATH_MFMA);
    CHECK(polykv_attend_path(&l, 17, 4) == POLYKV_PATH_MFMA);   // 68 rows: two passes
    CHECK(polykv_attend_path(&l, 1 << 20, 1 << 12) == POLYKV_ERR_SHAPE);
    CHECK(polykv_attend_workspace_bytes(&l, 15, 4, 2) == 0);
    g_stub.n_passes = 0;
    CHECK(polykv_attend_shared(pool, &l, nullptr, q, out, 15, 4, 0.088f, 0, 2, nullptr, 0, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "attend_mfma") == 0 && g_stub.a0 == 15 && g_stub.a1 == 4);
    CHECK(g_stub.n_passes == 1 && g_stub.row_begin[0] == 0 && g_stub.n_rows[0] == 60);
    // rows beyond one pass: consecutive ranges of at most POLYKV_ROWS_PER_PASS rows, every
    // launch with the full agent count (the strides of q, out and lse)
    struct RowCase { int agents, gqa; int passes; int last; };
    for (const RowCase& rc : {RowCase{16, 4, 1, 64}, RowCase{17, 4, 2, 4}, RowCase{33, 4, 3, 4},
                              RowCase{1, 130, 3, 2}, RowCase{200, 1, 4, 8}}) {
        for (int path : {POLYKV_PATH_AUTO, POLYKV_PATH_VALU, POLYKV_PATH_MFMA}) {
            g_stub.n_passes = 0;
            CHECK(polykv_attend_shared_path(pool, &l, nullptr, q, out, rc.agents, rc.gqa, 0.088f, 0, 2, nullptr, 0,
                                            nullptr, path) == POLYKV_OK);
            CHECK(g_stub.n_passes == rc.passes);
            CHECK(g_stub.a0 == rc.agents && g_stub.a1 == rc.gqa);
            for (int i = 0; i < g_stub.n_passes && i < 16; ++i) {
                CHECK(g_stub.row_begin[i] == POLYKV_ROWS_PER_PASS * i);
                CHECK(g_stub.n_rows[i] == (i + 1 < rc.passes ? POLYKV_ROWS_PER_PASS : rc.last));
            }
        }
    }
    // a failing launch stops the passes and is reported
    g_stub.n_passes = 0;
    g_stub.launch_status = hipErrorLaunchFailure;
    CHECK(polykv_attend_shared(pool, &l, nullptr, q, out, 33, 4, 0.088f, 0, 2, nullptr, 0, nullptr) ==
          POLYKV_ERR_LAUNCH);
    CHECK(g_stub.n_passes == 1);
    g_stub.launch_status = hipSuccess;
    // an argument error is found before the first pass
    g_stub.n_passes = 0;
    CHECK(polykv_attend_shared_path(pool, &l, nullptr, q, out, 33, 4, 0.088f, 0, 2, nullptr, 0, nullptr, 7) ==
          POLYKV_ERR_ARG);
    CHECK(g_stub.n_passes == 0);
    CHECK(polykv_attend_shared_path(pool, &l, nullptr, q, out, 15, 4, 0.088f, 0, 2, nullptr, 0, nullptr,
                                    POLYKV_PATH_VALU) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "attend_valu") == 0);
    CHECK(polykv_attend_shared_lse(pool, &l, nullptr, q, out, lse, 15, 4, 0.088f, 0, 2, nullptr, 0, nullptr,
                                   POLYKV_PATH_AUTO) == POLYKV_OK);
    CHECK(polykv_attend_shared_prefix(pool, &l, nullptr, q, out, lse, 37, 15, 4, 0.088f, 0, 2, nullptr, 0,
                                      nullptr, POLYKV_PATH_AUTO) == POLYKV_OK);
    CHECK(g_stub.geom.n_tokens == 37 && g_stub.geom.n_groups == 2);
    const int before = g_stub.calls;
    CHECK(polykv_attend_shared_prefix(pool, &l, nullptr, q, out, lse, 0, 15, 4, 0.088f, 0, 2, nullptr, 0,
                                      nullptr, POLYKV_PATH_AUTO) == POLYKV_ERR_RANGE);
    CHECK(polykv_attend_shared_prefix(pool, &l, nullptr, q, out, lse, 101, 15, 4, 0.088f, 0, 2, nullptr, 0,
                                      nullptr, POLYKV_PATH_AUTO) == POLYKV_ERR_RANGE);
    CHECK(polykv_attend_shared(pool, &l, nullptr, nullptr, out, 15, 4, 0.088f, 0, 2, nullptr, 0, nullptr) == POLYKV_ERR_NULL);
    CHECK(polykv_attend_shared(pool, &l, nullptr, q, out, 0, 4, 0.088f, 0, 2, nullptr, 0, nullptr) < 0);
    CHECK(polykv_attend_shared(pool, &l, nullptr, q, out, 15, 4, 0.088f, 1, 2, nullptr, 0, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_attend_shared(pool, &l, nullptr, q, out, 15, 4, NAN, 0, 2, nullptr, 0, nullptr) < 0);
    CHECK(polykv_attend_shared_path(pool, &l, nullptr, q, out, 15, 4, 0.088f, 0, 2, nullptr, 0, nullptr, 7) < 0);
    CHECK(g_stub.calls == before);

    // the private-tail merge
    const int32_t* len = static_cast<const int32_t*>(P(0x600000));
    CHECK(polykv_attend_tail_merge(&l, q, out, lse, P(0x700000), P(0x800000), len, 128, 15, 4, 0.088f, 2,
                                   nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "attend_tail") == 0 && g_stub.a0 == 128 && g_stub.a1 == 15);
    CHECK(polykv_attend_tail_merge(&l, q, out, lse, P(0x700000), P(0x800000), len, -1, 15, 4, 0.088f, 2,
                                   nullptr) < 0);
    CHECK(polykv_attend_tail_merge(&l, q, out, nullptr, P(0x700000), P(0x800000), len, 128, 15, 4, 0.088f,
                                   2, nullptr) == POLYKV_ERR_NULL);
}

static void dequant_and_project() {
    polykv_layout_t l = layout(2, 8, 128, 4096);
    void* pool = P(0x100000);
    CHECK(polykv_dequant_k(pool, &l, P(0x200000), 0, 2, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "dequant_k") == 0);
    CHECK(polykv_dequant_v(pool, &l, nullptr, P(0x200000), 1, 1, nullptr) == POLYKV_OK && g_stub.a0 == 1);
    CHECK(polykv_dequant_v(pool, &l, nullptr, P(0x200000), 1, 2, nullptr) == POLYKV_ERR_RANGE);
    CHECK(polykv_project_kv(P(0x300000), P(0x400000), P(0x500000), P(0x600000), P(0x700000), 4096, 4096, 8,
                            128, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "project") == 0 && g_stub.a0 == 4096 && g_stub.a1 == 4096);
    CHECK(polykv_project_kv(P(0x300000), P(0x400000), P(0x500000), P(0x600000), P(0x700000), 4096, 100, 8,
                            128, nullptr) < 0);
    CHECK(polykv_project_compress(P(0x300000), P(0x400000), P(0x500000), pool, &l, nullptr, 1, 512, 1024,
                                  4096, nullptr) == POLYKV_OK);
    CHECK(std::strcmp(g_stub.last, "project_compress") == 0 && g_stub.a0 == 1 && g_stub.a1 == 512);
    CHECK(polykv_project_compress(P(0x300000), P(0x400000), P(0x500000), pool, &l, nullptr, 1, 500, 100,
                                  4096, nullptr) == POLYKV_ERR_RANGE);     // token_begin % 32
    CHECK(polykv_project_compress(P(0x300000), P(0x400000), P(0x500000), pool, &l, nullptr, 1, 4064, 64,
                                  4096, nullptr) == POLYKV_ERR_RANGE);     // past the capacity
}

static void devices_and_errors() {
    polykv_layout_t l = layout(1, 1, 64, 10);
    g_stub.have_device = false;
    CHECK(polykv_compress_k(P(0x200000), P(0x100000), &l, 0, 1, nullptr) == POLYKV_ERR_DEVICE);
    g_stub.have_device = true;
    g_stub.launch_status = hipErrorLaunchFailure;
    CHECK(polykv_compress_k(P(0x200000), P(0x100000), &l, 0, 1, nullptr) == POLYKV_ERR_LAUNCH);
    g_stub.launch_status = hipSuccess;
    for (int c = 1; c >= -12; --c) {
        const char* s = polykv_strerror(c);
        CHECK(s != nullptr && std::strlen(s) > 0);
    }
}

int main() {
    layouts();
    codebook();
    compress_and_append();
    decode();
    dequant_and_project();
    devices_and_errors();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host layer under sanitizers: all checks passed\n");
    return 0;
}
