// Link-time stand-ins for the kernel launchers and the three HIP runtime calls that the
// host layer (host.cpp) makes, so that the host layer can be built host-only with the
// address and undefined-behaviour sanitizers and driven on a machine without a GPU. Every
// launcher records its call (which one, and a few of its arguments) and returns the
// configured status; the device queries report one gfx950 device, or none.

#include <hip/hip_runtime.h>

#include <cstring>

#include "polykv_internal.h"
#include "stubs.h"

StubState g_stub;

extern "C" hipError_t hipGetDevice(int* dev) {
    if (!g_stub.have_device) return hipErrorNoDevice;
    *dev = 0;
    return hipSuccess;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int dev) {
    if (!g_stub.have_device || dev != 0) return hipErrorInvalidDevice;
    std::memset(prop, 0, sizeof(*prop));
    std::strncpy(prop->gcnArchName, g_stub.arch, sizeof(prop->gcnArchName) - 1);
    return hipSuccess;
}

extern "C" hipError_t hipGetLastError() { return hipSuccess; }

namespace polykv {

static hipError_t record(const char* what, const PoolGeom* g, int32_t a0, int32_t a1) {
    g_stub.calls++;
    std::strncpy(g_stub.last, what, sizeof(g_stub.last) - 1);
    if (g) g_stub.geom = *g;
    g_stub.a0 = a0;
    g_stub.a1 = a1;
    return g_stub.launch_status;
}

hipError_t launch_compress_k(const void*, uint8_t*, const PoolGeom& g, int32_t lb, int32_t lc, hipStream_t) {
    return record("compress_k", &g, lb, lc);
}
hipError_t launch_compress_k_range(const void*, uint8_t*, const PoolGeom& g, int32_t tok0, int32_t n_tok,
                                   int32_t, int32_t, hipStream_t) {
    return record("compress_k_range", &g, tok0, n_tok);
}
hipError_t launch_compress_v_range(const void*, uint8_t*, const PoolGeom& g, const CodebookHalf& cb,
                                   int32_t tok0, int32_t n_tok, int32_t, int32_t, hipStream_t, bool valu) {
    g_stub.valu = valu;
    g_stub.cb = cb;
    return record("compress_v_range", &g, tok0, n_tok);
}
hipError_t launch_compress_v(const void*, uint8_t*, const PoolGeom& g, const CodebookHalf& cb, int32_t lb,
                             int32_t lc, hipStream_t, bool valu) {
    g_stub.valu = valu;
    g_stub.cb = cb;
    return record("compress_v", &g, lb, lc);
}
hipError_t launch_compress_kv_range(const void*, const void*, uint8_t*, const PoolGeom& g, const CodebookHalf& cb,
                                    int32_t tok0, int32_t n_tok, int32_t, int32_t, hipStream_t) {
    g_stub.cb = cb;
    return record("compress_kv_range", &g, tok0, n_tok);
}
hipError_t launch_attend_tail(const TailArgs& a, hipStream_t) {
    return record("attend_tail", nullptr, a.tail_cap, a.n_agents);
}
hipError_t launch_project(const __half*, const __half*, const __half*, __half*, __half*, int32_t n_tok,
                          int32_t hidden, int32_t, int32_t, hipStream_t) {
    return record("project", nullptr, n_tok, hidden);
}
hipError_t launch_project_compress(const __half*, const __half*, const __half*, uint8_t*, const PoolGeom& g,
                                   const CodebookHalf&, int32_t layer, int32_t tok0, int32_t, int32_t, hipStream_t) {
    return record("project_compress", &g, layer, tok0);
}
hipError_t launch_dequant_k(const uint8_t*, void*, const PoolGeom& g, int32_t lb, int32_t lc, hipStream_t) {
    return record("dequant_k", &g, lb, lc);
}
hipError_t launch_dequant_v(const uint8_t*, void*, const PoolGeom& g, const CodebookHalf&, int32_t lb, int32_t lc,
                            hipStream_t) {
    return record("dequant_v", &g, lb, lc);
}
size_t attend_workspace_bytes(const PoolGeom&, int32_t, int32_t, int32_t, int32_t) { return 0; }
static void record_pass(const AttendArgs& a) {
    if (g_stub.n_passes < 16) {
        g_stub.row_begin[g_stub.n_passes] = a.row_begin;
        g_stub.n_rows[g_stub.n_passes] = a.n_rows;
    }
    g_stub.n_passes++;
}
hipError_t launch_attend_valu(const AttendArgs& a, hipStream_t) {
    record_pass(a);
    return record("attend_valu", &a.g, a.n_agents, a.gqa);
}
hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t) {
    record_pass(a);
    return record("attend_mfma", &a.g, a.n_agents, a.gqa);
}
bool attend_mfma_supported(const PoolGeom& g, int32_t rows) {
    return (g.head_dim == 64 || g.head_dim == 128) && rows >= 1 && rows <= 64;
}

}  // namespace polykv
