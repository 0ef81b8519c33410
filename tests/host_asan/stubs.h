// Shared state of the host-layer stand-ins (stubs.cpp) and the driver (driver.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "polykv_internal.h"

struct StubState {
    bool have_device = true;
    const char* arch = "gfx950:sramecc+:xnack-";
    hipError_t launch_status = hipSuccess;
    int calls = 0;
    char last[32] = {0};
    polykv::PoolGeom geom = {};
    polykv::CodebookHalf cb = {};
    int32_t a0 = 0, a1 = 0;
    bool valu = false;
    // row ranges of the decode launches since the driver last cleared n_passes
    int n_passes = 0;
    int32_t row_begin[16] = {0}, n_rows[16] = {0};
};

extern StubState g_stub;
