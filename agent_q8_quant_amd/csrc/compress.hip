// Write-once compression of fp16 K and V into the shared pool (gfx950).
//
// Keys, q8_0 (PolyKV abstract: keys at int8, q8_0 format): blocks of 32 along
// head_dim, fp16 scale RNE16(amax/127), codes RNE(x/s) clamped to [-127, 127].
// Values, TurboQuant MSE (PolyKV abstract: FWHT rotation, then 3-bit Lloyd-Max codes for
// N(0,1)): y = H v / ||v||, code = #{k : y > b_k}, stored as three bit-planes over groups
// of 32 tokens plus an fp16 norm.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

// ---------------------------------------------------------------------------------------
// Keys. One thread owns 8 consecutive entries (one 16-B load); the 4 threads of a quad
// own one 32-entry block and combine their |x| maxima through two lane exchanges.
// Grid: x over 8-entry vectors of a tile, y over the tiles of the layer range.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_compress_k(const uint4* __restrict__ k,
                                                    uint8_t* __restrict__ pool, PoolGeom g,
                                                    int32_t layer_begin, uint32_t vec_per_tile) {
    const uint32_t tile_local = blockIdx.y;
    const uint32_t v = blockIdx.x * 256u + threadIdx.x;
    // vec_per_tile is a multiple of 4, so a quad is either wholly active or wholly idle
    const bool active = v < vec_per_tile;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (active) raw = k[(size_t)tile_local * vec_per_tile + v];

    const __half* hv = reinterpret_cast<const __half*>(&raw);
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = __half2float(hv[e]);
        amax = fmaxf(amax, fabsf(x[e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));

    const float s32 = amax / 127.0f;            // IEEE float32 division
    const __half s16 = __float2half_rn(s32);    // round to nearest even
    const float s = __half2float(s16);

    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float q = 0.0f;
        if (s != 0.0f) q = rintf(x[e] / s);     // exact division, half to even
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
        packed[e >> 2] |= b << (8 * (e & 3));
    }
    if (!active) return;
    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;
    uint2* codes = reinterpret_cast<uint2*>(pool + g.k_codes_off + tile * g.k_codes_stride);
    codes[v] = make_uint2(packed[0], packed[1]);
    if ((threadIdx.x & 3) == 0) {
        __half* scales = reinterpret_cast<__half*>(pool + g.k_scales_off + tile * g.k_scales_stride);
        scales[v >> 2] = s16;
    }
}

// ---------------------------------------------------------------------------------------
// Values. One lane owns one token's whole head vector in registers, so the FWHT runs
// entirely in registers. A wave covers two groups of 32 tokens ("items"): lanes 0-31 the
// first, lanes 32-63 the second. The plane words of a coordinate are wave ballots: the
// low 32 bits belong to the first item, the high 32 bits to the second.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_compress_v(const __half* __restrict__ v,
                                                    uint8_t* __restrict__ pool, PoolGeom g,
                                                    CodebookHalf cb, int32_t layer_begin,
                                                    uint32_t n_items) {
    constexpr int NW = D / 64;  // coordinates per lane in the word buffer
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
    const uint32_t G = (uint32_t)g.n_groups;
    const uint32_t T = (uint32_t)g.n_tokens;

    const uint32_t item = wave * 2u + (uint32_t)(lane >> 5);
    const uint32_t tile_local = item / G;
    const uint32_t grp = item - tile_local * G;
    const uint32_t token = grp * 32u + (uint32_t)(lane & 31);
    const bool valid = item < n_items && token < T;

    float x[D];
    if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(v + ((size_t)tile_local * T + token) * D);
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            uint4 r = src[c];
            const __half* h = reinterpret_cast<const __half*>(&r);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * c + e] = __half2float(h[e]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < D; ++i) x[i] = 0.0f;
    }

    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) ss = fmaf(x[i], x[i], ss);
    const float n = sqrtf(ss);

    // unnormalised Sylvester FWHT: y = H v
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (!(i & h)) {
                const float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
        }
    }

    // y / n > b  <=>  y > b * n for n > 0. For n = 0 the rotated vector is 0 by definition:
    // infinite magnitude thresholds make every coordinate code 3.
    const float t4 = n > 0.0f ? cb.boundary_pos[0] * n : INFINITY;
    const float t5 = n > 0.0f ? cb.boundary_pos[1] * n : INFINITY;
    const float t6 = n > 0.0f ? cb.boundary_pos[2] * n : INFINITY;

    uint32_t wlo[3][NW], whi[3][NW];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int c = 0; c < NW; ++c) wlo[p][c] = whi[p][c] = 0u;

#pragma unroll
    for (int i = 0; i < D; ++i) {
        const float y = x[i];
        const float a = fabsf(y);
        int code;
        if (y > 0.0f) {
            code = 4 + (a > t4) + (a > t5) + (a > t6);
        } else {
            // y > -t  <=>  |y| < t for y <= 0
            code = (a < t4) + (a < t5) + (a < t6);
        }
        const uint64_t m0 = __ballot(valid && (code & 1));
        const uint64_t m1 = __ballot(valid && (code & 2));
        const uint64_t m2 = __ballot(valid && (code & 4));
        if (lane == (i & 63)) {
            wlo[0][i >> 6] = (uint32_t)m0;
            wlo[1][i >> 6] = (uint32_t)m1;
            wlo[2][i >> 6] = (uint32_t)m2;
            whi[0][i >> 6] = (uint32_t)(m0 >> 32);
            whi[1][i >> 6] = (uint32_t)(m1 >> 32);
            whi[2][i >> 6] = (uint32_t)(m2 >> 32);
        }
    }

    // stores: every lane writes the words of its own coordinates for both items
    const size_t tile_base = (size_t)layer_begin * g.n_kv_heads;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t it = wave * 2u + (uint32_t)half;
        if (it >= n_items) continue;
        const uint32_t tl = it / G;
        const uint32_t gr = it - tl * G;
        uint32_t* words = reinterpret_cast<uint32_t*>(pool + g.v_planes_off +
                                                      (tile_base + tl) * g.v_planes_stride) +
                          (size_t)gr * 3 * D;
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                words[p * D + c * 64 + lane] = half ? whi[p][c] : wlo[p][c];
            }
    }
    if (valid) {
        __half* norms = reinterpret_cast<__half*>(pool + g.v_norms_off +
                                                  (tile_base + tile_local) * g.v_norms_stride);
        norms[token] = __float2half_rn(n);
    }
}

}  // namespace

hipError_t launch_compress_k(const void* k_fp16, uint8_t* pool, const PoolGeom& g,
                             int32_t layer_begin, int32_t layer_count, hipStream_t s) {
    const uint32_t vec_per_tile = (uint32_t)((uint64_t)g.n_tokens * g.head_dim / 8);
    const uint32_t tiles = (uint32_t)layer_count * (uint32_t)g.n_kv_heads;
    dim3 grid((vec_per_tile + 255) / 256, tiles);
    hipLaunchKernelGGL(k_compress_k, grid, dim3(256), 0, s, (const uint4*)k_fp16, pool, g,
                       layer_begin, vec_per_tile);
    return hipGetLastError();
}

hipError_t launch_compress_v(const void* v_fp16, uint8_t* pool, const PoolGeom& g,
                             const CodebookHalf& cb, int32_t layer_begin, int32_t layer_count,
                             hipStream_t s) {
    const uint64_t items = (uint64_t)layer_count * g.n_kv_heads * g.n_groups;
    const uint64_t waves = (items + 1) / 2;
    const uint32_t blocks = (uint32_t)((waves + 3) / 4);
    const __half* v = (const __half*)v_fp16;
    switch (g.head_dim) {
        case 64: hipLaunchKernelGGL(k_compress_v<64>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items); break;
        case 128: hipLaunchKernelGGL(k_compress_v<128>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items); break;
        case 256: hipLaunchKernelGGL(k_compress_v<256>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace polykv
