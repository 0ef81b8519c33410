// Write-once compression of fp16 K and V into the shared pool (gfx950).
//
// Keys, q8_0 (PolyKV abstract: keys at int8, q8_0 format): blocks of 32 along
// head_dim, fp16 scale RNE16(amax/127), codes RNE(x/s) clamped to [-127, 127].
// Values, TurboQuant MSE (PolyKV abstract: FWHT rotation, then 3-bit Lloyd-Max codes for
// N(0,1)): y = H v / ||v||, code = #{k : y > b_k}, stored as three bit-planes over groups
// of 32 tokens plus an fp16 norm.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "codec.h"
#include "polykv_internal.h"

namespace polykv {
namespace {

using codec::h8;
using codec::encode_v_group;
using codec::q8_encode8;

// ---------------------------------------------------------------------------------------
// Keys. One thread owns 8 consecutive entries (one 16-B load); the 4 threads of a quad
// own one 32-entry block and combine their |x| maxima through two lane exchanges.
// Grid: x over the 8-entry vectors of a tile's token range, y over the tiles of the layer
// range. The input holds that token range only: [layer_count][H][n_tok][d].
//
// The codec is codec::q8_encode8.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_compress_k(const uint4* __restrict__ k,
                                                    uint8_t* __restrict__ pool, PoolGeom g,
                                                    int32_t layer_begin, uint32_t vec_per_tile,
                                                    uint32_t tok0) {
    const uint32_t tile_local = blockIdx.y;
    const uint32_t v = blockIdx.x * 256u + threadIdx.x;
    // vec_per_tile is a multiple of 4, so a quad is either wholly active or wholly idle
    const bool active = v < vec_per_tile;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (active) raw = k[(size_t)tile_local * vec_per_tile + v];

    uint32_t packed[2];
    const __half s16 = q8_encode8(raw, packed);
    if (!active) return;
    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;
    const size_t v0 = (size_t)tok0 * (g.head_dim / 8);  // first 8-entry vector of the range
    uint2* codes = reinterpret_cast<uint2*>(pool + g.k_codes_off + tile * g.k_codes_stride);
    codes[v0 + v] = make_uint2(packed[0], packed[1]);
    if ((threadIdx.x & 3) == 0) {
        __half* scales = reinterpret_cast<__half*>(pool + g.k_scales_off + tile * g.k_scales_stride);
        scales[(v0 + v) >> 2] = s16;
    }
}

// Token range [tok0, tok0 + n_tok) of every tile (the whole tile for a one-shot compress,
// one prefill chunk for an append) and the 32-token groups it touches. The input holds the
// range only, [layer_count][H][n_tok][d]. A group the range covers only in part keeps the
// plane bits of its other tokens below the tile's length: the new words are
// (old & keep) | new bits. Bits of tokens at or past the tile's length are always 0.
struct TokRange {
    uint32_t tok0, n_tok, g_first, n_grp;
};

__device__ __forceinline__ uint32_t keep_mask(const TokRange& r, uint32_t grp, uint32_t T) {
    uint32_t keep = 0u;
    const uint32_t t_base = grp * 32u;
    // tokens of the group below the range, and those past it but below T
    if (r.tok0 > t_base) keep |= (r.tok0 - t_base >= 32u) ? 0xFFFFFFFFu : ((1u << (r.tok0 - t_base)) - 1u);
    const uint32_t end = r.tok0 + r.n_tok, lim = min(T, t_base + 32u);
    if (lim > end) {
        const uint32_t lo = max(end, t_base) - t_base, hi = lim - t_base;  // [lo, hi)
        const uint32_t upto_hi = hi >= 32u ? 0xFFFFFFFFu : ((1u << hi) - 1u);
        keep |= upto_hi & ~((1u << lo) - 1u);
    }
    return keep;
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
                                                    uint32_t n_items, TokRange rg) {
    constexpr int NW = D / 64;  // coordinates per lane in the word buffer
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
    const uint32_t T = (uint32_t)g.n_tokens;

    const uint32_t item = wave * 2u + (uint32_t)(lane >> 5);
    const uint32_t tile_local = item / rg.n_grp;
    const uint32_t grp = rg.g_first + (item - tile_local * rg.n_grp);
    const uint32_t token = grp * 32u + (uint32_t)(lane & 31);
    const bool valid = item < n_items && token >= rg.tok0 && token < rg.tok0 + rg.n_tok;

    float x[D];
    if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(v + ((size_t)tile_local * rg.n_tok + (token - rg.tok0)) * D);
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
        const uint32_t tl = it / rg.n_grp;
        const uint32_t gr = rg.g_first + (it - tl * rg.n_grp);
        const uint32_t keep = keep_mask(rg, gr, T);
        uint32_t* words = reinterpret_cast<uint32_t*>(pool + g.v_planes_off +
                                                      (tile_base + tl) * g.v_planes_stride) +
                          (size_t)gr * 3 * D;
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int c = 0; c < NW; ++c) {
                const uint32_t nw = half ? whi[p][c] : wlo[p][c];
                uint32_t* dst = &words[p * D + c * 64 + lane];
                *dst = keep ? ((*dst & keep) | nw) : nw;
            }
    }
    if (valid) {
        __half* norms = reinterpret_cast<__half*>(pool + g.v_norms_off +
                                                  (tile_base + tile_local) * g.v_norms_stride);
        norms[token] = __float2half_rn(n);
    }
}

// ---------------------------------------------------------------------------------------
// Values on the matrix cores (head_dim 64 and 128): one wave per 32-token group of one
// tile, encoded by codec::encode_v_group from the fp16 values loaded as its B operand.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_compress_v_mfma(const __half* __restrict__ v,
                                                         uint8_t* __restrict__ pool, PoolGeom g,
                                                         CodebookHalf cb, int32_t layer_begin,
                                                         uint32_t n_items, TokRange rg) {
    constexpr int KK = D / 16;        // k steps of the rotation
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hl = lane >> 5;
    // wave-uniform (and known to be so: scalar registers and branches)
    const uint32_t item = (uint32_t)__builtin_amdgcn_readfirstlane((int)((blockIdx.x * 256u + threadIdx.x) >> 6));
    if (item >= n_items) return;  // whole waves only
    const uint32_t T = (uint32_t)g.n_tokens;
    const uint32_t tile_local = item / rg.n_grp;
    const uint32_t grp = rg.g_first + (item - tile_local * rg.n_grp);
    const uint32_t token = grp * 32u + (uint32_t)l32;
    const bool valid = token >= rg.tok0 && token < rg.tok0 + rg.n_tok;

    // B operand: token l % 32, dims 16 kk + 8 (l / 32) .. +7 (16 contiguous bytes)
    h8 vb[KK];
    {
        const h8* src = reinterpret_cast<const h8*>(v + ((size_t)tile_local * rg.n_tok + (valid ? token - rg.tok0 : 0u)) * D + 8 * hl);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) vb[kk] = valid ? src[2 * kk] : h8{};
    }

    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;
    uint32_t* words = reinterpret_cast<uint32_t*>(pool + g.v_planes_off + tile * g.v_planes_stride) +
                      (size_t)grp * 3 * D;
    __half* norms = reinterpret_cast<__half*>(pool + g.v_norms_off + tile * g.v_norms_stride);
    encode_v_group<D>(vb, valid, cb, words, keep_mask(rg, grp, T), norms, token, lane);
}

}  // namespace

hipError_t launch_compress_k_range(const void* k_fp16, uint8_t* pool, const PoolGeom& g,
                                   int32_t tok0, int32_t n_tok, int32_t layer_begin,
                                   int32_t layer_count, hipStream_t s) {
    const uint32_t vec_per_tile = (uint32_t)((uint64_t)n_tok * g.head_dim / 8);
    const uint32_t tiles = (uint32_t)layer_count * (uint32_t)g.n_kv_heads;
    dim3 grid((vec_per_tile + 255) / 256, tiles);
    hipLaunchKernelGGL(k_compress_k, grid, dim3(256), 0, s, (const uint4*)k_fp16, pool, g,
                       layer_begin, vec_per_tile, (uint32_t)tok0);
    return hipGetLastError();
}

hipError_t launch_compress_v_range(const void* v_fp16, uint8_t* pool, const PoolGeom& g,
                                   const CodebookHalf& cb, int32_t tok0, int32_t n_tok,
                                   int32_t layer_begin, int32_t layer_count, hipStream_t s,
                                   bool valu) {
    TokRange rg;
    rg.tok0 = (uint32_t)tok0;
    rg.n_tok = (uint32_t)n_tok;
    rg.g_first = (uint32_t)tok0 / 32u;
    rg.n_grp = (uint32_t)(tok0 + n_tok - 1) / 32u - rg.g_first + 1u;
    const uint64_t items = (uint64_t)layer_count * g.n_kv_heads * rg.n_grp;
    const uint64_t waves = (items + 1) / 2;
    const uint32_t blocks = (uint32_t)((waves + 3) / 4);
    const __half* v = (const __half*)v_fp16;
    const uint32_t mblocks = (uint32_t)((items + 3) / 4);  // one wave per 32-token group
    if (valu) {
        switch (g.head_dim) {
            case 64: hipLaunchKernelGGL(k_compress_v<64>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
            case 128: hipLaunchKernelGGL(k_compress_v<128>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
            case 256: hipLaunchKernelGGL(k_compress_v<256>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (g.head_dim) {
        case 64: hipLaunchKernelGGL(k_compress_v_mfma<64>, dim3(mblocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        case 128: hipLaunchKernelGGL(k_compress_v_mfma<128>, dim3(mblocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        case 256: hipLaunchKernelGGL(k_compress_v<256>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_compress_k(const void* k_fp16, uint8_t* pool, const PoolGeom& g,
                             int32_t layer_begin, int32_t layer_count, hipStream_t s) {
    return launch_compress_k_range(k_fp16, pool, g, 0, g.n_tokens, layer_begin, layer_count, s);
}

hipError_t launch_compress_v(const void* v_fp16, uint8_t* pool, const PoolGeom& g,
                             const CodebookHalf& cb, int32_t layer_begin, int32_t layer_count,
                             hipStream_t s, bool valu) {
    return launch_compress_v_range(v_fp16, pool, g, cb, 0, g.n_tokens, layer_begin, layer_count, s, valu);
}

}  // namespace polykv
