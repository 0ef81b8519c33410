// Dequantisation of the shared pool back to fp16 K and V (gfx950), the form a model's
// ordinary KV cache holds.
//
// PolyKV abstract: keys are held as int8 q8_0 and values as TurboQuant MSE codes; the
// integration on the pages hands the decompressed cache to the model as an ordinary
// per-layer cache. Reconstruction, per token-head:
// - key:   k_hat = code * s (the stored fp16 block scale), rounded once to fp16. The
//          product of an int8 code and an fp16 scale is exact in fp32, so the result is
//          the correctly rounded fp16 of the exact reconstruction;
// - value: v_hat = (n / d) * H c[code] with n the stored fp16 norm, c the codebook's
//          centroids and H the +-1 Sylvester matrix (the inverse of y = H v / ||v||; H is
//          symmetric and H H = d I). The transform runs in fp32 (error far below one fp16
//          ulp), then one rounding to fp16.

#include <algorithm>

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Keys: one thread per 8 consecutive entries (8 codes in, one 16-byte fp16 store out).
// Grid: x over the 8-entry pieces of a tile, y over the tiles of the layer range.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_k(const uint8_t* __restrict__ pool, PoolGeom g,
                                                   int32_t layer_begin, uint32_t vec_per_tile,
                                                   u4* __restrict__ out) {
    const uint32_t tile_local = blockIdx.y;
    const uint32_t v = blockIdx.x * 256u + threadIdx.x;
    if (v >= vec_per_tile) return;
    const uint32_t D = (uint32_t)g.head_dim;
    const uint32_t per_row = D / 8;
    const uint32_t t = v / per_row, c8 = v - t * per_row;
    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;
    const uint8_t* codes = pool + g.k_codes_off + tile * g.k_codes_stride + (size_t)t * D + 8 * c8;
    const __half* scales = reinterpret_cast<const __half*>(pool + g.k_scales_off + tile * g.k_scales_stride);
    const uint2 raw = *reinterpret_cast<const uint2*>(codes);
    const float s = __half2float(scales[(size_t)t * (D / 32) + c8 / 4]);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t word = e < 2 ? raw.x : raw.y;
        const int8_t lo = (int8_t)((word >> (16 * (e & 1))) & 0xFFu);
        const int8_t hi = (int8_t)((word >> (16 * (e & 1) + 8)) & 0xFFu);
        const __half a = __float2half_rn((float)lo * s), b = __float2half_rn((float)hi * s);
        w[e] = (uint32_t)__half_as_ushort(a) | ((uint32_t)__half_as_ushort(b) << 16);
    }
    out[(size_t)tile_local * vec_per_tile + v] = u4{w[0], w[1], w[2], w[3]};
}

// ---------------------------------------------------------------------------------------
// Values. An item is one 32-token group of a tile for head_dim 128 and 256 (lane l holds
// token l % 32, coordinates (l / 32) * d/2 .. + d/2 - 1) and two consecutive groups for
// head_dim 64 (lane l holds token l % 32 of group l / 32, all 64 coordinates). Each wave
// walks items with a grid stride and keeps the next item's plane words and norm in
// registers while it works on the current one. Per item:
// 1. the plane words (3 x d per group, as stored) go from registers to the wave's LDS area;
// 2. lane l reads, per coordinate, the three words of its half and takes bit l % 32 of
//    each: the code, whose centroid comes from an 8-entry LDS table;
// 3. the FWHT runs in registers over the lane's coordinates, and for d >= 128 one last
//    butterfly pairs lane l with lane l ^ 32 (the other coordinate half), one register
//    swap per two coordinates;
// 4. times n / d, rounded to fp16, stored as 16-byte pieces.
// ---------------------------------------------------------------------------------------
template <int D>
struct DqCfg {
    static constexpr int HALVES = D == 64 ? 1 : 2;   // lanes per token
    static constexpr int CPL = D / HALVES;           // coordinates per lane
    static constexpr int GPW = D == 64 ? 2 : 1;      // groups per item
    static constexpr int WORDS = GPW * 3 * D;        // plane words per item
    static constexpr int PIECES = WORDS / 4;         // 16-byte pieces per item
    static constexpr int PPL = (PIECES + 63) / 64;   // pieces per lane
};

// Where item `item` lives, and its plane words and this lane's norm fetched into registers.
template <int D>
struct DqItem {
    uint32_t tile_local;
    int g0, n_grp, token;
    bool valid;
};

template <int D>
__device__ __forceinline__ DqItem<D> dq_item(uint32_t item, uint32_t items_per_tile, const PoolGeom& g, int lane) {
    using C = DqCfg<D>;
    DqItem<D> it;
    it.tile_local = item / items_per_tile;
    const uint32_t gi = item - it.tile_local * items_per_tile;
    it.g0 = (int)gi * C::GPW;
    it.n_grp = min(C::GPW, g.n_groups - it.g0);
    const int half = lane >> 5, t = lane & 31;
    it.token = 32 * (C::GPW == 2 ? it.g0 + half : it.g0) + t;
    it.valid = it.token < g.n_tokens && (C::GPW == 1 || half < it.n_grp);
    return it;
}

template <int D>
__device__ __forceinline__ void dq_fetch(const DqItem<D>& it, const uint8_t* pool, const PoolGeom& g,
                                         int32_t layer_begin, int lane, u4 (&pf)[DqCfg<D>::PPL],
                                         uint32_t& norm_bits) {
    using C = DqCfg<D>;
    const size_t tile = (size_t)layer_begin * g.n_kv_heads + it.tile_local;
    const u4* src = reinterpret_cast<const u4*>(pool + g.v_planes_off + tile * g.v_planes_stride +
                                                (size_t)it.g0 * (3 * D * 4));
    const int n_pieces = it.n_grp * 3 * D / 4;
#pragma unroll
    for (int i = 0; i < C::PPL; ++i) {
        const int piece = lane + 64 * i;
        if (piece < n_pieces) pf[i] = src[piece];
    }
    const uint16_t* norms = reinterpret_cast<const uint16_t*>(pool + g.v_norms_off + tile * g.v_norms_stride);
    norm_bits = it.valid ? norms[it.token] : 0u;
}

template <int D>
__global__ __launch_bounds__(256) void k_dequant_v(const uint8_t* __restrict__ pool, PoolGeom g,
                                                   CodebookHalf cb, int32_t layer_begin,
                                                   uint32_t items_per_tile, uint32_t n_items,
                                                   __half* __restrict__ out) {
    using C = DqCfg<D>;
    constexpr int CPL = C::CPL;
    __shared__ __attribute__((aligned(16))) uint32_t words[4][C::WORDS];
    __shared__ float ctab[8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < 8) {
        const int m = tid >= 4 ? tid - 4 : 3 - tid;
        const float mag = m == 0 ? cb.centroid_pos[0] : m == 1 ? cb.centroid_pos[1]
                        : m == 2 ? cb.centroid_pos[2] : cb.centroid_pos[3];
        ctab[tid] = tid >= 4 ? mag : -mag;
    }
    __syncthreads();  // the only workgroup barrier: waves without an item leave after it
    const uint32_t stride = gridDim.x * 4u;
    uint32_t item = (uint32_t)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4u + (uint32_t)w));
    if (item >= n_items) return;
    const int T = g.n_tokens;
    const int half = lane >> 5, t = lane & 31;
    const int coord0 = C::GPW == 2 ? 0 : half * CPL;
    const uint32_t* wb = &words[w][(C::GPW == 2 ? half * 3 * D : 0) + coord0];
    u4* stage = reinterpret_cast<u4*>(&words[w][0]);

    u4 pf[C::PPL];
    uint32_t norm_bits;
    DqItem<D> it = dq_item<D>(item, items_per_tile, g, lane);
    dq_fetch<D>(it, pool, g, layer_begin, lane, pf, norm_bits);
    while (true) {
        // 1. this item's words into LDS (the previous item's reads are complete: their
        //    results were consumed before its stores)
        {
            const int n_pieces = it.n_grp * 3 * D / 4;
#pragma unroll
            for (int i = 0; i < C::PPL; ++i) {
                const int piece = lane + 64 * i;
                if (piece < n_pieces) stage[piece] = pf[i];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const DqItem<D> cur = it;
        const float f = __half2float(__ushort_as_half((unsigned short)norm_bits)) * (1.0f / (float)D);
        const uint32_t next = item + stride;
        if (next < n_items) {
            it = dq_item<D>(next, items_per_tile, g, lane);
            dq_fetch<D>(it, pool, g, layer_begin, lane, pf, norm_bits);  // in flight meanwhile
        }

        // 2. codes -> centroids
        float x[CPL];
#pragma unroll
        for (int c = 0; c < CPL; c += 4) {
            const u4 p0 = *reinterpret_cast<const u4*>(wb + c);
            const u4 p1 = *reinterpret_cast<const u4*>(wb + D + c);
            const u4 p2 = *reinterpret_cast<const u4*>(wb + 2 * D + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t code = __builtin_amdgcn_ubfe(p0[e], t, 1) | (__builtin_amdgcn_ubfe(p1[e], t, 1) << 1) |
                                      (__builtin_amdgcn_ubfe(p2[e], t, 1) << 2);
                x[c + e] = ctab[code];
            }
        }
        // 3. Sylvester FWHT over the lane's coordinates (pairs at distance h become (a+b, a-b))
#pragma unroll
        for (int h = 1; h < CPL; h <<= 1)
#pragma unroll
            for (int e = 0; e < CPL; ++e)
                if (!(e & h)) {
                    const float a = x[e], b = x[e + h];
                    x[e] = a + b;
                    x[e + h] = a - b;
                }
        // 4. scale by n / d and store 16-byte pieces of `n` consecutive coordinates
        auto store = [&](const float* v, int first, int n) {
            u4* o = reinterpret_cast<u4*>(out + ((size_t)cur.tile_local * T + cur.token) * D + first);
#pragma unroll
            for (int c = 0; c < n; c += 8) {
                uint32_t q[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    q[e] = (uint32_t)__half_as_ushort(__float2half_rn(v[c + 2 * e] * f)) |
                           ((uint32_t)__half_as_ushort(__float2half_rn(v[c + 2 * e + 1] * f)) << 16);
                o[c / 8] = u4{q[0], q[1], q[2], q[3]};
            }
        };
        if constexpr (C::HALVES == 2) {
            // the last butterfly pairs coordinate i (lane l, lower half) with i + d/2 (lane
            // l ^ 32). One swap of registers e and e + HP (HP = d/4) hands the lower lane both
            // values of coordinate e and the upper lane both values of coordinate e + HP:
            // sw[0] is the lower half's value and sw[1] the upper half's in either lane. So
            // lane l finishes coordinates base + e and base + e + d/2 (e < HP), base = HP for
            // the upper lane: one swap and two additions per pair.
            constexpr int HP = CPL / 2;
            float lo[HP], hi[HP];
#pragma unroll
            for (int e = 0; e < HP; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[e]), __float_as_uint(x[e + HP]), false, false);
                const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
                lo[e] = a + b;
                hi[e] = a - b;
            }
            if (cur.valid) {
                const int base = half * HP;
                store(lo, base, HP);
                store(hi, base + CPL, HP);
            }
        } else {
            if (cur.valid) store(x, coord0, CPL);
        }
        if (next >= n_items) break;
        item = next;
    }
}

}  // namespace

hipError_t launch_dequant_k(const uint8_t* pool, void* k_fp16, const PoolGeom& g,
                            int32_t layer_begin, int32_t layer_count, hipStream_t s) {
    const uint32_t vec_per_tile = (uint32_t)((uint64_t)g.n_tokens * g.head_dim / 8);
    const uint32_t tiles = (uint32_t)layer_count * (uint32_t)g.n_kv_heads;
    dim3 grid((vec_per_tile + 255) / 256, tiles);
    hipLaunchKernelGGL(k_dequant_k, grid, dim3(256), 0, s, pool, g, layer_begin, vec_per_tile,
                       (u4*)k_fp16);
    return hipGetLastError();
}

hipError_t launch_dequant_v(const uint8_t* pool, void* v_fp16, const PoolGeom& g,
                            const CodebookHalf& cb, int32_t layer_begin, int32_t layer_count,
                            hipStream_t s) {
    const uint32_t gpw = g.head_dim == 64 ? 2u : 1u;
    const uint32_t items_per_tile = ((uint32_t)g.n_groups + gpw - 1) / gpw;
    const uint64_t items = (uint64_t)layer_count * g.n_kv_heads * items_per_tile;
    // waves walk the items with a grid stride; 2048 workgroups (8 per CU) cover the chip
    const uint32_t blocks = (uint32_t)std::min<uint64_t>((items + 3) / 4, 2048);
    __half* out = (__half*)v_fp16;
    switch (g.head_dim) {
        case 64: hipLaunchKernelGGL(k_dequant_v<64>, dim3(blocks), dim3(256), 0, s, pool, g, cb, layer_begin, items_per_tile, (uint32_t)items, out); break;
        case 128: hipLaunchKernelGGL(k_dequant_v<128>, dim3(blocks), dim3(256), 0, s, pool, g, cb, layer_begin, items_per_tile, (uint32_t)items, out); break;
        case 256: hipLaunchKernelGGL(k_dequant_v<256>, dim3(blocks), dim3(256), 0, s, pool, g, cb, layer_begin, items_per_tile, (uint32_t)items, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace polykv
