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
// Values. An item is one 32-token group of a tile; each wave walks items with a grid stride
// and keeps the next item's plane words and norms in registers while it works on the
// current one. Every lane holds 32 coordinates of one token: LPT = d/32 lanes per token,
// lane l = t + TPP q (TPP = 64/LPT tokens per pass) holds token t of the pass and
// coordinates 32 q .. 32 q + 31, and the wave covers its group in 32/TPP passes. Per item:
// 1. the plane words (3 x d per group, as stored) go from registers to the wave's LDS area;
// 2. per coordinate, the lane takes bit t of its three words: the code, whose centroid
//    comes from an 8-entry LDS table;
// 3. the FWHT runs in registers up to distance 16, then across lanes: for d = 256 first
//    distance 32 between lanes l and l ^ 8 (a DPP row rotation), then, for the two highest
//    bits of q, distances 32 (d = 128) or 64 (d = 256) between l and l ^ 16 and d/2 between
//    l and l ^ 32 (d = 64: only the last), one register swap and two additions per
//    coordinate pair each. A swap of registers e and e + 16 hands the lane with the lower
//    bit both values of its local coordinate e and the other lane both values of e + 16, so
//    each swap stage halves the run a lane holds; a lane ends with two runs of 16 coordinates,
//    c0 .. c0 + 15 and d/2 + c0 .. + 15;
// 4. times n / d, rounded to fp16; for d >= 128 through the wave's LDS rows out to memory:
//    each lane places its two runs in its token's row, then lane l writes pieces l, l + 64,
//    ... of the pass's rows, so every store instruction covers 1 KB of consecutive bytes (a
//    lane's own runs are 16-byte pieces 32 bytes apart, which a store instruction would
//    scatter over 16 rows at d = 128); at d = 64 the lanes store their own runs.
// Keeping 32 coordinates per lane (not d/2) halves the registers of d = 128 and so doubles
// the waves a SIMD holds, which hides the latency of the lookup and shuffle chains.
// ---------------------------------------------------------------------------------------
template <int D>
struct DqCfg {
    static constexpr int LPT = D / 32;               // lanes per token
    static constexpr int TPP = 64 / LPT;             // tokens per pass
    static constexpr int PASSES = 32 / TPP;
    static constexpr int WORDS = 3 * D;              // plane words per group
    static constexpr int PIECES = WORDS / 4;         // 16-byte pieces per group
    static constexpr int PPL = (PIECES + 63) / 64;   // pieces per lane
    // output staging of one pass (TPP tokens x D fp16): rows padded by 16 bytes so that the
    // 16 lanes of one 16-byte LDS access (same q, consecutive t) hit distinct banks
    static constexpr int ROW_BYTES = 2 * D + 16;
    static constexpr int OUT_BYTES = TPP * ROW_BYTES;
    static constexpr int OUT_PIECES = TPP * D / 8;    // 16-byte pieces of a pass (= 4 per lane)
    static_assert(OUT_PIECES == 256, "four pieces per lane");
};

// first coordinate of the lane's lower run after the cross-lane stages (q: the lane's
// 32-coordinate slot before them)
template <int D>
__device__ __forceinline__ int dq_run_start(int q) {
    if constexpr (D == 64) return 16 * q;
    else if constexpr (D == 128) return 16 * (q & 1) + 32 * (q >> 1);
    else return 32 * (q & 1) + 16 * ((q >> 1) & 1) + 64 * (q >> 2);
}

// one cross-lane butterfly stage by register swaps (see above)
template <bool ROW16>
__device__ __forceinline__ void dq_swap_stage(float (&x)[32]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t a0 = __float_as_uint(x[e]), b0 = __float_as_uint(x[e + 16]);
        const auto sw = ROW16 ? __builtin_amdgcn_permlane16_swap(a0, b0, false, false)
                              : __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const float a = __uint_as_float(sw[0]), b = __uint_as_float(sw[1]);
        x[e] = a + b;
        x[e + 16] = a - b;
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_dequant_v(const uint8_t* __restrict__ pool, PoolGeom g,
                                                   CodebookHalf cb, int32_t layer_begin,
                                                   uint32_t items_per_tile, uint32_t n_items,
                                                   __half* __restrict__ out) {
    using C = DqCfg<D>;
    constexpr int TPP = C::TPP, PASSES = C::PASSES;
    __shared__ __attribute__((aligned(16))) uint32_t words[4][C::WORDS];
    __shared__ __attribute__((aligned(16))) uint8_t ostage[4][D >= 128 ? C::OUT_BYTES : 16];
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
    const int tl = lane % TPP, q = lane / TPP;
    const uint32_t* wb = &words[w][32 * q];
    u4* stage = reinterpret_cast<u4*>(&words[w][0]);
    const int run0 = dq_run_start<D>(q);

    // the item's plane words and this lane's norms (one per pass), fetched one item ahead
    u4 pf[C::PPL];
    uint32_t nb[PASSES];
    uint32_t tile_next = 0;
    int g_next = 0;
    auto fetch = [&](uint32_t it) {
        tile_next = it / items_per_tile;
        g_next = (int)(it - tile_next * items_per_tile);
        const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_next;
        const u4* src = reinterpret_cast<const u4*>(pool + g.v_planes_off + tile * g.v_planes_stride +
                                                    (size_t)g_next * (3 * D * 4));
#pragma unroll
        for (int i = 0; i < C::PPL; ++i) {
            const int piece = lane + 64 * i;
            if (piece < C::PIECES) pf[i] = src[piece];
        }
        const uint16_t* nrm = reinterpret_cast<const uint16_t*>(pool + g.v_norms_off + tile * g.v_norms_stride);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int tok = 32 * g_next + TPP * p + tl;
            nb[p] = tok < T ? nrm[tok] : 0u;
        }
    };
    fetch(item);
    while (true) {
        // 1. this item's words into LDS (the previous item's reads are complete: their
        //    results were consumed before its stores)
#pragma unroll
        for (int i = 0; i < C::PPL; ++i) {
            const int piece = lane + 64 * i;
            if (piece < C::PIECES) stage[piece] = pf[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t tile_local = tile_next;
        const int g0 = g_next;
        uint32_t ncur[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) ncur[p] = nb[p];
        const uint32_t next = item + stride;
        if (next < n_items) fetch(next);  // in flight meanwhile
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int t = TPP * pass + tl;  // token within the group
            const float f = __half2float(__ushort_as_half((unsigned short)ncur[pass])) * (1.0f / (float)D);
            // 2. codes -> centroids
            float x[32];
#pragma unroll
            for (int c = 0; c < 32; c += 4) {
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
            // 3. Sylvester FWHT: pairs at distance h become (a + b, a - b)
#pragma unroll
            for (int h = 1; h < 32; h <<= 1)
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    if (!(e & h)) {
                        const float a = x[e], b = x[e + h];
                        x[e] = a + b;
                        x[e + h] = a - b;
                    }
            if constexpr (D == 256) {
                // distance 32 between lanes l and l ^ 8 (rotation by 8 within a row of 16):
                // the lane with bit 3 clear keeps a + b, the other b' - a' of its own pair
                const float sg = (q & 1) ? -1.0f : 1.0f;
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(x[e]), 0x128, 0xF, 0xF, false);
                    x[e] = __builtin_fmaf(sg, x[e], __int_as_float(o));
                }
            }
            if constexpr (D >= 128) dq_swap_stage<true>(x);
            dq_swap_stage<false>(x);
            // 4. times n / d, rounded once to fp16. For d >= 128 the lane's two runs of 16
            //    coordinates go to their places in the pass's rows in LDS (row tl), and the
            //    wave then writes the rows out as consecutive 16-byte pieces (one store
            //    instruction covers 1 KB); for d = 64 (128-byte rows) each lane stores its
            //    runs itself.
            const int tok0 = 32 * g0 + TPP * pass;                // first token of the pass
            auto put = [&](const float* v, int first, uint8_t* row_base) {
#pragma unroll
                for (int c = 0; c < 16; c += 8) {
                    uint32_t qq[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        qq[e] = (uint32_t)__half_as_ushort(__float2half_rn(v[c + 2 * e] * f)) |
                                ((uint32_t)__half_as_ushort(__float2half_rn(v[c + 2 * e + 1] * f)) << 16);
                    *reinterpret_cast<u4*>(row_base + 2 * (first + c)) = u4{qq[0], qq[1], qq[2], qq[3]};
                }
            };
            if constexpr (D >= 128) {
                uint8_t* rowp = &ostage[w][0] + tl * C::ROW_BYTES;
                put(x, run0, rowp);
                put(x + 16, D / 2 + run0, rowp);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                u4* ob = reinterpret_cast<u4*>(out + ((size_t)tile_local * T + tok0) * D);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int piece = 64 * k + lane, row = piece / (D / 8), pc = piece % (D / 8);
                    const u4 val = *reinterpret_cast<const u4*>(&ostage[w][0] + row * C::ROW_BYTES + 16 * pc);
                    if (tok0 + row < T) ob[piece] = val;
                }
                // the next pass rewrites the rows: these reads are complete once their values
                // are stored (each store waits for its value)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            } else if (tok0 + tl < T) {
                uint8_t* rowp = reinterpret_cast<uint8_t*>(out + ((size_t)tile_local * T + tok0 + tl) * D);
                put(x, run0, rowp);
                put(x + 16, D / 2 + run0, rowp);
            }
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
    const uint32_t items_per_tile = (uint32_t)g.n_groups;
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
