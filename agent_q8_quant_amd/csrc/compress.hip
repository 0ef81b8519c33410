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
// Values on the vector ALU (every head_dim): one wave per 32-token group of one tile.
// Lane l holds token l % 32 of the group and its dims [h D / 2, (h + 1) D / 2), h = l / 32,
// in registers, so the rotation y = H v is log2(D) - 1 butterfly stages inside each lane
// (dims i and i + s, s < D / 2) and a last stage across the lane pair l, l ^ 32 (dims i
// and i + D / 2), in the order s = 1, 2, ..., D / 2 of the Sylvester recursion. A ballot
// of register j is then the plane words of dims j (low lanes) and j + D / 2 (high lanes),
// coded and packed by codec::put_code_words.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_compress_v(const __half* __restrict__ v,
                                                    uint8_t* __restrict__ pool, PoolGeom g,
                                                    CodebookHalf cb, int32_t layer_begin,
                                                    uint32_t n_items, TokRange rg) {
    constexpr int DH = D / 2;         // dims per lane
    constexpr int WPL = 3 * D / 64;   // plane words per lane of the store
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

    float x[DH];
    if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(v + ((size_t)tile_local * rg.n_tok + (token - rg.tok0)) * D + hl * DH);
#pragma unroll
        for (int c = 0; c < DH / 8; ++c) {
            const uint4 r = src[c];
            const __half* h = reinterpret_cast<const __half*>(&r);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * c + e] = __half2float(h[e]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < DH; ++i) x[i] = 0.0f;
    }

    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < DH; ++i) ss = fmaf(x[i], x[i], ss);
    {
        const uint32_t u = __float_as_uint(ss);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float n = sqrtf(ss);

    // unnormalised Sylvester FWHT: the stages inside the lane, then the one across the pair
    // (the low lane keeps a + b, the high lane a - b, a the low lane's value)
#pragma unroll
    for (int h = 1; h < DH; h <<= 1) {
#pragma unroll
        for (int i = 0; i < DH; ++i) {
            if (!(i & h)) {
                const float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < DH; ++i) {
        const uint32_t u = __float_as_uint(x[i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        // lane l < 32: sw[0] = own value, sw[1] = partner's; lane l >= 32: the reverse
        const float lo = __uint_as_float(sw[0]), hi = __uint_as_float(sw[1]);
        x[i] = hl ? lo - hi : lo + hi;
    }

    const codec::VThresh t = codec::v_thresholds(n, valid, cb);
    uint32_t wv[WPL];
#pragma unroll
    for (int r = 0; r < WPL; ++r) wv[r] = 0u;
#pragma unroll
    for (int j = 0; j < DH; ++j) codec::put_code_words<D>(x[j], t, j, j + DH, wv);

    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;
    uint32_t* words = reinterpret_cast<uint32_t*>(pool + g.v_planes_off + tile * g.v_planes_stride) +
                      (size_t)grp * 3 * D;
    codec::store_group_words<D>(words, keep_mask(rg, grp, T), wv, lane);
    if (hl == 0 && valid) {
        __half* norms = reinterpret_cast<__half*>(pool + g.v_norms_off + tile * g.v_norms_stride);
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

// ---------------------------------------------------------------------------------------
// Keys and values of the same token range in one launch (head_dim 64 and 128). Wave w takes
// the 32-token group w / 2 of the range (tile-major, as the value kernels number them):
// even waves its keys, odd waves its values, so every SIMD holds both kinds and the value
// waves' vector work overlaps the key waves' memory traffic.
// Keys: 32 tokens x D entries are 4 D pieces of 8 entries; lane l takes pieces l + 64 i,
// which keeps every load instruction on 1 KB of contiguous input and every quad of lanes on
// one 32-entry block (codec::q8_encode8). All of a lane's loads are issued before the first
// encode. Values: as k_compress_v_mfma.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_compress_kv(const __half* __restrict__ k,
                                                     const __half* __restrict__ v,
                                                     uint8_t* __restrict__ pool, PoolGeom g,
                                                     CodebookHalf cb, int32_t layer_begin,
                                                     uint32_t n_items, TokRange rg) {
    constexpr int KK = D / 16;        // k steps of the rotation; also key pieces per lane
    constexpr int PPT = D / 8;        // 8-entry pieces per token row
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)((blockIdx.x * 256u + threadIdx.x) >> 6));
    const uint32_t item = wave >> 1;
    if (item >= n_items) return;  // whole waves only
    const uint32_t T = (uint32_t)g.n_tokens;
    const uint32_t tile_local = item / rg.n_grp;
    const uint32_t grp = rg.g_first + (item - tile_local * rg.n_grp);
    const size_t tile = (size_t)layer_begin * g.n_kv_heads + tile_local;

    if ((wave & 1u) == 0u) {
        // keys of the group's tokens in the range
        const uint4* src = reinterpret_cast<const uint4*>(k + (size_t)tile_local * rg.n_tok * D);
        uint4 raw[KK];
#pragma unroll
        for (int i = 0; i < KK; ++i) {
            const uint32_t pc = (uint32_t)lane + 64u * i;
            const uint32_t token = grp * 32u + pc / PPT;
            const bool ok = token >= rg.tok0 && token < rg.tok0 + rg.n_tok;
            raw[i] = ok ? src[(size_t)(token - rg.tok0) * PPT + pc % PPT] : make_uint4(0, 0, 0, 0);
        }
        uint2* codes = reinterpret_cast<uint2*>(pool + g.k_codes_off + tile * g.k_codes_stride);
        __half* scales = reinterpret_cast<__half*>(pool + g.k_scales_off + tile * g.k_scales_stride);
#pragma unroll
        for (int i = 0; i < KK; ++i) {
            uint32_t packed[2];
            const __half s16 = q8_encode8(raw[i], packed);
            const uint32_t pc = (uint32_t)lane + 64u * i;
            const uint32_t token = grp * 32u + pc / PPT;
            if (token >= rg.tok0 && token < rg.tok0 + rg.n_tok) {
                const size_t piece = (size_t)token * PPT + pc % PPT;
                codes[piece] = make_uint2(packed[0], packed[1]);
                if ((lane & 3) == 0) scales[piece >> 2] = s16;
            }
        }
        return;
    }

    const int l32 = lane & 31, hl = lane >> 5;
    const uint32_t token = grp * 32u + (uint32_t)l32;
    const bool valid = token >= rg.tok0 && token < rg.tok0 + rg.n_tok;
    h8 vb[KK];
    {
        const h8* src = reinterpret_cast<const h8*>(v + ((size_t)tile_local * rg.n_tok + (valid ? token - rg.tok0 : 0u)) * D + 8 * hl);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) vb[kk] = valid ? src[2 * kk] : h8{};
    }
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
    const __half* v = (const __half*)v_fp16;
    const uint32_t blocks = (uint32_t)((items + 3) / 4);  // one wave per 32-token group
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
        case 64: hipLaunchKernelGGL(k_compress_v_mfma<64>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        case 128: hipLaunchKernelGGL(k_compress_v_mfma<128>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        case 256: hipLaunchKernelGGL(k_compress_v<256>, dim3(blocks), dim3(256), 0, s, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_compress_kv_range(const void* k_fp16, const void* v_fp16, uint8_t* pool,
                                    const PoolGeom& g, const CodebookHalf& cb, int32_t tok0,
                                    int32_t n_tok, int32_t layer_begin, int32_t layer_count,
                                    hipStream_t s) {
    if (g.head_dim == 256) {  // no matrix-core value kernel: the two launches
        hipError_t e = launch_compress_k_range(k_fp16, pool, g, tok0, n_tok, layer_begin, layer_count, s);
        if (e != hipSuccess) return e;
        return launch_compress_v_range(v_fp16, pool, g, cb, tok0, n_tok, layer_begin, layer_count, s, true);
    }
    TokRange rg;
    rg.tok0 = (uint32_t)tok0;
    rg.n_tok = (uint32_t)n_tok;
    rg.g_first = (uint32_t)tok0 / 32u;
    rg.n_grp = (uint32_t)(tok0 + n_tok - 1) / 32u - rg.g_first + 1u;
    const uint64_t items = (uint64_t)layer_count * g.n_kv_heads * rg.n_grp;
    const uint32_t blocks = (uint32_t)((2 * items + 3) / 4);  // two waves per group
    const __half* k = (const __half*)k_fp16;
    const __half* v = (const __half*)v_fp16;
    switch (g.head_dim) {
        case 64: hipLaunchKernelGGL(k_compress_kv<64>, dim3(blocks), dim3(256), 0, s, k, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
        case 128: hipLaunchKernelGGL(k_compress_kv<128>, dim3(blocks), dim3(256), 0, s, k, v, pool, g, cb, layer_begin, (uint32_t)items, rg); break;
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
