// K/V projection with the pool compression fused into its epilogue (gfx950).
//
// PolyKV abstract: the shared KV cache is compressed a single time, when it is written.
// The K and V of a prefill chunk are the projections x W_k^T and x W_v^T of the layer's
// input; this kernel computes them on the matrix cores and compresses every 32-token x
// head tile straight from its accumulators into the pool, so the fp16 K and V never go
// to HBM. Each projection output is rounded to fp16 first (the value an fp16 cache would
// hold), so the pool bytes are exactly those of an fp16 projection followed by
// polykv_append_k/v. The same kernel without the compression (mode STORE) writes the fp16
// projection, head-major [H][n_tok][d], for that unfused path.
//
// Work layout: one workgroup per (128-token tile, head, K or V), four waves; wave w owns
// tokens 32 w .. 32 w + 31 of the tile and all d columns of the head. The reduction over
// the hidden size runs in 64-wide steps: both operand tiles ([128 tokens][64] of x and
// [d outputs][64] of W, k-contiguous, 16-byte pieces XOR-swizzled by row) go through two
// LDS stages, and every thread holds the pieces of the step after next in registers while
// the current step is multiplied (v_mfma_f32_32x32x16_f16: 32 tokens x 32 outputs per instruction, fp16
// operands, fp32 accumulation). After the last step each wave rounds its 32 x d block to
// fp16 into LDS and encodes it: keys with the q8_0 codec (one lane per 8 entries), values
// with the matrix-core TurboQuant codec (the wave's 32 tokens are one 32-token group).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "codec.h"
#include "polykv_internal.h"

namespace polykv {
namespace {

using codec::h8;
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;   // tokens per workgroup
constexpr int BK = 64;    // hidden entries per step

template <int D>
struct PjCfg {
    static constexpr int NT = D / 32;                 // 32-column output tiles per wave
    static constexpr int X_PIECES = BM * BK / 8;      // 16-byte pieces of the x tile
    static constexpr int W_PIECES = D * BK / 8;
    static constexpr int XPT = X_PIECES / 256;        // per thread
    static constexpr int WPT = W_PIECES / 256;
    static constexpr int OFF_X = 0;                                  // two stages of x and W
    static constexpr int OFF_W = OFF_X + BM * BK * 2;
    static constexpr int STAGE_BYTES = OFF_W + D * BK * 2;
    static constexpr int LDS_MAIN = 2 * STAGE_BYTES;
    static constexpr int STAGE = 32 * D * 2;          // one wave's fp16 block (epilogue)
    static constexpr int LDS = LDS_MAIN > 4 * STAGE ? LDS_MAIN : 4 * STAGE;
    static_assert(XPT >= 1 && WPT >= 1, "whole pieces per thread");
};

// LDS offset (bytes) of the 16-byte piece c (0..7) of row r of a [rows][64] fp16 tile
__device__ __forceinline__ uint32_t sw_off(uint32_t r, uint32_t c) { return r * 128u + ((c ^ (r & 7u)) << 4); }

struct PjArgs {
    const __half* x;        // [n_tok][hidden]
    const __half* w[2];     // [n_heads * d][hidden] for K (0) and V (1)
    __half* out[2];         // mode STORE: [n_heads][n_tok][d] for K and V
    uint8_t* pool;
    PoolGeom g;
    CodebookHalf cb;
    int32_t layer, tok0, n_tok, hidden, n_heads;
};

enum { MODE_STORE = 0, MODE_POOL = 1 };

template <int D, int MODE>
__global__ __launch_bounds__(256) void k_project(PjArgs a) {
    using C = PjCfg<D>;
    constexpr int NT = C::NT;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t_tile = blockIdx.x * BM;                    // first token of the tile (chunk-relative)
    const int h = blockIdx.y;
    const int which = blockIdx.z;                          // 0: K, 1: V
    const int n_tok = a.n_tok, hidden = a.hidden;
    const __half* wmat = a.w[which] + (size_t)h * D * hidden;

    // global -> register pieces of step k0: piece p of x is row p / 8, column piece p % 8;
    // rows past the chunk read its last row (valid memory; their results are not stored)
    u4 px[C::XPT], pw[C::WPT];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int p = tid + 256 * i, r = p >> 3, c = p & 7;
            const int row = min(t_tile + r, n_tok - 1);
            px[i] = *reinterpret_cast<const u4*>(a.x + (size_t)row * hidden + k0 + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < C::WPT; ++i) {
            const int p = tid + 256 * i, r = p >> 3, c = p & 7;
            pw[i] = *reinterpret_cast<const u4*>(wmat + (size_t)r * hidden + k0 + 8 * c);
        }
    };

    f16v acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f16v{};

    // two LDS stages: step ks multiplies stage ks % 2 while the registers of step ks + 1 go
    // into the other stage and the loads of step ks + 2 are in flight; one barrier per step
    const int steps = hidden / BK;
    auto put = [&](int st) {
        uint8_t* base = lds + st * C::STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) {
            const int p = tid + 256 * i;
            *reinterpret_cast<u4*>(base + C::OFF_X + sw_off(p >> 3, p & 7)) = px[i];
        }
#pragma unroll
        for (int i = 0; i < C::WPT; ++i) {
            const int p = tid + 256 * i;
            *reinterpret_cast<u4*>(base + C::OFF_W + sw_off(p >> 3, p & 7)) = pw[i];
        }
    };
    fetch(0);
    put(0);
    if (steps > 1) fetch(BK);
    __syncthreads();
    for (int ks = 0; ks < steps; ++ks) {
        const uint8_t* base = lds + (ks & 1) * C::STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            // lane l: row l % 32 of its block, k = 16 s + 8 (l / 32) .. + 7 (piece 2 s + l / 32)
            const uint32_t c = 2u * s + (uint32_t)(lane >> 5);
            const h8 av = *reinterpret_cast<const h8*>(base + C::OFF_X + sw_off(32u * w + (lane & 31), c));
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const h8 bv = *reinterpret_cast<const h8*>(base + C::OFF_W + sw_off(32u * j + (lane & 31), c));
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[j], 0, 0, 0);
            }
        }
        if (ks + 1 < steps) {
            put((ks + 1) & 1);                          // its readers finished before the last barrier
            if (ks + 2 < steps) fetch((ks + 2) * BK);
        }
        __syncthreads();
    }

    // ---- epilogue: the wave's 32 x D block, rounded to fp16, into its LDS stage (the
    // loop's last barrier: every wave is done with the operand tiles) ----
    __half* stage = reinterpret_cast<__half*>(lds + w * C::STAGE);   // [32 tokens][D]
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // register i: token 8 (i / 4) + 4 (l / 32) + i % 4, output column l % 32 of tile j
            const int m = 8 * (i / 4) + 4 * (lane >> 5) + (i & 3);
            stage[m * D + 32 * j + (lane & 31)] = __float2half_rn(acc[j][i]);
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const int t_wave = t_tile + 32 * w;                    // chunk-relative first token
    if (t_wave >= n_tok) return;                           // wave-uniform
    constexpr int PPR = D / 8;                             // 16-byte pieces per token row
    if constexpr (MODE == MODE_STORE) {
        __half* out = a.out[which] + (size_t)h * n_tok * D;
        for (int p = lane; p < 32 * PPR; p += 64) {
            const int m = p / PPR, c = p % PPR;
            if (t_wave + m < n_tok)
                *reinterpret_cast<u4*>(out + (size_t)(t_wave + m) * D + 8 * c) =
                    *reinterpret_cast<const u4*>(stage + m * D + 8 * c);
        }
        return;
    } else {
        const PoolGeom& g = a.g;
        const size_t tile = (size_t)a.layer * g.n_kv_heads + h;
        const uint32_t tok = (uint32_t)(a.tok0 + t_wave);   // pool token of the wave's row 0
        if (which == 0) {
            // keys: lane = 8 entries; a quad = one 32-entry block of one token
            uint2* codes = reinterpret_cast<uint2*>(a.pool + g.k_codes_off + tile * g.k_codes_stride);
            __half* scales = reinterpret_cast<__half*>(a.pool + g.k_scales_off + tile * g.k_scales_stride);
#pragma unroll
            for (int it = 0; it < 32 * PPR / 64; ++it) {
                const int p = lane + 64 * it, m = p / PPR, c = p % PPR;
                const uint4 raw = *reinterpret_cast<const uint4*>(stage + m * D + 8 * c);
                uint32_t packed[2];
                const __half s16 = codec::q8_encode8(raw, packed);
                if (t_wave + m < n_tok) {
                    const size_t v = (size_t)(tok + m) * PPR + c;
                    codes[v] = make_uint2(packed[0], packed[1]);
                    if ((lane & 3) == 0) scales[v >> 2] = s16;
                }
            }
        } else {
            // values: the wave's 32 tokens are the 32-token group tok / 32
            h8 vb[D / 16];
            const int t32 = lane & 31;
            const bool valid = t_wave + t32 < n_tok;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                vb[kk] = valid ? *reinterpret_cast<const h8*>(stage + t32 * D + 16 * kk + 8 * (lane >> 5)) : h8{};
            const uint32_t grp = tok / 32u;
            // tokens of the group past the chunk but below the pool length keep their bits
            const uint32_t end = (uint32_t)(a.tok0 + n_tok), T = (uint32_t)g.n_tokens;
            const uint32_t lim = min(T, grp * 32u + 32u);
            uint32_t keep = 0u;
            if (lim > end) {
                const uint32_t lo = end - grp * 32u, hi = lim - grp * 32u;
                keep = (hi >= 32u ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
            }
            uint32_t* words = reinterpret_cast<uint32_t*>(a.pool + g.v_planes_off + tile * g.v_planes_stride) +
                              (size_t)grp * 3 * D;
            __half* norms = reinterpret_cast<__half*>(a.pool + g.v_norms_off + tile * g.v_norms_stride);
            codec::encode_v_group<D>(vb, valid, a.cb, words, keep, norms, tok + (uint32_t)t32, lane);
        }
    }
}

template <int D, int MODE>
hipError_t launch_t(const PjArgs& a, int nz, hipStream_t s) {
    using C = PjCfg<D>;
    auto kern = k_project<D, MODE>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    dim3 grid((a.n_tok + BM - 1) / BM, a.n_heads, nz);
    hipLaunchKernelGGL(kern, grid, dim3(256), C::LDS, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const __half* x, const __half* w_k, const __half* w_v, __half* k_out,
                          __half* v_out, int32_t n_tok, int32_t hidden, int32_t n_heads,
                          int32_t head_dim, hipStream_t s) {
    PjArgs a = {};
    a.x = x;
    a.w[0] = w_k;
    a.w[1] = w_v;
    a.out[0] = k_out;
    a.out[1] = v_out;
    a.n_tok = n_tok;
    a.hidden = hidden;
    a.n_heads = n_heads;
    if (!w_v) {  // K only
        if (head_dim == 64) return launch_t<64, MODE_STORE>(a, 1, s);
        if (head_dim == 128) return launch_t<128, MODE_STORE>(a, 1, s);
        return hipErrorInvalidValue;
    }
    if (head_dim == 64) return launch_t<64, MODE_STORE>(a, 2, s);
    if (head_dim == 128) return launch_t<128, MODE_STORE>(a, 2, s);
    return hipErrorInvalidValue;
}

hipError_t launch_project_compress(const __half* x, const __half* w_k, const __half* w_v,
                                   uint8_t* pool, const PoolGeom& g, const CodebookHalf& cb,
                                   int32_t layer, int32_t tok0, int32_t n_tok, int32_t hidden,
                                   hipStream_t s) {
    PjArgs a = {};
    a.x = x;
    a.w[0] = w_k;
    a.w[1] = w_v;
    a.pool = pool;
    a.g = g;
    a.cb = cb;
    a.layer = layer;
    a.tok0 = tok0;
    a.n_tok = n_tok;
    a.hidden = hidden;
    a.n_heads = g.n_kv_heads;
    if (g.head_dim == 64) return launch_t<64, MODE_POOL>(a, 2, s);
    if (g.head_dim == 128) return launch_t<128, MODE_POOL>(a, 2, s);
    return hipErrorInvalidValue;
}

}  // namespace polykv
