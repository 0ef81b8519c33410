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
// Work layout: one workgroup per (256-token tile, head, K or V), eight waves. The reduction
// over the hidden size runs in 64-wide steps: both operand tiles ([256 tokens][64] of x and
// [d outputs][64] of W, k-contiguous, 16-byte pieces XOR-swizzled by row) stream into a
// three-deep LDS ring by direct-to-LDS loads issued two steps ahead, spread over the
// sub-steps of the step in between, with one barrier per step.
// Wave w multiplies a 64-token x 64-output block (32-token x 64-output for d = 64) with
// v_mfma_f32_32x32x16_f16 (fp16 operands, fp32 accumulation), two by two 32 x 32 tiles, so
// every operand fragment read from LDS feeds two products. After the last step the
// workgroup rounds its 256 x d block to fp16 into LDS, and wave w encodes tokens
// 32 w .. 32 w + 31: keys with the q8_0 codec (one lane per 8 entries), values with the
// matrix-core TurboQuant codec (the wave's 32 tokens are one 32-token group).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "codec.h"
#include "lds_dma.h"
#include "polykv_internal.h"

namespace polykv {
namespace {

using codec::h8;
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;     // tokens per workgroup
constexpr int BK = 64;      // hidden entries per step
constexpr int NST = 3;      // LDS ring depth (steps)
static_assert(NST == 3, "the ring waits assume loads two steps ahead");
template <int D>
struct PjCfg {
    static constexpr int WAVES = 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WN = D / 64;                 // waves across the outputs
    static constexpr int WM = WAVES / WN;             // waves across the tokens
    static constexpr int MT = BM / WM / 32;           // 32-token tiles per wave
    static constexpr int NT = D / 32 / WN;            // 32-output tiles per wave
    static constexpr int X_BYTES = BM * BK * 2;       // one step of x
    static constexpr int W_BYTES = D * BK * 2;        // one step of W
    static constexpr int X_INSTR = X_BYTES / 1024 / WAVES;   // DMA instructions per wave and step
    static constexpr int W_INSTR = W_BYTES / 1024 / WAVES;
    static constexpr int LOADS = X_INSTR + W_INSTR;
    static constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
    static constexpr int LDS_MAIN = NST * STAGE_BYTES;
    static constexpr int LDS_OUT = BM * D * 2;        // the fp16 block (epilogue)
    static constexpr int LDS = LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT;
    static_assert(WM * WN == WAVES && MT >= 1 && NT >= 1 && 32 * NT * WN == D, "wave grid");
    static_assert(X_INSTR * WAVES * 1024 == X_BYTES && W_INSTR * WAVES * 1024 == W_BYTES, "whole DMA instructions");
    static_assert((NST - 1) * LOADS <= 63 && LDS <= 160 * 1024, "vmcnt and LDS budgets");
    static_assert(STAGE_BYTES % 256 == 0 && X_BYTES % 256 == 0, "256-byte aligned DMA destinations");
};

// LDS offset (bytes) of the 16-byte piece c (0..7) of row r of a [rows][64] fp16 tile. The
// XOR with bits 1..3 of the row puts the 16 rows one fragment read touches (same piece) on
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t sw_off(uint32_t r, uint32_t c) { return r * 128u + ((c ^ ((r >> 1) & 7u)) << 4); }

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

// A step's operand tiles go into a ring stage by direct-to-LDS loads, LOADS instructions per
// wave: instruction j < X_INSTR is x-tile instruction w + WAVES j, the others W-tile
// instructions. Destination piece P (16 bytes, lane-linear within each 1 KB instruction) is
// row P / 8, slot P % 8 of its tile; it holds global piece (P % 8) ^ ((row >> 1) & 7) of
// that row, which realises the swizzle of sw_off. Rows past the chunk read its last row
// (valid memory; their results are not stored). The per-lane offsets are fixed over the
// reduction (the scalar base moves by k0), so they are computed once.
template <class C>
struct DmaOffs {
    uint32_t o[C::LOADS];
};
template <class C>
__device__ __forceinline__ DmaOffs<C> dma_offsets(int hidden, int rows_valid, int w, int lane) {
    DmaOffs<C> d;
    const uint32_t row_bytes = (uint32_t)hidden * 2u;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
        const bool isx = j < C::X_INSTR;
        const int q = w + C::WAVES * (isx ? j : j - C::X_INSTR);
        const uint32_t P = 64u * (uint32_t)q + (uint32_t)lane, r = P >> 3, c = (P & 7u) ^ ((r >> 1) & 7u);
        const uint32_t rr = isx ? min(r, (uint32_t)rows_valid - 1u) : r;
        d.o[j] = rr * row_bytes + 16u * c;
    }
    return d;
}
// Instruction j of a step's loads is issued during sub-step sched(j) (1, 2 or 3) of the step
// two before, between that sub-step's fragment reads and its products. Issued in one burst
// after the barrier, every wave's loads (40 or 48 instructions) queue at the CU's memory
// unit at once and a wave held at one of them issues no products; spread out, they overlap
// the products. Sub-step 0 is left out: every wave reads its first fragments right after
// the barrier.
template <class C>
__device__ __forceinline__ constexpr int sched(int j) { return 1 + j * (BK / 16 - 1) / C::LOADS; }
template <class C>
__device__ __forceinline__ void issue_one(const __half* xt, const __half* wmat, int k0, int j, int w,
                                          const DmaOffs<C>& d, uint8_t* stage) {
    const bool isx = j < C::X_INSTR;
    const int q = w + C::WAVES * (isx ? j : j - C::X_INSTR);
    if (isx) lds_dma::dma16(xt + k0, d.o[j], lds_dma::lds_addr(stage + 1024 * q));
    else lds_dma::dma16(wmat + k0, d.o[j], lds_dma::lds_addr(stage + C::X_BYTES + 1024 * q));
}

// One 32-token group of the projected block (fp16 in LDS, [32 tokens][D]): written as fp16
// (mode STORE) or encoded into the pool.
template <int D, int MODE>
__device__ __forceinline__ void encode_group(const PjArgs& a, const __half* stage, int t_wave, int which,
                                             int h, int lane) {
    const int n_tok = a.n_tok;
    constexpr int PPR = D / 8;                             // 16-byte pieces per token row
    if constexpr (MODE == MODE_STORE) {
        __half* out = a.out[which] + (size_t)h * n_tok * D;
        for (int p = lane; p < 32 * PPR; p += 64) {
            const int m = p / PPR, c = p % PPR;
            if (t_wave + m < n_tok)
                *reinterpret_cast<u4*>(out + (size_t)(t_wave + m) * D + 8 * c) =
                    *reinterpret_cast<const u4*>(stage + m * D + 8 * c);
        }
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
__global__ __launch_bounds__(PjCfg<D>::THREADS, 1) void k_project(PjArgs a) {
    using C = PjCfg<D>;
    constexpr int MT = C::MT, NT = C::NT;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t_tile = blockIdx.x * BM;                    // first token of the tile (chunk-relative)
    const int h = blockIdx.y;
    const int which = blockIdx.z;                          // 0: K, 1: V
    const int n_tok = a.n_tok, hidden = a.hidden;
    const __half* wmat = a.w[which] + (size_t)h * D * hidden;
    const __half* xt = a.x + (size_t)t_tile * hidden;
    const int rows_valid = min(BM, n_tok - t_tile);
    const int wm = w / C::WN, wn = w - wm * C::WN;
    const uint32_t row0 = 32u * MT * wm, col0 = 32u * NT * wn;  // the wave's block in the tile

    f16v acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f16v{};

    // ring of NST stages: step ks multiplies stage ks % NST; the loads of step ks + NST - 1
    // go into the stage step ks - 1 used, after the barrier that ends every wave's reads of
    // it, spread over the sub-steps of step ks
    const DmaOffs<C> dof = dma_offsets<C>(hidden, rows_valid, w, lane);
    const int steps = hidden / BK;
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < steps)
#pragma unroll
            for (int j = 0; j < C::LOADS; ++j) issue_one<C>(xt, wmat, s * BK, j, w, dof, lds + s * C::STAGE_BYTES);
    for (int ks = 0; ks < steps; ++ks) {
        // this step's loads (and those of every earlier step) have landed, in every wave:
        // only the next step's may still be in flight
        if (ks + 1 < steps) lds_dma::wait_vm<C::LOADS>();
        else lds_dma::wait_vm<0>();
        __syncthreads();
        const bool more = ks + NST - 1 < steps;
        uint8_t* nst = lds + ((ks + NST - 1) % NST) * C::STAGE_BYTES;
        const int nk0 = (ks + NST - 1) * BK;
        const uint8_t* xs = lds + (ks % NST) * C::STAGE_BYTES;
        const uint8_t* ws = xs + C::X_BYTES;
#pragma unroll
        for (int ss = 0; ss < BK / 16; ++ss) {
            // lane l: row l % 32 of a tile, k = 16 ss + 8 (l / 32) .. + 7 (piece 2 ss + l / 32)
            const uint32_t c = 2u * ss + (uint32_t)(lane >> 5);
            h8 av[MT], bv[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                av[i] = *reinterpret_cast<const h8*>(xs + sw_off(row0 + 32u * i + (lane & 31), c));
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bv[j] = *reinterpret_cast<const h8*>(ws + sw_off(col0 + 32u * j + (lane & 31), c));
            if (more)
#pragma unroll
                for (int j = 0; j < C::LOADS; ++j)
                    if (sched<C>(j) == ss) issue_one<C>(xt, wmat, nk0, j, w, dof, nst);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with the ring: the fp16 block reuses it

    // the workgroup's BM x D block, rounded to fp16, into LDS [BM tokens][D]
    __half* blk = reinterpret_cast<__half*>(lds);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // register e: token 8 (e / 4) + 4 (l / 32) + e % 4, output column l % 32 of the tile
                const uint32_t m = row0 + 32u * i + 8u * (e / 4) + 4u * (lane >> 5) + (e & 3);
                blk[m * D + col0 + 32u * j + (lane & 31)] = __float2half_rn(acc[i][j][e]);
            }
    __syncthreads();

    // ---- epilogue: the tile's 32-token groups, wave w taking groups w, w + WAVES, ... ----
    for (int grp32 = w; grp32 < BM / 32; grp32 += C::WAVES) {
        const int t_wave = t_tile + 32 * grp32;            // chunk-relative first token
        if (t_wave >= n_tok) break;                        // wave-uniform
        encode_group<D, MODE>(a, blk + 32 * grp32 * D, t_wave, which, h, lane);
    }
}

template <int D, int MODE>
hipError_t launch_t(const PjArgs& a, int nz, hipStream_t s) {
    using C = PjCfg<D>;
    auto kern = k_project<D, MODE>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once((const void*)kern, C::LDS, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((a.n_tok + BM - 1) / BM, a.n_heads, nz);
    hipLaunchKernelGGL(kern, grid, dim3(C::THREADS), C::LDS, s, a);
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
