// Shared-pool decode attention on the gfx950 matrix cores.
//
// PolyKV abstract: N agents decode against one compressed pool. For a pool tile (layer,
// KV head) the query rows of every agent that reads that head (agents x GQA) form the
// M side of two contractions against the tile's tokens: scores S = scale * q . k_hat
// (keys: int8 q8_0 codes times their fp16 block scale) and P.V in the Hadamard-rotated
// domain, acc = sum_t p_t n_t c[code_t]; one inverse FWHT per output row at the end
// replaces the per-token inverse rotation.
//
// Layout of the work:
// - one workgroup (4 waves) per tile; the tile's tokens are cut into 32-token chunks (one
//   value bit-plane group each) and wave w takes chunks w, w+4, w+8, ...;
// - each wave streams its chunks from HBM into its own 4-stage LDS ring with
//   global_load_lds (direct to LDS, no registers), issued three chunks ahead;
// - scores: v_mfma_f32_16x16x32_f16 with 16 tokens x one 32-wide q8 block as A (codes
//   converted to fp16 exactly) and 16 query rows as B. The query is split q = q_hi + q_lo
//   (both fp16, q_lo carrying the rounding error of q_hi), so two MFMAs per block give
//   ~22-bit query precision with exact products and fp32 accumulation; the block scale is
//   applied per token with v_fma_mix (fp16 scale, fp32 accumulate);
// - online softmax in base 2 with a lazy maximum: a row's reference m is only raised when a
//   score exceeds it by more than 8, so P stays in (0, 1] after an offset of 2^-8 and the
//   accumulators are rarely rescaled;
// - P.V: A = p * n_t in fp16 (the 8 tokens a lane holds after the score MFMA are exactly
//   the 8 K-slots it must supply, so P never leaves its registers); B = fp16 centroids
//   decoded from the bit-planes through a 4096-entry LDS table indexed by one nibble of
//   each plane (4 tokens per lookup);
// - the 4 waves' (m, l, acc) are merged through LDS, then each row gets H acc / (d l).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int CHUNK = 32;
constexpr int NSTAGE = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;  // log2 units a score may exceed the reference maximum

template <int D>
struct MCfg {
    static constexpr int NB = D / 32;                  // q8 blocks per row
    static constexpr int NDB = D / 16;                 // 16-wide dimension blocks
    static constexpr int SLOTS = D / 16;               // 16-byte slots in a key row
    static constexpr int K_BYTES = CHUNK * D;
    static constexpr int V_BYTES = 3 * D * 4;
    static constexpr int S_BYTES = CHUNK * NB * 2;
    static constexpr int N_BYTES = CHUNK * 2;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = OFF_K + K_BYTES;
    static constexpr int OFF_S = OFF_V + V_BYTES;
    static constexpr int OFF_N = OFF_S + S_BYTES;
    static constexpr int STAGE = (OFF_N + N_BYTES + 255) / 256 * 256;
    static constexpr int RING = NSTAGE * STAGE;
    static constexpr int K_INSTR = K_BYTES / 1024;           // dwordx4 DMA instructions
    static constexpr int V_INSTR = (V_BYTES + 1023) / 1024;
    static constexpr int V_TAIL_LANES = (V_BYTES % 1024) / 16;  // lanes of the last V instr
    static constexpr int S_LANES = S_BYTES / 4;               // dword DMA lanes for scales
    static constexpr int LOADS = K_INSTR + V_INSTR + 2;       // DMA instructions per chunk
    static constexpr int LUT_BYTES = 4096 * 8;
    static constexpr int OFF_LUT = 0;
    static constexpr int OFF_RING = LUT_BYTES;
    static constexpr int LDS = OFF_RING + WAVES * RING;
    static_assert(K_BYTES % 1024 == 0, "key stage is whole DMA instructions");
    static_assert(S_LANES <= 64, "scales fit one dword DMA");
};

// ---- direct-to-LDS DMA through inline asm: the compiler does not track these loads, so
// it inserts no vmcnt(0) before LDS reads; the kernel waits with explicit vmcnt counts.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

struct TileSrc {
    const int8_t* kcodes;
    const uint8_t* kscales;
    const uint8_t* vplanes;
    const uint8_t* vnorms;
    int T;
};

// Issue the DMA of chunk c into one ring stage. Every lane calls it; partial instructions
// are exec-masked. Rows past the end of the tile are clamped to the last token (valid
// memory; those tokens are masked out of the softmax).
template <int D>
__device__ __forceinline__ void issue_chunk(const TileSrc& ts, int c, uint8_t* stage, int lane) {
    using C = MCfg<D>;
    const int t0 = c * CHUNK;
    const int T = ts.T;
#pragma unroll
    for (int i = 0; i < C::K_INSTR; ++i) {
        const int o = i * 1024 + 16 * lane;
        const int tt = o / D;
        const int slot = (o % D) / 16;
        const int seg = slot ^ (tt & (C::SLOTS - 1));
        const int tok = min(t0 + tt, T - 1);
        dma16(ts.kcodes + (size_t)tok * D + seg * 16, lds_addr(stage + C::OFF_K + i * 1024));
    }
    const uint8_t* vg = ts.vplanes + (size_t)c * C::V_BYTES;
#pragma unroll
    for (int i = 0; i < C::V_INSTR; ++i) {
        const bool tail = (i == C::V_INSTR - 1) && C::V_TAIL_LANES != 0;
        if (!tail || lane < C::V_TAIL_LANES)
            dma16(vg + i * 1024 + 16 * lane, lds_addr(stage + C::OFF_V + i * 1024));
    }
    if (lane < C::S_LANES) {
        const int per_tok = C::NB * 2;
        const int o = 4 * lane;
        const int tok = min(t0 + o / per_tok, T - 1);
        dma4(ts.kscales + (size_t)tok * per_tok + (o % per_tok), lds_addr(stage + C::OFF_S));
    }
    if (lane < 16) {
        int tok = t0 + 2 * lane;
        if (tok > T - 1) tok = (T - 1) & ~1;
        dma4(ts.vnorms + (size_t)tok * 2, lds_addr(stage + C::OFF_N));
    }
}

// vmcnt wait for "n chunks issued after the one needed" (n known only at run time).
template <int LOADS>
__device__ __forceinline__ void wait_chunks_after(int n) {
    if (n >= 3) wait_vm<3 * LOADS>();
    else if (n == 2) wait_vm<2 * LOADS>();
    else if (n == 1) wait_vm<LOADS>();
    else wait_vm<0>();
}

__device__ __forceinline__ float centroid_full(uint32_t code, const CodebookHalf& cb) {
    const uint32_t m = code >= 4u ? code - 4u : 3u - code;
    const float mag = (m & 2u) ? ((m & 1u) ? cb.centroid_pos[3] : cb.centroid_pos[2])
                               : ((m & 1u) ? cb.centroid_pos[1] : cb.centroid_pos[0]);
    return code >= 4u ? mag : -mag;
}

template <int D, int NRB>
__global__ __launch_bounds__(256, 1) void k_attend_mfma(AttendArgs a) {
    using C = MCfg<D>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int l16 = lane & 15;   // row (scores) / token (key operand) / dim (values) index
    const int j = lane >> 4;     // lane group 0..3

    const PoolGeom& g = a.g;
    const int H = g.n_kv_heads, T = g.n_tokens, G = a.gqa, A = a.n_agents;
    const int R = A * G;
    const int tile_local = blockIdx.x;
    const int l_local = tile_local / H, h = tile_local - l_local * H;
    const size_t tile = (size_t)(a.layer_begin + l_local) * H + h;
    TileSrc ts;
    ts.kcodes = reinterpret_cast<const int8_t*>(a.pool + g.k_codes_off + tile * g.k_codes_stride);
    ts.kscales = a.pool + g.k_scales_off + tile * g.k_scales_stride;
    ts.vplanes = a.pool + g.v_planes_off + tile * g.v_planes_stride;
    ts.vnorms = a.pool + g.v_norms_off + tile * g.v_norms_stride;
    ts.T = T;

    const int NC = (T + CHUNK - 1) / CHUNK;
    const int nk = w < NC ? (NC - w + WAVES - 1) / WAVES : 0;  // chunks of this wave
    uint8_t* ring = lds + C::OFF_RING + w * C::RING;

    // start streaming before anything else
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nk) issue_chunk<D>(ts, w + WAVES * s, ring + s * C::STAGE, lane);

    // value lookup table: entry e -> the fp16 centroids of 4 tokens whose plane bits are
    // the nibbles (e & 15, (e >> 4) & 15, e >> 8)
    {
        h4* lut = reinterpret_cast<h4*>(lds + C::OFF_LUT);
        for (int e = tid; e < 4096; e += 256) {
            h4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t code = ((e >> u) & 1) | (((e >> (4 + u)) & 1) << 1) | (((e >> (8 + u)) & 1) << 2);
                v[u] = (_Float16)centroid_full(code, a.cb);
            }
            lut[e] = v;
        }
    }

    // query rows (B operand of the score MFMA): lane holds row 16*rb + l16, dims
    // 32*b + 8*j .. +7, pre-multiplied by scale * log2(e) and split into fp16 hi + lo
    const size_t HG = (size_t)H * G;
    const float qs = a.softmax_scale * kLog2e;
    h8 qh[NRB][C::NB], ql[NRB][C::NB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int r = 16 * rb + l16;
        const float* qrow = nullptr;
        if (r < R) {
            const int ag = r / G, jj = r - ag * G;
            qrow = a.q + (((size_t)l_local * A + ag) * HG + (size_t)h * G + jj) * D;
        }
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
            float x[8];
            if (qrow) {
                const float4 u0 = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * j);
                const float4 u1 = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * j + 4);
                x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
                x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = x[e] * qs;
                const _Float16 hi = (_Float16)v;
                qh[rb][b][e] = hi;
                ql[rb][b][e] = (_Float16)(v - (float)hi);
            }
        }
    }
    __syncthreads();  // lookup table complete

    const h4* lut = reinterpret_cast<const h4*>(lds + C::OFF_LUT);
    float m_ref[NRB], l_run[NRB];
    f4 O[NRB][C::NDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_ref[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) O[rb][db] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    for (int k = 0; k < nk; ++k) {
        const int c = w + WAVES * k;
        const int t0 = c * CHUNK;
        if (k + NSTAGE - 1 < nk)
            issue_chunk<D>(ts, c + WAVES * (NSTAGE - 1), ring + ((k + NSTAGE - 1) % NSTAGE) * C::STAGE, lane);
        wait_chunks_after<C::LOADS>(min(NSTAGE - 1, nk - 1 - k));
        const uint8_t* st = ring + (k % NSTAGE) * C::STAGE;

        // norms of the lane's 8 token slots: tokens 4j..4j+3 and 16+4j..16+4j+3
        const h4 n_lo = *reinterpret_cast<const h4*>(st + C::OFF_N + 8 * j);
        const h4 n_hi = *reinterpret_cast<const h4*>(st + C::OFF_N + 32 + 8 * j);

        // ---- scores ----
        f4 S[2][NRB];
        const bool first = (k == 0);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            // block scales of tokens 16tb + 4j + i (i = 0..3), NB per token, as h8 vectors
            h8 scv[C::NB / 2];
            {
                const h8* sp = reinterpret_cast<const h8*>(st + C::OFF_S + (16 * tb + 4 * j) * C::NB * 2);
#pragma unroll
                for (int v = 0; v < C::NB / 2; ++v) scv[v] = sp[v];
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const float init = first ? 0.0f : -(m_ref[rb] + kSlack);
                S[tb][rb] = f4{init, init, init, init};
            }
            const int tt = 16 * tb + l16;
#pragma unroll
            for (int b = 0; b < C::NB; ++b) {
                const int seg = 2 * b + (j >> 1);
                const int slot = seg ^ (tt & (C::SLOTS - 1));
                const uint2 raw = *reinterpret_cast<const uint2*>(st + C::OFF_K + tt * D + slot * 16 + 8 * (j & 1));
                h8 ak;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ak[e] = (_Float16)(int8_t)(raw.x >> (8 * e));
                    ak[4 + e] = (_Float16)(int8_t)(raw.y >> (8 * e));
                }
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    f4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qh[rb][b], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, ql[rb][b], acc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int si = i * C::NB + b;
                        S[tb][rb][i] = __builtin_fmaf(acc[i], (float)scv[si >> 3][si & 7], S[tb][rb][i]);
                    }
                }
            }
        }
        // tokens past the end of the tile
        if (t0 + CHUNK > T) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + 16 * tb + 4 * j + i >= T)
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) S[tb][rb][i] = -INFINITY;
        }
        // reference maximum: exact on the first chunk, raised lazily afterwards
        bool over = first;
        if (!first) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) over |= S[tb][rb][i] > 0.0f;
        }
        if (__any(over)) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                float cm = -INFINITY;
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) cm = fmaxf(cm, S[tb][rb][i]);
                cm = fmaxf(cm, __shfl_xor(cm, 16));
                cm = fmaxf(cm, __shfl_xor(cm, 32));
                // scores are S' = S - (m_ref + slack) (or S itself on the first chunk)
                float shift;  // amount subtracted from this chunk's scores
                if (first) {
                    m_ref[rb] = cm;
                    shift = cm + kSlack;
                } else {
                    const float up = fmaxf(cm, 0.0f);  // raise m_ref so that S' <= 0
                    m_ref[rb] += up;
                    shift = up;
                    const float alpha = exp2f(-up);
                    l_run[rb] *= alpha;
                    // accumulator rows 4j + i live in lanes whose l16 is 4j + i
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = __shfl(alpha, 4 * j + i);
#pragma unroll
                        for (int db = 0; db < C::NDB; ++db) O[rb][db][i] *= ai;
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[tb][rb][i] -= shift;
            }
        }
        // probabilities (scaled by 2^-slack), row sums, and the P.V operand p * n
        h8 ap[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            float p[8];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[4 * tb + i] = __builtin_amdgcn_exp2f(S[tb][rb][i]);
            float ls = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ls += p[e];
            l_run[rb] += ls;
            const h8 ph = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                           (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
            const h8 nn = {n_lo[0], n_lo[1], n_lo[2], n_lo[3], n_hi[0], n_hi[1], n_hi[2], n_hi[3]};
            ap[rb] = ph * nn;
        }

        // ---- P.V in the rotated domain ----
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(st + C::OFF_V);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int dim = 16 * db + l16;
            const uint32_t w0 = vw[dim], w1 = vw[D + dim], w2 = vw[2 * D + dim];
            const uint32_t sh = 4u * (uint32_t)j;
            const uint32_t ilo = ((w0 >> sh) & 15u) | (((w1 >> sh) & 15u) << 4) | (((w2 >> sh) & 15u) << 8);
            const uint32_t ihi = ((w0 >> (sh + 16u)) & 15u) | (((w1 >> (sh + 16u)) & 15u) << 4) |
                                 (((w2 >> (sh + 16u)) & 15u) << 8);
            const h4 vlo = lut[ilo], vhi = lut[ihi];
            const h8 bv = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                O[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb], bv, O[rb][db], 0, 0, 0);
        }
    }

    // ---- merge the waves and finish the rows ----
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        l_run[rb] += __shfl_xor(l_run[rb], 16);
        l_run[rb] += __shfl_xor(l_run[rb], 32);
    }
    constexpr int ROWS = 16 * NRB;
    __syncthreads();  // every ring is drained; the ring area is reused below
    float* mw = reinterpret_cast<float*>(lds + C::OFF_RING);  // [WAVES][ROWS]
    float* lw = mw + WAVES * ROWS;                             // [WAVES][ROWS]
    float* ob = lw + WAVES * ROWS;                             // [2][ROWS][D]
    if (j == 0) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            mw[w * ROWS + 16 * rb + l16] = m_ref[rb];
            lw[w * ROWS + 16 * rb + l16] = l_run[rb];
        }
    }
    __syncthreads();
    // this wave's weight for accumulator rows 16rb + 4j + i
    float fo[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * j + i;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < WAVES; ++v) M = fmaxf(M, mw[v * ROWS + row]);
            const float mine = mw[w * ROWS + row];
            fo[rb][i] = mine == -INFINITY ? 0.0f : exp2f(mine - M);
        }
    float* mybuf = ob + (w & 1) * ROWS * D;
    if (w < 2) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) mybuf[(16 * rb + 4 * j + i) * D + 16 * db + l16] = O[rb][db][i] * fo[rb][i];
    }
    __syncthreads();
    if (w >= 2) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) mybuf[(16 * rb + 4 * j + i) * D + 16 * db + l16] += O[rb][db][i] * fo[rb][i];
    }
    __syncthreads();

    // four threads per row, D/4 dimensions each; FWHT stages below D/4 in registers, the
    // last two across the four threads
    constexpr int QD = D / 4;
    const int row = tid >> 2, qtr = tid & 3;
    if (row < ROWS) {
        float x[QD];
#pragma unroll
        for (int e = 0; e < QD; ++e) x[e] = ob[row * D + qtr * QD + e] + ob[ROWS * D + row * D + qtr * QD + e];
#pragma unroll
        for (int hh = 1; hh < QD; hh <<= 1)
#pragma unroll
            for (int e = 0; e < QD; ++e)
                if (!(e & hh)) {
                    const float u = x[e], v = x[e + hh];
                    x[e] = u + v;
                    x[e + hh] = u - v;
                }
#pragma unroll
        for (int st = 1; st <= 2; st <<= 1) {
            const bool upper = (qtr & st) != 0;
#pragma unroll
            for (int e = 0; e < QD; ++e) {
                const float other = __shfl_xor(x[e], st);
                x[e] = upper ? other - x[e] : x[e] + other;
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) M = fmaxf(M, mw[v * ROWS + row]);
        float L = 0.0f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            const float mv = mw[v * ROWS + row];
            if (mv != -INFINITY) L += lw[v * ROWS + row] * exp2f(mv - M);
        }
        if (row < R) {
            const float inv = 1.0f / ((float)D * L);
            const int ag = row / G, jj = row - ag * G;
            float* o = a.out + (((size_t)l_local * A + ag) * HG + (size_t)h * G + jj) * D + qtr * QD;
#pragma unroll
            for (int e = 0; e < QD; e += 4)
                *reinterpret_cast<float4*>(o + e) = make_float4(x[e] * inv, x[e + 1] * inv, x[e + 2] * inv, x[e + 3] * inv);
        }
    }
}

template <int D, int NRB>
hipError_t launch_t(const AttendArgs& a, hipStream_t s) {
    using C = MCfg<D>;
    static_assert(C::LDS >= C::OFF_RING + (2 * WAVES * 16 * NRB + 2 * 16 * NRB * D) * 4, "merge space");
    auto kern = k_attend_mfma<D, NRB>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    const uint32_t tiles = (uint32_t)a.layer_count * (uint32_t)a.g.n_kv_heads;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), C::LDS, s, a);
    return hipGetLastError();
}

}  // namespace

bool attend_mfma_supported(const PoolGeom& g, int32_t rows) {
    return (g.head_dim == 64 || g.head_dim == 128) && rows >= 1 && rows <= 64;
}

hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s) {
    const int rows = a.n_agents * a.gqa;
    const int nrb = (rows + 15) / 16;
    if (a.g.head_dim == 128) {
        if (nrb == 1) return launch_t<128, 1>(a, s);
        if (nrb == 2) return launch_t<128, 2>(a, s);
        return launch_t<128, 4>(a, s);
    }
    if (a.g.head_dim == 64) {
        if (nrb == 1) return launch_t<64, 1>(a, s);
        if (nrb == 2) return launch_t<64, 2>(a, s);
        return launch_t<64, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace polykv
