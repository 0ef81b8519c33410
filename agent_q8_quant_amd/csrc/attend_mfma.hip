// Shared-pool decode attention on the gfx950 matrix cores.
//
// PolyKV abstract: N agents decode against one compressed pool. For a pool tile (layer,
// KV head) the query rows of every agent that reads that head (agents x GQA) form the
// M side of two contractions against the tile's tokens: scores S = scale * q . k_hat
// (keys: int8 q8_0 codes times their fp16 block scale) and P.V in the Hadamard-rotated
// domain, acc = sum_t p_t n_t c[code_t]; one inverse FWHT per output row at the end
// replaces the per-token inverse rotation.
//
// Layout of the work (one workgroup of 8 waves per tile):
// - the tile's tokens are cut into 32-token chunks (one value bit-plane group each); pair
//   p of waves (p = 0..3, sharing SIMD p) takes chunks p, p+4, p+8, ...;
// - in each pair, a score wave streams keys, block scales and norms into its LDS ring
//   (direct-to-LDS DMA), computes S with v_mfma_f32_16x16x32_f16 (16 tokens x one
//   32-wide q8 block as A, codes converted to fp16 exactly; 16 query rows as B, the query
//   split q = q_hi + q_lo in fp16 for ~22-bit precision), applies the block scales with
//   v_fma_mix, runs a lazy-max online softmax in base 2 and writes p * n_t as fp16 to a
//   double-buffered LDS slot; a value wave streams the value bit-planes, decodes them to
//   fp16 centroids through a 4096-entry table (one nibble of each plane = 4 tokens) and
//   accumulates P.V in fp32 one chunk behind the score wave. The two waves of a pair sit
//   on one SIMD, so the matrix work of one overlaps the vector work of the other;
// - a row's reference maximum is raised only when a score exceeds it by more than 8
//   (log2 units); the score wave then passes per-row rescale factors to the value wave;
// - at the end the pairs' (m, l, acc) are merged through LDS and each row becomes
//   H acc / (d l).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int PAIRS = 4;
constexpr int CHUNK = 32;
constexpr int NSTAGE = 3;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;  // log2 units a score may exceed the reference maximum

template <int D, int NRB>
struct MCfg {
    static constexpr int NB = D / 32;                  // q8 blocks per row
    static constexpr int NDB = D / 16;                 // 16-wide dimension blocks
    static constexpr int SLOTS = D / 16;               // 16-byte slots in a key row
    static constexpr int ROWS = 16 * NRB;
    // score-wave stage: key codes, block scales, value norms
    static constexpr int K_BYTES = CHUNK * D;
    static constexpr int S_BYTES = CHUNK * NB * 2;
    static constexpr int N_BYTES = CHUNK * 2;
    static constexpr int A_OFF_K = 0;
    static constexpr int A_OFF_S = K_BYTES;
    static constexpr int A_OFF_N = A_OFF_S + S_BYTES;
    static constexpr int A_STAGE = (A_OFF_N + N_BYTES + 255) / 256 * 256;
    // value-wave stage: the three bit-planes of the chunk
    static constexpr int V_BYTES = 3 * D * 4;
    static constexpr int B_STAGE = (V_BYTES + 255) / 256 * 256;
    // probabilities p * n (fp16 A operand of P.V), per row block one h8 per lane, and the
    // per-row rescale factors with a flag
    static constexpr int P_BYTES = NRB * 64 * 16;
    static constexpr int ALPHA_BYTES = ROWS * 4 + 16;
    // per pair
    static constexpr int PAIR_OFF_A = 0;
    static constexpr int PAIR_OFF_B = PAIR_OFF_A + NSTAGE * A_STAGE;
    static constexpr int PAIR_OFF_P = PAIR_OFF_B + NSTAGE * B_STAGE;
    static constexpr int PAIR_OFF_AL = PAIR_OFF_P + 2 * P_BYTES;
    static constexpr int PAIR_BYTES = (PAIR_OFF_AL + 2 * ALPHA_BYTES + 255) / 256 * 256;
    static constexpr int LUT_BYTES = 4096 * 8;
    static constexpr int OFF_LUT = 0;
    static constexpr int OFF_PAIRS = LUT_BYTES;
    static constexpr int LDS = OFF_PAIRS + PAIRS * PAIR_BYTES;
    // DMA instructions per chunk
    static constexpr int K_INSTR = K_BYTES / 1024;
    static constexpr int S_LANES = S_BYTES / 4;
    static constexpr int A_LOADS = K_INSTR + 2;
    static constexpr int V_INSTR = (V_BYTES + 1023) / 1024;
    static constexpr int V_TAIL_LANES = (V_BYTES % 1024) / 16;
    static constexpr int B_LOADS = V_INSTR;
    // merge area (reuses the pair area at the end)
    static constexpr int MERGE_BYTES = (2 * PAIRS * ROWS + 2 * ROWS * D) * 4;
    static_assert(K_BYTES % 1024 == 0, "key stage is whole DMA instructions");
    static_assert(S_LANES <= 64, "scales fit one dword DMA");
    static_assert(MERGE_BYTES <= PAIRS * PAIR_BYTES, "merge area fits");
};

// ---- direct-to-LDS DMA through inline asm: the compiler does not track these loads, so
// it inserts no vmcnt(0) before LDS reads; each wave waits on its own loads with explicit
// vmcnt counts. Address = 64-bit scalar base + 32-bit per-lane offset; LDS destination =
// M0 + 16 * lane (4 * lane for dwords).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// wait until at most n later chunks (of LOADS instructions each) are still in flight
template <int LOADS>
__device__ __forceinline__ void wait_chunks_after(int n) {
    if (n >= 2) wait_vm<2 * LOADS>();
    else if (n == 1) wait_vm<LOADS>();
    else wait_vm<0>();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// 8 int8 codes -> 8 fp16 (exact): sign-extending byte selects, two results per dword.
__device__ __forceinline__ h8 codes_to_h8(uint2 raw) {
    uint32_t d0, d1, d2, d3;
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(d0) : "v"(raw.x));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1" : "+v"(d0) : "v"(raw.x));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(d1) : "v"(raw.x));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3" : "+v"(d1) : "v"(raw.x));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(d2) : "v"(raw.y));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1" : "+v"(d2) : "v"(raw.y));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(d3) : "v"(raw.y));
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3" : "+v"(d3) : "v"(raw.y));
    const uint4 u = make_uint4(d0, d1, d2, d3);
    return __builtin_bit_cast(h8, u);
}

__device__ __forceinline__ float centroid_full(uint32_t code, const CodebookHalf& cb) {
    const uint32_t m = code >= 4u ? code - 4u : 3u - code;
    const float mag = (m & 2u) ? ((m & 1u) ? cb.centroid_pos[3] : cb.centroid_pos[2])
                               : ((m & 1u) ? cb.centroid_pos[1] : cb.centroid_pos[0]);
    return code >= 4u ? mag : -mag;
}

struct TileSrc {
    const int8_t* kcodes;
    const uint8_t* kscales;
    const uint8_t* vplanes;
    const uint8_t* vnorms;
    int T;
};

// Score wave: DMA of the keys, block scales and norms of chunk c. Key rows keep their
// 16-byte slots XOR-swizzled by the row index, so the 16 rows one fragment read touches
// fall into distinct LDS banks. Rows past the end of the tile are clamped to the last
// token (valid memory; those tokens are masked out of the softmax).
template <int D, int NRB>
__device__ __forceinline__ void issue_keys(const TileSrc& ts, const uint32_t (&krow)[MCfg<D, NRB>::K_INSTR],
                                           const uint32_t (&kseg)[MCfg<D, NRB>::K_INSTR], int c,
                                           uint8_t* stage, int lane) {
    using C = MCfg<D, NRB>;
    const int t0 = c * CHUNK;
    const int T = ts.T;
    const bool full = t0 + CHUNK <= T;
    const int8_t* kb = ts.kcodes + (size_t)t0 * D;
#pragma unroll
    for (int i = 0; i < C::K_INSTR; ++i) {
        uint32_t row = krow[i];
        if (!full) row = min(row, (uint32_t)(T - 1 - t0));
        dma16(kb, row * D + kseg[i], lds_addr(stage + C::A_OFF_K + i * 1024));
    }
    constexpr int per_tok = C::NB * 2;
    if (lane < C::S_LANES) {
        const int o = 4 * lane;
        int row = o / per_tok;
        if (!full) row = min(row, T - 1 - t0);
        dma4(ts.kscales + (size_t)t0 * per_tok, (uint32_t)(row * per_tok + (o % per_tok)),
             lds_addr(stage + C::A_OFF_S));
    }
    if (lane < 16) {
        int row = 2 * lane;
        if (!full && row > T - 1 - t0) row = (T - 1 - t0) & ~1;
        dma4(ts.vnorms + (size_t)t0 * 2, (uint32_t)(row * 2), lds_addr(stage + C::A_OFF_N));
    }
}

// Value wave: DMA of the three bit-planes of chunk c (always inside the tile).
template <int D, int NRB>
__device__ __forceinline__ void issue_values(const TileSrc& ts, int c, uint8_t* stage, int lane) {
    using C = MCfg<D, NRB>;
    const uint8_t* vg = ts.vplanes + (size_t)c * C::V_BYTES;
#pragma unroll
    for (int i = 0; i < C::V_INSTR; ++i) {
        const bool tail = (i == C::V_INSTR - 1) && C::V_TAIL_LANES != 0;
        if (!tail || lane < C::V_TAIL_LANES)
            dma16(vg, (uint32_t)(i * 1024 + 16 * lane), lds_addr(stage + i * 1024));
    }
}

template <int D, int NRB>
__global__ __launch_bounds__(512, 1) void k_attend_mfma(AttendArgs a) {
    using C = MCfg<D, NRB>;
    constexpr int NB = C::NB, NDB = C::NDB, ROWS = C::ROWS;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int pair = w & (PAIRS - 1);
    const bool score_wave = w < PAIRS;
    const int l16 = lane & 15;
    const int j = lane >> 4;

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
    const int nk = pair < NC ? (NC - pair + PAIRS - 1) / PAIRS : 0;  // chunks of this pair
    const int nk_max = (NC + PAIRS - 1) / PAIRS;                      // same for every wave
    uint8_t* pbase = lds + C::OFF_PAIRS + pair * C::PAIR_BYTES;
    uint8_t* aring = pbase + C::PAIR_OFF_A;
    uint8_t* bring = pbase + C::PAIR_OFF_B;
    h8* pbuf = reinterpret_cast<h8*>(pbase + C::PAIR_OFF_P);          // [2][NRB][64]
    float* albuf = reinterpret_cast<float*>(pbase + C::PAIR_OFF_AL);  // [2][ROWS + 4]
    constexpr int AL_STRIDE = ROWS + 4;

    // per-lane DMA offsets of the key rows (independent of the chunk)
    uint32_t krow[C::K_INSTR], kseg[C::K_INSTR];
#pragma unroll
    for (int i = 0; i < C::K_INSTR; ++i) {
        const int o = i * 1024 + 16 * lane;
        const int tt = o / D;
        const int slot = (o % D) / 16;
        krow[i] = (uint32_t)tt;
        kseg[i] = (uint32_t)((slot ^ (tt & (C::SLOTS - 1))) * 16);
    }
    // start streaming: the score wave two chunks ahead, the value wave likewise
    if (score_wave) {
        for (int s = 0; s < NSTAGE - 1; ++s)
            if (s < nk) issue_keys<D, NRB>(ts, krow, kseg, pair + PAIRS * s, aring + s * C::A_STAGE, lane);
    } else {
        for (int s = 0; s < NSTAGE - 1; ++s)
            if (s < nk) issue_values<D, NRB>(ts, pair + PAIRS * s, bring + s * C::B_STAGE, lane);
    }

    // value lookup table: entry e -> lambda * the centroids of the 4 tokens whose plane bits
    // are the nibbles (e & 15, (e >> 4) & 15, e >> 8), in fp16
    {
        h4* lut = reinterpret_cast<h4*>(lds + C::OFF_LUT);
        const float lam = a.cb.fp16_scale;
        for (int e = tid; e < 4096; e += 512) {
            h4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t code = ((e >> u) & 1) | (((e >> (4 + u)) & 1) << 1) | (((e >> (8 + u)) & 1) << 2);
                v[u] = (_Float16)(lam * centroid_full(code, a.cb));
            }
            lut[e] = v;
        }
    }
    __syncthreads();

    const size_t HG = (size_t)H * G;
    float m_ref[NRB], l_run[NRB];  // score wave: per row l16 of each row block
    f4 O[NRB][NDB];                // value wave: rows 16rb + 4j + i, dim 16db + l16
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        m_ref[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) O[rb][db] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    if (score_wave) {
        // ===================== score wave =====================
        // query rows (B operand): lane holds row 16rb + l16, dims 32b + 8j .. +7, times
        // scale * log2(e), as fp16 hi + lo
        const float qs = a.softmax_scale * kLog2e;
        h8 qh[NRB][NB], ql[NRB][NB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = 16 * rb + l16;
            const float* qrow = nullptr;
            if (r < R) {
                const int ag = r / G, jj = r - ag * G;
                qrow = a.q + (((size_t)l_local * A + ag) * HG + (size_t)h * G + jj) * D;
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
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
        // LDS offsets (within a stage) of the key fragments: token 16tb + l16, dims
        // 32b + 8j .. +7, through the row swizzle
        uint32_t kfrag[2][NB];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int tt = 16 * tb + l16;
                const int seg = 2 * b + (j >> 1);
                const int slot = seg ^ (tt & (C::SLOTS - 1));
                kfrag[tb][b] = (uint32_t)(C::A_OFF_K + tt * D + slot * 16 + 8 * (j & 1));
            }

        for (int k = 0; k < nk_max; ++k) {
            if (k < nk) {
                const int c = pair + PAIRS * k;
                const int t0 = c * CHUNK;
                if (k + NSTAGE - 1 < nk)
                    issue_keys<D, NRB>(ts, krow, kseg, c + PAIRS * (NSTAGE - 1),
                                       aring + ((k + NSTAGE - 1) % NSTAGE) * C::A_STAGE, lane);
                wait_chunks_after<C::A_LOADS>(min(NSTAGE - 1, nk - 1 - k));
                const uint8_t* st = aring + (k % NSTAGE) * C::A_STAGE;
                const h4 n_lo = *reinterpret_cast<const h4*>(st + C::A_OFF_N + 8 * j);
                const h4 n_hi = *reinterpret_cast<const h4*>(st + C::A_OFF_N + 32 + 8 * j);
                const bool first = k == 0;
                f4 S[2][NRB];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    h8 scv[NB / 2];
                    const h8* sp = reinterpret_cast<const h8*>(st + C::A_OFF_S + (16 * tb + 4 * j) * NB * 2);
#pragma unroll
                    for (int v = 0; v < NB / 2; ++v) scv[v] = sp[v];
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const float init = first ? 0.0f : -(m_ref[rb] + kSlack);
                        S[tb][rb] = f4{init, init, init, init};
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const h8 ak = codes_to_h8(*reinterpret_cast<const uint2*>(st + kfrag[tb][b]));
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) {
                            f4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qh[rb][b], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, ql[rb][b], acc, 0, 0, 0);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int si = i * NB + b;
                                S[tb][rb][i] = __builtin_fmaf(acc[i], (float)scv[si >> 3][si & 7], S[tb][rb][i]);
                            }
                        }
                    }
                }
                if (t0 + CHUNK > T) {
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (t0 + 16 * tb + 4 * j + i >= T)
#pragma unroll
                                for (int rb = 0; rb < NRB; ++rb) S[tb][rb][i] = -INFINITY;
                }
                // reference maxima: exact on the first chunk; afterwards raised only when a
                // score exceeds m_ref + slack (then the value wave rescales its rows)
                float mx = -INFINITY;
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[tb][rb][i]);
                float* al = albuf + (k & 1) * AL_STRIDE;
                const bool raise = __any(first || mx > 0.0f);
                if (raise) {
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        float cm = -INFINITY;
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) cm = fmaxf(cm, S[tb][rb][i]);
                        cm = fmaxf(cm, __shfl_xor(cm, 16));
                        cm = fmaxf(cm, __shfl_xor(cm, 32));
                        float shift, alpha;
                        if (first) {
                            m_ref[rb] = cm;
                            shift = cm + kSlack;
                            alpha = 1.0f;
                        } else {
                            shift = fmaxf(cm, 0.0f);
                            m_ref[rb] += shift;
                            alpha = __builtin_amdgcn_exp2f(-shift);
                            l_run[rb] *= alpha;
                        }
                        if (j == 0) al[16 * rb + l16] = alpha;
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) S[tb][rb][i] -= shift;
                    }
                }
                if (lane == 0) al[ROWS] = (raise && !first) ? 1.0f : 0.0f;
                // probabilities (scaled by 2^-slack), row sums, P.V operand p * n
                const h8 nn = {n_lo[0], n_lo[1], n_lo[2], n_lo[3], n_hi[0], n_hi[1], n_hi[2], n_hi[3]};
                h8* pb = pbuf + (k & 1) * NRB * 64;
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    float p[8];
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) p[4 * tb + i] = __builtin_amdgcn_exp2f(S[tb][rb][i]);
                    l_run[rb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                    const h8 ph = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                                   (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
                    pb[rb * 64 + lane] = ph * nn;
                }
            }
            __syncthreads();  // probabilities of chunk k are visible to the value wave
        }
        __syncthreads();      // matches the value wave's extra (last) step
    } else {
        // ===================== value wave =====================
        const h4* lut = reinterpret_cast<const h4*>(lds + C::OFF_LUT);
        const uint32_t sh = 4u * (uint32_t)j;
        __syncthreads();  // step -1: nothing to consume yet
        for (int k = 0; k < nk_max; ++k) {
            if (k < nk) {
                if (k + NSTAGE - 1 < nk)
                    issue_values<D, NRB>(ts, pair + PAIRS * (k + NSTAGE - 1),
                                         bring + ((k + NSTAGE - 1) % NSTAGE) * C::B_STAGE, lane);
                wait_chunks_after<C::B_LOADS>(min(NSTAGE - 1, nk - 1 - k));
                const float* al = albuf + (k & 1) * AL_STRIDE;
                if (al[ROWS] != 0.0f) {
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float ai = al[16 * rb + 4 * j + i];
#pragma unroll
                            for (int db = 0; db < NDB; ++db) O[rb][db][i] *= ai;
                        }
                }
                const h8* pb = pbuf + (k & 1) * NRB * 64;
                h8 ap[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) ap[rb] = pb[rb * 64 + lane];
                const uint32_t* vw = reinterpret_cast<const uint32_t*>(bring + (k % NSTAGE) * C::B_STAGE);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int dim = 16 * db + l16;
                    const uint32_t w0 = vw[dim], w1 = vw[D + dim], w2 = vw[2 * D + dim];
                    const uint32_t ilo = __builtin_amdgcn_ubfe(w0, sh, 4) | (__builtin_amdgcn_ubfe(w1, sh, 4) << 4) |
                                         (__builtin_amdgcn_ubfe(w2, sh, 4) << 8);
                    const uint32_t ihi = __builtin_amdgcn_ubfe(w0, sh + 16u, 4) |
                                         (__builtin_amdgcn_ubfe(w1, sh + 16u, 4) << 4) |
                                         (__builtin_amdgcn_ubfe(w2, sh + 16u, 4) << 8);
                    const h4 vlo = lut[ilo], vhi = lut[ihi];
                    const h8 bv = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
                        O[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb], bv, O[rb][db], 0, 0, 0);
                }
            }
            __syncthreads();  // done with the probabilities of chunk k
        }
    }

    // ---- merge the pairs and finish the rows ----
    float* mw = reinterpret_cast<float*>(lds + C::OFF_PAIRS);  // [PAIRS][ROWS]
    float* lw = mw + PAIRS * ROWS;                              // [PAIRS][ROWS]
    float* ob = lw + PAIRS * ROWS;                              // [2][ROWS][D]
    if (score_wave) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            float l = l_run[rb];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            if (j == 0) {
                mw[pair * ROWS + 16 * rb + l16] = m_ref[rb];
                lw[pair * ROWS + 16 * rb + l16] = l;
            }
        }
    }
    __syncthreads();
    // the value wave of pair p weights its rows by 2^(m_p - M)
    float fo[NRB][4];
    if (!score_wave) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rb + 4 * j + i;
                float M = -INFINITY;
#pragma unroll
                for (int v = 0; v < PAIRS; ++v) M = fmaxf(M, mw[v * ROWS + row]);
                const float mine = mw[pair * ROWS + row];
                fo[rb][i] = mine == -INFINITY ? 0.0f : exp2f(mine - M);
            }
        if (pair < 2) {
            float* mybuf = ob + pair * ROWS * D;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mybuf[(16 * rb + 4 * j + i) * D + 16 * db + l16] = O[rb][db][i] * fo[rb][i];
        }
    }
    __syncthreads();
    if (!score_wave && pair >= 2) {
        float* mybuf = ob + (pair - 2) * ROWS * D;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
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
        for (int stp = 1; stp <= 2; stp <<= 1) {
            const bool upper = (qtr & stp) != 0;
#pragma unroll
            for (int e = 0; e < QD; ++e) {
                const float other = __shfl_xor(x[e], stp);
                x[e] = upper ? other - x[e] : x[e] + other;
            }
        }
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < PAIRS; ++v) M = fmaxf(M, mw[v * ROWS + row]);
        float L = 0.0f;
#pragma unroll
        for (int v = 0; v < PAIRS; ++v) {
            const float mv = mw[v * ROWS + row];
            if (mv != -INFINITY) L += lw[v * ROWS + row] * exp2f(mv - M);
        }
        if (row < R) {
            const float inv = 1.0f / ((float)D * L * a.cb.fp16_scale);
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
    using C = MCfg<D, NRB>;
    auto kern = k_attend_mfma<D, NRB>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    const uint32_t tiles = (uint32_t)a.layer_count * (uint32_t)a.g.n_kv_heads;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(512), C::LDS, s, a);
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
