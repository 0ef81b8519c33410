// Shared-pool decode attention on the gfx950 matrix cores.
//
// PolyKV abstract: N agents decode against one compressed pool. For a pool tile (layer,
// KV head) the query rows of every agent that reads that head (agents x GQA) form the
// M side of two contractions against the tile's tokens: scores S = scale * q . k_hat
// (keys: int8 q8_0 codes times their fp16 block scale) and P.V in the Hadamard-rotated
// domain, acc = sum_t p_t n_t c[code_t]; one inverse FWHT per output row at the end
// replaces the per-token inverse rotation. A launch serves up to 64 of a tile's rows (a
// range given by the launch arguments); more rows are served by further launches.
//
// Layout of the work (one workgroup per tile, four token streams, one per SIMD):
// - the tile's tokens are cut into 32-token chunks (one value bit-plane group each);
//   stream s takes chunks s, s+4, s+8, ...;
// - each stream has score waves and two value waves, all on the stream's SIMD. A score
//   wave owns a block of query rows: it computes S for its rows with
//   v_mfma_f32_16x16x32_f16 (16 tokens x one 32-wide q8 block as A, codes converted to
//   fp16 exactly; 16 query rows as B, the query split q = q_hi + q_lo in fp16 for ~22-bit
//   precision), applies the block scales with v_fma_mix, runs a lazy-max online softmax
//   in base 2 and writes p * n_t as fp16 to a double-buffered LDS slot. A value wave owns
//   half of the head dimensions: it decodes the value bit-planes of its dimensions to
//   fp16 centroids through a 4096-entry table (one nibble of each plane = 4 tokens) and
//   accumulates P.V for every row in fp32, one chunk behind the score waves. Four waves
//   of similar register size per SIMD hide each other's latencies;
// - small workgroups (d = 64, at most 16 rows) run one value wave per stream for all the
//   dimensions, read the 64-entry pair table the big table is built from (two tokens per
//   lookup) and use a three-deep key ring, so that three of them fit one CU;
// - the first score wave of a stream streams the keys, block scales and norms of its
//   chunks into a four-deep LDS ring by direct-to-LDS DMA (256-byte aligned
//   destinations); each value wave streams its share of the planes into a three-deep
//   ring. One workgroup barrier per chunk step publishes keys and probabilities;
// - a row's reference maximum is raised only when a score exceeds it by more than 8
//   (log2 units); the score wave then passes per-row rescale factors to the value waves;
// - start-up: the first chunks are requested, then the queries, and the queries are
//   converted only after the lookup tables are built, so that the latencies overlap;
//   score waves issue at a raised priority (their chain is the longer one);
// - at the end the streams' (m, l, acc) are merged through LDS in a bank-padded layout and
//   each row becomes H acc / (d l), the last two FWHT stages across a quad of lanes (DPP).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>


#include "lds_dma.h"
#include "polykv_internal.h"

namespace polykv {
namespace {

using lds_dma::dma16;
using lds_dma::dma4;
using lds_dma::lane_id;
using lds_dma::lds_addr;
using lds_dma::wait_vm;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int STREAMS = 4;
constexpr int CHUNK = 32;
constexpr int NSV = 3;  // plane ring depth (chunks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Reference maxima of the online softmax (log2 units): a row's reference puts the largest
// p * n of the chunk that places it at 2^kPlace, and is raised when some p * n could exceed
// 2^(kPlace + kSlack) or some p could exceed 2^kPmax.
constexpr float kPlace = 6.0f;
constexpr float kSlack = 8.0f;
constexpr float kPmax = 64.0f;

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

// D: head_dim; SRB: 16-row blocks per score wave; NSW: score waves per stream; LUT: value
// decode through the 4096-entry table (else through the 64-entry pair table, which keeps
// the LDS small enough for two workgroups per CU).
template <int D, int SRB, int NSW, bool LUT>
struct MCfg {
    // The small workgroups (the pair-table variant, at most 16 rows) run one value wave per
    // stream and a three-deep key ring, so that three of them share a CU (LDS and
    // registers): a pool of many small tiles then runs in one round.
    static constexpr int NVW = LUT ? 2 : 1;            // value waves per stream
    static constexpr int NSK = LUT ? 4 : 3;            // key ring depth (chunks)
    static constexpr int K_PRE = 2;                    // key chunks requested before the first step
    static constexpr int WG_PER_CU = LUT ? 1 : 3;
    static constexpr int NB = D / 32;                  // q8 blocks per row
    static constexpr int NRB = SRB * NSW;              // 16-row blocks per tile
    static constexpr int ROWS = 16 * NRB;
    static constexpr int WAVES = STREAMS * (NSW + NVW);
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int SLOTS = D / 16;               // 16-byte slots in a key row
    static constexpr int HD = D / NVW;                 // dimensions per value wave
    static constexpr int VDB = HD / 16;                // 16-column blocks per value wave
    // Every DMA destination below is 256-byte aligned.
    // key stage: key codes, rows XOR-swizzled by 16-byte slot
    static constexpr int K_BYTES = CHUNK * D;
    // meta stage: block scales at 0, value norms at 256
    static constexpr int S_BYTES = CHUNK * NB * 2;
    static constexpr int N_BYTES = CHUNK * 2;
    static constexpr int M_OFF_S = 0;
    static constexpr int M_OFF_N = 256;
    static constexpr int M_STAGE = 512;
    // plane stage: [value wave][plane][HD] words, each value wave's share 256-B aligned
    static constexpr int VH_BYTES = 3 * HD * 4;
    static constexpr int VH_SLOT = round_up(VH_BYTES, 256);
    static constexpr int V_LANES = VH_BYTES / 16;      // lanes of the one DMA instruction
    static constexpr int LPP = HD * 4 / 16;            // lanes per plane
    static constexpr int B_STAGE = NVW * VH_SLOT;
    // probabilities p * n (fp16 A operand of P.V, one h8 per lane and row block) and the
    // per-row rescale factors, then one flag per score wave
    static constexpr int P_BYTES = NRB * 64 * 16;
    static constexpr int AL_STRIDE = ROWS + 4;
    static constexpr int ST_OFF_K = 0;
    static constexpr int ST_OFF_M = ST_OFF_K + NSK * K_BYTES;
    static constexpr int ST_OFF_B = ST_OFF_M + NSK * M_STAGE;
    static constexpr int ST_OFF_P = ST_OFF_B + NSV * B_STAGE;
    static constexpr int ST_OFF_AL = ST_OFF_P + 2 * P_BYTES;
    static constexpr int STREAM_BYTES = round_up(ST_OFF_AL + 2 * AL_STRIDE * 4, 256);
    static constexpr int LUT_BYTES = LUT ? 4096 * 8 : 0;
    static constexpr int OFF_LUT = 0;
    static constexpr int OFF_MASK = LUT_BYTES;                 // fp16 [2][CHUNK] token weights
    static constexpr int OFF_PAIR = OFF_MASK + 256;            // fp16 [64][2] pair table
    static constexpr int OFF_STREAMS = OFF_PAIR + 256;
    static constexpr int LDS = OFF_STREAMS + STREAMS * STREAM_BYTES;
    // DMA instructions per chunk
    static constexpr int K_INSTR = K_BYTES / 1024;
    static constexpr int S_LANES = S_BYTES / 4;
    static constexpr int A_LOADS = K_INSTR + 2;
    // merge area (reuses the stream areas at the end)
    // merge area: m and l per stream and row, then two partial accumulators of ROWS rows;
    // a row takes MRS floats and each 32-dim quarter of it MQS, so that 16-byte accesses
    // of consecutive lanes (4 dims of rows 4 apart, or quarters of neighbouring rows)
    // fall into distinct LDS banks
    static constexpr int MQS = 36;
    static constexpr int MRS = round_up(NB * MQS, 32) + 16;
    static constexpr int MERGE_BYTES = (2 * STREAMS * ROWS + 2 * ROWS * MRS) * 4;
    static_assert(K_BYTES % 1024 == 0, "key stage is whole DMA instructions");
    static_assert(S_LANES <= 64 && V_LANES <= 64, "one DMA instruction each");
    static_assert(MERGE_BYTES <= STREAMS * STREAM_BYTES, "merge area fits");
    static_assert(!(LUT && NRB == STREAMS) || 2 * NRB * NB * 64 * 16 <= LUT_BYTES, "shared query halves fit the table area");
    static_assert(MQS % 4 == 0 && MRS % 4 == 0 && (2 * STREAMS * ROWS) % 4 == 0, "16-byte merge accesses");
    static_assert(WG_PER_CU * LDS <= 160 * 1024, "WG_PER_CU workgroups fit the LDS of one CU");
    static_assert(NSK <= 4 && NSV <= 4 && 3 * A_LOADS <= 63, "wait_chunks_after covers the rings");
    static_assert(S_BYTES <= 256 && N_BYTES <= 256 && K_BYTES % 256 == 0 && OFF_STREAMS % 256 == 0,
                  "256-byte aligned DMA destinations");
    static_assert(ROWS % 4 == 0 && D % 64 == 0, "whole rows per wave and whole float4 of dims per finishing thread");
    static_assert(SLOTS <= 16 && 1024 % D == 0, "the key swizzle repeats every 1 KB");
};

// wait until at most n (0..3) later chunks of LOADS instructions each are still in flight
template <int LOADS>
__device__ __forceinline__ void wait_chunks_after(int n) {
    if (n >= 3) wait_vm<3 * LOADS>();
    else if (n == 2) wait_vm<2 * LOADS>();
    else if (n == 1) wait_vm<LOADS>();
    else wait_vm<0>();
}


// 8 int8 codes -> 8 fp16 (exact): sign-extending byte selects, two results per dword.
// One asm block, because the compiler's hazard tracking does not look inside inline asm:
// - a half-dword (dst_sel) write must not be read by the very next VALU instruction, so
//   the four low-half writes come first and each high-half write (which reads the
//   preserved low half) is four instructions behind its low-half write;
// - a VALU result read by a matrix-core instruction needs two wait states, given by the
//   closing s_nop 1 (the results feed v_mfma directly).
__device__ __forceinline__ h8 codes_to_h8(uint2 raw) {
    uint32_t d0, d1, d2, d3;
    asm("v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
        "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
        "s_nop 1"
        : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
        : "v"(raw.x), "v"(raw.y));
    const uint4 u = make_uint4(d0, d1, d2, d3);
    return __builtin_bit_cast(h8, u);
}

// maximum and sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (cross-lane swaps, no LDS)
__device__ __forceinline__ float max_over_j(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ uint32_t max_over_j_u32(uint32_t u) {
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t v = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(b[0], b[1]);
}
__device__ __forceinline__ float sum_over_j(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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

// Keys, block scales and norms of chunk c into one key stage. Key rows keep their
// 16-byte slots XOR-swizzled by the row index, so the 16 rows one fragment read touches
// fall into distinct LDS banks; one DMA instruction moves 1 KB, and the swizzle repeats
// every 1 KB, so instruction i reads koff + 1 KB * i. In the tile's last, partial chunk,
// rows past the end of the tile are clamped to the last token (valid memory; those
// tokens get weight 0 in the softmax).

// The lane offsets are derived from the lane id where they are used, so that nothing
// stays live across the score loop for them.
template <class C, bool FULL>
__device__ __forceinline__ void issue_keys(const TileSrc& ts, int c, uint8_t* stage, uint8_t* meta) {
    constexpr int D = C::SLOTS * 16;
    constexpr int per_tok = C::NB * 2;
    constexpr int ROWS_PER_INSTR = 1024 / D;
    const uint32_t lane = lane_id();
    const uint32_t krow = 16u * lane / D;
    const uint32_t koff = krow * D + (((16u * lane) % D) / 16 ^ (krow & (C::SLOTS - 1))) * 16;
    const uint32_t soff = 4u * lane, noff = 4u * lane;
    const int t0 = c * CHUNK;
    const int8_t* kb = ts.kcodes + (size_t)t0 * D;
    const uint8_t* sb = ts.kscales + (size_t)t0 * per_tok;
    const uint8_t* nb = ts.vnorms + (size_t)t0 * 2;
    if constexpr (FULL) {
#pragma unroll
        for (int i = 0; i < C::K_INSTR; ++i) dma16(kb + 1024 * i, koff, lds_addr(stage + i * 1024));
        if (lane < (uint32_t)C::S_LANES) dma4(sb, soff, lds_addr(meta + C::M_OFF_S));
        if (lane < 16u) dma4(nb, noff, lds_addr(meta + C::M_OFF_N));
    } else {
        // from the chunk base: the clamped row plus the lane's swizzled slot (which is the
        // same in every instruction); never a negative offset
        const uint32_t last = (uint32_t)(ts.T - 1 - t0);
        const uint32_t slot16 = koff - krow * D;
#pragma unroll
        for (int i = 0; i < C::K_INSTR; ++i) {
            const uint32_t row = krow + ROWS_PER_INSTR * i;
            dma16(kb, min(row, last) * D + slot16, lds_addr(stage + i * 1024));
        }
        if (lane < (uint32_t)C::S_LANES) {
            const uint32_t row = soff / per_tok;
            dma4(sb, soff - (row - min(row, last)) * per_tok, lds_addr(meta + C::M_OFF_S));
        }
        if (lane < 16u) {
            const uint32_t row = noff / 2;
            dma4(nb, row > last ? 2 * (last & ~1u) : noff, lds_addr(meta + C::M_OFF_N));
        }
    }
}
template <class C>
__device__ __forceinline__ void issue_keys_any(const TileSrc& ts, int c, uint8_t* stage, uint8_t* meta) {
    if ((c + 1) * CHUNK <= ts.T) issue_keys<C, true>(ts, c, stage, meta);
    else issue_keys<C, false>(ts, c, stage, meta);
}

// Value wave `half`: its half of the three bit-planes of chunk c (always inside the tile),
// as [plane][HD] words at the start of its half of the plane stage.
template <class C>
__device__ __forceinline__ void issue_planes(const TileSrc& ts, int c, int half, uint8_t* stage) {
    constexpr int D = C::SLOTS * 16;
    const int lane = (int)lane_id();
    if (lane < C::V_LANES) {
        const int p = lane / C::LPP, seg = lane - p * C::LPP;
        const uint8_t* vg = ts.vplanes + (size_t)c * (3 * D * 4);
        dma16(vg, (uint32_t)(p * D * 4 + half * C::HD * 4 + 16 * seg), lds_addr(stage + half * C::VH_SLOT));
    }
}

template <int D, int SRB, int NSW, bool LUT>
__global__ __launch_bounds__((MCfg<D, SRB, NSW, LUT>::THREADS))
__attribute__((amdgpu_waves_per_eu(MCfg<D, SRB, NSW, LUT>::WG_PER_CU * MCfg<D, SRB, NSW, LUT>::WAVES / STREAMS)))
void k_attend_mfma(AttendArgs a) {
    using C = MCfg<D, SRB, NSW, LUT>;
    constexpr int NB = C::NB, NRB = C::NRB, ROWS = C::ROWS, VDB = C::VDB, HD = C::HD;
    constexpr int AL_STRIDE = C::AL_STRIDE;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int tid = threadIdx.x;
    // from mbcnt (not from the thread index) so that the lane-derived values below can
    // be recomputed where they are used instead of being held across the chunk loop
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int stream = w % STREAMS;
    const int role = w / STREAMS;                            // < NSW: score wave
    const bool score_wave = role < NSW;
    const int l16 = lane & 15;
    const int j = lane >> 4;

    const PoolGeom& g = a.g;
    const int H = g.n_kv_heads, T = g.n_tokens, G = a.gqa, A = a.n_agents;
    const int R = a.n_rows;  // rows of this launch; row r is row a.row_begin + r of the tile
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
    const int nk = stream < NC ? (NC - stream + STREAMS - 1) / STREAMS : 0;  // this stream
    const int nk_max = (NC + STREAMS - 1) / STREAMS;                         // every stream
    uint8_t* sbase = lds + C::OFF_STREAMS + stream * C::STREAM_BYTES;
    uint8_t* kring = sbase + C::ST_OFF_K;
    uint8_t* mring = sbase + C::ST_OFF_M;
    uint8_t* bring = sbase + C::ST_OFF_B;
    h8* pbuf = reinterpret_cast<h8*>(sbase + C::ST_OFF_P);          // [2][NRB][64]
    float* albuf = reinterpret_cast<float*>(sbase + C::ST_OFF_AL);  // [2][AL_STRIDE]
    const size_t HG = (size_t)H * G;

    const bool key_wave = score_wave && role == 0;
    // ---- score waves: queries (B operand). Lane holds row 16 rb + l16 of its row
    // blocks, dims 32b + 8j .. +7, times scale * log2(e), as fp16 hi + lo. With the big
    // table (LUT) the query loads are shared: the first score wave of stream s loads row
    // block s, splits it and writes both halves into the table's area, from which every
    // score wave reads its own row blocks before the table is built (a tile's queries are
    // loaded once instead of once per stream).
    constexpr bool QSHARE = LUT && NRB == STREAMS;
    constexpr int QRB = QSHARE ? 1 : SRB;     // row blocks loaded by this wave
    h8 qh[SRB][NB], ql[SRB][NB];
    float m_ref[SRB], l_run[SRB];
    float4 qraw[QRB][NB][2];
    const bool q_loader = score_wave && (!QSHARE || role == 0);
    if (score_wave) {
#pragma unroll
        for (int rb = 0; rb < SRB; ++rb) {
            m_ref[rb] = -INFINITY;
            l_run[rb] = 0.0f;
        }
    }
    if (q_loader) {
#pragma unroll
        for (int qb = 0; qb < QRB; ++qb) {
            const int r = 16 * (QSHARE ? stream : SRB * role + qb) + l16;
            if (r < R) {
                const int gr = a.row_begin + r, ag = gr / G, jj = gr - ag * G;
                const float* qrow = a.q + (((size_t)l_local * A + ag) * HG + (size_t)h * G + jj) * D;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    qraw[qb][b][0] = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * j);
                    qraw[qb][b][1] = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * j + 4);
                }
            } else {
#pragma unroll
                for (int b = 0; b < NB; ++b) qraw[qb][b][0] = qraw[qb][b][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }

    // The start-up latencies overlap: the query loads go out first (nothing can be scored
    // before they land), then the first chunks: K_PRE key chunks and NSV - 1 plane chunks
    // (the key ring's remaining chunks follow in the first chunk step, which keeps the
    // burst of requests at launch small); the lookup tables are built meanwhile, and the
    // queries are converted afterwards.
    if (key_wave) {
        for (int s = 0; s < C::K_PRE; ++s)
            if (s < nk) issue_keys_any<C>(ts, stream + STREAMS * s, kring + s * C::K_BYTES, mring + s * C::M_STAGE);
    } else if (!score_wave) {
        for (int s = 0; s < NSV - 1; ++s)
            if (s < nk) issue_planes<C>(ts, stream + STREAMS * s, role - NSW, bring + s * C::B_STAGE);
    }

    // value lookup table, built in two steps. Pair table: entry x (6 bits: plane 0, 1 and 2
    // bits of token A at bits 0, 2, 4 and of token B at bits 1, 3, 5) -> lambda * the
    // centroids of A and B in fp16. Main table: entry e -> the centroids of the 4 tokens whose
    // plane bits are the nibbles (e & 15, (e >> 4) & 15, e >> 8), i.e. two pair entries.
    if (tid < 64) {
        const float lam = a.cb.fp16_scale;
        const uint32_t ca = (tid & 1) | (((tid >> 2) & 1) << 1) | (((tid >> 4) & 1) << 2);
        const uint32_t cbb = ((tid >> 1) & 1) | (((tid >> 3) & 1) << 1) | (((tid >> 5) & 1) << 2);
        reinterpret_cast<h2*>(lds + C::OFF_PAIR)[tid] =
            h2{(_Float16)(lam * centroid_full(ca, a.cb)), (_Float16)(lam * centroid_full(cbb, a.cb))};
    }
    // token weights of a full chunk (all 1) and of the tile's last chunk (1 below T)
    if (tid < 2 * CHUNK) {
        const int t = tid & (CHUNK - 1);
        const bool tail = tid >= CHUNK;
        reinterpret_cast<_Float16*>(lds + C::OFF_MASK)[tid] =
            (!tail || (NC - 1) * CHUNK + t < T) ? (_Float16)1.0f : (_Float16)0.0f;
    }
    // split the loaded queries into fp16 hi + lo
    h8* qsh = reinterpret_cast<h8*>(lds + C::OFF_LUT);  // shared halves: [hi, lo][rb][b][lane]
    if (q_loader) {
        const float qs = a.softmax_scale * kLog2e;
#pragma unroll
        for (int qb = 0; qb < QRB; ++qb)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float4 u0 = qraw[qb][b][0], u1 = qraw[qb][b][1];
                const float x[8] = {u0.x * qs, u0.y * qs, u0.z * qs, u0.w * qs,
                                    u1.x * qs, u1.y * qs, u1.z * qs, u1.w * qs};
                h8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) hi[e] = (_Float16)x[e];
                // lo must be formed from the hi that is stored. Left to itself the compiler
                // recomputes hi for this subtraction from the unrounded product q * qs (a
                // mixed-precision fma), which rounds differently from the stored hi whenever
                // the fp32 x falls on an fp16 tie; hi + lo then misses x by one fp16 ulp.
                // The empty asm makes the stored hi opaque, so it is the one used.
                uint4 hu = __builtin_bit_cast(uint4, hi);
                asm volatile("" : "+v"(hu.x), "+v"(hu.y), "+v"(hu.z), "+v"(hu.w));
                hi = __builtin_bit_cast(h8, hu);
#pragma unroll
                for (int e = 0; e < 8; ++e) lo[e] = (_Float16)(x[e] - (float)hi[e]);
                if constexpr (QSHARE) {
                    qsh[(stream * NB + b) * 64 + lane] = hi;
                    qsh[((NRB + stream) * NB + b) * 64 + lane] = lo;
                } else {
                    qh[qb][b] = hi;
                    ql[qb][b] = lo;
                }
            }
    }
    __syncthreads();  // pair table (and shared query halves) complete
    if constexpr (QSHARE) {
        if (score_wave) {
#pragma unroll
            for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    qh[rb][b] = qsh[((SRB * role + rb) * NB + b) * 64 + lane];
                    ql[rb][b] = qsh[((NRB + SRB * role + rb) * NB + b) * 64 + lane];
                }
        }
        __syncthreads();  // query halves read before the table overwrites them
    }
    if constexpr (LUT) {
        const uint32_t* pair = reinterpret_cast<const uint32_t*>(lds + C::OFF_PAIR);
        uint2* lut = reinterpret_cast<uint2*>(lds + C::OFF_LUT);
        for (int e = tid; e < 4096; e += C::THREADS) {
            const uint32_t i01 = (e & 3) | ((e >> 2) & 0xC) | ((e >> 4) & 0x30);
            const uint32_t i23 = ((e >> 2) & 3) | ((e >> 4) & 0xC) | ((e >> 6) & 0x30);
            lut[e] = make_uint2(pair[i01], pair[i23]);
        }
    }
    // the first key chunk must have landed before the barrier publishes it
    if (key_wave) wait_chunks_after<C::A_LOADS>(min(C::K_PRE - 1, nk - 1));
    __syncthreads();

    f4 O[NRB][VDB];  // value waves: rows 16 rb + 4j + i, dims HD * half + VDB * l16 + db
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < VDB; ++db) O[rb][db] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    if (score_wave) {
        // ===================== score waves =====================
        // the score waves carry the longer dependency chain of a chunk step: their
        // instructions go first when both kinds of wave are ready to issue
        __builtin_amdgcn_s_setprio(1);
        // LDS offsets (within a stage) of the key fragments: token l16, dims 32b + 8j .. +7,
        // through the row swizzle
        // (token block tb adds 16 * D: the swizzle depends only on the low row bits)
        uint32_t kfrag[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int seg = 2 * b + (j >> 1);
            const int slot = seg ^ (l16 & (C::SLOTS - 1));
            kfrag[b] = (uint32_t)(l16 * D + slot * 16 + 8 * (j & 1));
        }

        for (int k = 0; k <= nk_max; ++k) {
            if (k < nk) {
                const int c = stream + STREAMS * k;
                const int t0 = c * CHUNK;
                if (key_wave) {
                    // the rest of the ring's initial chunks, then one chunk per step, NSK - 1 ahead
                    if (k == 0)
                        for (int s2 = C::K_PRE; s2 < C::NSK - 1; ++s2)
                            if (s2 < nk) issue_keys_any<C>(ts, stream + STREAMS * s2, kring + s2 * C::K_BYTES, mring + s2 * C::M_STAGE);
                    if (k + C::NSK - 1 < nk)
                        issue_keys_any<C>(ts, c + STREAMS * (C::NSK - 1), kring + ((k + C::NSK - 1) % C::NSK) * C::K_BYTES,
                                          mring + ((k + C::NSK - 1) % C::NSK) * C::M_STAGE);
                }
                // stage offset in LDS: wave-uniform, so every lane address below is one
                // scalar + vector add
                const uint32_t st_off = (uint32_t)__builtin_amdgcn_readfirstlane(
                    (int)(C::OFF_STREAMS + stream * C::STREAM_BYTES + C::ST_OFF_K + (k % C::NSK) * C::K_BYTES));
                const uint32_t mt_off = (uint32_t)__builtin_amdgcn_readfirstlane(
                    (int)(C::OFF_STREAMS + stream * C::STREAM_BYTES + C::ST_OFF_M + (k % C::NSK) * C::M_STAGE));
                const uint8_t* st = lds + st_off;
                const uint8_t* mt = lds + mt_off;
                const h4 n_lo = *reinterpret_cast<const h4*>(mt + C::M_OFF_N + 8 * j);
                const h4 n_hi = *reinterpret_cast<const h4*>(mt + C::M_OFF_N + 32 + 8 * j);
                // token weights: 1, or 0 for the tokens past T in the tile's last chunk
                const uint8_t* wm = lds + (uint32_t)__builtin_amdgcn_readfirstlane(C::OFF_MASK + (t0 + CHUNK > T ? 64 : 0));
                const h4 m_lo = *reinterpret_cast<const h4*>(wm + 8 * j);
                const h4 m_hi = *reinterpret_cast<const h4*>(wm + 32 + 8 * j);
                const bool first = k == 0;
                f4 S[2][SRB];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    h8 scv[(NB + 1) / 2];
                    const h8* sp = reinterpret_cast<const h8*>(mt + C::M_OFF_S + (16 * tb + 4 * j) * NB * 2);
#pragma unroll
                    for (int v = 0; v < (NB + 1) / 2; ++v) scv[v] = sp[v];
#pragma unroll
                    for (int rb = 0; rb < SRB; ++rb) {
                        const float init = first ? 0.0f : -m_ref[rb];
                        S[tb][rb] = f4{init, init, init, init};
                    }
                    // two-stage pipeline over the q8 blocks: block b+1's conversion and its
                    // hi products are issued before block b's scale FMAs read its results
                    const uint8_t* kt = st + 16 * D * tb;
                    h8 ak = codes_to_h8(*reinterpret_cast<const uint2*>(kt + kfrag[0]));
                    f4 acc[SRB];
#pragma unroll
                    for (int rb = 0; rb < SRB; ++rb)
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qh[rb][0], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                    for (int rb = 0; rb < SRB; ++rb)
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, ql[rb][0], acc[rb], 0, 0, 0);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        f4 accn[SRB];
                        h8 akn;
                        if (b + 1 < NB) {
                            akn = codes_to_h8(*reinterpret_cast<const uint2*>(kt + kfrag[b + 1]));
#pragma unroll
                            for (int rb = 0; rb < SRB; ++rb)
                                accn[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(akn, qh[rb][b + 1], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                        }
#pragma unroll
                        for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int si = i * NB + b;
                                S[tb][rb][i] = __builtin_fmaf(acc[rb][i], (float)scv[si >> 3][si & 7], S[tb][rb][i]);
                            }
                        if (b + 1 < NB) {
#pragma unroll
                            for (int rb = 0; rb < SRB; ++rb)
                                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(akn, ql[rb][b + 1], accn[rb], 0, 0, 0);
                            ak = akn;
                        }
                    }
                }
                // Probabilities p = 2^(score - m) with one reference m per row; the P.V operand
                // is p * n rounded once to fp16 (n the token's value norm), the row sums take
                // p in fp32. m is placed so that the row's largest p * n in the chunk that
                // places it is 2^kPlace, and raised only when some p * n could exceed
                // 2^(kPlace + kSlack) or some p could exceed 2^kPmax: the operand then holds
                // every weight within 2^-(14 + kPlace) of the row's largest as a normal fp16
                // number and never overflows, and p stays finite (zero norms included). The
                // per-chunk check is conservative: the largest score - m of the wave's rows
                // against kPlace + kSlack - log2 of the chunk's largest norm. The tile's last
                // chunk always takes the exact path (its norm slots past T may hold any bits;
                // its rows past T repeat the last token, so they never raise m).
                float mx = -INFINITY;
#pragma unroll
                for (int rb = 0; rb < SRB; ++rb)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[tb][rb][i]);
                // the chunk's largest norm: non-negative fp16 bit patterns order as integers
                const u16x4 nmv = __builtin_elementwise_max(__builtin_bit_cast(u16x4, n_lo), __builtin_bit_cast(u16x4, n_hi));
                const uint32_t nmb = max_over_j_u32(max(max((uint32_t)nmv[0], (uint32_t)nmv[1]),
                                                        max((uint32_t)nmv[2], (uint32_t)nmv[3])));
                const float thr = fminf(kPlace + kSlack - __builtin_log2f((float)__builtin_bit_cast(_Float16, (uint16_t)nmb)), kPmax);
                float* al = albuf + (k & 1) * AL_STRIDE;
                const bool raise = __any(first || t0 + CHUNK > T || mx > thr);
                if (raise) {
                    asm volatile("" ::: "memory");  // rare: keep it out of the common path
                    // norms and weights of the lane's tokens (slots past T may hold any bits)
                    const h8 nr = {n_lo[0], n_lo[1], n_lo[2], n_lo[3], n_hi[0], n_hi[1], n_hi[2], n_hi[3]};
                    const h8 wt = {m_lo[0], m_lo[1], m_lo[2], m_lo[3], m_hi[0], m_hi[1], m_hi[2], m_hi[3]};
#pragma unroll
                    for (int rb = 0; rb < SRB; ++rb) {
                        // the row's largest log2(p * n) and largest score - m in this chunk
                        float cw = -INFINITY, cs = -INFINITY;
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                cs = fmaxf(cs, S[tb][rb][i]);
                                cw = fmaxf(cw, wt[4 * tb + i] != (_Float16)0.0f ? S[tb][rb][i] + __builtin_log2f((float)nr[4 * tb + i]) : -INFINITY);
                            }
                        cw = max_over_j(cw);
                        cs = max_over_j(cs);
                        // zero norms give -inf in cw; the second term keeps p <= 2^kPmax
                        const float want = fmaxf(cw - kPlace, cs - kPmax);
                        float shift, alpha;
                        if (first) {
                            shift = want;
                            m_ref[rb] = shift;
                            alpha = 1.0f;
                        } else {
                            shift = (cw > kPlace + kSlack || cs > kPmax) ? want : 0.0f;
                            m_ref[rb] += shift;
                            alpha = __builtin_amdgcn_exp2f(-shift);
                            l_run[rb] *= alpha;
                        }
                        if (j == 0) al[16 * (SRB * role + rb) + l16] = alpha;
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) S[tb][rb][i] -= shift;
                    }
                }
                if (lane == 0) al[ROWS + role] = (raise && !first) ? 1.0f : 0.0f;
                // p into the row sums (weight 0 past T), p * n into the P.V operand
                const h8 wt = {m_lo[0], m_lo[1], m_lo[2], m_lo[3], m_hi[0], m_hi[1], m_hi[2], m_hi[3]};
                h8 nv = h8{n_lo[0], n_lo[1], n_lo[2], n_lo[3], n_hi[0], n_hi[1], n_hi[2], n_hi[3]};
                if (t0 + CHUNK > T) {
                    // the tile's last chunk: norm slots past T may hold any bits (padding, or
                    // tokens not written yet), so they are replaced by 0, not multiplied by it
#pragma unroll
                    for (int e = 0; e < 8; ++e) nv[e] = wt[e] != (_Float16)0.0f ? nv[e] : (_Float16)0.0f;
                }
                h8* pb = pbuf + (k & 1) * NRB * 64;
#pragma unroll
                for (int rb = 0; rb < SRB; ++rb) {
                    h8 ph;
                    float l = l_run[rb];
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float p = __builtin_amdgcn_exp2f(S[tb][rb][i]);
                            l = __builtin_fmaf(p, (float)wt[4 * tb + i], l);
                            ph[4 * tb + i] = (_Float16)(p * (float)nv[4 * tb + i]);
                        }
                    l_run[rb] = l;
                    pb[(SRB * role + rb) * 64 + lane] = ph;
                }
                // the next key chunk must have landed before the barrier publishes it
                if (key_wave) wait_chunks_after<C::A_LOADS>(max(0, min(C::NSK - 2, nk - 2 - k)));
            }
            __syncthreads();
        }
    } else {
        // ===================== value waves =====================
        const int half = role - NSW;
        const h4* lut = reinterpret_cast<const h4*>(lds + C::OFF_LUT);
        const h2* pairs = reinterpret_cast<const h2*>(lds + C::OFF_PAIR);
        const uint32_t sh = 4u * (uint32_t)j;
        for (int k = 0; k <= nk_max; ++k) {
            const int kk = k - 1;  // one chunk behind the score waves
            if (kk >= 0 && kk < nk) {
                if (kk + NSV - 1 < nk)
                    issue_planes<C>(ts, stream + STREAMS * (kk + NSV - 1), half,
                                    bring + ((kk + NSV - 1) % NSV) * C::B_STAGE);
                wait_chunks_after<1>(min(NSV - 1, nk - 1 - kk));
                const float* al = albuf + (kk & 1) * AL_STRIDE;
#pragma unroll
                for (int r = 0; r < NSW; ++r) {
                    if (al[ROWS + r] != 0.0f) {
#pragma unroll
                        for (int rb = SRB * r; rb < SRB * (r + 1); ++rb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float ai = al[16 * rb + 4 * j + i];
#pragma unroll
                                for (int db = 0; db < VDB; ++db) O[rb][db][i] *= ai;
                            }
                    }
                }
                const h8* pb = pbuf + (kk & 1) * NRB * 64;
                h8 ap[NRB];
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) ap[rb] = pb[rb * 64 + lane];
                // plane words of this lane's VDB consecutive dimensions
                const uint32_t vs_off = (uint32_t)__builtin_amdgcn_readfirstlane(
                    (int)(C::OFF_STREAMS + stream * C::STREAM_BYTES + C::ST_OFF_B + (kk % NSV) * C::B_STAGE + half * C::VH_SLOT));
                const uint8_t* vs = lds + vs_off + 4 * VDB * l16;
                uint32_t wv[3][VDB];
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    if constexpr (VDB == 4) {
                        const uint4 u = *reinterpret_cast<const uint4*>(vs + p * HD * 4);
                        wv[p][0] = u.x; wv[p][1] = u.y; wv[p][2] = u.z; wv[p][3] = u.w;
                    } else {
                        const uint2 u = *reinterpret_cast<const uint2*>(vs + p * HD * 4);
                        wv[p][0] = u.x; wv[p][1] = u.y;
                    }
                }
#pragma unroll
                for (int db = 0; db < VDB; ++db) {
                    const uint32_t w0 = wv[0][db], w1 = wv[1][db], w2 = wv[2][db];
                    h8 bv;
                    if constexpr (LUT) {
                        // tokens 4j .. 4j + 3 and 16 + 4j .. + 3: one table entry each
                        const uint32_t ilo = __builtin_amdgcn_ubfe(w0, sh, 4) | (__builtin_amdgcn_ubfe(w1, sh, 4) << 4) |
                                             (__builtin_amdgcn_ubfe(w2, sh, 4) << 8);
                        const uint32_t ihi = __builtin_amdgcn_ubfe(w0, sh + 16u, 4) |
                                             (__builtin_amdgcn_ubfe(w1, sh + 16u, 4) << 4) |
                                             (__builtin_amdgcn_ubfe(w2, sh + 16u, 4) << 8);
                        const h4 vlo = lut[ilo], vhi = lut[ihi];
                        bv = h8{vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
                    } else {
                        // the same tokens two at a time through the pair table
                        auto pidx = [&](uint32_t b) {
                            return __builtin_amdgcn_ubfe(w0, b, 2) | (__builtin_amdgcn_ubfe(w1, b, 2) << 2) |
                                   (__builtin_amdgcn_ubfe(w2, b, 2) << 4);
                        };
                        const h2 p0 = pairs[pidx(sh)], p1 = pairs[pidx(sh + 2u)];
                        const h2 p2 = pairs[pidx(sh + 16u)], p3 = pairs[pidx(sh + 18u)];
                        bv = h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                    }
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
                        O[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[rb], bv, O[rb][db], 0, 0, 0);
                }
            }
            __syncthreads();
        }
    }

    // ---- merge the streams and finish the rows ----
    constexpr int MQS = C::MQS, MRS = C::MRS;
    float* mw = reinterpret_cast<float*>(lds + C::OFF_STREAMS);  // [STREAMS][ROWS]
    float* lw = mw + STREAMS * ROWS;                              // [STREAMS][ROWS]
    float* ob = lw + STREAMS * ROWS;                              // [2][ROWS][MRS]
    if (score_wave) {
#pragma unroll
        for (int rb = 0; rb < SRB; ++rb) {
            const float l = sum_over_j(l_run[rb]);
            if (j == 0) {
                const int row = 16 * (SRB * role + rb) + l16;
                mw[stream * ROWS + row] = m_ref[rb];
                lw[stream * ROWS + row] = l;
            }
        }
    }
    __syncthreads();
    // the value waves of stream s weight their rows by 2^(m_s - M); a lane's VDB
    // consecutive dims lie inside one 32-dim quarter
    float fo[NRB][4];
    const int dq = HD * (role - NSW) + VDB * l16;
    const int qoff = (dq >> 5) * MQS + (dq & 31);
    if (!score_wave) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rb + 4 * j + i;
                float M = -INFINITY;
#pragma unroll
                for (int v = 0; v < STREAMS; ++v) M = fmaxf(M, mw[v * ROWS + row]);
                const float mine = mw[stream * ROWS + row];
                fo[rb][i] = mine == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mine - M);
            }
        if (stream < 2) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* pp = ob + (stream * ROWS + 16 * rb + 4 * j + i) * MRS + qoff;
                    if constexpr (VDB == 4)
                        *reinterpret_cast<float4*>(pp) = make_float4(O[rb][0][i] * fo[rb][i], O[rb][1][i] * fo[rb][i],
                                                                     O[rb][2][i] * fo[rb][i], O[rb][3][i] * fo[rb][i]);
                    else
                        *reinterpret_cast<float2*>(pp) = make_float2(O[rb][0][i] * fo[rb][i], O[rb][1][i] * fo[rb][i]);
                }
        }
    }
    __syncthreads();
    if (!score_wave && stream >= 2) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float* pp = ob + ((stream - 2) * ROWS + 16 * rb + 4 * j + i) * MRS + qoff;
                if constexpr (VDB == 4) {
                    float4 u = *reinterpret_cast<const float4*>(pp);
                    u.x += O[rb][0][i] * fo[rb][i];
                    u.y += O[rb][1][i] * fo[rb][i];
                    u.z += O[rb][2][i] * fo[rb][i];
                    u.w += O[rb][3][i] * fo[rb][i];
                    *reinterpret_cast<float4*>(pp) = u;
                } else {
                    float2 u = *reinterpret_cast<const float2*>(pp);
                    u.x += O[rb][0][i] * fo[rb][i];
                    u.y += O[rb][1][i] * fo[rb][i];
                    *reinterpret_cast<float2*>(pp) = u;
                }
            }
    }
    __syncthreads();

    // Sixteen threads per row, every wave of the workgroup: lane q + 4 a + 16 b of wave w
    // (q, a, b in 0..3) holds dims FD * (q + 4 b) .. + FD - 1 of row 4 w + a (and of the rows
    // 4 * WAVES further on, while any are left). The FWHT stages
    // below FD run in registers; the four above, partners lane ^ 1 and ^ 2 (a quad
    // permutation, DPP) and lane ^ 16 and ^ 32 (row swaps), across lanes. (The indices are
    // rebuilt from the lane id here rather than kept live, and spilled, across the loop.)
    constexpr int FD = D / 16;
    const int fq = lane & 3, fa = (lane >> 2) & 3, fb = lane >> 4;
    const int ft = fq + 4 * fb;
    for (int row0 = 4 * w; row0 < ROWS; row0 += 4 * C::WAVES) {
        const int row = row0 + fa;
        float x[FD];
        const int d0 = FD * ft;
        const float* p0 = ob + min(row, ROWS - 1) * MRS + (d0 >> 5) * MQS + (d0 & 31);
        const float* p1 = p0 + ROWS * MRS;
#pragma unroll
        for (int e = 0; e < FD; e += 4) {
            const float4 u = *reinterpret_cast<const float4*>(p0 + e);
            const float4 v = *reinterpret_cast<const float4*>(p1 + e);
            x[e] = u.x + v.x;
            x[e + 1] = u.y + v.y;
            x[e + 2] = u.z + v.z;
            x[e + 3] = u.w + v.w;
        }
#pragma unroll
        for (int hh = 1; hh < FD; hh <<= 1)
#pragma unroll
            for (int e = 0; e < FD; ++e)
                if (!(e & hh)) {
                    const float u = x[e], v = x[e + hh];
                    x[e] = u + v;
                    x[e + hh] = u - v;
                }
        // the lower lane of a pair keeps own + other, the upper one other - own
#pragma unroll
        for (int stp = 1; stp <= 2; stp <<= 1) {
            const float sg = (fq & stp) ? -1.0f : 1.0f;
#pragma unroll
            for (int e = 0; e < FD; ++e) {
                const int xi = __float_as_int(x[e]);
                const int oi = stp == 1 ? __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false)   // lanes 1,0,3,2
                                        : __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false);  // lanes 2,3,0,1
                x[e] = __builtin_fmaf(sg, x[e], __int_as_float(oi));
            }
        }
        // row swaps: the first result is the lower lane's value, the second the upper's
#pragma unroll
        for (int e = 0; e < FD; ++e) {
            const uint32_t xu = __float_as_uint(x[e]);
            const auto r = __builtin_amdgcn_permlane16_swap(xu, xu, false, false);
            x[e] = __builtin_fmaf((fb & 1) ? -1.0f : 1.0f, __uint_as_float(r[1]), __uint_as_float(r[0]));
        }
#pragma unroll
        for (int e = 0; e < FD; ++e) {
            const uint32_t xu = __float_as_uint(x[e]);
            const auto r = __builtin_amdgcn_permlane32_swap(xu, xu, false, false);
            x[e] = __builtin_fmaf((fb & 2) ? -1.0f : 1.0f, __uint_as_float(r[1]), __uint_as_float(r[0]));
        }
        if (row < R) {
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < STREAMS; ++v) M = fmaxf(M, mw[v * ROWS + row]);
            float L = 0.0f;
#pragma unroll
            for (int v = 0; v < STREAMS; ++v) {
                const float mv = mw[v * ROWS + row];
                if (mv != -INFINITY) L += lw[v * ROWS + row] * __builtin_amdgcn_exp2f(mv - M);
            }
            const float inv = 1.0f / ((float)D * L * a.cb.fp16_scale);
            const int gr = a.row_begin + row, ag = gr / G, jj = gr - ag * G;
            // scores are in log2 units and every p carries 2^-m
            if (a.lse && ft == 0)
                a.lse[((size_t)l_local * A + ag) * HG + (size_t)h * G + jj] =
                    kLn2 * (M + __builtin_log2f(L));
            float* o = a.out + (((size_t)l_local * A + ag) * HG + (size_t)h * G + jj) * D + d0;
#pragma unroll
            for (int e = 0; e < FD; e += 4)
                *reinterpret_cast<float4*>(o + e) = make_float4(x[e] * inv, x[e + 1] * inv, x[e + 2] * inv, x[e + 3] * inv);
        }
    }
}

template <int D, int SRB, int NSW, bool LUT = true>
hipError_t launch_t(const AttendArgs& a, hipStream_t s) {
    using C = MCfg<D, SRB, NSW, LUT>;
    auto kern = k_attend_mfma<D, SRB, NSW, LUT>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once((const void*)kern, C::LDS, lds_set);
    if (e != hipSuccess) return e;
    const uint32_t tiles = (uint32_t)a.layer_count * (uint32_t)a.g.n_kv_heads;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(C::THREADS), C::LDS, s, a);
    return hipGetLastError();
}

}  // namespace

bool attend_mfma_supported(const PoolGeom& g, int32_t rows) {
    return (g.head_dim == 64 || g.head_dim == 128) && rows >= 1 && rows <= 64;
}

hipError_t launch_attend_mfma(const AttendArgs& a, hipStream_t s) {
    const int nrb = (a.n_rows + 15) / 16;
    if (a.g.head_dim == 128) {
        if (nrb == 1) return launch_t<128, 1, 1>(a, s);
        if (nrb == 2) return launch_t<128, 1, 2>(a, s);
        return launch_t<128, 2, 2>(a, s);
    }
    if (a.g.head_dim == 64) {
        // up to 16 rows at d = 64 the workgroup fits 2 per CU without the big table
        if (nrb == 1) return launch_t<64, 1, 1, false>(a, s);
        if (nrb == 2) return launch_t<64, 1, 2>(a, s);
        return launch_t<64, 2, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace polykv
