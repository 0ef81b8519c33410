// Shared-pool decode attention, fp32 vector-ALU path (gfx950).
//
// PolyKV abstract: N agents read one compressed pool concurrently. For a pool tile (layer, KV head) every agent's query rows of that KV head are
// scored against every pool token: S = scale * q . (code * s), an online softmax runs over
// token chunks, and P.V is accumulated in the Hadamard-rotated domain as
// acc = sum_t p_t * n_t * c[code_t]; each output row is H acc / (d * l) with a single
// inverse FWHT per row instead of one per token. A launch serves up to 64 of a tile's rows
// (a range given by the launch arguments); more rows are served by further launches.
//
// One workgroup (256 threads) owns one tile. Per chunk of C tokens the keys are expanded
// to fp32 (already multiplied by their block scale and scale * log2 e) and the values to
// n_t * c[code] in LDS; threads own 4 query rows each and a slice of the chunk's tokens
// (scores) or of the head dimensions (P.V).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float centroid_of(uint32_t code, const CodebookHalf& cb) {
    // code >= 4: +c[code - 4] of the positive half; code <= 3: -c[3 - code]
    const uint32_t m = code >= 4u ? code - 4u : 3u - code;
    const float mag = (m & 2u) ? ((m & 1u) ? cb.centroid_pos[3] : cb.centroid_pos[2])
                               : ((m & 1u) ? cb.centroid_pos[1] : cb.centroid_pos[0]);
    return code >= 4u ? mag : -mag;
}

template <int D, int NRQ>
struct ValuCfg {
    static constexpr int RP = 4 * NRQ;                        // padded rows
    static constexpr int C = (D == 256 && NRQ == 16) ? 32 : 64;  // tokens per chunk
    static constexpr int TQN = 256 / NRQ;                     // thread groups per row quad
    static constexpr int TPT = C / TQN;                       // tokens per thread (scores)
    static constexpr int DPT = D / TQN;                       // dims per thread (P.V)
    static constexpr int QS = RP + 4;                         // padded stride of qT rows
    // LDS carve-up, in floats
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + D * QS;
    static constexpr int OFF_V = OFF_K + D * C;
    static constexpr int OFF_P = OFF_V + C * D;
    static constexpr int OFF_N = OFF_P + C * RP;
    static constexpr int OFF_L = OFF_N + C;
    static constexpr int OFF_M = OFF_L + RP;
    static constexpr int FLOATS = OFF_M + RP;
    static_assert(TPT >= 1 && DPT >= 1, "thread mapping");
    static_assert(RP * D <= D * C + C * D, "final accumulator must fit the K and V stages");
};

template <int D, int NRQ>
__global__ __launch_bounds__(256) void k_attend_valu(AttendArgs a) {
    using Cfg = ValuCfg<D, NRQ>;
    constexpr int RP = Cfg::RP, C = Cfg::C, TQN = Cfg::TQN, TPT = Cfg::TPT, DPT = Cfg::DPT,
                  QS = Cfg::QS;
    extern __shared__ float lds[];
    float* qT = lds + Cfg::OFF_Q;   // [D][QS]   query rows, transposed
    float* kT = lds + Cfg::OFF_K;   // [D][C]    scaled keys, transposed
    float* vh = lds + Cfg::OFF_V;   // [C][D]    n_t * c[code], rotated domain
    float* pT = lds + Cfg::OFF_P;   // [C][RP]   softmax numerators
    float* nrm = lds + Cfg::OFF_N;  // [C]       value norms
    float* lrow = lds + Cfg::OFF_L; // [RP]      row sums at the end
    float* mrow = lds + Cfg::OFF_M; // [RP]      row maxima at the end (log2 units)

    const PoolGeom& g = a.g;
    const int tid = threadIdx.x;
    const int H = g.n_kv_heads, T = g.n_tokens, G = a.gqa, A = a.n_agents;
    const int R = a.n_rows;  // rows of this launch; row r is row a.row_begin + r of the tile
    const int tile_local = blockIdx.x;
    const int l_local = tile_local / H, h = tile_local - l_local * H;
    const size_t tile = (size_t)(a.layer_begin + l_local) * H + h;
    const int8_t* kcodes = reinterpret_cast<const int8_t*>(a.pool + g.k_codes_off + tile * g.k_codes_stride);
    const __half* kscales = reinterpret_cast<const __half*>(a.pool + g.k_scales_off + tile * g.k_scales_stride);
    const uint32_t* vplanes = reinterpret_cast<const uint32_t*>(a.pool + g.v_planes_off + tile * g.v_planes_stride);
    const __half* vnorms = reinterpret_cast<const __half*>(a.pool + g.v_norms_off + tile * g.v_norms_stride);
    const size_t HG = (size_t)H * G;

    // query rows: row_begin + r = agent * G + j  ->  q[l_local][agent][h * G + j][:]
    for (int idx = tid; idx < RP * D; idx += 256) {
        const int r = idx / D, i = idx - r * D;
        float val = 0.0f;
        if (r < R) {
            const int gr = a.row_begin + r, ag = gr / G, j = gr - ag * G;
            val = a.q[(((size_t)l_local * A + ag) * HG + (size_t)h * G + j) * D + i];
        }
        qT[i * QS + r] = val;
    }

    const int rq = tid / TQN, tq = tid - rq * TQN;
    const float sl2 = a.softmax_scale * kLog2e;
    float m_run[4], l_run[4], acc[4][DPT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[r][e] = 0.0f;
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        __syncthreads();  // previous chunk fully consumed (and qT written on entry)
        // keys: 16 codes per load, expanded with their block scale
        for (int li = tid; li < C * (D / 16); li += 256) {
            const int t = li % C, part = li / C;
            const int tok = t0 + t;
            float vals[16];
            if (tok < T) {
                const uint4 raw = *reinterpret_cast<const uint4*>(kcodes + (size_t)tok * D + 16 * part);
                const int8_t* cb8 = reinterpret_cast<const int8_t*>(&raw);
                const float s = __half2float(kscales[(size_t)tok * (D / 32) + part / 2]) * sl2;
#pragma unroll
                for (int e = 0; e < 16; ++e) vals[e] = (float)cb8[e] * s;
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) vals[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) kT[(16 * part + e) * C + t] = vals[e];
        }
        if (tid < C) nrm[tid] = (t0 + tid < T) ? __half2float(vnorms[t0 + tid]) : 0.0f;
        __syncthreads();
        // values: one (token group, coordinate) pair per thread step
        for (int it = tid; it < (C / 32) * D; it += 256) {
            const int gi = it / D, i = it - gi * D;
            const int grp = t0 / 32 + gi;
            uint32_t w0 = 0, w1 = 0, w2 = 0;
            if (grp < g.n_groups) {
                const uint32_t* wp = vplanes + (size_t)grp * 3 * D + i;
                w0 = wp[0];
                w1 = wp[D];
                w2 = wp[2 * D];
            }
#pragma unroll 8
            for (int j = 0; j < 32; ++j) {
                const uint32_t code = ((w0 >> j) & 1u) | (((w1 >> j) & 1u) << 1) | (((w2 >> j) & 1u) << 2);
                vh[(gi * 32 + j) * D + i] = nrm[gi * 32 + j] * centroid_of(code, a.cb);
            }
        }
        __syncthreads();

        // scores for rows 4rq..4rq+3 and tokens tq*TPT ..
        float s[4][TPT];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < TPT; ++t) s[r][t] = 0.0f;
        for (int i = 0; i < D; ++i) {
            const float4 q4 = *reinterpret_cast<const float4*>(qT + i * QS + 4 * rq);
            float kv[TPT];
#pragma unroll
            for (int t = 0; t < TPT; ++t) kv[t] = kT[i * C + tq * TPT + t];
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                s[0][t] = fmaf(q4.x, kv[t], s[0][t]);
                s[1][t] = fmaf(q4.y, kv[t], s[1][t]);
                s[2][t] = fmaf(q4.z, kv[t], s[2][t]);
                s[3][t] = fmaf(q4.w, kv[t], s[3][t]);
            }
        }
        // online softmax (base 2); the TQN lanes of a row quad are consecutive lanes
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float cm = -INFINITY;
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                if (t0 + tq * TPT + t >= T) s[r][t] = -INFINITY;
                cm = fmaxf(cm, s[r][t]);
            }
#pragma unroll
            for (int off = 1; off < TQN; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
            const float m_new = fmaxf(m_run[r], cm);
            alpha[r] = exp2f(m_run[r] - m_new);
            float ps = 0.0f;
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                const float p = exp2f(s[r][t] - m_new);
                ps += p;
                pT[(tq * TPT + t) * RP + 4 * rq + r] = p;
            }
            l_run[r] = l_run[r] * alpha[r] + ps;
            m_run[r] = m_new;
        }
        __syncthreads();
        // P.V for rows 4rq.. and dims tq*DPT ..
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[r][e] *= alpha[r];
        for (int t = 0; t < C; ++t) {
            const float4 p4 = *reinterpret_cast<const float4*>(pT + t * RP + 4 * rq);
            const float* vr = vh + t * D + tq * DPT;
#pragma unroll
            for (int e = 0; e < DPT; ++e) {
                const float vv = vr[e];
                acc[0][e] = fmaf(p4.x, vv, acc[0][e]);
                acc[1][e] = fmaf(p4.y, vv, acc[1][e]);
                acc[2][e] = fmaf(p4.z, vv, acc[2][e]);
                acc[3][e] = fmaf(p4.w, vv, acc[3][e]);
            }
        }
    }

    // row sums: partials of the TQN lanes of a row quad
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float l = l_run[r];
#pragma unroll
        for (int off = 1; off < TQN; off <<= 1) l += __shfl_xor(l, off);
        l_run[r] = l;
    }
    __syncthreads();
    float* accs = lds + Cfg::OFF_K;  // [RP][D], reuses the key and value stages
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < DPT; ++e) accs[(4 * rq + r) * D + tq * DPT + e] = acc[r][e];
    if (tq == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lrow[4 * rq + r] = l_run[r];
            mrow[4 * rq + r] = m_run[r];
        }
    }
    __syncthreads();
    if (tid < R) {
        float x[D];
#pragma unroll
        for (int i = 0; i < D; ++i) x[i] = accs[tid * D + i];
#pragma unroll
        for (int hh = 1; hh < D; hh <<= 1) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                if (!(i & hh)) {
                    const float u = x[i], w = x[i + hh];
                    x[i] = u + w;
                    x[i + hh] = u - w;
                }
            }
        }
        const float inv = 1.0f / ((float)D * lrow[tid]);
        const int gr = a.row_begin + tid, ag = gr / G, j = gr - ag * G;
        // scores are in log2 units (scale * log2 e folded into q)
        if (a.lse)
            a.lse[((size_t)l_local * A + ag) * HG + (size_t)h * G + j] =
                kLn2 * (mrow[tid] + __builtin_log2f(lrow[tid]));
        float* o = a.out + (((size_t)l_local * A + ag) * HG + (size_t)h * G + j) * D;
#pragma unroll
        for (int i = 0; i < D; i += 4)
            *reinterpret_cast<float4*>(o + i) = make_float4(x[i] * inv, x[i + 1] * inv, x[i + 2] * inv, x[i + 3] * inv);
    }
}

template <int D, int NRQ>
hipError_t launch_valu_t(const AttendArgs& a, hipStream_t s) {
    using Cfg = ValuCfg<D, NRQ>;
    const size_t lds = (size_t)Cfg::FLOATS * sizeof(float);
    auto kern = k_attend_valu<D, NRQ>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once((const void*)kern, (int)lds, lds_set);
    if (e != hipSuccess) return e;
    const uint32_t tiles = (uint32_t)a.layer_count * (uint32_t)a.g.n_kv_heads;
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

size_t attend_workspace_bytes(const PoolGeom&, int32_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_attend_valu(const AttendArgs& a, hipStream_t s) {
    const bool small = a.n_rows <= 16;
    switch (a.g.head_dim) {
        case 64: return small ? launch_valu_t<64, 4>(a, s) : launch_valu_t<64, 16>(a, s);
        case 128: return small ? launch_valu_t<128, 4>(a, s) : launch_valu_t<128, 16>(a, s);
        case 256: return small ? launch_valu_t<256, 4>(a, s) : launch_valu_t<256, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace polykv
