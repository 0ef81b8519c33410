// Private-tail merge (gfx950): every agent also attends over its own uncompressed fp16
// tokens (the tail it generated after the shared pool was written), and that partial is
// merged with the shared-pool result by log-sum-exp.
//
// PolyKV abstract: the compressed pool is handed to N separate agent contexts; each
// context then continues on its own. The pool result (normalised output o_p and
// lse_p = ln sum_pool exp(scale q . k)) and the tail partial (o_t, lse_t) combine as
//   M = max(lse_p, lse_t), w_p = exp(lse_p - M), w_t = exp(lse_t - M),
//   o = (w_p o_p + w_t o_t) / (w_p + w_t),  lse = M + ln(w_p + w_t),
// which is the softmax attention over the union of pool and tail tokens.
//
// One workgroup per (layer, agent, KV head), four waves; wave w serves query row w of a
// group of four of that head's gqa rows. The tail streams through LDS in chunks of 64
// tokens, and every thread holds the next chunk's 16-byte pieces in registers while the
// current chunk is used, so the loads of one chunk overlap the arithmetic of the previous
// one. Lane t scores token t against its wave's row (fp32 q from LDS, fp16 keys read 8 at
// a time), the wave runs an online softmax in base 2, and then each lane accumulates P.V
// for D/64 dimensions.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // 16 bytes, a plain vector

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int TCH = 64;  // tail tokens per chunk

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int D>
struct TailCfg {
    static constexpr int KS = D + 8;            // padded fp16 stride of a key row in LDS
    static constexpr int DPL = D / 64;          // dimensions per lane in P.V
    static constexpr int PPT = TCH * D / 8 / 256;  // 16-byte pieces of K (and of V) per thread
    static constexpr int OFF_Q = 0;                                  // fp32 [4][D]
    static constexpr int OFF_K = OFF_Q + 4 * D * 4;                  // fp16 [TCH][KS]
    static constexpr int OFF_V = OFF_K + TCH * KS * 2;               // fp16 [TCH][D]
    static constexpr int OFF_P = OFF_V + TCH * D * 2;                // fp32 [4][TCH]
    static constexpr int LDS = OFF_P + 4 * TCH * 4;
    static_assert(PPT >= 1 && TCH * D / 8 == 256 * PPT, "whole pieces per thread");
};

// The 16-byte pieces of chunk t0 that this thread moves: piece i is token (tid + 256 i) / PR,
// column (tid + 256 i) % PR of the chunk (PR pieces per token row); tokens past the tail
// read the last tail token instead (valid memory; their scores are masked).
template <int PPT, int PR>
__device__ __forceinline__ void fetch_chunk(u4 (&nk)[PPT], u4 (&nv)[PPT], const u4* tk,
                                            const u4* tv, int t0, int n, int tid) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int piece = tid + 256 * i;
        const size_t row = (size_t)min(t0 + piece / PR, n - 1);
        nk[i] = tk[row * PR + piece % PR];
        nv[i] = tv[row * PR + piece % PR];
    }
}

template <int D>
__global__ __launch_bounds__(256) void k_attend_tail(TailArgs a) {
    using C = TailCfg<D>;
    constexpr int DPL = C::DPL, PPT = C::PPT, PR = D / 8;  // PR: pieces per token row
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float* qs = reinterpret_cast<float*>(lds + C::OFF_Q);
    _Float16* ks = reinterpret_cast<_Float16*>(lds + C::OFF_K);
    _Float16* vs = reinterpret_cast<_Float16*>(lds + C::OFF_V);
    float* ps = reinterpret_cast<float*>(lds + C::OFF_P);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.n_kv_heads, G = a.gqa, A = a.n_agents;
    const int h = blockIdx.x % H;
    const int ag = (blockIdx.x / H) % A;
    const int l = blockIdx.x / (H * A);
    // tail length from device memory; values outside [0, cap] are clamped
    const int n = min(max(a.tail_len[ag], 0), a.tail_cap);
    if (n == 0) return;  // the pool result stands (uniform over the workgroup)

    const size_t HG = (size_t)H * G;
    const size_t tail_base = (((size_t)ag * a.layer_count + l) * H + h) * (size_t)a.tail_cap * D;
    const u4* tk = reinterpret_cast<const u4*>(reinterpret_cast<const __half*>(a.tail_k) + tail_base);
    const u4* tv = reinterpret_cast<const u4*>(reinterpret_cast<const __half*>(a.tail_v) + tail_base);
    const float qscale = a.softmax_scale * kLog2e;

    u4 nk[PPT], nv[PPT];

    for (int rg = 0; rg < G; rg += 4) {
        const int row = rg + w;                 // query head h * G + row of this agent
        const bool live = row < G;              // wave-uniform
        const size_t qi = ((size_t)l * A + ag) * HG + (size_t)h * G + (live ? row : 0);
        fetch_chunk<PPT, PR>(nk, nv, tk, tv, 0, n, tid);
        // the pool partial of this row, loaded now so that its latency overlaps the tail's
        float* orow = a.out + qi * D + DPL * lane;
        float o_pool[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o_pool[e] = orow[e];
        const float lse_p = a.lse[qi];
        __syncthreads();                        // previous row group is done with qs
        if (live)
            for (int e = lane; e < D; e += 64) qs[w * D + e] = a.q[qi * D + e] * qscale;
        float m = -INFINITY, lsum = 0.0f;
        float o[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;

        for (int t0 = 0; t0 < n; t0 += TCH) {
            const int cnt = min(TCH, n - t0);
            __syncthreads();                    // previous chunk is consumed
#pragma unroll
            for (int i = 0; i < PPT; ++i) {
                const int piece = tid + 256 * i;
                const int t = piece / PR, c = piece % PR;
                *reinterpret_cast<u4*>(ks + t * C::KS + 8 * c) = nk[i];
                *reinterpret_cast<u4*>(vs + t * D + 8 * c) = nv[i];
            }
            __syncthreads();
            if (t0 + TCH < n) fetch_chunk<PPT, PR>(nk, nv, tk, tv, t0 + TCH, n, tid);  // in flight meanwhile
            if (live) {
                // score of token `lane` against this wave's row, in log2 units; rows past the
                // tail hold a copy of the last token (finite) and are masked here
                float acc = 0.0f;
                {
                    const h8* kr = reinterpret_cast<const h8*>(ks + lane * C::KS);
                    const float4* qr = reinterpret_cast<const float4*>(qs + w * D);
#pragma unroll
                    for (int b = 0; b < D / 8; ++b) {
                        const h8 kk = kr[b];
                        const float4 q0 = qr[2 * b], q1 = qr[2 * b + 1];
                        acc = __builtin_fmaf(q0.x, (float)kk[0], acc);
                        acc = __builtin_fmaf(q0.y, (float)kk[1], acc);
                        acc = __builtin_fmaf(q0.z, (float)kk[2], acc);
                        acc = __builtin_fmaf(q0.w, (float)kk[3], acc);
                        acc = __builtin_fmaf(q1.x, (float)kk[4], acc);
                        acc = __builtin_fmaf(q1.y, (float)kk[5], acc);
                        acc = __builtin_fmaf(q1.z, (float)kk[6], acc);
                        acc = __builtin_fmaf(q1.w, (float)kk[7], acc);
                    }
                }
                const float s = lane < cnt ? acc : -INFINITY;
                const float m_new = fmaxf(m, wave_max(s));
                const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // m = -inf: 0
                const float p = lane < cnt ? __builtin_amdgcn_exp2f(s - m_new) : 0.0f;
                lsum = lsum * alpha + wave_sum(p);
                m = m_new;
                ps[w * TCH + lane] = p;
#pragma unroll
                for (int e = 0; e < DPL; ++e) o[e] *= alpha;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // P.V over the whole chunk (p = 0 past the tail), unrolled so that the LDS
                // reads are issued ahead of their use
                const float4* pr = reinterpret_cast<const float4*>(ps + w * TCH);
#pragma unroll
                for (int t4 = 0; t4 < TCH / 4; ++t4) {
                    const float4 p4 = pr[t4];
                    const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const _Float16* vr = vs + (4 * t4 + u) * D + DPL * lane;
#pragma unroll
                        for (int e = 0; e < DPL; ++e) o[e] = __builtin_fmaf(pv[u], (float)vr[e], o[e]);
                    }
                }
            }
        }
        if (live) {
            // merge with the shared-pool partial (natural-log lse, normalised output)
            const float lse_t = kLn2 * (m + __builtin_log2f(lsum));
            const float M = fmaxf(lse_p, lse_t);
            const float wp = __expf(lse_p - M), wt = __expf(lse_t - M);
            const float inv = 1.0f / (wp + wt);
#pragma unroll
            for (int e = 0; e < DPL; ++e) orow[e] = (wp * o_pool[e] + wt * (o[e] / lsum)) * inv;
            if (lane == 0) a.lse[qi] = M + __logf(wp + wt);
        }
    }
}

template <int D>
hipError_t launch_tail_t(const TailArgs& a, hipStream_t s) {
    using C = TailCfg<D>;
    auto kern = k_attend_tail<D>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_limit_once((const void*)kern, C::LDS, lds_set);
    if (e != hipSuccess) return e;
    const uint32_t blocks = (uint32_t)a.layer_count * (uint32_t)a.n_agents * (uint32_t)a.n_kv_heads;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), C::LDS, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_tail(const TailArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 64: return launch_tail_t<64>(a, s);
        case 128: return launch_tail_t<128>(a, s);
        case 256: return launch_tail_t<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace polykv
