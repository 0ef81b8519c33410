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
// tokens: lane t scores token t against its wave's row (fp32), the wave runs an online
// softmax in base 2, and then each lane accumulates P.V for D/64 dimensions.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace {

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
    static constexpr int OFF_Q = 0;                                  // fp32 [4][D]
    static constexpr int OFF_K = OFF_Q + 4 * D * 4;                  // fp16 [TCH][KS]
    static constexpr int OFF_V = OFF_K + TCH * KS * 2;               // fp16 [TCH][D]
    static constexpr int OFF_P = OFF_V + TCH * D * 2;                // fp32 [4][TCH]
    static constexpr int LDS = OFF_P + 4 * TCH * 4;
};

template <int D>
__global__ __launch_bounds__(256) void k_attend_tail(TailArgs a) {
    using C = TailCfg<D>;
    constexpr int DPL = C::DPL;
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
    const __half* tk = reinterpret_cast<const __half*>(a.tail_k) + tail_base;
    const __half* tv = reinterpret_cast<const __half*>(a.tail_v) + tail_base;
    const float qscale = a.softmax_scale * kLog2e;

    for (int rg = 0; rg < G; rg += 4) {
        const int row = rg + w;                 // query head h * G + row of this agent
        const bool live = row < G;              // wave-uniform
        const size_t qi = ((size_t)l * A + ag) * HG + (size_t)h * G + (live ? row : 0);
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
            // stage keys and values: 16-byte pieces, rows past the tail are not loaded
            for (int i = tid; i < TCH * D / 8; i += 256) {
                const int t = i / (D / 8), c = i - t * (D / 8);
                if (t < cnt) {
                    const uint4 kk = *reinterpret_cast<const uint4*>(tk + (size_t)(t0 + t) * D + 8 * c);
                    const uint4 vv = *reinterpret_cast<const uint4*>(tv + (size_t)(t0 + t) * D + 8 * c);
                    *reinterpret_cast<uint4*>(ks + t * C::KS + 8 * c) = kk;
                    *reinterpret_cast<uint4*>(vs + t * D + 8 * c) = vv;
                }
            }
            __syncthreads();
            if (live) {
                // score of token lane against this wave's row, in log2 units
                float s = -INFINITY;
                if (lane < cnt) {
                    float acc = 0.0f;
                    const _Float16* kr = ks + lane * C::KS;
                    const float* qr = qs + w * D;
#pragma unroll 8
                    for (int e = 0; e < D; ++e) acc = __builtin_fmaf(qr[e], (float)kr[e], acc);
                    s = acc;
                }
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
                for (int t = 0; t < cnt; ++t) {
                    const float pt = ps[w * TCH + t];
#pragma unroll
                    for (int e = 0; e < DPL; ++e)
                        o[e] = __builtin_fmaf(pt, (float)vs[t * D + DPL * lane + e], o[e]);
                }
            }
        }
        if (live) {
            // merge with the shared-pool partial (natural-log lse, normalised output)
            const float lse_t = kLn2 * (m + __builtin_log2f(lsum));
            const float lse_p = a.lse[qi];
            const float M = fmaxf(lse_p, lse_t);
            const float wp = __expf(lse_p - M), wt = __expf(lse_t - M);
            const float inv = 1.0f / (wp + wt);
            float* orow = a.out + qi * D + DPL * lane;
#pragma unroll
            for (int e = 0; e < DPL; ++e) orow[e] = (wp * orow[e] + wt * (o[e] / lsum)) * inv;
            if (lane == 0) a.lse[qi] = M + __logf(wp + wt);
        }
    }
}

template <int D>
hipError_t launch_tail_t(const TailArgs& a, hipStream_t s) {
    using C = TailCfg<D>;
    auto kern = k_attend_tail<D>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
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
