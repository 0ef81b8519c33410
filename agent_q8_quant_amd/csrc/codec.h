// Device-side codecs of one key block and one value group, shared by the compress kernels
// (input from HBM) and the fused projection kernel (input from LDS).
//
// PolyKV abstract: keys are quantised at int8 in the q8_0 format; values are rotated by a
// fast Walsh-Hadamard transform and coded with a 3-bit Lloyd-Max quantiser for N(0,1).
// The finer definitions (block of 32 along head_dim, fp16 scale RNE16(amax / 127), codes
// RNE(x / s) clamped to [-127, 127]; y = H v / ||v||, code = #{k : y > b_k}, three
// bit-planes per 32-token group) are the library's format.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "polykv_internal.h"

namespace polykv {
namespace codec {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------------------
// q8_0 of 8 consecutive key entries (one 16-byte fp16 piece) per lane; the four lanes of
// a quad hold one 32-entry block and combine their |x| maxima through two lane exchanges.
// Returns the block's fp16 scale; packed[0..1] receive the 8 int8 codes.
// Arithmetic, equal to the definition (IEEE amax / 127, round-half-even of x / s):
// - m / 127 for an fp16 m lies at least 1/254 of an fp16 ulp from every fp16 rounding
//   midpoint, so amax * fl(1/127) (relative error < 2^-22) rounds to the same fp16 scale;
// - x and s are fp16, so every quotient x / s that is not a tie lies at least 2^-13 from
//   a half-integer, and a tie is exactly representable in fp32. The quotient below,
//   t = x r with r = rcp(s), refined once by t + (x - t s) r, is within ~2^-40 relative
//   of x / s: it equals the quotient whenever that is representable (every tie), and is
//   far closer than 2^-13 otherwise, so rint gives round-half-even of the exact x / s.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ __half q8_encode8(uint4 raw, uint32_t (&packed)[2]) {
    const __half* hv = reinterpret_cast<const __half*>(&raw);
    float x[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = __half2float(hv[e]);
        amax = fmaxf(amax, fabsf(x[e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));

    const __half s16 = __float2half_rn(amax * (1.0f / 127.0f));   // = RNE16(amax / 127)
    const float s = __half2float(s16);
    const float r = s > 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;   // s = 0: every code 0

    packed[0] = packed[1] = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = x[e] * r;
        const float t2 = __builtin_fmaf(__builtin_fmaf(-t, s, x[e]), r, t);
        const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(t2), -127.0f, 127.0f);
        const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
        packed[e >> 2] |= b << (8 * (e & 3));
    }
    return s16;
}

// lane `lane` (a constant once the loops are unrolled) of w := the wave-uniform value x
__device__ __forceinline__ void put_lane(uint32_t& w, uint32_t x, int lane) {
    asm("v_writelane_b32 %0, %1, %2" : "+v"(w) : "s"(x), "i"(lane));
}

// Thresholds b_k n (k = 4, 5, 6) a token's rotated coordinates y are compared with:
// y / n > b  <=>  y > b n for n > 0; n = 0 gives y = 0 and infinite thresholds (every code
// 3). Tokens outside the encoded range have y = 0 and get thresholds -1: then every plane
// bit of put_code_words comes out 0 (bits past T must be 0; others are merged back by
// the caller's keep mask).
struct VThresh {
    float t4, t5, t6;
};
__device__ __forceinline__ VThresh v_thresholds(float n, bool valid, const CodebookHalf& cb) {
    const float inv_t = valid ? (n > 0.0f ? 1.0f : INFINITY) : -1.0f;
    VThresh t;
    t.t4 = n > 0.0f ? cb.boundary_pos[0] * n : inv_t;
    t.t5 = n > 0.0f ? cb.boundary_pos[1] * n : inv_t;
    t.t6 = n > 0.0f ? cb.boundary_pos[2] * n : inv_t;
    return t;
}

// Codes of one register of rotated coordinates, one per lane, into the group's plane
// words. A ballot over the wave is two whole plane words: the low 32 lanes hold dim d_lo of
// tokens 0..31, the high 32 lanes dim d_hi. Word (p, d) of the group (3 x D words) goes to
// lane (p D + d) % 64 of wv[(p D + d) / 64]; d_lo and d_hi are constants once unrolled.
// Codes from four compares (sign and |y| against the three positive thresholds):
// code = 4 + m for y > 0, 3 - m otherwise, m = c4 + c5 + c6 (thermometer), so
// bit 2 = sign, bit 1 = c5 xnor sign, bit 0 = (c4 ^ c5 ^ c6) xnor sign
// (for y < 0 exactly on a boundary this gives the higher code).
template <int D>
__device__ __forceinline__ void put_code_words(float yy, const VThresh& t, int d_lo, int d_hi,
                                               uint32_t (&wv)[3 * D / 64]) {
    const float ay = fabsf(yy);
    const uint64_t pos = __ballot(yy > 0.0f);
    const uint64_t c4 = __ballot(ay > t.t4);
    const uint64_t c5 = __ballot(ay > t.t5);
    const uint64_t c6 = __ballot(ay > t.t6);
    uint64_t pl[3];
    pl[2] = pos;
    pl[1] = ~(c5 ^ pos);
    pl[0] = ~(c4 ^ c5 ^ c6 ^ pos);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int w0 = p * D + d_lo, w1 = p * D + d_hi;
        put_lane(wv[w0 / 64], (uint32_t)pl[p], w0 % 64);
        put_lane(wv[w1 / 64], (uint32_t)(pl[p] >> 32), w1 % 64);
    }
}

// The group's plane words from wv (lane-linear per register); bits in `keep`
// (wave-uniform) are read back and kept, the others written.
template <int D>
__device__ __forceinline__ void store_group_words(uint32_t* words, uint32_t keep,
                                                  const uint32_t (&wv)[3 * D / 64], int lane) {
    constexpr int WPL = 3 * D / 64;
    if (keep) {
#pragma unroll
        for (int r = 0; r < WPL; ++r) words[64 * r + lane] = (words[64 * r + lane] & keep) | wv[r];
    } else {
#pragma unroll
        for (int r = 0; r < WPL; ++r) words[64 * r + lane] = wv[r];
    }
}

// ---------------------------------------------------------------------------------------
// One 32-token value group on the matrix cores (head_dim 64 or 128), one wave. vb holds
// the B operand: lane l has token l % 32 of the group, dims 16 kk + 8 (l / 32) .. + 7 in
// vb[kk] (zeros for tokens not encoded here; valid is false for them). The rotation
// y = H v runs as v_mfma_f32_32x32x16_f16 with the +-1 Sylvester matrix as the A operand
// (exact in fp16; accumulation in fp32), so lane l ends up holding token l % 32 at output
// dims 32 mb + 8 (i / 4) + 4 (l / 32) + i % 4 (register i of block mb): a ballot of one
// register covers dims d0 (low half) and d0 + 4 (high half).
// H[m][k] = (-1)^popcount(m & k); for the A fragment of output block mb and k step kk,
// lane l holds m = 32 mb + l % 32, k = 16 kk + 8 (l / 32) + e, and the sign factors into
// (-1)^(popcount(a & b) + (a >> 4) * (kk & 1)) * (-1)^popcount(mb & (kk >> 1)) with
// a = l % 32 and b = 8 (l / 32) + e.
// words: the group's 3 x D plane words (keep: as in store_group_words). norms: the
// tile's norms; token: this lane's token index.
// ---------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void encode_v_group(const h8 (&vb)[D / 16], bool valid, const CodebookHalf& cb,
                                               uint32_t* words, uint32_t keep, __half* norms,
                                               uint32_t token, int lane) {
    constexpr int KK = D / 16;        // k steps of the rotation
    constexpr int MB = D / 32;        // 32-dim output blocks
    constexpr int WPL = 3 * D / 64;   // plane words per lane of the store
    const int l32 = lane & 31, hl = lane >> 5;
    // Sylvester fragments for even and odd k steps
    h8 F[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int b = 8 * hl + e;
        const int base = __builtin_popcount(l32 & b) & 1;
        F[0][e] = base ? (_Float16)-1.0f : (_Float16)1.0f;
        F[1][e] = (base ^ (l32 >> 4)) ? (_Float16)-1.0f : (_Float16)1.0f;
    }

    // squared norm in fp32 (each lane holds half of the token's dims)
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const h2 x = {vb[kk][e], vb[kk][e + 1]};
            ss = __builtin_amdgcn_fdot2(x, x, ss, false);
        }
    {
        const uint32_t u = __float_as_uint(ss);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float n = sqrtf(ss);
    const VThresh t = v_thresholds(n, valid, cb);

    uint32_t wv[WPL];
#pragma unroll
    for (int r = 0; r < WPL; ++r) wv[r] = 0u;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        f16v y = {};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bool neg = __builtin_popcount(mb & (kk >> 1)) & 1;
            const h8 a = neg ? -F[kk & 1] : F[kk & 1];
            y = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, vb[kk], y, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d0 = 32 * mb + 8 * (i / 4) + (i % 4);
            put_code_words<D>(y[i], t, d0, d0 + 4, wv);
        }
    }

    store_group_words<D>(words, keep, wv, lane);
    if (hl == 0 && valid) norms[token] = __float2half_rn(n);
}

}  // namespace codec
}  // namespace polykv
