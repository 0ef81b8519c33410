// Direct global-to-LDS loads (gfx950) through inline assembly, shared by the kernels that
// stream operand tiles into LDS rings.
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight into LDS:
// address = 64-bit scalar base + 32-bit per-lane offset, LDS destination = M0 + 16 * lane
// (4 * lane for the dword form), so one wave instruction fills 1 KB of LDS. The compiler
// does not track these loads: it inserts no vmcnt wait for them, so each wave waits on its
// own loads with explicit vmcnt counts (wait_vm) before a barrier publishes the data.
// Destinations must be 256-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace polykv {
namespace lds_dma {

// M0 is a reserved register that the compiler does not let inline asm clobber: each asm
// block saves it, points it at the LDS destination for the load (which reads it at issue)
// and restores it.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}
// at most N vector-memory instructions of this wave still in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// lane id, recomputed at every use: volatile so that the compiler neither hoists it (and
// the offsets derived from it) out of a loop nor keeps it live across the loop
__device__ __forceinline__ uint32_t lane_id() {
    uint32_t r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

}  // namespace lds_dma
}  // namespace polykv
