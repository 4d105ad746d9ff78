// Direct global->LDS copies and explicit vector-memory waits shared by the
// decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// s_waitcnt with vmcnt <= N (lgkmcnt / expcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave-wide global->LDS copies: lane i's 16 (resp. 4) bytes land at
// lds_base + 16*i (resp. 4*i).  Issued from inline asm so that the
// compiler's wait-count pass does not stall every later LDS read on them (it
// cannot tell which buffer a copy targets); the kernels order them with
// explicit vmcnt waits.  M0 carries the LDS base; nothing else in these
// kernels uses M0 (the asm sets it before every copy), so listing the
// reserved register is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// A uniform 64-bit address kept in scalar registers (inside divergent code
// the compiler may otherwise hold it in vector registers).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}
// The same 16-byte copy addressed as a uniform 64-bit base plus a per-lane
// 32-bit byte offset (one VGPR per copy instead of a 64-bit address pair).
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace mla
