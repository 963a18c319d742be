// Building blocks of the HBM -> LDS tile rings of the attention and LM-head
// kernels: direct global -> LDS loads, waits on the vector-memory counter,
// and workgroup barriers without a memory fence.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace orthrus {

typedef void __attribute__((address_space(3)))* lds_void_ptr;

// Workgroup barrier without a memory fence: no wait for outstanding global
// loads is implied (the tile ring waits for exactly the loads it needs); the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS byte address lds + 16 l.  It is written as assembly so
// that the compiler does not track these LDS writes: lacking proof that a
// later LDS read touches another ring stage, it would wait for every load in
// flight before that read, draining the ring.  The ring's own vmcnt waits
// and barriers order each read after the loads that fill its stage.
// m0 is a register the compiler reserves; nothing else in these kernels takes
// an m0 operand (the LDS reads, barriers and lane reads here do not), so the
// clobber is safe and the warning about it is silenced for this function.
// NT selects the non-temporal (streaming) cache policy, for data that no
// other workgroup reads again: it keeps a one-pass stream from displacing
// what the caches still hold (measured faster for the bf16 K/V stream and
// for LM-head weights read once; slower where weight tiles are shared).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT = false>
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt"
        :
        : "s"(lds), "v"(src)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds), "v"(src)
        : "memory", "m0");
  }
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(p)));
}

}  // namespace orthrus
