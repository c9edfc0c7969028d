// Direct-to-LDS buffer loads and the barrier that waits for them, shared by
// the kernels that stream operands through an LDS ring.
#pragma once

#include <stdint.h>

#include "common.h"

namespace mlr {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// A buffer offset past every range the kernels use (all below 2 GiB): a load
// from it returns zero and touches no memory.
constexpr uint32_t kOob = 0x80000000u;

// Byte address in LDS of a __shared__ array (pass the array itself: a cast
// of a generic pointer would add a null check).
#define lds_address(arr) \
  __builtin_amdgcn_readfirstlane(                                                        \
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(arr))))

// Buffer resource (raw, 32-bit elements, no stride) as four scalar words, for
// the inline DMA below.
__device__ __forceinline__ i32x4_t dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r.y = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(int(bytes));
  r.w = 0x00020000;
  return r;
}

// One 16-byte-per-lane buffer load written straight to LDS: lane i's chunk
// lands at byte lds + 16 i.  Written as inline assembly so that the compiler
// does not see an LDS store in flight; it would otherwise wait for every
// outstanding stage before each LDS read.  The waits for these loads are the
// explicit ones in stage_barrier.  M0 (the LDS base) is saved and restored.
// NT: a non-temporal (evict-first) load, for bytes no other workgroup reads.
template <bool NT = false>
__device__ __forceinline__ void dma16(i32x4_t r, uint32_t lds, uint32_t voff) {
  int saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
}

// Wait until at most VM vector memory operations of this wavefront are
// outstanding and its LDS operations are done, then meet the workgroup.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier; no release fence is used, since one would also wait for
// the stages still in flight.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt is a 6-bit field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mlr
