// Direct HBM -> LDS transfers and LDS transpose reads for gfx950.
#pragma once

#include "device_common.hpp"

namespace tpcol {

#define TP_AS1 __attribute__((address_space(1)))
#define TP_AS3 __attribute__((address_space(3)))
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// One wave-wide DMA: lane i's 16 bytes at g land at LDS byte address
// lds + 16*i.  Issued as inline assembly on purpose: the compiler then does
// not count it as a pending LDS write, so it neither drains it at every
// barrier nor before every ds_read; callers order it explicitly with
// wait_vmcnt + barrier.  The compiler does not insert hazard wait states
// into inline assembly, so the s_nop 4 supplies them: five wait states
// cover both a VALU write of an SGPR operand (e.g. v_readfirstlane of the
// base) and the M0 write that a vector-memory read of it must not follow
// directly.
__device__ __forceinline__ void dma16(const uint16_t *g, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte
// offset: the per-block address arithmetic stays on the scalar unit.
__device__ __forceinline__ void dma16s(uint32_t voff, const void *sbase, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Same, nontemporal: for data read once (decode weights), which should not
// displace cached lines.
__device__ __forceinline__ void dma16s_nt(uint32_t voff, const void *sbase, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// LDS byte address of a __shared__ pointer (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const uint16_t *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(TP_AS3 const void *)p);
}

// Wait until at most N of this wave's vector-memory ops are still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j & 3) of the 8-byte chunks addressed by lanes 4e + (j >> 2), e = 0..3.
__device__ __forceinline__ uint2 tr_read(const uint16_t *p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_AS3 i16x4_t *)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace tpcol
