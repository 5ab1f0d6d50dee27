// gfx950 memory helpers shared by kernels that stage global data in LDS with the
// asynchronous LDS-DMA loads (global_load_lds_dwordx4) and wait for them with explicit
// vmcnt counts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sv {
namespace gmem {

// Wait until at most N vector-memory loads of this wave are outstanding. Loads complete
// in issue order, so afterwards every load but the newest N has landed (LDS-DMA loads
// included).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits [3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] at maximum.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  // a C-style cast is the address-space conversion (generic -> LDS)
  return static_cast<uint32_t>(
      (uintptr_t)((__attribute__((address_space(3))) char*)(const_cast<void*>(p))));
}

// One 16-byte LDS-DMA load per lane: lane i's 16 bytes at base + off land at LDS byte
// address lds + 16 * i. base and lds must be wave-uniform. Both pass through
// readfirstlane so they sit in SGPRs even where the register allocator kept a uniform
// value (one derived from the wave index, say) in VGPRs; each 32-bit half of the base is
// converted to uint32_t before widening, so a low word with bit 31 set is not
// sign-extended into the high word.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint64_t sa = (static_cast<uint64_t>(hi) << 32) | lo;
  const uint32_t sl = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
  // The LDS address goes in through an M0 operand, so the compiler writes M0 itself and
  // knows this instruction reads it. The compiler cannot see that the asm is a vector
  // memory instruction, so the asm provides the wait states its operands need: a VMEM
  // instruction must not read an SGPR within 5 wait states of a VALU write to it (the
  // base halves come from v_readfirstlane) and an LDS DMA must not read M0 in the wait
  // state after an SALU write to it. s_nop 4 gives 5 after whatever precedes the asm.
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(reinterpret_cast<const void*>(sa)), "{m0}"(sl)
               : "memory");
}

}  // namespace gmem
}  // namespace sv
