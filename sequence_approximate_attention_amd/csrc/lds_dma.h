// Device helpers shared by the bf16 kernels that stage tiles in LDS with
// direct-to-LDS buffer loads (gfx950).
#pragma once

#include "spava_common.h"

namespace spava {

// K-tile rows are read in a permuted order (bits 2 and 3 of the row index
// swapped) so that the accumulators of S^T = K Q^T already have the B-operand
// layout of a following V^T P^T product with keys in natural order.
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte slot of chunk c in a swizzled LDS row r of RB bytes: the 16 rows
// one ds_read_b128 phase touches land in distinct banks.  The map is an
// involution in c, so it also gives the chunk stored in slot c.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB == 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most N
// vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer descriptor (gfx9 family: stride 0, word 3 = 0x00020000) over
// `bytes` bytes from `base`, as four scalar words.  The kernels keep every
// lane's address of a direct-to-LDS copy inside its tensor and do not rely on
// the range check: copies whose lanes pointed past the end of a tensor that
// ended on an allocation boundary have faulted the GPU.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((unsigned)b);
  r.y = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}

// One buffer_load_dwordx4 ... lds: every lane's 16 bytes at byte offset
// soff + voff of the buffer land at lds + 16 * lane.  Written as inline
// assembly so that the compiler keeps no wait bookkeeping of its own for these
// copies: their completion is awaited explicitly (wait_vm) before the barrier
// that publishes a ring slot.  M0 carries the LDS address; it needs one wait
// state before the load.  The compiler does not accept M0 (a reserved
// register) as a clobber, so it cannot be told that this statement writes
// it: no other code in the kernels that use this copy may rely on M0, which
// tests/test_device_asm.py checks in their generated assembly.
__device__ __forceinline__ void copy16_to_lds(const u32x4& rsrc, unsigned soff, unsigned voff,
                                              unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "memory");
}

}  // namespace spava
