// Tile loads that write LDS directly (LDS DMA), issued through inline
// assembly.
//
// Why asm: for the builtin forms of these loads the compiler cannot tell
// which LDS bytes a load in flight will write, so before the first LDS read
// that follows one it waits for every vector load in flight (vmcnt(0)). In a
// double-buffered loop that is the next stage's tile: each stage would wait
// for its successor's data before it could start. The kernels order tile
// loads and LDS reads themselves (a vmcnt wait and a workgroup barrier per
// stage), so the loads here are invisible to the compiler's wait insertion.
// Waits the compiler inserts for its own loads stay correct: vector loads
// complete in issue order, so waiting for an older load never needs to know
// about younger ones.
//
// The LDS address goes to M0 as an asm operand ("{m0}"), so the compiler
// writes M0 itself and knows its value is replaced. Hazards the compiler
// would handle for the real instructions are written out here, because it
// schedules around asm without looking inside:
//   * a VALU write of an SGPR followed by a memory instruction that reads it
//     needs 5 wait states (the compiler may restore a spilled SGPR with
//     v_readlane right before the asm);
//   * an M0 write followed by an LDS-DMA instruction needs 1.
// The leading s_nop 4 covers both.
#pragma once

#include <stdint.h>

#include "fwd_common.hpp"

namespace fa {
namespace hw {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for raw (unformatted, unswizzled) dword access.
constexpr int kRawBufferFlags = 0x00020000;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// raw buffer descriptor: base, stride 0, num_records bytes
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a & 0xffffffffu), static_cast<int>((a >> 32) & 0xffffu),
               num_records, kRawBufferFlags};
}

// buffer_load_dwordx4 ... offen lds: lane L's 16 bytes at voffset + soffset
// land at LDS address lds + 16 L. The buffer range check covers the sum of
// both offsets: bytes at or past num_records read as zeros.
__device__ __forceinline__ void dma_tile16(i32x4 rsrc, uint32_t lds, uint32_t voffset,
                                           uint32_t soffset) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds)
               : "memory");
}
// global_load_lds_dword: lane L's 4 bytes at base + voffset land at lds + 4 L.
__device__ __forceinline__ void dma_dword(const int* base, uint32_t lds, uint32_t voffset) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voffset), "s"(base), "{m0}"(lds)
               : "memory");
}

// A pointer that is the same in every lane, stated as such (so that loads
// through it are scalar and descriptors built from it are SGPRs).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// x as an SGPR value the compiler cannot see through: computations that
// depend on it stay where they are written (they are not hoisted out of
// loops and kept live in scalar registers).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

}  // namespace hw
}  // namespace fa
