// Building blocks of the grouped-GEMM kernels on gfx950: LDS-DMA operand
// loads (buffer_load ... lds), the XOR swizzle of 128-byte LDS rows, and
// explicit vmcnt waits.
//
// A 16-byte LDS-DMA load writes lane l's 16 bytes at LDS address
// M0 + 16 * l, so one wave instruction fills 1 KiB = 8 rows of 128 bytes.
// Lane l serves row l / 8 and physical 16-byte chunk l % 8 of that row; the
// swizzle decides which logical K chunk it fetches from global memory.
//
// The loads are issued through inline asm: the compiler does not see them,
// so it does not force vmcnt(0) before every LDS read (it must assume an
// LDS-DMA may alias any LDS access). The kernels wait with explicit vmcnt
// counts instead. The compiler's own waits for its loads stay correct
// because vmcnt only over-counts the extra loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mok {

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef short i16x8v __attribute__((vector_size(16)));

// Physical chunk = logical chunk ^ swz(row). 16-byte reads of 16
// consecutive rows at one logical chunk hit 16 distinct 16-byte bank groups
// with 64 banks, and 8 consecutive rows hit 8 distinct groups with 32.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row & 1) << 2)) & 7; }

// LDS byte address of a shared-memory object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Raw buffer resource (stride 0) in SGPRs: loads at offsets >= bytes return 0.
__device__ __forceinline__ i32x4v rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  i32x4v r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// The resource as SGPR operands (wave-uniform by construction).
__device__ __forceinline__ i32x4v sgpr(i32x4v r) {
  return i32x4v{__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}

// 16 bytes per lane from buffer offset voff + soff into LDS at m0 + 16 * lane.
__device__ __forceinline__ void lds_dma16(i32x4v rs, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(sgpr(rs)), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory", "m0");
}

// 4 bytes per lane into LDS at m0 + 4 * lane (the MXFP8 block-scale dword
// of one row per lane).
__device__ __forceinline__ void lds_dma4(i32x4v rs, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(sgpr(rs)), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace mok
