// Building blocks of the persistent producer/consumer GEMM kernels: global ->
// LDS copies, explicit memory-counter waits, the workgroup barrier without a
// memory fence, and scalar-cache reads of small uniform data.
//
// Copies (global_load_lds) are issued from inline assembly so that the
// compiler does not add its own waits on them: each copying wave tracks its
// copies with explicit vmcnt waits, and a workgroup barrier then publishes the
// landed stage to the consuming waves.  A wave's vmcnt drains in issue order,
// so every wave keeps a single stream of copies with a fixed count per stage.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe_mx {

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (gfx9 encoding; expcnt left at its maximum).
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Asynchronous copies global -> LDS (global_load_lds): lane i of the wave writes
// its `size` bytes at lds + size*i; `lds` is a wave-uniform LDS byte address.
// M0 carries the LDS address; one wait state separates its write from the copy.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}

// The same copies from a wave-uniform base (scalar registers) plus a 32-bit
// per-lane byte offset: no 64-bit per-lane address.
__device__ __forceinline__ void lds_copy16_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void lds_copy4_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(base) : "memory");
}

// Workgroup barrier with no memory fence (the waits above do the ordering).
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Tile-list entry through the scalar cache: a scalar load counts on lgkmcnt,
// not on the vector memory counter that tracks the copies in flight, so
// reading the next item's geometry never waits for them.  The load and its
// wait sit in one asm block.
__device__ __forceinline__ Tile load_tile(const Tile* tiles, int ti) {
  const Tile* ptr = tiles + __builtin_amdgcn_readfirstlane(ti);
  int4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  Tile t;
  t.expert = v.x;
  t.p0 = v.y;
  t.rows = v.z;
  t.pad = v.w;
  return t;
}

// 16 consecutive dwords at a wave-uniform, 4-byte aligned address, through the
// scalar cache (load and wait in one asm block).
struct Dw16 {
  int v[16];
};
__device__ __forceinline__ Dw16 load_dw16(const void* p) {
  typedef int i16v __attribute__((ext_vector_type(16)));
  i16v r;
  asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
  Dw16 d;
#pragma unroll
  for (int i = 0; i < 16; ++i) d.v[i] = r[i];
  return d;
}

}  // namespace moe_mx
