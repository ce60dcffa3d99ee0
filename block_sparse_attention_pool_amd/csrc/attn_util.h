// Device helpers shared by the attention kernels (block-sparse, dense,
// cluster-chunk and micro): output stores, LDS addresses, scalar index
// loads, compile-time loops and the direct global->LDS tile copy.
#pragma once

#include <type_traits>

#include "bsa_device.h"

namespace bsa {

template <bool OUT_BF16>
__device__ __forceinline__ void store4(void* O, int64_t off, float x0, float x1, float x2, float x3) {
  if constexpr (OUT_BF16) {
    const u32x2 v = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
    *(u32x2*)((uint16_t*)O + off) = v;
  } else {
    const f32x4 v = {x0, x1, x2, x3};
    *(f32x4*)((float*)O + off) = v;
  }
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u16*)p;
}

// Read-only index arrays in the constant address space: uniform loads of
// them become scalar loads.
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Compile-time loop: f(std::integral_constant<int, U>) for U in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One direct global->LDS copy of 16 bytes per lane: lane l's bytes from
// sbase + voff land at LDS byte (m0base + OFF) + 16*l.  Written as asm (no
// output registers; M0, SCC and memory declared clobbered) so that the
// compiler does not order later LDS reads behind it: completion is awaited
// explicitly with s_waitcnt vmcnt before the tile is read.
template <int OFF>
__device__ __forceinline__ void dma16(uint32_t m0base, const void* sbase, uint32_t voff) {
  asm volatile("s_add_u32 m0, %0, %3\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0base), "v"(voff), "s"(sbase), "i"(OFF)
               : "memory", "m0", "scc");
}

// A pointer whose value is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Sum of the two fp16 halves of a packed word added to acc (fp32).
__device__ __forceinline__ float add_f16x2(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace bsa
