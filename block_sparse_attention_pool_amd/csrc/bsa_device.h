// Device-side helpers shared by the gfx950 kernels: vector types for the
// matrix-core builtins, bf16 <-> f32 conversion and wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;  // macro block (tokens)
constexpr int kMicro = 16;  // micro tile (tokens)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round-to-nearest-even float -> bf16 bits (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> packed bf16x2 (low half = a), one round-to-nearest-even
// conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Two floats -> packed fp16x2 (low half = a), round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// bf16 bits -> fp16 bits.  Exact for |x| in [2^-14, 65504]; smaller
// magnitudes round to fp16 subnormals (absolute error <= 2^-25).
__device__ __forceinline__ uint32_t bf16_bits_to_f16_bits(uint32_t h) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(h));
}

// Staged V^T: position p (0..15) inside a 16-key chunk holds key
// 8*((p%8)/4) + 4*(p/8) + (p%4): lane group g = p/8, slot j = p%8 of the
// 32x32x16 operand maps to key 8*(j/4) + 4*g + j%4, which is the key order
// of the 32x32 accumulator rows the lane holds.
__device__ __forceinline__ int vt_key_of_pos(int p) {
  return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}

// Monotone map of a float to uint32: a < b  <=>  key(a) < key(b), and
// a == b  <=>  key(a) == key(b): adding +0 turns -0 into +0, so the two
// zeros (equal values) get one key and tie like any other equal scores.
__device__ __forceinline__ uint32_t float_order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

}  // namespace bsa
