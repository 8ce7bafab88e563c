// Device helpers used by several kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Bit position of two-bit field u (0..15) in a byte-sliced word.
__host__ __device__ constexpr int field_shift(int u) { return 8 * (u & 3) + 2 * (u >> 2); }

// Byte-sliced code word -> four int8 values (fields 4j..4j+3), one v_perm:
// selector bytes are the 2-bit codes, the pool maps 0->0x00, 1->0x01, 3->0xFF.
__device__ __forceinline__ uint32_t expand_codes(uint32_t word, int j) {
  const uint32_t sel = (word >> (2 * j)) & 0x03030303u;
  return __builtin_amdgcn_perm(0u, 0xFF000100u, sel);
}

// Wave-wide max of a uint32 (64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Wave-wide sum of a uint64 (64 lanes, modulo 2^64).
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
    v += ((unsigned long long)hi << 32) | lo;
  }
  return v;
}

}  // namespace sbl
