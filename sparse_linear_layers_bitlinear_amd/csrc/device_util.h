// Device helpers used by several kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
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

// Wave-wide sum of a uint32 (64 lanes, modulo 2^32).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
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


// Per-token activation scale (absmax quantizer): from the bit pattern of the
// row's largest |x| (fp32), the quantizer multiplies by q = 127 / (max + eps)
// and the dequantizer uses s = (max + eps) / 127, both in IEEE fp32.
struct ActScale {
  float q, s;
};
__device__ __forceinline__ ActScale act_scale(uint32_t max_bits, float eps) {
  const float d = __uint_as_float(max_bits) + eps;
  return ActScale{127.0f / d, d / 127.0f};
}

// One activation code: f * q rounded to the nearest integer, ties to even,
// clipped to [-128, 127]. The rounding is read off the bit pattern of
// f * q + 1.5 * 2^23 (unit in the last place 1 there), whose low byte is the
// two's-complement code. The clip never acts: q = fp32(127 / d) with d >= max|x|,
// so |f * q| <= 127 * (1 + 2^-23) and the rounded value lies in [-127, 127].
// (A row of zeros with a scale that overflowed gives 0 * inf = NaN, whose low
// byte is 0: zeros quantize to zeros for any eps.) Returns the code in bits 7:0.
__device__ __forceinline__ uint32_t act_code_bits(float f, float q) {
  return __float_as_uint(f * q + 12582912.0f);
}
__device__ __forceinline__ int act_code(float f, float q) {
  return (int)(int8_t)(act_code_bits(f, q) & 0xFFu);
}

// bytes 7:0 of a, b, c, d -> one little-endian word {a, b, c, d}
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

// max |x| of one 16-byte vector, as an fp32 bit pattern (|x| compared as
// uint32, exact for non-negative floats; bf16 values widen exactly).
template <bool BF16>
__device__ __forceinline__ uint32_t absmax_vec(const uint4& d) {
  if constexpr (BF16) {
    const uint32_t m = 0x7FFF7FFFu;
    const uint32_t a = d.x & m, b = d.y & m, c = d.z & m, e = d.w & m;
    const uint32_t lo = max(max(a & 0xFFFFu, b & 0xFFFFu), max(c & 0xFFFFu, e & 0xFFFFu));
    const uint32_t hi = max(max(a >> 16, b >> 16), max(c >> 16, e >> 16));
    return max(lo, hi) << 16;
  } else {
    return max(max(d.x & 0x7FFFFFFFu, d.y & 0x7FFFFFFFu), max(d.z & 0x7FFFFFFFu, d.w & 0x7FFFFFFFu));
  }
}

// 16 bytes of activations (8 bf16 or 4 fp32) -> their codes, packed little-endian.
template <bool BF16>
__device__ __forceinline__ uint2 act_codes_vec(const uint4& d, float q) {
  if constexpr (BF16) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
    uint32_t c[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      c[2 * h] = act_code_bits(__uint_as_float(w[h] << 16), q);
      c[2 * h + 1] = act_code_bits(__uint_as_float(w[h] & 0xFFFF0000u), q);
    }
    return make_uint2(pack_low_bytes(c[0], c[1], c[2], c[3]), pack_low_bytes(c[4], c[5], c[6], c[7]));
  } else {
    return make_uint2(pack_low_bytes(act_code_bits(__uint_as_float(d.x), q),
                                     act_code_bits(__uint_as_float(d.y), q),
                                     act_code_bits(__uint_as_float(d.z), q),
                                     act_code_bits(__uint_as_float(d.w), q)), 0u);
  }
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + 2 GiB - 1): loads take a per-lane
// 32-bit offset plus a wave-uniform scalar offset, so address arithmetic
// costs no VALU. Offsets are always in bounds by construction (callers keep
// every buffer below 2^31 bytes; no reliance on the hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF,
                                           0x00020000);
}

// Epilogue of one 16x16 tile slice held by a lane: outputs o..o+3 of token t.
// y = fp32(fp32(acc * sx[t]) * sw[o]), rounded to bf16 (RNE) or kept fp32.
template <bool YBF16>
__device__ __forceinline__ void store_tile(void* __restrict__ y, int32_t* __restrict__ acc_out,
                                           const v4i& c, int t, int o, int O, float s_t,
                                           const float* __restrict__ sw, int sw_inc) {
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = (float)c[r] * s_t;
    v[r] = a * sw[min(o + r, O - 1) * sw_inc];
  }
  const int64_t base = (int64_t)t * O + o;
  if (o + 3 < O && (O & 3) == 0) {
    if constexpr (YBF16) {
      const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *(uint2*)((uint16_t*)y + base) = make_uint2(lo, hi);
    } else {
      *(float4*)((float*)y + base) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (acc_out) *(int4*)(acc_out + base) = make_int4(c[0], c[1], c[2], c[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (o + r >= O) break;
      if constexpr (YBF16) ((uint16_t*)y)[base + r] = (uint16_t)f32_to_bf16_bits(v[r]);
      else ((float*)y)[base + r] = v[r];
      if (acc_out) acc_out[base + r] = c[r];
    }
  }
}

// store_tile with the four weight scales of rows o..o+3 already in registers
// (sw[r] for row min(o + r, O - 1)).
template <bool YBF16>
__device__ __forceinline__ void store_tile_sw(void* __restrict__ y, int32_t* __restrict__ acc_out,
                                           const v4i& c, int t, int o, int O, float s_t,
                                           const float (&sw)[4]) {
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = (float)c[r] * s_t;
    v[r] = a * sw[r];
  }
  const int64_t base = (int64_t)t * O + o;
  if (o + 3 < O && (O & 3) == 0) {
    if constexpr (YBF16) {
      const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *(uint2*)((uint16_t*)y + base) = make_uint2(lo, hi);
    } else {
      *(float4*)((float*)y + base) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (acc_out) *(int4*)(acc_out + base) = make_int4(c[0], c[1], c[2], c[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (o + r >= O) break;
      if constexpr (YBF16) ((uint16_t*)y)[base + r] = (uint16_t)f32_to_bf16_bits(v[r]);
      else ((float*)y)[base + r] = v[r];
      if (acc_out) acc_out[base + r] = c[r];
    }
  }
}

}  // namespace sbl
