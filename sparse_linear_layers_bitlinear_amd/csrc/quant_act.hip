// a1: per-token absmax int8 activation quantization.
//
// Sparse-BitNet summary, section 3.4 "Activation quantization":
// x~ = Clip(x * 127 / (max|x| + eps), -128, 127); BitNet b1.58 2B4T summary,
// section 3.4 "Activation Quantization: Per-Token Absmax": one scale per
// token, nearest-integer rounding.
//
// One wavefront owns one token row. It issues all 16-byte loads of the row at
// once (rows of up to 8192 bf16 / 4096 fp32 values stay in registers), reduces
// max|x| across the wave (|x| compared as uint32 bit patterns, exact for
// non-negative floats) and writes the int8 codes from registers; longer rows
// re-read their tail from L2. HBM traffic is the algorithmic 3 bytes/element
// (bf16) + 4 bytes/token.
#include "sbl_internal.h"
#include "device_util.cuh"

namespace sbl {

constexpr int kActRowsPerBlock = 4;  // 4 wavefronts, one row each

// Quantize V values with scale s and store them as V int8 at q.
template <int V>
__device__ __forceinline__ void quant_store(const float* f, float s, int8_t* q) {
  uint32_t packed[V / 4];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    float v = rintf(f[e] * s);
    v = fminf(fmaxf(v, -128.0f), 127.0f);
    const uint32_t b = (uint32_t)((int)v) & 0xFFu;
    if (e % 4 == 0) packed[e / 4] = b; else packed[e / 4] |= b << (8 * (e % 4));
  }
  if constexpr (V == 8) *(uint2*)q = make_uint2(packed[0], packed[1]);
  else *(uint32_t*)q = packed[0];
}

template <bool BF16>
__device__ __forceinline__ void unpack_vec(const uint4& d, float* f) {
  if constexpr (BF16) {
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f[2 * h] = bf16_bits_to_f32(w[h] & 0xFFFFu);
      f[2 * h + 1] = bf16_bits_to_f32(w[h] >> 16);
    }
  } else {
    f[0] = __uint_as_float(d.x); f[1] = __uint_as_float(d.y);
    f[2] = __uint_as_float(d.z); f[3] = __uint_as_float(d.w);
  }
}

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

// Vector path. Rows of up to 64 * kActCache vectors stay in registers: all
// loads are issued before the reduction, and the codes come from registers.
// Longer rows take a second pass (served from L2).
constexpr int kActCache = 16;

template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_act_vec(const void* __restrict__ xv, int64_t T,
                                                       int64_t K, int64_t ldx, float eps,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ sx) {
  constexpr int V = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kActRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t nvec = K / V;
  const uint4* row = (const uint4*)((const char*)xv + t * ldx * (BF16 ? 2 : 4));
  int8_t* qrow = xq + t * K;

  uint4 d[kActCache];
  uint32_t mx = 0;
#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    d[u] = i < nvec ? row[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kActCache; ++u) mx = max(mx, absmax_vec<BF16>(d[u]));
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) mx = max(mx, absmax_vec<BF16>(row[i]));
  mx = wave_max_u32(mx);

  // scale in IEEE fp32: d = m + eps, s = 127 / d
  const float dd = __uint_as_float(mx) + eps;
  const float s = 127.0f / dd;
  if (lane == 0) sx[t] = dd / 127.0f;

  float f[V];
#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    if (i < nvec) {
      unpack_vec<BF16>(d[u], f);
      quant_store<V>(f, s, qrow + i * V);
    }
  }
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) {
    unpack_vec<BF16>(row[i], f);
    quant_store<V>(f, s, qrow + i * V);
  }
}

// Scalar path for rows that are not 16-byte aligned or not whole vectors.
template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_act_scalar(const void* __restrict__ xv, int64_t T,
                                                          int64_t K, int64_t ldx, float eps,
                                                          int8_t* __restrict__ xq,
                                                          float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kActRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xb = BF16 ? (const uint16_t*)xv + t * ldx : nullptr;
  const float* xf = BF16 ? nullptr : (const float*)xv + t * ldx;
  int8_t* qrow = xq + t * K;
  uint32_t mx = 0;
  for (int64_t i = lane; i < K; i += 64) {
    const uint32_t u = BF16 ? ((uint32_t)xb[i] << 16) : __float_as_uint(xf[i]);
    mx = max(mx, u & 0x7FFFFFFFu);
  }
  mx = wave_max_u32(mx);
  const float dd = __uint_as_float(mx) + eps;
  const float s = 127.0f / dd;
  if (lane == 0) sx[t] = dd / 127.0f;
  for (int64_t i = lane; i < K; i += 64) {
    const float f = BF16 ? bf16_bits_to_f32(xb[i]) : xf[i];
    float v = rintf(f * s);
    v = fminf(fmaxf(v, -128.0f), 127.0f);
    qrow[i] = (int8_t)(int)v;
  }
}

hipError_t launch_quant_act(const void* x, bool bf16, int64_t T, int64_t K, int64_t ldx,
                            float eps, int8_t* xq, float* sx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int es = bf16 ? 2 : 4;
  const int V = bf16 ? 8 : 4;
  // 16-byte vectors need every row start aligned and whole vectors per row;
  // xq rows (K bytes) need K % 4 (fp32) or K % 8 (bf16) for the packed stores.
  const bool vec = ((ldx * es) % 16 == 0) && (K % V == 0);
  const dim3 grid((unsigned)cdiv(T, kActRowsPerBlock)), block(256);
  if (bf16) {
    if (vec) hipLaunchKernelGGL(k_quant_act_vec<true>, grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
    else hipLaunchKernelGGL(k_quant_act_scalar<true>, grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
  } else {
    if (vec) hipLaunchKernelGGL(k_quant_act_vec<false>, grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
    else hipLaunchKernelGGL(k_quant_act_scalar<false>, grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
  }
  return hipGetLastError();
}

}  // namespace sbl
