// a1: per-token absmax int8 activation quantization.
//
// Sparse-BitNet summary, section 3.4 "Activation quantization":
// x~ = Clip(x * 127 / (max|x| + eps), -128, 127); BitNet b1.58 2B4T summary,
// section 3.4 "Activation Quantization: Per-Token Absmax": one scale per
// token, nearest-integer rounding.
//
// One wavefront owns one token row. Pass 1 streams the row from HBM with
// 16-byte loads and reduces max|x| across the wave (|x| compared as uint32
// bit patterns, exact for non-negative floats). Pass 2 re-reads the row
// (served from L2: a row is at most a few tens of KB) and writes int8 codes.
// HBM traffic is the algorithmic 3 bytes/element (bf16) + 4 bytes/token.
#include "sbl_internal.h"
#include "device_util.cuh"

namespace sbl {

constexpr int kActRowsPerBlock = 4;  // 4 wavefronts, one row each

template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_quant_act(const void* __restrict__ xv, int64_t T,
                                                   int64_t K, int64_t ldx, float eps,
                                                   int8_t* __restrict__ xq,
                                                   float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kActRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  // elements per 16-byte vector
  constexpr int V = VEC ? (BF16 ? 8 : 4) : 1;
  const int64_t nvec = K / V;

  const uint16_t* xb = BF16 ? (const uint16_t*)xv + t * ldx : nullptr;
  const float* xf = BF16 ? nullptr : (const float*)xv + t * ldx;
  int8_t* qrow = xq + t * K;

  // ---- pass 1: max |x| ----
  uint32_t mx = 0;
  for (int64_t i = lane; i < nvec; i += 64) {
    if constexpr (VEC) {
      const uint4 d = BF16 ? *(const uint4*)(xb + i * V) : *(const uint4*)(xf + i * V);
      if constexpr (BF16) {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t lo = (w[h] & 0x7FFFu) << 16, hi = (w[h] >> 16 & 0x7FFFu) << 16;
          mx = max(mx, max(lo, hi));
        }
      } else {
        mx = max(mx, max(max(d.x & 0x7FFFFFFFu, d.y & 0x7FFFFFFFu),
                         max(d.z & 0x7FFFFFFFu, d.w & 0x7FFFFFFFu)));
      }
    } else {
      uint32_t u = BF16 ? ((uint32_t)xb[i] << 16) : __float_as_uint(xf[i]);
      mx = max(mx, u & 0x7FFFFFFFu);
    }
  }
  mx = wave_max_u32(mx);

  // scale in IEEE fp32: d = m + eps, s = 127 / d
  const float d = __uint_as_float(mx) + eps;
  const float s = 127.0f / d;
  if (lane == 0) sx[t] = d / 127.0f;

  // ---- pass 2: codes ----
  for (int64_t i = lane; i < nvec; i += 64) {
    if constexpr (VEC) {
      float f[V];
      if constexpr (BF16) {
        const uint4 dv = *(const uint4*)(xb + i * V);
        const uint32_t w[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          f[2 * h] = bf16_bits_to_f32(w[h] & 0xFFFFu);
          f[2 * h + 1] = bf16_bits_to_f32(w[h] >> 16);
        }
      } else {
        const float4 dv = *(const float4*)(xf + i * V);
        f[0] = dv.x; f[1] = dv.y; f[2] = dv.z; f[3] = dv.w;
      }
      uint32_t packed[V / 4];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float v = rintf(f[e] * s);
        v = fminf(fmaxf(v, -128.0f), 127.0f);
        const uint32_t b = (uint32_t)((int)v) & 0xFFu;
        if (e % 4 == 0) packed[e / 4] = b; else packed[e / 4] |= b << (8 * (e % 4));
      }
      if constexpr (V == 8) *(uint2*)(qrow + i * V) = make_uint2(packed[0], packed[1]);
      else *(uint32_t*)(qrow + i * V) = packed[0];
    } else {
      const float f = BF16 ? bf16_bits_to_f32(xb[i]) : xf[i];
      float v = rintf(f * s);
      v = fminf(fmaxf(v, -128.0f), 127.0f);
      qrow[i] = (int8_t)(int)v;
    }
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
    if (vec) hipLaunchKernelGGL((k_quant_act<true, true>), grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
    else hipLaunchKernelGGL((k_quant_act<true, false>), grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
  } else {
    if (vec) hipLaunchKernelGGL((k_quant_act<false, true>), grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
    else hipLaunchKernelGGL((k_quant_act<false, false>), grid, block, 0, s, x, T, K, ldx, eps, xq, sx);
  }
  return hipGetLastError();
}

}  // namespace sbl
