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
#include "device_util.h"
#include "exact_sum.h"

namespace sbl {

constexpr int kActRowsPerBlock = 4;  // 4 wavefronts, one row each

// codes of one 16-byte input vector: 8 bytes (bf16) or 4 bytes (fp32)
template <bool BF16>
__device__ __forceinline__ void store_codes(const uint2& c, int8_t* q) {
  if constexpr (BF16) *(uint2*)q = c;
  else *(uint32_t*)q = c.x;
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

  const ActScale sc = act_scale(mx, eps);
  if (lane == 0) sx[t] = sc.s;

#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    if (i < nvec) store_codes<BF16>(act_codes_vec<BF16>(d[u], sc.q), qrow + i * V);
  }
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64)
    store_codes<BF16>(act_codes_vec<BF16>(row[i], sc.q), qrow + i * V);
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
  const ActScale sc = act_scale(mx, eps);
  if (lane == 0) sx[t] = sc.s;
  for (int64_t i = lane; i < K; i += 64) {
    const float f = BF16 ? bf16_bits_to_f32(xb[i]) : xf[i];
    qrow[i] = (int8_t)act_code(f, sc.q);
  }
}

// ---------------------------------------------------------------------------
// RMS normalization fused into the quantizer: x~ = Q_a(Norm(x)).
// Sparse-BitNet summary, section 3.4 (Algorithm 1 walk-through: the input is
// normalized, RMSNorm in the BitNet architecture, then quantized); BitNet
// b1.58 2B4T summary, section 3.2 (subln normalization, no bias terms).
// The pages fix no arithmetic; this kernel computes, per row:
//   sq_k = fp32(x_k * x_k),
//   S = sum_k sq_k, exactly, rounded once to the nearest fp64 -- the result
//       does not depend on the order of the terms (see exact_sum.h),
//   r = fp32(1 / sqrt(S / K + eps_n))   (fp64 division, square root, division)
//   z_k = fp32(fp32(x_k * r) * g_k)     (without g: z_k = fp32(x_k * r))
// and then exactly the quantizer above on z. x is read once (plus g, which
// stays in L2) and only the int8 codes are written: the HBM round trip of a
// separate normalized tensor is gone.
//
// The exact sum: every lane marks the 32-binade windows its squares fall in;
// for each window present in the row (a wave-uniform loop, usually two or
// three windows) every lane adds its squares of that window as integers into
// a 96-bit register accumulator, the wave sums the accumulators exactly, and
// the row's 16 window bins are turned into the fp64 S.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void unpack_f32(const uint4& d, float* f) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  if constexpr (BF16) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f[2 * h] = __uint_as_float(w[h] << 16);
      f[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) f[h] = __uint_as_float(w[h]);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_rmsnorm_quant_act(const void* __restrict__ xv,
                                                           const float* __restrict__ gain,
                                                           int64_t T, int64_t K, int64_t ldx,
                                                           float eps_n, float eps,
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
#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    d[u] = i < nvec ? row[i] : make_uint4(0, 0, 0, 0);   // zeros add +0 to S
  }
  // square of element e of a vector, as a sign-free fp32 bit pattern
  auto sq_bits = [&](const uint4& v, int e) -> uint32_t {
    float f[V];
    unpack_f32<BF16>(v, f);
    const float p = f[e] * f[e];
    return __float_as_uint(p);
  };
  // windows holding a nonzero square (per lane, then over the wave)
  uint32_t tags = 0;
  auto mark = [&](const uint4& v) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      uint32_t tg;
      uint64_t tv;
      exact_term(sq_bits(v, e), tg, tv);
      tags |= (tv != 0 ? 1u : 0u) << tg;
    }
  };
#pragma unroll
  for (int u = 0; u < kActCache; ++u) mark(d[u]);
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) mark(row[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tags |= (uint32_t)__shfl_xor((int)tags, off, 64);
  tags = __builtin_amdgcn_readfirstlane(tags);
  unsigned long long bins[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) bins[j] = 0;
  while (tags) {                                         // (wave-uniform)
    const uint32_t tw = 31u - __clz(tags);
    tags &= ~(1u << tw);
    uint32_t a0 = 0, a1 = 0, a2 = 0;
    auto add = [&](const uint4& v) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        uint32_t tg;
        uint64_t tv;
        exact_term(sq_bits(v, e), tg, tv);
        add96(a0, a1, a2, tg == tw ? tv : 0ull);
      }
    };
#pragma unroll
    for (int u = 0; u < kActCache; ++u) add(d[u]);
    for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) add(row[i]);
    const unsigned long long lo = wave_sum_u64(a0);
    const unsigned long long hi = wave_sum_u64((unsigned long long)a1 | ((unsigned long long)a2 << 32));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == (int)tw) {
        bins[2 * j] = lo;
        bins[2 * j + 1] = hi;
      }
  }
  const double S = exact_bins_to_f64(bins);
  const float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));

  // z of vector i (V values)
  auto norm = [&](const uint4& v, int64_t i, float* z) {
    unpack_f32<BF16>(v, z);
#pragma unroll
    for (int e = 0; e < V; ++e) z[e] = z[e] * r;
    if (gain) {
#pragma unroll
      for (int e4 = 0; e4 < V; e4 += 4) {
        const float4 g4 = *(const float4*)(gain + i * V + e4);
        z[e4] = z[e4] * g4.x;
        z[e4 + 1] = z[e4 + 1] * g4.y;
        z[e4 + 2] = z[e4 + 2] * g4.z;
        z[e4 + 3] = z[e4 + 3] * g4.w;
      }
    }
  };
  uint32_t mx = 0;
  float z[V];
#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    if (i < nvec) {
      norm(d[u], i, z);
#pragma unroll
      for (int e = 0; e < V; ++e) mx = max(mx, __float_as_uint(z[e]) & 0x7FFFFFFFu);
    }
  }
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) {
    norm(row[i], i, z);
#pragma unroll
    for (int e = 0; e < V; ++e) mx = max(mx, __float_as_uint(z[e]) & 0x7FFFFFFFu);
  }
  mx = wave_max_u32(mx);
  const ActScale sc = act_scale(mx, eps);
  if (lane == 0) sx[t] = sc.s;
  auto put = [&](int64_t i, const float* zz) {
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < V; ++e) c[e] = act_code_bits(zz[e], sc.q);
    if constexpr (BF16)
      *(uint2*)(qrow + i * V) = make_uint2(pack_low_bytes(c[0], c[1], c[2], c[3]),
                                           pack_low_bytes(c[4], c[5], c[6], c[7]));
    else
      *(uint32_t*)(qrow + i * V) = pack_low_bytes(c[0], c[1], c[2], c[3]);
  };
#pragma unroll
  for (int u = 0; u < kActCache; ++u) {
    const int64_t i = lane + 64 * u;
    if (i < nvec) {
      norm(d[u], i, z);
      put(i, z);
    }
  }
  for (int64_t i = lane + 64 * kActCache; i < nvec; i += 64) {
    norm(row[i], i, z);
    put(i, z);
  }
}

hipError_t launch_rmsnorm_quant_act(const void* x, bool bf16, const float* gain, int64_t T,
                                    int64_t K, int64_t ldx, float eps_n, float eps, int8_t* xq,
                                    float* sx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(T, kActRowsPerBlock)), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_rmsnorm_quant_act<true>, grid, block, 0, s, x, gain, T, K, ldx, eps_n,
                       eps, xq, sx);
  else
    hipLaunchKernelGGL(k_rmsnorm_quant_act<false>, grid, block, 0, s, x, gain, T, K, ldx, eps_n,
                       eps, xq, sx);
  return hipGetLastError();
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
