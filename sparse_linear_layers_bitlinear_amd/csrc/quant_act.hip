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

constexpr int kActRowsPerBlock = 4;

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
// The exact sum, fast case: a square of a bf16 value has at most 16
// significant bits (fp32 input: 24), so the squares whose exponents lie in a
// window of W binades are integer multiples of the window's lowest unit, and
// a sum of at most K of them stays below K * 2^(W - 1 + SB) of that unit.
// With W = 54 - SB - ceil(log2 K) every partial sum is an integer below 2^53
// units: fp64 accumulation of the window's squares is exact in any order.
// A first pass finds the largest square; if every nonzero square is normal
// and lies in the two windows below the largest, each window is summed in
// fp64 (per lane, then over the wave) and the two exact sums are added once:
// one IEEE addition, so S is the exact sum rounded once to the nearest fp64.
// Other rows (squares spread over more binades, subnormal squares, overflow)
// take the general sum: every lane marks the 32-binade windows its squares
// fall in; for each window present in the row (a wave-uniform loop) every
// lane adds its squares of that window as integers into a 96-bit register
// accumulator, the wave sums the accumulators exactly, and the row's 16
// window bins are turned into the fp64 S. That path re-reads the row from
// L2 so that it holds few registers.
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

// The fused kernel keeps 8 vectors per lane in registers (with 16 its four
// passes need more than 256 registers) and re-reads the rest of a row from L2
// in batches of kRmsBatch loads issued together.
constexpr int kRmsCache = 8;
constexpr int kRmsBatch = 8;

// fp64 sum over the wave (any order: the callers' terms sum exactly)
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v < o ? v : o;
  }
  return v;
}

// the general exact sum of fp32(x * x) over a row (see above)
template <bool BF16>
__device__ __attribute__((noinline)) double row_square_sum_windows(const uint4* __restrict__ row,
                                                                   int64_t nvec, int lane) {
  constexpr int V = BF16 ? 8 : 4;
  uint32_t tags = 0;
#pragma unroll 1
  for (int64_t i = lane; i < nvec; i += 64) {
    float f[V];
    unpack_f32<BF16>(row[i], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      uint32_t tg;
      uint64_t tv;
      exact_term(__float_as_uint(f[e] * f[e]), tg, tv);
      tags |= (tv != 0 ? 1u : 0u) << tg;
    }
  }
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
#pragma unroll 1
    for (int64_t i = lane; i < nvec; i += 64) {
      float f[V];
      unpack_f32<BF16>(row[i], f);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        uint32_t tg;
        uint64_t tv;
        exact_term(__float_as_uint(f[e] * f[e]), tg, tv);
        add96(a0, a1, a2, tg == tw ? tv : 0ull);
      }
    }
    const unsigned long long lo = wave_sum_u64(a0);
    const unsigned long long hi = wave_sum_u64((unsigned long long)a1 | ((unsigned long long)a2 << 32));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == (int)tw) {
        bins[2 * j] = lo;
        bins[2 * j + 1] = hi;
      }
  }
  return exact_bins_to_f64(bins);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_rmsnorm_quant_act(const void* __restrict__ xv,
                                                           const float* __restrict__ gain,
                                                           int64_t T, int64_t K, int64_t ldx,
                                                           float eps_n, float eps,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ sx, int stage) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];   // the gain, when staged
  constexpr int V = BF16 ? 8 : 4;
  constexpr int SB = BF16 ? 16 : 24;                    // significant bits of a square
  const int lane = threadIdx.x & 63;
  const int64_t tw = (int64_t)blockIdx.x * kActRowsPerBlock + (threadIdx.x >> 6);
  // a wave past the last row computes row T - 1 again and stores nothing (every
  // wave takes part in the barrier that publishes the staged gain)
  const bool own = tw < T;
  const int64_t t = own ? tw : T - 1;
  const int64_t nvec = K / V;
  const uint4* row = (const uint4*)((const char*)xv + t * ldx * (BF16 ? 2 : 4));
  int8_t* qrow = xq + t * K;

  uint4 d[kRmsCache];
#pragma unroll
  for (int u = 0; u < kRmsCache; ++u) {
    const int64_t i = lane + 64 * u;
    d[u] = i < nvec ? row[i] : make_uint4(0, 0, 0, 0);   // zero squares change nothing
  }
  // the gain into LDS by DMA (one instruction: 64 float4), read by the last two passes
  if (stage) {
    const int wave = threadIdx.x >> 6;
    const int64_t nq = K / 4;
    for (int64_t c = wave; 64 * c < nq; c += kActRowsPerBlock)
      if (64 * c + lane < nq)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(gain + 4 * (64 * c + lane)),
            (__attribute__((address_space(3))) void*)(gsm + 256 * c), 16, 0, 0);
  }
  // f(v, i) for the vectors past the register cache, kRmsBatch loads in flight
  auto tail = [&](auto&& f) {
    for (int64_t i0 = lane + 64 * kRmsCache; i0 < nvec; i0 += 64 * kRmsBatch) {
      uint4 w[kRmsBatch];
#pragma unroll
      for (int b = 0; b < kRmsBatch; ++b) {
        const int64_t i = i0 + 64 * b;
        w[b] = i < nvec ? row[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < kRmsBatch; ++b)
        if (i0 + 64 * b < nvec) f(w[b], i0 + 64 * b);
    }
  };
  // largest square and smallest nonzero square (bit patterns of non-negative
  // floats order as their values)
  uint32_t smax = 0, smin = 0xFFFFFFFFu;
  auto range = [&](const uint4& v) {
    float f[V];
    unpack_f32<BF16>(v, f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const uint32_t b = __float_as_uint(f[e] * f[e]);
      smax = max(smax, b);
      smin = min(smin, b != 0 ? b : 0xFFFFFFFFu);
    }
  };
#pragma unroll
  for (int u = 0; u < kRmsCache; ++u) range(d[u]);
  tail([&](const uint4& v, int64_t) { range(v); });
  smax = __builtin_amdgcn_readfirstlane(wave_max_u32(smax));
  smin = __builtin_amdgcn_readfirstlane(wave_min_u32(smin));
  int lk = 0;                                            // ceil(log2 K)
  while ((int64_t)1 << lk < K) ++lk;
  const int W = 54 - SB - lk;                            // window width (binades)
  const int emax = (int)(smax >> 23), emin = (int)(smin >> 23);
  double S;
  if (smax == 0) {
    S = 0.0;
  } else if (smax < 0x7F800000u && emin >= 1 && W >= 1 && emax - emin < 2 * W) {
    // squares at or above 2^(emax - W + 1) (biased exponents) in one window,
    // the rest in the window below
    const uint32_t split = (uint32_t)(emax - W + 1) << 23;
    double shi = 0.0, slo = 0.0;
    auto acc = [&](const uint4& v) {
      float f[V];
      unpack_f32<BF16>(v, f);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float p = f[e] * f[e];
        const double dp = (double)p;
        if (__float_as_uint(p) >= split) shi += dp;
        else slo += dp;
      }
    };
#pragma unroll
    for (int u = 0; u < kRmsCache; ++u) acc(d[u]);
    tail([&](const uint4& v, int64_t) { acc(v); });
    S = wave_sum_f64(shi) + wave_sum_f64(slo);
  } else {
    S = row_square_sum_windows<BF16>(row, nvec, lane);
  }
  const float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));

  if (stage) {
    __builtin_amdgcn_s_waitcnt(0);                       // this wave's gain copies landed ...
    __syncthreads();                                     // ... and every wave's
  }

  // the absmax of z and the codes, with the gain read through gp (LDS when
  // staged, else global memory)
  auto finish = [&](const float* __restrict__ gp) {
    // z of vector i (V values)
    auto norm = [&](const uint4& v, int64_t i, float* z) {
      unpack_f32<BF16>(v, z);
#pragma unroll
      for (int e = 0; e < V; ++e) z[e] = z[e] * r;
      if (gp) {
#pragma unroll
        for (int e4 = 0; e4 < V; e4 += 4) {
          const float4 g4 = *(const float4*)(gp + i * V + e4);
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
    for (int u = 0; u < kRmsCache; ++u) {
      const int64_t i = lane + 64 * u;
      if (i < nvec) {
        norm(d[u], i, z);
#pragma unroll
        for (int e = 0; e < V; ++e) mx = max(mx, __float_as_uint(z[e]) & 0x7FFFFFFFu);
      }
    }
    tail([&](const uint4& v, int64_t i) {
      norm(v, i, z);
#pragma unroll
      for (int e = 0; e < V; ++e) mx = max(mx, __float_as_uint(z[e]) & 0x7FFFFFFFu);
    });
    mx = wave_max_u32(mx);
    const ActScale sc = act_scale(mx, eps);
    if (!own) return;                                    // (wave-uniform)
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
    for (int u = 0; u < kRmsCache; ++u) {
      const int64_t i = lane + 64 * u;
      if (i < nvec) {
        norm(d[u], i, z);
        put(i, z);
      }
    }
    tail([&](const uint4& v, int64_t i) {
      norm(v, i, z);
      put(i, z);
    });
  };
  if (stage) finish(gsm);
  else finish(gain);
}

hipError_t launch_rmsnorm_quant_act(const void* x, bool bf16, const float* gain, int64_t T,
                                    int64_t K, int64_t ldx, float eps_n, float eps, int8_t* xq,
                                    float* sx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(T, kActRowsPerBlock)), block(256);
  // the gain goes through LDS for rows of 4096 to 16384 values (one copy per
  // block of four rows instead of two reads from L2 per row: Qwen2.5-3B down
  // input, K = 11008, 151 -> 135 us; on 2048-value rows the copy and its
  // barrier cost more than they save, 34 -> 38 us)
  const int stage = gain != nullptr && K >= 4096 && K * 4 <= 65536 ? 1 : 0;
  const size_t lds = stage ? (size_t)K * 4 : 0;
  if (bf16)
    hipLaunchKernelGGL(k_rmsnorm_quant_act<true>, grid, block, lds, s, x, gain, T, K, ldx, eps_n,
                       eps, xq, sx, stage);
  else
    hipLaunchKernelGGL(k_rmsnorm_quant_act<false>, grid, block, lds, s, x, gain, T, K, ldx, eps_n,
                       eps, xq, sx, stage);
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
