// Exact, order-free sums of non-negative fp32 values, correctly rounded to
// fp64 once at the end. Used where a floating-point sum decides integers
// later on (the absmean scale gamma decides every ternary code; the RMS of a
// token decides its activation codes), so the result must not depend on how
// the work is split over threads, workgroups or launches.
//
// A finite non-negative fp32 value with bit pattern u is m * 2^(e' - 150),
// where e' = max(e, 1) for the biased exponent e and m is the 24-bit
// significand (hidden bit included for normals). With tag = e' >> 5 (0..7)
// and sh = e' & 31, the value is (m << sh) * 2^(32 tag - 150) and m << sh <
// 2^55. A sum is kept as 16 unsigned 64-bit "bins": bins[2 tag] and
// bins[2 tag + 1] hold the low and high 32-bit-aligned parts of the integer
// sum of window `tag` (value = (bins[2 tag] + bins[2 tag + 1] * 2^32) *
// 2^(32 tag - 150)), so that adding 32-bit pieces of up to 2^31 terms can
// never overflow a bin.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbl {

// (a2:a1:a0) += v, a 96-bit unsigned accumulator in three registers
__device__ __forceinline__ void add96(uint32_t& a0, uint32_t& a1, uint32_t& a2, uint64_t v) {
  uint64_t lo = (uint64_t)a0 + (uint32_t)v;
  uint64_t mid = (uint64_t)a1 + (uint32_t)(v >> 32) + (lo >> 32);
  a0 = (uint32_t)lo;
  a1 = (uint32_t)mid;
  a2 += (uint32_t)(mid >> 32);
}

// Window and integer term of a non-negative finite fp32 bit pattern u (sign
// bit clear): tag = e' >> 5 and v = m << (e' & 31). Zero gives v = 0.
__device__ __forceinline__ void exact_term(uint32_t u, uint32_t& tag, uint64_t& v) {
  const uint32_t ee = max(u >> 23, 1u);
  const uint32_t m = u - ((ee - 1u) << 23);
  tag = ee >> 5;
  v = (uint64_t)m << (ee & 31u);
}

// The 16 bins of an exact sum -> that sum rounded to the nearest fp64 (ties
// to even). Registers only (constant indices); bins may live in LDS or in a
// local array.
__device__ inline double exact_bins_to_f64(const unsigned long long* bins) {
  // exact sum in units of 2^-150 as 32-bit limbs
  constexpr int NL = 12;
  uint32_t L[NL];
  {
    unsigned long long w[NL + 1];
#pragma unroll
    for (int i = 0; i <= NL; ++i) w[i] = 0;
#pragma unroll
    for (int tag = 0; tag < 8; ++tag) {
      const unsigned long long lo = bins[2 * tag], hi = bins[2 * tag + 1];
      w[tag] += lo & 0xFFFFFFFFull;
      w[tag + 1] += (lo >> 32) + (hi & 0xFFFFFFFFull);
      w[tag + 2] += hi >> 32;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      w[i + 1] += w[i] >> 32;
      L[i] = (uint32_t)w[i];
    }
  }
  int top = -1;
#pragma unroll
  for (int i = 0; i < NL; ++i)
    if (L[i]) top = i;
  if (top < 0) return 0.0;
  // 96-bit window of the three highest limbs, plus a sticky bit for the rest
  uint32_t h = 0, m = 0, l = 0;
  bool below = false;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (i == top) h = L[i];
    if (i == top - 1) m = L[i];
    if (i == top - 2) l = L[i];
    if (i < top - 2 && L[i]) below = true;
  }
  const int c = __clz(h);                               // h != 0
  unsigned __int128 V = ((unsigned __int128)h << 64) | ((unsigned __int128)m << 32) | l;
  V <<= c;                                              // bit 95 set
  unsigned long long mant = (unsigned long long)(V >> 43) & ((1ull << 53) - 1);
  const bool rb = (V >> 42) & 1;
  const bool sticky = below || ((V & (((unsigned __int128)1 << 42) - 1)) != 0);
  if (rb && (sticky || (mant & 1ull))) ++mant;          // nearest, ties to even
  // value = V_window * 2^(32*(top-2)) * 2^-150, V_window = mant * 2^(43 - c)
  return ldexp((double)mant, 43 - c + 32 * (top - 2) - 150);
}

}  // namespace sbl
