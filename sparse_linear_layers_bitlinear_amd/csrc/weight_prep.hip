// a2-a4: absmean scale, N:M mask, RoundClip, mask application, packing.
//
// Sparse-BitNet summary, section 3.4: "Step 1: Compute the Rescaling Factor"
// (gamma = ||W||_1 / (d_out d_in)), "Step 2: Rescale and RoundClip" (Eq. 1),
// "N:M Mask Generation" (keep the N largest |W| of each M-group along the
// input dimension, ranked on master weights), "Composition Order:
// Quant-Then-Mask" (gamma over the full W; mask applied to the codes).
//
// Pipeline (all on the caller's stream, no host sync):
//   k_absmean_partial  grid-stride over W; exact sum of |W| as integer
//                      mantissa bins per 32-exponent window (order-free)
//   k_absmean_finalize one workgroup: bins -> exact big integer -> RN fp64
//                      -> / n -> fp32 gamma, sw = gamma + eps, and the
//                      RoundClip threshold t (smallest |w| whose code is +-1)
//   k_qmp              one thread per 32-wide chunk of a row, W staged
//                      through LDS with coalesced 16-byte loads; rank-based
//                      top-N-of-M mask, code = sign(w) * (|w| >= t), packing.
#include "sbl_internal.h"
#include "device_util.cuh"

namespace sbl {

// ---------------------------------------------------------------------------
// Exact sum of |W|.
// |w| = m * 2^(e' - 150) with m the 24-bit significand (hidden bit added for
// normals) and e' = max(e, 1). With tag = e' >> 5 and sh = e' & 31 every
// element contributes (m << sh) < 2^55 to window `tag` (weight 2^(32 tag)).
// A thread keeps one 96-bit register accumulator for its first window and
// sends any other window's terms to LDS bins (rare for weight tensors, whose
// magnitudes span far fewer than 32 binades). Bins hold (low 32 bits, rest)
// pairs so that u64 LDS atomics cannot overflow for n < 2^31.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void add96(uint32_t& a0, uint32_t& a1, uint32_t& a2, uint64_t v) {
  uint64_t lo = (uint64_t)a0 + (uint32_t)v;
  uint64_t mid = (uint64_t)a1 + (uint32_t)(v >> 32) + (lo >> 32);
  a0 = (uint32_t)lo;
  a1 = (uint32_t)mid;
  a2 += (uint32_t)(mid >> 32);
}

struct AbsSlot {
  uint32_t tag = 0xFFFFFFFFu, a0 = 0, a1 = 0, a2 = 0;
};

__device__ __forceinline__ void abs_accumulate(AbsSlot& st, unsigned long long* bins, uint32_t u) {
  u &= 0x7FFFFFFFu;
  if (u == 0) return;
  const uint32_t e = u >> 23;
  const uint32_t m = (u & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  const uint32_t ee = e ? e : 1u;
  const uint32_t tag = ee >> 5;
  const uint64_t v = (uint64_t)m << (ee & 31u);
  if (st.tag == 0xFFFFFFFFu) st.tag = tag;
  if (tag == st.tag) {
    add96(st.a0, st.a1, st.a2, v);
  } else {
    atomicAdd(&bins[2 * tag], (unsigned long long)(uint32_t)v);
    atomicAdd(&bins[2 * tag + 1], (unsigned long long)(v >> 32));
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_absmean_partial(const void* __restrict__ wv, int64_t n,
                                                         unsigned long long* __restrict__ partials) {
  __shared__ unsigned long long bins[16];
  if (threadIdx.x < 16) bins[threadIdx.x] = 0;
  __syncthreads();
  AbsSlot st;
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte load
  const int64_t nvec = n / V;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const uint4 d = *((const uint4*)wv + i);
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if constexpr (BF16) {
        abs_accumulate(st, bins, (w[h] & 0xFFFFu) << 16);
        abs_accumulate(st, bins, w[h] & 0xFFFF0000u);
      } else {
        abs_accumulate(st, bins, w[h]);
      }
    }
  }
  // tail elements (n % V) by block 0
  if (blockIdx.x == 0) {
    for (int64_t i = nvec * V + threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t u = BF16 ? ((uint32_t)((const uint16_t*)wv)[i] << 16)
                              : ((const uint32_t*)wv)[i];
      abs_accumulate(st, bins, u);
    }
  }
  if (st.tag != 0xFFFFFFFFu) {
    atomicAdd(&bins[2 * st.tag], (unsigned long long)st.a0);
    atomicAdd(&bins[2 * st.tag + 1], (unsigned long long)st.a1 | ((unsigned long long)st.a2 << 32));
  }
  __syncthreads();
  if (threadIdx.x < 16) partials[(int64_t)blockIdx.x * 16 + threadIdx.x] = bins[threadIdx.x];
}

// Device scalars written by the finalize kernel (inside the workspace).
struct PrepScalars {
  float gamma;
  float sw;
  uint32_t t_bits;  // RoundClip threshold: code != 0  <=>  |w| bits >= t_bits
  uint32_t pad;
};

// Smallest non-negative fp32 t with rint(fp32(t / sw)) >= 1, i.e. the
// boundary of the zero code. fp32 division is monotone in t, so the set of
// |w| with a nonzero code is exactly [t, inf).
__device__ float roundclip_threshold(float sw) {
  float t = 0.5f * sw;
  for (int it = 0; it < 64 && t > 0.0f; ++it) {
    const float p = __uint_as_float(__float_as_uint(t) - 1u);
    if (rintf(p / sw) >= 1.0f) t = p; else break;
  }
  for (int it = 0; it < 64 && rintf(t / sw) < 1.0f; ++it)
    t = __uint_as_float(__float_as_uint(t) + 1u);
  return t;
}

__global__ __launch_bounds__(256) void k_absmean_finalize(const unsigned long long* __restrict__ partials,
                                                          int nblocks, int64_t n, float eps,
                                                          float* __restrict__ gamma_sw,
                                                          PrepScalars* __restrict__ scal) {
  __shared__ unsigned long long red[16][256];
  unsigned long long acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0;
  for (int b = threadIdx.x; b < nblocks; b += 256) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] += partials[(int64_t)b * 16 + j];
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) red[j][threadIdx.x] = acc[j];
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) {
#pragma unroll
      for (int j = 0; j < 16; ++j) red[j][threadIdx.x] += red[j][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;

  // Exact sum in units of 2^-150 as 32-bit limbs.
  unsigned long long limb[14];
#pragma unroll
  for (int i = 0; i < 14; ++i) limb[i] = 0;
  for (int tag = 0; tag < 8; ++tag) {
    const unsigned long long lo = red[2 * tag][0], hi = red[2 * tag + 1][0];
    limb[tag] += lo & 0xFFFFFFFFull;
    limb[tag + 1] += lo >> 32;
    limb[tag + 1] += hi & 0xFFFFFFFFull;
    limb[tag + 2] += hi >> 32;
  }
  for (int i = 0; i < 13; ++i) {
    limb[i + 1] += limb[i] >> 32;
    limb[i] &= 0xFFFFFFFFull;
  }
  int top = -1;
  for (int i = 13; i >= 0; --i)
    if (limb[i]) { top = i; break; }
  double S = 0.0;
  if (top >= 0) {
    const int p = 32 * top + (31 - __clz((uint32_t)limb[top]));  // highest set bit
    auto bit = [&](int i) -> unsigned long long {
      return i < 0 ? 0ull : (limb[i >> 5] >> (i & 31)) & 1ull;
    };
    if (p <= 52) {
      unsigned long long v = 0;
      for (int i = p; i >= 0; --i) v = (v << 1) | bit(i);
      S = ldexp((double)v, -150);
    } else {
      unsigned long long mant = 0;
      for (int i = p; i >= p - 52; --i) mant = (mant << 1) | bit(i);
      const unsigned long long rb = bit(p - 53);
      bool sticky = false;
      for (int i = p - 54; i >= 0; --i)
        if (bit(i)) { sticky = true; break; }
      if (rb && (sticky || (mant & 1ull))) ++mant;  // round to nearest, ties to even
      S = ldexp((double)mant, p - 52 - 150);
    }
  }
  const double q = S / (double)n;
  const float gamma = (float)q;
  const float sw = gamma + eps;
  const float t = roundclip_threshold(sw);
  gamma_sw[0] = gamma;
  gamma_sw[1] = sw;
  scal->gamma = gamma;
  scal->sw = sw;
  scal->t_bits = __float_as_uint(t);
  scal->pad = 0;
}

// ---------------------------------------------------------------------------
// Mask + RoundClip + pack. One thread per 32-wide chunk (o, c), c in
// [0, ceil(K/128)*4), which covers every byte of a packed row record.
// A block's 256 chunks are staged through LDS (row stride 33 words, so the
// per-thread reads below are bank-conflict free) with 16-byte loads in which
// consecutive lanes read consecutive addresses.
// ---------------------------------------------------------------------------
constexpr int kChunksPerBlock = 256;
constexpr int kLdsStride = 33;

template <int M>
__device__ __forceinline__ uint32_t topn_keep_bits(const uint32_t* a, int N) {
  // rank_i = #{j : |w_j| > |w_i|} + #{j < i : |w_j| == |w_i|}; keep iff rank_i < N
  int rank[M];
#pragma unroll
  for (int i = 0; i < M; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = i + 1; j < M; ++j) {
      if (a[j] > a[i]) ++rank[i]; else ++rank[j];
    }
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) keep |= (rank[i] < N ? 1u : 0u) << i;
  return keep;
}

template <bool BF16, int M, bool IDX>
__global__ __launch_bounds__(256) void k_qmp(const void* __restrict__ wv, int64_t O, int64_t K,
                                             int N, int64_t C, const PrepScalars* __restrict__ scal,
                                             uint8_t* __restrict__ packed, int64_t pitch,
                                             int64_t code_chunks, int64_t mask_off,
                                             int8_t* __restrict__ w_eff,
                                             uint8_t* __restrict__ mask_out,
                                             float* __restrict__ sw_rows) {
  __shared__ uint32_t lds[kChunksPerBlock * kLdsStride];
  const int64_t total = O * C;
  const int64_t base = (int64_t)blockIdx.x * kChunksPerBlock;

  // ---- stage: |w| bits (sign kept) of 256 chunks x 32 elements ----
  constexpr int V = BF16 ? 8 : 4;              // elements per 16-byte piece
  constexpr int PIECES = 32 / V;               // pieces per chunk
  for (int p = threadIdx.x; p < kChunksPerBlock * PIECES; p += 256) {
    const int lc = p / PIECES, pc = p % PIECES;
    const int64_t ch = base + lc;
    uint32_t vals[V];
#pragma unroll
    for (int e = 0; e < V; ++e) vals[e] = 0;
    if (ch < total) {
      const int64_t o = ch / C, c = ch % C;
      const int64_t k = 32 * c + (int64_t)V * pc;
      if (k < K) {  // K % 4 == 0; a piece is whole when k + V <= K
        if (k + V <= K && ((K * (BF16 ? 2 : 4)) % 16 == 0)) {
          const uint4 d = BF16 ? *(const uint4*)((const uint16_t*)wv + o * K + k)
                               : *(const uint4*)((const float*)wv + o * K + k);
          const uint32_t w[4] = {d.x, d.y, d.z, d.w};
          if constexpr (BF16) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              vals[2 * h] = (w[h] & 0xFFFFu) << 16;
              vals[2 * h + 1] = w[h] & 0xFFFF0000u;
            }
          } else {
#pragma unroll
            for (int h = 0; h < 4; ++h) vals[h] = w[h];
          }
        } else {
          for (int e = 0; e < V && k + e < K; ++e)
            vals[e] = BF16 ? ((uint32_t)((const uint16_t*)wv)[o * K + k + e] << 16)
                           : ((const uint32_t*)wv)[o * K + k + e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) lds[lc * kLdsStride + pc * V + e] = vals[e];
  }
  __syncthreads();

  const int64_t ch = base + threadIdx.x;
  if (ch >= total) return;
  const int64_t o = ch / C, c = ch % C;
  const int64_t k0 = 32 * c;
  const uint32_t tb = scal->t_bits;

  uint32_t a[32], sgn = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t u = lds[threadIdx.x * kLdsStride + e];
    a[e] = u & 0x7FFFFFFFu;
    sgn |= (u >> 31) << e;
  }
  // valid elements of this chunk: k0 + e < K
  const int64_t rem = K - k0;
  const uint32_t valid = rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));

  uint32_t keep = 0;
#pragma unroll
  for (int g = 0; g < 32 / M; ++g) keep |= topn_keep_bits<M>(a + g * M, N) << (g * M);
  uint32_t nz = 0;  // code != 0
#pragma unroll
  for (int e = 0; e < 32; ++e) nz |= (a[e] >= tb ? 1u : 0u) << e;
  const uint32_t kept_nz = nz & keep & valid;

  // optional unpacked outputs (k < K only)
  if (w_eff || mask_out) {
    for (int e = 0; e < 32; ++e) {
      if (!((valid >> e) & 1u)) break;
      const int64_t idx = o * K + k0 + e;
      if (w_eff) w_eff[idx] = ((kept_nz >> e) & 1u) ? (((sgn >> e) & 1u) ? (int8_t)-1 : (int8_t)1) : (int8_t)0;
      if (mask_out) mask_out[idx] = (uint8_t)((keep & valid) >> e & 1u);
    }
  }
  if (sw_rows && c == 0) sw_rows[o] = scal->sw;

  uint8_t* rec = packed ? packed + o * pitch : nullptr;
  if (!rec) return;
  if constexpr (IDX) {
    // 8 groups of 4: kept slots i0 < i1 (exactly two; padding groups keep 0,1)
    uint32_t cw = 0, iw = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t kb = (keep >> (4 * q)) & 0xFu;
      const uint32_t i0 = __builtin_ctz(kb | 0x10u);
      const uint32_t i1 = 31u - __builtin_clz(kb | 1u);
      iw |= (i0 | (i1 << 2)) << (4 * q);
      const uint32_t s0 = 4 * q + i0, s1 = 4 * q + i1;
      const uint32_t f0 = ((kept_nz >> s0) & 1u) ? (((sgn >> s0) & 1u) ? 3u : 1u) : 0u;
      const uint32_t f1 = ((kept_nz >> s1) & 1u) ? (((sgn >> s1) & 1u) ? 3u : 1u) : 0u;
      cw |= f0 << field_shift(2 * q);
      cw |= f1 << field_shift(2 * q + 1);
    }
    *(uint2*)(rec + 8 * c) = make_uint2(cw, iw);
  } else {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t f0 = ((kept_nz >> u) & 1u) ? (((sgn >> u) & 1u) ? 3u : 1u) : 0u;
      const uint32_t f1 = ((kept_nz >> (u + 16)) & 1u) ? (((sgn >> (u + 16)) & 1u) ? 3u : 1u) : 0u;
      w0 |= f0 << field_shift(u);
      w1 |= f1 << field_shift(u);
    }
    if (c < code_chunks) *(uint2*)(rec + 8 * c) = make_uint2(w0, w1);
    *(uint32_t*)(rec + mask_off + 4 * c) = keep & valid;
  }
}

template <bool BF16>
static hipError_t launch_qmp_typed(const void* w, int64_t O, int64_t K, int N, int M,
                                   const PrepScalars* scal, uint8_t* packed, int8_t* w_eff,
                                   uint8_t* mask, float* sw_rows, hipStream_t s) {
  const int64_t C = row_chunks(K);
  const int64_t pitch = row_pitch(K, N, M);
  const int64_t code_chunks = dense_code_bytes(K) / 8;
  const int64_t mask_off = dense_code_bytes(K);
  const dim3 grid((unsigned)cdiv(O * C, kChunksPerBlock)), block(256);
  if (index_form(N, M))
    hipLaunchKernelGGL((k_qmp<BF16, 4, true>), grid, block, 0, s, w, O, K, N, C, scal, packed,
                       pitch, code_chunks, mask_off, w_eff, mask, sw_rows);
  else if (M == 4)
    hipLaunchKernelGGL((k_qmp<BF16, 4, false>), grid, block, 0, s, w, O, K, N, C, scal, packed,
                       pitch, code_chunks, mask_off, w_eff, mask, sw_rows);
  else
    hipLaunchKernelGGL((k_qmp<BF16, 8, false>), grid, block, 0, s, w, O, K, N, C, scal, packed,
                       pitch, code_chunks, mask_off, w_eff, mask, sw_rows);
  return hipGetLastError();
}

hipError_t launch_quant_mask_weight(const void* w, bool bf16, int64_t O, int64_t K, int N, int M,
                                    float eps, int8_t* w_eff, uint8_t* mask, void* packed,
                                    float* gamma_sw, float* sw_rows, void* ws, hipStream_t s) {
  const int64_t n = O * K;
  auto* partials = (unsigned long long*)ws;
  auto* scal = (PrepScalars*)((char*)ws + (size_t)kAbsmeanMaxBlocks * 16 * sizeof(unsigned long long));
  const int V = bf16 ? 8 : 4;
  int64_t want = cdiv(cdiv(n, V), 256 * 8);  // >= 8 vectors per thread
  int nblocks = (int)(want < 1 ? 1 : (want > kAbsmeanMaxBlocks ? kAbsmeanMaxBlocks : want));
  if (bf16)
    hipLaunchKernelGGL((k_absmean_partial<true>), dim3(nblocks), dim3(256), 0, s, w, n, partials);
  else
    hipLaunchKernelGGL((k_absmean_partial<false>), dim3(nblocks), dim3(256), 0, s, w, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_absmean_finalize, dim3(1), dim3(256), 0, s, partials, nblocks, n, eps,
                     gamma_sw, scal);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return bf16 ? launch_qmp_typed<true>(w, O, K, N, M, scal, (uint8_t*)packed, w_eff, mask, sw_rows, s)
              : launch_qmp_typed<false>(w, O, K, N, M, scal, (uint8_t*)packed, w_eff, mask, sw_rows, s);
}

// ---------------------------------------------------------------------------
// Standalone pack / unpack, one thread per 32-wide chunk of a row record.
// ---------------------------------------------------------------------------
template <bool IDX>
__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ w_eff,
                                              const uint8_t* __restrict__ mask, int64_t O,
                                              int64_t K, int64_t C, uint8_t* __restrict__ packed,
                                              int64_t pitch, int64_t code_chunks, int64_t mask_off) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= O * C) return;
  const int64_t o = ch / C, c = ch % C, k0 = 32 * c;
  uint32_t keep = 0;
  uint64_t fw = 0;  // 2-bit code of element e at bits [2e+1:2e]
  for (int e = 0; e < 32; ++e) {
    if (k0 + e < K) {
      const int64_t idx = o * K + k0 + e;
      keep |= (mask[idx] ? 1u : 0u) << e;
      fw |= (uint64_t)((uint32_t)w_eff[idx] & 3u) << (2 * e);
    }
  }
  auto f = [&](uint32_t e) -> uint32_t { return (uint32_t)(fw >> (2 * e)) & 3u; };
  uint8_t* rec = packed + o * pitch;
  if constexpr (IDX) {
    if (k0 >= K) keep = 0x33333333u;            // padding groups keep slots (0, 1)
    else if (K - k0 < 32) keep |= 0x33333333u & ~((1u << (K - k0)) - 1u);
    uint32_t cw = 0, iw = 0;
    for (int q = 0; q < 8; ++q) {
      const uint32_t kb = (keep >> (4 * q)) & 0xFu;
      const uint32_t i0 = __builtin_ctz(kb | 0x10u);
      const uint32_t i1 = 31u - __builtin_clz(kb | 1u);
      iw |= (i0 | (i1 << 2)) << (4 * q);
      cw |= f(4 * q + (i0 & 3)) << field_shift(2 * q);
      cw |= f(4 * q + (i1 & 3)) << field_shift(2 * q + 1);
    }
    *(uint2*)(rec + 8 * c) = make_uint2(cw, iw);
  } else {
    uint32_t w0 = 0, w1 = 0;
    for (int u = 0; u < 16; ++u) {
      w0 |= f(u) << field_shift(u);
      w1 |= f(u + 16) << field_shift(u);
    }
    if (c < code_chunks) *(uint2*)(rec + 8 * c) = make_uint2(w0, w1);
    *(uint32_t*)(rec + mask_off + 4 * c) = keep;
  }
}

template <bool IDX>
__global__ __launch_bounds__(256) void k_unpack(const uint8_t* __restrict__ packed, int64_t O,
                                                int64_t K, int64_t C, int64_t pitch,
                                                int64_t mask_off, int8_t* __restrict__ w_eff,
                                                uint8_t* __restrict__ mask) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= O * C) return;
  const int64_t o = ch / C, c = ch % C, k0 = 32 * c;
  if (k0 >= K) return;
  const uint8_t* rec = packed + o * pitch;
  int8_t wv[32];
  uint32_t keep = 0;
  if constexpr (IDX) {
    const uint2 r = *(const uint2*)(rec + 8 * c);
    for (int e = 0; e < 32; ++e) wv[e] = 0;
    for (int q = 0; q < 8; ++q) {
      const uint32_t i0 = (r.y >> (4 * q)) & 3u, i1 = (r.y >> (4 * q + 2)) & 3u;
      const uint32_t f0 = (r.x >> field_shift(2 * q)) & 3u, f1 = (r.x >> field_shift(2 * q + 1)) & 3u;
      wv[4 * q + i0] = (int8_t)(f0 == 3u ? -1 : (int)f0);
      wv[4 * q + i1] = (int8_t)(f1 == 3u ? -1 : (int)f1);
      keep |= ((1u << i0) | (1u << i1)) << (4 * q);
    }
  } else {
    const uint2 r = *(const uint2*)(rec + 8 * c);
    for (int u = 0; u < 16; ++u) {
      const uint32_t f0 = (r.x >> field_shift(u)) & 3u, f1 = (r.y >> field_shift(u)) & 3u;
      wv[u] = (int8_t)(f0 == 3u ? -1 : (int)f0);
      wv[u + 16] = (int8_t)(f1 == 3u ? -1 : (int)f1);
    }
    keep = *(const uint32_t*)(rec + mask_off + 4 * c);
  }
  for (int e = 0; e < 32 && k0 + e < K; ++e) {
    const int64_t idx = o * K + k0 + e;
    w_eff[idx] = wv[e];
    mask[idx] = (uint8_t)((keep >> e) & 1u);
  }
}

hipError_t launch_pack(const int8_t* w_eff, const uint8_t* mask, int64_t O, int64_t K, int N,
                       int M, void* packed, hipStream_t s) {
  const int64_t C = row_chunks(K);
  const dim3 grid((unsigned)cdiv(O * C, 256)), block(256);
  if (index_form(N, M))
    hipLaunchKernelGGL((k_pack<true>), grid, block, 0, s, w_eff, mask, O, K, C, (uint8_t*)packed,
                       row_pitch(K, N, M), dense_code_bytes(K) / 8, dense_code_bytes(K));
  else
    hipLaunchKernelGGL((k_pack<false>), grid, block, 0, s, w_eff, mask, O, K, C, (uint8_t*)packed,
                       row_pitch(K, N, M), dense_code_bytes(K) / 8, dense_code_bytes(K));
  return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, int64_t O, int64_t K, int N, int M, int8_t* w_eff,
                         uint8_t* mask, hipStream_t s) {
  const int64_t C = row_chunks(K);
  const dim3 grid((unsigned)cdiv(O * C, 256)), block(256);
  if (index_form(N, M))
    hipLaunchKernelGGL((k_unpack<true>), grid, block, 0, s, (const uint8_t*)packed, O, K, C,
                       row_pitch(K, N, M), dense_code_bytes(K), w_eff, mask);
  else
    hipLaunchKernelGGL((k_unpack<false>), grid, block, 0, s, (const uint8_t*)packed, O, K, C,
                       row_pitch(K, N, M), dense_code_bytes(K), w_eff, mask);
  return hipGetLastError();
}

}  // namespace sbl
