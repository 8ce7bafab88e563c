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
  constexpr int U = 8;             // loads in flight per thread
  const int64_t nvec = n / V;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto consume = [&](const uint4& d) {
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
  };
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < nvec; i += U * stride) {
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = *((const uint4*)wv + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) consume(d[u]);
  }
  for (; i < nvec; i += stride) consume(*((const uint4*)wv + i));
  // tail elements (n % V) by block 0
  if (blockIdx.x == 0) {
    for (int64_t j = nvec * V + threadIdx.x; j < n; j += blockDim.x) {
      const uint32_t u = BF16 ? ((uint32_t)((const uint16_t*)wv)[j] << 16)
                              : ((const uint32_t*)wv)[j];
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
  // thread t sums the 16 bins of blocks t, t + 256, ... (all loads independent),
  // then a wave reduction and a 4-way combine in LDS
  __shared__ unsigned long long red[4][16];
  unsigned long long acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0;
  for (int b = threadIdx.x; b < nblocks; b += 256) {
    const uint4* p = (const uint4*)(partials + (int64_t)b * 16);
    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = p[q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      acc[2 * q] += (unsigned long long)v[q].x | ((unsigned long long)v[q].y << 32);
      acc[2 * q + 1] += (unsigned long long)v[q].z | ((unsigned long long)v[q].w << 32);
    }
  }
  // two-level reduction through LDS: 256 x 16 -> 16 x 16 -> 16
  __shared__ unsigned long long part[16][257];
#pragma unroll
  for (int j = 0; j < 16; ++j) part[j][threadIdx.x] = acc[j];
  __syncthreads();
  {
    const int col = threadIdx.x & 15, grp = threadIdx.x >> 4;  // 16 groups of 16 rows
    unsigned long long sum = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += part[col][grp * 16 + r];
    __syncthreads();
    part[col][grp] = sum;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    unsigned long long sum = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += part[threadIdx.x][r];
    red[0][threadIdx.x] = sum;
    red[1][threadIdx.x] = red[2][threadIdx.x] = red[3][threadIdx.x] = 0;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;

  // Exact sum in units of 2^-150 as 32-bit limbs (registers only: constant indices).
  constexpr int NL = 12;
  uint32_t L[NL];
  {
    unsigned long long w[NL + 1];
#pragma unroll
    for (int i = 0; i <= NL; ++i) w[i] = 0;
#pragma unroll
    for (int tag = 0; tag < 8; ++tag) {
      const unsigned long long lo = red[0][2 * tag] + red[1][2 * tag] + red[2][2 * tag] + red[3][2 * tag];
      const unsigned long long hi = red[0][2 * tag + 1] + red[1][2 * tag + 1] + red[2][2 * tag + 1] +
                                    red[3][2 * tag + 1];
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
  double S = 0.0;
  if (top >= 0) {
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
    S = ldexp((double)mant, 43 - c + 32 * (top - 2) - 150);
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

// Keep bits of one group of M magnitudes (bit i = slot i kept):
// rank_i = #{j : |w_j| > |w_i|} + #{j < i : |w_j| == |w_i|}; keep iff rank_i < N.
// With c = [a_j > a_i] for a pair i < j: rank_i gains c and rank_j gains 1 - c,
// so rank = sum_i i<<4i-style base + sum over pairs of c * (field_i - field_j),
// held as 4-bit fields of one register (final values are in [0, M-1]).
template <int M>
__device__ __forceinline__ uint32_t topn_keep_bits(const uint32_t* a, int N) {
  uint32_t R = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) R += (uint32_t)i << (4 * i);
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = i + 1; j < M; ++j)
      R += (a[j] > a[i]) ? ((1u << (4 * i)) - (1u << (4 * j))) : 0u;
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) keep |= (((R >> (4 * i)) & 15u) < (uint32_t)N ? 1u : 0u) << i;
  return keep;
}

// Byte-slice 16 two-bit fields: bit u of lo (u = 4b + a) -> bit 8a + 2b, and
// the same for hi one position up; i.e. a 4x4 transpose of 2-bit cells.
__device__ __forceinline__ uint32_t byte_slice16(uint32_t lo, uint32_t hi) {
  // interleave: bit u of lo -> 2u, bit u of hi -> 2u + 1
  auto spread = [](uint32_t x) {
    x &= 0xFFFFu;
    x = (x | (x << 8)) & 0x00FF00FFu;
    x = (x | (x << 4)) & 0x0F0F0F0Fu;
    x = (x | (x << 2)) & 0x33333333u;
    x = (x | (x << 1)) & 0x55555555u;
    return x;
  };
  uint32_t v = spread(lo) | (spread(hi) << 1);   // cell (b, a) at 8b + 2a
  // transpose the 4x4 matrix of 2-bit cells: (b, a) -> (a, b)
  uint32_t t = (v ^ (v >> 6)) & 0x00CC00CCu;      // swap cells at distance (1,-1)
  v ^= t ^ (t << 6);
  t = (v ^ (v >> 12)) & 0x0000F0F0u;              // swap 2x2 blocks
  v ^= t ^ (t << 12);
  return v;
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
  // all chunk/row indices fit in 32 bits: O * C < 2^31 (O * K < 2^31)
  const uint32_t total = (uint32_t)(O * C), C32 = (uint32_t)C, K32 = (uint32_t)K;
  const uint32_t base = blockIdx.x * kChunksPerBlock;

  // ---- stage: raw bits of 256 chunks x 32 elements ----
  constexpr int V = BF16 ? 8 : 4;              // elements per 16-byte piece
  constexpr int PIECES = 32 / V;               // pieces per chunk = pieces per thread
  const bool rows16 = ((K32 * (BF16 ? 2u : 4u)) % 16u) == 0;
  uint4 d[PIECES];
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const uint32_t p = threadIdx.x + 256u * q;
    const uint32_t ch = base + p / PIECES, pc = p % PIECES;
    d[q] = make_uint4(0, 0, 0, 0);
    if (ch < total) {
      const uint32_t o = ch / C32, c = ch - o * C32;
      const uint32_t k = 32u * c + V * pc;
      const int64_t off = (int64_t)o * K + k;
      if (k + V <= K32 && rows16) {
        d[q] = BF16 ? *(const uint4*)((const uint16_t*)wv + off)
                    : *(const uint4*)((const float*)wv + off);
      } else if (k < K32) {  // K % 4 == 0: a partial piece holds whole 4-element groups
        uint32_t t[4] = {0, 0, 0, 0};
        for (uint32_t e = 0; e < (uint32_t)V && k + e < K32; ++e) {
          const uint32_t u = BF16 ? (uint32_t)((const uint16_t*)wv)[off + e]
                                  : ((const uint32_t*)wv)[off + e];
          if constexpr (BF16) t[e >> 1] |= u << (16 * (e & 1)); else t[e] = u;
        }
        d[q] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const uint32_t p = threadIdx.x + 256u * q;
    const uint32_t lc = p / PIECES, pc = p % PIECES;
    const uint32_t w[4] = {d[q].x, d[q].y, d[q].z, d[q].w};
    uint32_t* dst = lds + lc * kLdsStride + pc * V;
    if constexpr (BF16) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        dst[2 * h] = (w[h] & 0xFFFFu) << 16;
        dst[2 * h + 1] = w[h] & 0xFFFF0000u;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) dst[h] = w[h];
    }
  }
  __syncthreads();

  const uint32_t ch = base + threadIdx.x;
  if (ch >= total) return;
  const uint32_t o = ch / C32, c = ch - o * C32;
  const uint32_t k0 = 32u * c;
  const uint32_t tb = scal->t_bits;

  uint32_t a[32], sgn = 0, nz = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t u = lds[threadIdx.x * kLdsStride + e];
    a[e] = u & 0x7FFFFFFFu;
    sgn |= (u >> 31) << e;
    nz |= ((tb - 1u - a[e]) >> 31) << e;          // a >= tb  (both < 2^31, tb >= 1)
  }
  const uint32_t valid = k0 >= K32 ? 0u : (K32 - k0 >= 32u ? 0xFFFFFFFFu : ((1u << (K32 - k0)) - 1u));

  uint32_t keep = 0;
#pragma unroll
  for (int g = 0; g < 32 / M; ++g) keep |= topn_keep_bits<M>(a + g * M, N) << (g * M);
  const uint32_t kn = nz & keep & valid;          // nonzero code, kept
  const uint32_t kneg = kn & sgn;                 // ... and negative

  // optional unpacked outputs (k < K only)
  if (w_eff || mask_out) {
    for (int e = 0; e < 32; ++e) {
      if (!((valid >> e) & 1u)) break;
      const int64_t idx = (int64_t)o * K + k0 + e;
      if (w_eff) w_eff[idx] = ((kn >> e) & 1u) ? (((kneg >> e) & 1u) ? (int8_t)-1 : (int8_t)1) : (int8_t)0;
      if (mask_out) mask_out[idx] = (uint8_t)((keep & valid) >> e & 1u);
    }
  }
  if (sw_rows && c == 0) sw_rows[o] = scal->sw;

  if (!packed) return;
  uint8_t* rec = packed + (int64_t)o * pitch;
  if constexpr (IDX) {
    // 8 groups of 4: kept slots i0 < i1 (exactly two; padding groups keep 0,1)
    uint32_t iw = 0, lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t kb = (keep >> (4 * q)) & 0xFu;
      const uint32_t i0 = __builtin_ctz(kb | 0x10u);
      const uint32_t i1 = 31u - __builtin_clz(kb | 1u);
      iw |= (i0 | (i1 << 2)) << (4 * q);
      lo |= ((kn >> (4 * q + i0)) & 1u) << (2 * q) | ((kn >> (4 * q + i1)) & 1u) << (2 * q + 1);
      hi |= ((kneg >> (4 * q + i0)) & 1u) << (2 * q) | ((kneg >> (4 * q + i1)) & 1u) << (2 * q + 1);
    }
    *(uint2*)(rec + 8 * c) = make_uint2(byte_slice16(lo, hi), iw);
  } else {
    const uint32_t w0 = byte_slice16(kn & 0xFFFFu, kneg & 0xFFFFu);
    const uint32_t w1 = byte_slice16(kn >> 16, kneg >> 16);
    if (c < (uint32_t)code_chunks) *(uint2*)(rec + 8 * c) = make_uint2(w0, w1);
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
  // about 8 vectors per thread, at most 512 blocks (two per CU)
  const int64_t want = cdiv(cdiv(n, V), 256 * 8);
  const int nblocks = (int)(want < 1 ? 1 : (want > 512 ? 512 : want));
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
