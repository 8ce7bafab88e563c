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
//                      mantissa bins per 32-exponent window (order-free),
//                      one vector of bins per block (at most 128 per tensor)
//   k_qmp              an extra wave per block sums the tensor's partial
//                      vectors into 16 bins and turns them into an exact big
//                      integer -> RN fp64 -> / n -> fp32 gamma, sw = gamma +
//                      eps, and the RoundClip threshold t (smallest |w| whose
//                      code is +-1); meanwhile one thread per 32-wide chunk of
//                      a row stages W through LDS with coalesced 16-byte
//                      loads and ranks it: top-N-of-M mask; then
//                      code = sign(w) * (|w| >= t), packing.
#include "sbl_internal.h"
#include "device_util.h"
#include "exact_sum.h"

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

// Register accumulator of one window. Window 3 holds every |w| in
// [2^-31, 2) (e' in [96, 127]), where practically all weights lie; any other
// term goes to the LDS bins, so the choice costs nothing in exactness.
constexpr uint32_t kAbsWindow = 3;
struct AbsSlot {
  uint32_t tag = kAbsWindow, a0 = 0, a1 = 0, a2 = 0;
};


// Accumulate one |w| (any sign bit): terms of the slot's window go to the
// 96-bit register accumulator with no branch (zeros add nothing, whatever
// their window); others (rare for weights) are added to the LDS bins.
__device__ __forceinline__ void abs_accumulate(AbsSlot& st, unsigned long long* bins, uint32_t u) {
  uint32_t tag;
  uint64_t v;
  exact_term(u & 0x7FFFFFFFu, tag, v);
  const bool here = tag == st.tag || v == 0;
  const uint64_t vh = here ? v : 0;
  add96(st.a0, st.a1, st.a2, vh);
  if (!here) {
    atomicAdd(&bins[2 * tag], (unsigned long long)(uint32_t)v);
    atomicAdd(&bins[2 * tag + 1], (unsigned long long)(v >> 32));
  }
}

// ---------------------------------------------------------------------------
// Batches: every kernel below serves up to kMaxPrepBatch weight tensors in
// one launch; a block finds its tensor from its index. The descriptor is a
// kernel argument (by value), so the launches can be captured in a graph.
// ---------------------------------------------------------------------------
struct PrepItemK {
  const void* w;
  int8_t* w_eff;
  uint8_t* mask;
  uint8_t* packed;
  float* gamma_sw;
  float* sw_rows;
  uint32_t* mask_bits;                       // optional mask diagnostics
  const uint32_t* prev_mask_bits;
  unsigned long long* flips;
  float* group_thr;
  int32_t variant, pad_v;
  int64_t O, K;
  int32_t C, pitch, code_chunks, mask_off;   // packed-record geometry
  int32_t part0, nparts;                     // its partial vectors (= its partial-pass blocks)
  int32_t blk1, blk3;                        // its first block in the partial / mask pass
};
struct PrepBatchK {
  int32_t count, pad;
  PrepItemK it[kMaxPrepBatch];
};

// Tensor of block `blk` given each tensor's first block (wave-uniform), and
// that tensor's descriptor, selected with constant indices only.
__device__ __forceinline__ int prep_index(const PrepBatchK& b, int blk, bool mask_pass) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kMaxPrepBatch; ++j)
    if (j < b.count && blk >= (mask_pass ? b.it[j].blk3 : b.it[j].blk1)) i = j;
  return i;
}
__device__ __forceinline__ PrepItemK prep_item(const PrepBatchK& b, int i) {
  PrepItemK r = b.it[0];
#pragma unroll
  for (int j = 1; j < kMaxPrepBatch; ++j)
    if (j == i) r = b.it[j];
  return r;
}

// Slow path: add |w| to the LDS bins if it lies outside window 3.
__device__ __forceinline__ void abs_accumulate_other(unsigned long long* bins, uint32_t u) {
  uint32_t tag;
  uint64_t v;
  exact_term(u & 0x7FFFFFFFu, tag, v);
  if (tag != kAbsWindow && v != 0) {
    atomicAdd(&bins[2 * tag], (unsigned long long)(uint32_t)v);
    atomicAdd(&bins[2 * tag + 1], (unsigned long long)(v >> 32));
  }
}

// One vector of 16 bins per block. Each thread walks its vectors in batches
// of kAbsBatch 16-byte loads, with the next batch in flight while the
// current one is accumulated.
//
// Fast path (branch-free): |w| with e in [96, 127] -- window 3, where
// practically every weight lies -- adds (m | 2^23) << (e & 31) to the 96-bit
// register slot; zeros add nothing; any other term only marks its lane. A
// marked lane re-reads its vectors afterwards and adds exactly those other
// terms to the LDS bins (the exact sum is order-free, so the split is exact).
// Few, large blocks: every mask-pass workgroup sums its tensor's partial
// vectors itself, so their number stays small.
constexpr int kAbsThreads = 1024;
constexpr int kAbsBatch = 8;
constexpr int kAbsBlocks = 256;        // partial vectors of a batch (at most)
constexpr int kAbsPerTensor = 128;     // partial vectors of one tensor (at most)
static_assert(kAbsBlocks <= kAbsmeanMaxBlocks,
              "partials must fit the weight-prep workspace");

// window-3 term of a sign-cleared |w| (0 outside window 3); `other` set if
// the value is nonzero and outside window 3
__device__ __forceinline__ uint64_t abs_term3(uint32_t u, bool& other) {
  const bool in3 = (u >> 28) == 3u;                          // e in [96, 127]
  other |= !in3 && u != 0u;
  const uint32_t m = in3 ? ((u & 0x7FFFFFu) | 0x800000u) : 0u;
  return (uint64_t)m << ((u >> 23) & 31u);
}

// A block's partial result (block p of the batch): its 16 bins, and a
// compact record {bin 2w, bin 2w + 1, any other bin nonzero, 0} of window
// w = 3, where practically every weight lies. The mask pass reads the
// 32-byte records and falls back to the full vectors only when a flag is set.
__device__ __forceinline__ void write_partial(unsigned long long* __restrict__ partials_all, int64_t p,
                                              const unsigned long long* bins) {
  if (threadIdx.x < 16) partials_all[p * 16 + threadIdx.x] = bins[threadIdx.x];
  if (threadIdx.x == 0) {
    unsigned long long other = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j != 2 * (int)kAbsWindow && j != 2 * (int)kAbsWindow + 1) other |= bins[j];
    unsigned long long* const c = partials_all + (int64_t)kAbsmeanMaxBlocks * 16 + p * 4;
    c[0] = bins[2 * kAbsWindow];
    c[1] = bins[2 * kAbsWindow + 1];
    c[2] = other != 0 ? 1ull : 0ull;
    c[3] = 0;
  }
}

template <bool BF16>
__global__ __launch_bounds__(kAbsThreads) void k_absmean_partial(const PrepBatchK batch,
                                                                 unsigned long long* __restrict__ partials_all) {
  const int item = prep_index(batch, blockIdx.x, false);
  const PrepItemK pi = prep_item(batch, item);
  const void* __restrict__ wv = pi.w;
  const int64_t n = pi.O * pi.K;
  const uint32_t lb = blockIdx.x - pi.blk1, nblk = pi.nparts;      // block within the tensor
  __shared__ unsigned long long bins[16];
  if (threadIdx.x < 16) bins[threadIdx.x] = 0;
  __syncthreads();
  uint32_t a0 = 0, a1 = 0, a2 = 0;                  // window-3 slot
  bool other = false;
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte load
  constexpr int U = kAbsBatch;
  // 32-bit indexing: n < 2^31. The trip count is uniform over the block
  // (its first thread has the most vectors) and every load is unconditional:
  // a lane past its own last vector re-reads that vector (distinct per lane)
  // and drops the terms, so no lane-divergent branch guards a prefetch.
  const uint32_t nvec = (uint32_t)(n / V);
  const uint32_t stride = nblk * blockDim.x;
  const uint32_t i0 = lb * blockDim.x + threadIdx.x;
  const uint4* src = (const uint4*)wv;
  auto consume = [&](const uint4& d, bool ok) {
    const uint32_t w[4] = {ok ? d.x : 0u, ok ? d.y : 0u, ok ? d.z : 0u, ok ? d.w : 0u};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if constexpr (BF16) {
        add96(a0, a1, a2, abs_term3((w[h] << 16) & 0x7FFFFFFFu, other));
        add96(a0, a1, a2, abs_term3(w[h] & 0x7FFF0000u, other));
      } else {
        add96(a0, a1, a2, abs_term3(w[h] & 0x7FFFFFFFu, other));
      }
    }
  };
  const uint32_t b0 = lb * blockDim.x;
  const uint32_t trips = b0 < nvec ? (nvec - b0 + stride - 1) / stride : 0;   // uniform
  const uint32_t cnt = i0 < nvec ? (nvec - i0 + stride - 1) / stride : 0;
  if (trips > 0) {
    const uint32_t last = min(i0 + (cnt > 0 ? cnt - 1 : 0) * stride, nvec - 1);
    auto load = [&](uint32_t k0, uint4 (&d)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = src[min(i0 + (k0 + u) * stride, last)];
    };
    uint4 d0[U], d1[U];
    load(0, d0);
    for (uint32_t k = 0; k < trips; k += 2 * U) {
      load(k + U, d1);
#pragma unroll
      for (int u = 0; u < U; ++u) consume(d0[u], k + u < cnt);
      if (k + U >= trips) break;
      load(k + 2 * U, d0);
#pragma unroll
      for (int u = 0; u < U; ++u) consume(d1[u], k + U + u < cnt);
    }
  }
  AbsSlot st;                                       // slow path: other windows
  st.a0 = st.a1 = st.a2 = 0;
  if (other) {
    for (uint32_t k = 0; k < cnt; ++k) {
      const uint4 d = src[i0 + k * stride];
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (BF16) {
          abs_accumulate_other(bins, w[h] << 16);
          abs_accumulate_other(bins, w[h] & 0xFFFF0000u);
        } else {
          abs_accumulate_other(bins, w[h]);
        }
      }
    }
  }
  // tail elements (n % V) by the tensor's first block
  if (lb == 0) {
    for (int64_t j = (int64_t)nvec * V + threadIdx.x; j < n; j += blockDim.x) {
      const uint32_t u = BF16 ? ((uint32_t)((const uint16_t*)wv)[j] << 16)
                              : ((const uint32_t*)wv)[j];
      abs_accumulate(st, bins, u);
    }
  }
  // Fold the window-3 slots: a wave-wide sum and one atomic pair per wave
  // (hundreds of same-address LDS atomics per block would serialize); the
  // tail slot of block 0 per lane.
  const unsigned long long lo = a0;
  const unsigned long long hi = (unsigned long long)a1 | ((unsigned long long)a2 << 32);
  const unsigned long long slo = wave_sum_u64(lo), shi = wave_sum_u64(hi);
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&bins[2 * kAbsWindow], slo);
    atomicAdd(&bins[2 * kAbsWindow + 1], shi);
  }
  if (lb == 0 && (st.a0 | st.a1 | st.a2)) {
    atomicAdd(&bins[2 * st.tag], (unsigned long long)st.a0);
    atomicAdd(&bins[2 * st.tag + 1], (unsigned long long)st.a1 | ((unsigned long long)st.a2 << 32));
  }
  __syncthreads();
  write_partial(partials_all, (int64_t)pi.part0 + lb, bins);
}

// Per-tensor scalars of the weight quantization.
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

// 16 summed bins -> correctly rounded fp64 sum -> gamma, sw, threshold.
// The bins are exact integers: bin 2w holds low parts and bin 2w+1 high parts
// of window w (weight 2^(32 w - 150)).
__device__ PrepScalars scalars_from_bins(const unsigned long long* bins, int64_t n, float eps) {
  const double S = exact_bins_to_f64(bins);
  const double q = S / (double)n;
  PrepScalars r;
  r.gamma = (float)q;
  r.sw = r.gamma + eps;
  r.t_bits = __float_as_uint(roundclip_threshold(r.sw));
  r.pad = 0;
  return r;
}

// ---------------------------------------------------------------------------
// Mask + RoundClip + pack. One thread per 32-wide chunk (o, c), c in
// [0, ceil(K/128)*4), which covers every byte of a packed row record.
// A block's chunks are staged through LDS (row stride 36 words: 16-byte
// accesses on both sides, bank-conflict free) with 16-byte global loads in
// which consecutive lanes read consecutive addresses.
// ---------------------------------------------------------------------------
constexpr int kChunksPerBlock = 128;
constexpr int kLdsStride = 36;   // words per staged chunk: 16-byte aligned, conflict-free

// The n lowest set bits of v (n <= 8).
__device__ __forceinline__ uint32_t lowest_bits(uint32_t v, int n) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < n) {
      const uint32_t b = v & (0u - v);
      r |= b;
      v ^= b;
    }
  }
  return r;
}

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

// Keep bits of a group of 8 when only D = 8 - N in {1, 2} slots are dropped:
// the D lowest in keep priority, where slot j ranks below an earlier slot i
// iff |w_j| <= |w_i| (equal magnitudes keep the lower index) -- the same set
// the rank rule above drops. One scan in index order tracks the lowest (and
// second lowest) slot as a one-hot mask: 3 (D = 1) or 6 (D = 2) operations
// per slot instead of 3 per pair.
template <int D>
__device__ __forceinline__ uint32_t drop_low_keep_bits8(const uint32_t* a) {
  uint32_t v1, b1, v2 = 0, b2 = 0;
  int j0;
  if constexpr (D == 1) {
    v1 = a[0];
    b1 = 1u;
    j0 = 1;
  } else {
    const bool c = a[1] <= a[0];            // slot 1 below slot 0
    v1 = c ? a[1] : a[0];
    b1 = c ? 2u : 1u;
    v2 = c ? a[0] : a[1];
    b2 = c ? 1u : 2u;
    j0 = 2;
  }
#pragma unroll
  for (int j = j0; j < 8; ++j) {
    const bool c1 = a[j] <= v1;
    if constexpr (D == 2) {
      const bool c2 = a[j] <= v2;
      v2 = c1 ? v1 : (c2 ? a[j] : v2);
      b2 = c1 ? b1 : (c2 ? (1u << j) : b2);
    }
    v1 = c1 ? a[j] : v1;
    b1 = c1 ? (1u << j) : b1;
  }
  return 0xFFu & ~(b1 | b2);
}

// Keep bits of a group of 8 from a short sorted list instead of all ranks:
// keep_topk_bits8<K> keeps the K highest (N = K), drop_lowk_keep_bits8<D>
// drops the D lowest (N = 8 - D). Keep priority as in the rank rule: a larger
// |w| first, equal magnitudes the lower index. One scan in index order
// inserts each slot into a list of K (or D) (magnitude, slot) entries that
// starts from sentinels: a later slot enters the kept list only if strictly
// larger than an entry, the dropped list if not larger. About 3K operations
// per slot and few registers, against 3 per pair for the rank rule.
template <int K>
__device__ __forceinline__ uint32_t keep_topk_bits8(const uint32_t* a) {
  int v[K];                                   // |w| < 2^31: every slot beats -1
  uint32_t b[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { v[k] = -1; b[k] = 0; }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int x = (int)a[j];
    bool c[K];
#pragma unroll
    for (int k = 0; k < K; ++k) c[k] = x > v[k];
#pragma unroll
    for (int k = K - 1; k >= 1; --k) {
      v[k] = c[k - 1] ? v[k - 1] : (c[k] ? x : v[k]);
      b[k] = c[k - 1] ? b[k - 1] : (c[k] ? (1u << j) : b[k]);
    }
    v[0] = c[0] ? x : v[0];
    b[0] = c[0] ? (1u << j) : b[0];
  }
  uint32_t keep = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) keep |= b[k];
  return keep;
}
template <int D>
__device__ __forceinline__ uint32_t drop_lowk_keep_bits8(const uint32_t* a) {
  uint32_t v[D], b[D];                        // every |w| is at most the sentinel
#pragma unroll
  for (int k = 0; k < D; ++k) { v[k] = 0xFFFFFFFFu; b[k] = 0; }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t x = a[j];
    bool c[D];
#pragma unroll
    for (int k = 0; k < D; ++k) c[k] = x <= v[k];
#pragma unroll
    for (int k = D - 1; k >= 1; --k) {
      v[k] = c[k - 1] ? v[k - 1] : (c[k] ? x : v[k]);
      b[k] = c[k - 1] ? b[k - 1] : (c[k] ? (1u << j) : b[k]);
    }
    v[0] = c[0] ? x : v[0];
    b[0] = c[0] ? (1u << j) : b[0];
  }
  uint32_t drop = 0;
#pragma unroll
  for (int k = 0; k < D; ++k) drop |= b[k];
  return 0xFFu & ~drop;
}

// The two slots an index-form group of 4 selects: its kept slots (bits 0..3
// of kb), completed by the lowest free slots while fewer than two are set.
__device__ __forceinline__ uint32_t select2(uint32_t kb) {
  kb &= 0xFu;
  if (__popc(kb) < 2) kb |= ~kb & (kb + 1u);
  if (__popc(kb) < 2) kb |= ~kb & (kb + 1u);
  return kb & 0xFu;
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

// ---------------------------------------------------------------------------
// Mask-then-quant (ablation, variant 2): gamma over the kept weights only.
// Sparse-BitNet summary, section 3.4 "Composition Order": W_eff =
// Q_t(W (.) M), whose scale comes from the Top-N active weights alone. The
// partial pass then needs the mask: one thread per 32-wide chunk (as in the
// mask pass) forms the keep bits with the same rank rule and adds exactly the
// kept |w| -- the same 96-bit window accumulator and LDS bins as
// k_absmean_partial, the same 16 partials per block. `vec`: every row starts
// 16-byte aligned, so whole chunks are read with 16-byte loads.
// ---------------------------------------------------------------------------
template <bool BF16, int M, int SEL>
__global__ __launch_bounds__(kAbsThreads) void k_absmean_partial_kept(
    const PrepBatchK batch, int N, bool vec, unsigned long long* __restrict__ partials_all) {
  const int item = prep_index(batch, blockIdx.x, false);
  const PrepItemK pi = prep_item(batch, item);
  const void* __restrict__ wv = pi.w;
  const uint32_t lb = blockIdx.x - pi.blk1, nblk = pi.nparts;
  __shared__ unsigned long long bins[16];
  if (threadIdx.x < 16) bins[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t C32 = (uint32_t)pi.C, K32 = (uint32_t)pi.K;
  const uint32_t total = (uint32_t)(pi.O * pi.C);
  uint32_t a0 = 0, a1 = 0, a2 = 0;
  for (uint32_t ch = lb * kAbsThreads + threadIdx.x; ch < total; ch += nblk * kAbsThreads) {
    const uint32_t o = ch / C32, c = ch - o * C32, k0 = 32u * c;
    uint32_t a[32];
    const int64_t row = (int64_t)o * pi.K + k0;
    if (vec && k0 + 32u <= K32) {
      constexpr int NV = BF16 ? 4 : 8;             // 16-byte vectors per chunk
      const uint4* src = (const uint4*)((const char*)wv + row * (BF16 ? 2 : 4));
      uint4 d[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) d[v] = src[v];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t w4[4] = {d[v].x, d[v].y, d[v].z, d[v].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if constexpr (BF16) {
            a[8 * v + 2 * h] = (w4[h] << 16) & 0x7FFFFFFFu;
            a[8 * v + 2 * h + 1] = w4[h] & 0x7FFF0000u;
          } else {
            a[4 * v + h] = w4[h] & 0x7FFFFFFFu;
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t k = k0 + (uint32_t)e;
        uint32_t u = 0;
        if (k < K32)
          u = BF16 ? ((uint32_t)((const uint16_t*)wv)[row + e] << 16) : ((const uint32_t*)wv)[row + e];
        a[e] = u & 0x7FFFFFFFu;
      }
    }
    uint32_t keep = 0;
#pragma unroll
    for (int g = 0; g < 32 / M; ++g) {
      uint32_t kb;
      if constexpr (SEL == 1) kb = drop_low_keep_bits8<1>(a + g * M);
      else if constexpr (SEL == 2) kb = drop_low_keep_bits8<2>(a + g * M);
      else if constexpr (SEL == 3) kb = 0xFFu;
      else if constexpr (SEL == 4) kb = keep_topk_bits8<2>(a + g * M);
      else if constexpr (SEL == 5) kb = keep_topk_bits8<3>(a + g * M);
      else if constexpr (SEL == 6) kb = drop_lowk_keep_bits8<3>(a + g * M);
      else if constexpr (SEL == 7) kb = keep_topk_bits8<4>(a + g * M);
      else kb = topn_keep_bits<M>(a + g * M, N);
      keep |= kb << (g * M);
    }
    bool other = false;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t u = ((keep >> e) & 1u) ? a[e] : 0u;    // dropped slots add nothing
      add96(a0, a1, a2, abs_term3(u, other));
    }
    if (other) {
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if ((keep >> e) & 1u) abs_accumulate_other(bins, a[e]);
    }
  }
  const unsigned long long lo = a0;
  const unsigned long long hi = (unsigned long long)a1 | ((unsigned long long)a2 << 32);
  const unsigned long long slo = wave_sum_u64(lo), shi = wave_sum_u64(hi);
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&bins[2 * kAbsWindow], slo);
    atomicAdd(&bins[2 * kAbsWindow + 1], shi);
  }
  __syncthreads();
  write_partial(partials_all, (int64_t)pi.part0 + lb, bins);
}

// Workgroup: one thread per chunk and one more wave that sums the tensor's
// partial records into the absmean bins and turns them into gamma, sw and the
// threshold (a serial computation) while the others stage W and rank the
// groups; the threshold is needed only for the codes.
constexpr int kQmpThreads = kChunksPerBlock + 64;
// Loads in flight when the extra wave sums full partial vectors (few
// registers: the wave shares the kernel's allocation).
constexpr int kSumUnroll = 8;
static_assert(kAbsPerTensor % 64 == 0, "compact records: whole loads per lane");

// SEL: how the mask is found -- 0: rank rule (any N); for M = 8 also
// 1: drop the lowest slot (N = 7), 2: drop the two lowest (N = 6), 3: keep
// all (N = 8), 4: keep the two highest (N = 2), 5: the three highest (N = 3),
// 6: drop the three lowest (N = 5), 7: keep the four highest (N = 4).

template <bool BF16, int M, bool IDX, int SEL>
__global__ __launch_bounds__(kQmpThreads) void k_qmp(const PrepBatchK batch, int N,
                                                     const unsigned long long* __restrict__ partials_all,
                                                     float eps) {
  const int item = prep_index(batch, blockIdx.x, true);
  const PrepItemK pi = prep_item(batch, item);
  const void* __restrict__ wv = pi.w;
  const int64_t O = pi.O, K = pi.K, C = pi.C, pitch = pi.pitch;
  const int64_t code_chunks = pi.code_chunks, mask_off = pi.mask_off;
  int8_t* __restrict__ w_eff = pi.w_eff;
  uint8_t* __restrict__ mask_out = pi.mask;
  uint8_t* __restrict__ packed = pi.packed;
  float* __restrict__ gamma_sw = pi.gamma_sw;
  float* __restrict__ sw_rows = pi.sw_rows;
  const uint32_t lb = blockIdx.x - pi.blk3;                // block within the tensor
  __shared__ __attribute__((aligned(16))) uint32_t lds[kChunksPerBlock * kLdsStride];
  __shared__ unsigned long long red[16];
  __shared__ PrepScalars scal;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave == kChunksPerBlock / 64) {
    // ---- scalar wave: partials -> 16 bins -> gamma, sw, threshold ----
    const int lane = threadIdx.x & 63;
    const int np = pi.nparts;
    const unsigned long long* __restrict__ cp =
        partials_all + (int64_t)kAbsmeanMaxBlocks * 16 + (int64_t)pi.part0 * 4;
    unsigned long long s0 = 0, s1 = 0, fl = 0;
    {
      uint4 a[kAbsPerTensor / 64], f[kAbsPerTensor / 64];   // all loads in flight
#pragma unroll
      for (int u = 0; u < kAbsPerTensor / 64; ++u) {
        const int64_t r = min(lane + 64 * u, np - 1);
        a[u] = *(const uint4*)(cp + r * 4);
        f[u] = *(const uint4*)(cp + r * 4 + 2);
      }
      // (1) W staged by the other waves. A plain barrier: this wave wrote
      // nothing they read, and its loads stay in flight across it, so the
      // sums below overlap the other waves' ranking.
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int u = 0; u < kAbsPerTensor / 64; ++u) {
        const unsigned long long m = lane + 64 * u < np ? ~0ull : 0ull;
        s0 += (((unsigned long long)a[u].y << 32) | a[u].x) & m;
        s1 += (((unsigned long long)a[u].w << 32) | a[u].z) & m;
        fl |= (unsigned long long)(f[u].x | f[u].y) & m;
      }
    }
    if (__ballot(fl != 0) == 0) {
      // every block's terms lie in window 3 (or are zero)
      s0 = wave_sum_u64(s0);
      s1 = wave_sum_u64(s1);
      if (lane < 16) red[lane] = lane == 2 * (int)kAbsWindow ? s0 : lane == 2 * (int)kAbsWindow + 1 ? s1 : 0ull;
    } else {
      // some block has terms elsewhere: sum the full vectors, 8 lanes per
      // vector (16 bytes, two bins, each), 8 vectors per load instruction
      const uint4* __restrict__ pv = (const uint4*)(partials_all + (int64_t)pi.part0 * 16);
      const int e = lane & 7, v0 = lane >> 3;
      s0 = s1 = 0;                                        // bins 2e, 2e + 1
      for (int b = 0; b < np; b += 8 * kSumUnroll) {
        uint4 d[kSumUnroll];
#pragma unroll
        for (int u = 0; u < kSumUnroll; ++u) d[u] = pv[min(b + v0 + 8 * u, np - 1) * 8 + e];
#pragma unroll
        for (int u = 0; u < kSumUnroll; ++u) {
          const unsigned long long m = b + v0 + 8 * u < np ? ~0ull : 0ull;
          s0 += (((unsigned long long)d[u].y << 32) | d[u].x) & m;
          s1 += (((unsigned long long)d[u].w << 32) | d[u].z) & m;
        }
      }
#pragma unroll
      for (int off = 8; off < 64; off <<= 1) {            // sum over the 8 vector slots
        s0 += ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(s0 >> 32), off, 64) << 32) |
              (uint32_t)__shfl_xor((int)(uint32_t)s0, off, 64);
        s1 += ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(s1 >> 32), off, 64) << 32) |
              (uint32_t)__shfl_xor((int)(uint32_t)s1, off, 64);
      }
      if (lane < 8) {
        red[2 * lane] = s0;
        red[2 * lane + 1] = s1;
      }
    }
    if (lb == 0 && lane == 0 && pi.flips) *pi.flips = 0;   // accumulated by the flips pass
    __builtin_amdgcn_wave_barrier();                    // red written (one wave: in order)
    if (lane == 0) {
      const int64_t n = pi.variant == 2 ? O * (K / M) * N : O * K;   // kept weights only
      const PrepScalars sc = scalars_from_bins(red, n, eps);
      scal = sc;
      if (lb == 0) {
        gamma_sw[0] = sc.gamma;
        gamma_sw[1] = sc.sw;
      }
    }
    __syncthreads();                                    // (2) scalars visible
    return;
  }
  // all chunk/row indices fit in 32 bits: O * C < 2^31 (O * K < 2^31)
  const uint32_t total = (uint32_t)(O * C), C32 = (uint32_t)C, K32 = (uint32_t)K;
  const uint32_t base = lb * kChunksPerBlock;

  // ---- stage: raw bits of the block's chunks x 32 elements ----
  constexpr int V = BF16 ? 8 : 4;              // elements per 16-byte piece
  constexpr int PIECES = 32 / V;               // pieces per chunk = pieces per thread
  const bool rows16 = ((K32 * (BF16 ? 2u : 4u)) % 16u) == 0;
  uint4 d[PIECES];
  if (K32 % 128u == 0 && rows16) {
    // every chunk lies inside its row and the rows are 32 * C elements long:
    // the block's chunks are one contiguous run of W. All loads unconditional
    // (clamped to the tensor's last piece; those chunks are inactive), so they
    // are all in flight together.
    const uint4* const src = (const uint4*)wv;
    const uint32_t last = total * PIECES - 1u;
#pragma unroll
    for (int q = 0; q < PIECES; ++q)
      d[q] = src[min(base * PIECES + threadIdx.x + (uint32_t)kChunksPerBlock * q, last)];
  } else {
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const uint32_t p = threadIdx.x + (uint32_t)kChunksPerBlock * q;
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
  }
#pragma unroll
  for (int q = 0; q < PIECES; ++q) {
    const uint32_t p = threadIdx.x + (uint32_t)kChunksPerBlock * q;
    const uint32_t lc = p / PIECES, pc = p % PIECES;
    const uint32_t w[4] = {d[q].x, d[q].y, d[q].z, d[q].w};
    uint32_t* dst = lds + lc * kLdsStride + pc * V;
    if constexpr (BF16) {
      *(uint4*)dst = make_uint4(w[0] << 16, w[0] & 0xFFFF0000u, w[1] << 16, w[1] & 0xFFFF0000u);
      *(uint4*)(dst + 4) =
          make_uint4(w[2] << 16, w[2] & 0xFFFF0000u, w[3] << 16, w[3] & 0xFFFF0000u);
    } else {
      *(uint4*)dst = d[q];
    }
  }
  __syncthreads();                                    // (1) W staged

  const uint32_t ch = base + threadIdx.x;
  const bool active = ch < total;
  const uint32_t o = active ? ch / C32 : 0u, c = ch - o * C32;
  const uint32_t k0 = 32u * c;

  // the mask and the signs need no scalar: computed before barrier (2)
  uint32_t a[32], sgn = 0, keep = 0;
  if (active) {
    uint32_t raw[32];
#pragma unroll
    for (int e4 = 0; e4 < 8; ++e4) {
      const uint4 v = *(const uint4*)(lds + threadIdx.x * kLdsStride + 4 * e4);
      raw[4 * e4] = v.x; raw[4 * e4 + 1] = v.y; raw[4 * e4 + 2] = v.z; raw[4 * e4 + 3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      a[e] = raw[e] & 0x7FFFFFFFu;
      sgn |= (raw[e] >> 31) << e;
    }
#pragma unroll
    for (int g = 0; g < 32 / M; ++g) {
      uint32_t kb;
      if constexpr (SEL == 1) kb = drop_low_keep_bits8<1>(a + g * M);
      else if constexpr (SEL == 2) kb = drop_low_keep_bits8<2>(a + g * M);
      else if constexpr (SEL == 3) kb = 0xFFu;
      else if constexpr (SEL == 4) kb = keep_topk_bits8<2>(a + g * M);
      else if constexpr (SEL == 5) kb = keep_topk_bits8<3>(a + g * M);
      else if constexpr (SEL == 6) kb = drop_lowk_keep_bits8<3>(a + g * M);
      else if constexpr (SEL == 7) kb = keep_topk_bits8<4>(a + g * M);
      else kb = topn_keep_bits<M>(a + g * M, N);
      keep |= kb << (g * M);
    }
  }
  __syncthreads();                                    // (2) scalars from the extra wave
  if (!active) return;
  const PrepScalars sc = scal;
  const uint32_t tb = sc.t_bits;
  uint32_t nz = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) nz |= ((tb - 1u - a[e]) >> 31) << e;   // a >= tb (both < 2^31, tb >= 1)
  const uint32_t valid = k0 >= K32 ? 0u : (K32 - k0 >= 32u ? 0xFFFFFFFFu : ((1u << (K32 - k0)) - 1u));
  if (pi.variant == 1) {
    // ablation: rank the ternary magnitudes |W_q| -- the nonzero codes first,
    // then the zero codes, each in index order
    constexpr uint32_t MM = (1u << M) - 1u;
    keep = 0;
#pragma unroll
    for (int g = 0; g < 32 / M; ++g) {
      const uint32_t z = (nz >> (g * M)) & MM;
      const int cnt = __popc(z);
      const uint32_t kg = cnt >= N ? lowest_bits(z, N) : (z | lowest_bits(~z & MM, N - cnt));
      keep |= kg << (g * M);
    }
  }
  // mask diagnostics
  {
    const uint32_t vbits = k0 >= K32 ? 0u : (K32 - k0 >= 32u ? 0xFFFFFFFFu : ((1u << (K32 - k0)) - 1u));
    if (pi.mask_bits) pi.mask_bits[(int64_t)o * C + c] = keep & vbits;
    if (pi.group_thr) {
      // largest dropped magnitude of each group (the (N+1)-th largest |w|
      // when the mask is ranked on |w|)
      constexpr int G = 32 / M;
      float* const thr = pi.group_thr + (int64_t)o * (K / M) + (int64_t)c * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint32_t t = 0;
#pragma unroll
        for (int e = 0; e < M; ++e)
          if (!((keep >> (g * M + e)) & 1u)) t = max(t, a[g * M + e]);
        if (k0 + (uint32_t)(g * M) < K32) thr[g] = __uint_as_float(t);
      }
    }
  }
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
  if (sw_rows && c == 0) sw_rows[o] = sc.sw;

  if (!packed) return;
  uint8_t* rec = packed + (int64_t)o * pitch;
  if constexpr (IDX) {
    // 8 groups of 4: selected slots i0 < i1 -- the kept ones (2:4: exactly
    // two; padding groups keep 0,1), for 2:8 completed by the lowest free
    // slots (code 0); the 2:8 mask itself goes to the mask words
    uint32_t iw = 0, lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t kb = M == 8 ? select2(keep >> (4 * q)) : (keep >> (4 * q)) & 0xFu;
      const uint32_t i0 = __builtin_ctz(kb | 0x10u);
      const uint32_t i1 = 31u - __builtin_clz(kb | 1u);
      iw |= (i0 | (i1 << 2)) << (4 * q);
      lo |= ((kn >> (4 * q + i0)) & 1u) << (2 * q) | ((kn >> (4 * q + i1)) & 1u) << (2 * q + 1);
      hi |= ((kneg >> (4 * q + i0)) & 1u) << (2 * q) | ((kneg >> (4 * q + i1)) & 1u) << (2 * q + 1);
    }
    *(uint2*)(rec + 8 * c) = make_uint2(byte_slice16(lo, hi), iw);
    if constexpr (M == 8) *(uint32_t*)(rec + mask_off + 4 * c) = keep & valid;
  } else {
    const uint32_t w0 = byte_slice16(kn & 0xFFFFu, kneg & 0xFFFFu);
    const uint32_t w1 = byte_slice16(kn >> 16, kneg >> 16);
    if (c < (uint32_t)code_chunks) *(uint2*)(rec + 8 * c) = make_uint2(w0, w1);
    *(uint32_t*)(rec + mask_off + 4 * c) = keep & valid;
  }
}

// Mask flips against the previous step's keep bits (both in the word layout
// of mask_bits), for the tensors that ask for them: a grid-stride popcount
// of (cur ^ prev), summed in LDS, one atomic per workgroup (the counter was
// zeroed by the mask pass). Same-address atomics from every workgroup of
// the mask pass would serialize; kFlipBlocks per tensor keeps them few.
constexpr int kFlipBlocks = 64;
__global__ __launch_bounds__(256) void k_mask_flips(const PrepBatchK batch) {
  const int item = blockIdx.x / kFlipBlocks, lb = blockIdx.x % kFlipBlocks;
  const PrepItemK pi = prep_item(batch, item);
  if (!pi.flips) return;                               // uniform per workgroup
  const int64_t n = pi.O * (int64_t)pi.C;
  uint32_t cnt = 0;
  for (int64_t i = (int64_t)lb * 256 + threadIdx.x; i < n; i += (int64_t)kFlipBlocks * 256)
    cnt += (uint32_t)__popc(pi.mask_bits[i] ^ pi.prev_mask_bits[i]);
  __shared__ uint32_t part[4];
  const uint32_t w = wave_sum_u32(cnt);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = part[0] + part[1] + part[2] + part[3];
    if (t) atomicAdd(pi.flips, (unsigned long long)t);
  }
}

hipError_t launch_quant_mask_weight(const PrepTensor* items, int count, bool bf16, int N, int M,
                                    float eps, void* ws, hipStream_t s) {
  PrepBatchK b{};
  b.count = count;
  const int V = bf16 ? 8 : 4;
  const int cap = std::min(kAbsPerTensor, kAbsBlocks / count);   // partial vectors per tensor
  int parts = 0, blk3 = 0;
  for (int i = 0; i < count; ++i) {
    const PrepTensor& t = items[i];
    PrepItemK& k = b.it[i];
    k.w = t.w;
    k.w_eff = t.w_eff;
    k.mask = t.mask;
    k.packed = (uint8_t*)t.packed;
    k.gamma_sw = t.gamma_sw;
    k.sw_rows = t.sw_rows;
    k.mask_bits = t.mask_bits;
    k.prev_mask_bits = t.prev_mask_bits;
    k.flips = t.flips;
    k.group_thr = t.group_thr;
    k.variant = t.variant;
    k.pad_v = 0;
    k.O = t.O;
    k.K = t.K;
    k.C = (int32_t)row_chunks(t.K);
    k.pitch = (int32_t)row_pitch(t.K, N, M);
    k.code_chunks = (int32_t)(dense_code_bytes(t.K) / 8);
    k.mask_off = (int32_t)mask_area_offset(t.K, N, M);
    // about one batch of loads per thread (the exact accumulation is VALU
    // work: spread it over many waves)
    // (variant 2: one chunk of 32 per thread and step)
    const int64_t want = t.variant == 2 ? cdiv(t.O * (int64_t)row_chunks(t.K), (int64_t)kAbsThreads)
                                        : cdiv(cdiv(t.O * t.K, V), (int64_t)kAbsThreads * kAbsBatch);
    const int nb = (int)(want < 1 ? 1 : (want > cap ? cap : want));
    k.part0 = parts;
    k.nparts = nb;
    k.blk1 = parts;
    parts += nb;
    k.blk3 = blk3;
    blk3 += (int)cdiv(t.O * (int64_t)k.C, kChunksPerBlock);
  }
  auto* partials = (unsigned long long*)ws;
  if (items[0].variant == 2) {   // a batch is all of variant 2 or none (checked by the caller)
    bool vec = true;               // (w itself is 16-byte aligned)
    for (int i = 0; i < count; ++i) vec = vec && (items[i].K * (bf16 ? 2 : 4)) % 16 == 0;
#define SBL_KEPT(BV, MV, SV) \
    hipLaunchKernelGGL((k_absmean_partial_kept<BV, MV, SV>), dim3(parts), dim3(kAbsThreads), 0, s, b, N, vec, partials)
#define SBL_KEPT_NM(BV)                                             \
    if (M == 4) SBL_KEPT(BV, 4, 0);                                   \
    else if (N == 8) SBL_KEPT(BV, 8, 3);                              \
    else if (N == 7) SBL_KEPT(BV, 8, 1);                              \
    else if (N == 6) SBL_KEPT(BV, 8, 2);                              \
    else if (N == 2) SBL_KEPT(BV, 8, 4);                              \
    else if (N == 3) SBL_KEPT(BV, 8, 5);                              \
    else if (N == 5) SBL_KEPT(BV, 8, 6);                              \
    else if (N == 4) SBL_KEPT(BV, 8, 7);                              \
    else SBL_KEPT(BV, 8, 0)
    if (bf16) { SBL_KEPT_NM(true); } else { SBL_KEPT_NM(false); }
#undef SBL_KEPT_NM
#undef SBL_KEPT
  } else if (bf16) {
    hipLaunchKernelGGL((k_absmean_partial<true>), dim3(parts), dim3(kAbsThreads), 0, s, b, partials);
  } else {
    hipLaunchKernelGGL((k_absmean_partial<false>), dim3(parts), dim3(kAbsThreads), 0, s, b, partials);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)blk3), block(kQmpThreads);
#define SBL_QMP(BV, MV, IV, SV) \
  hipLaunchKernelGGL((k_qmp<BV, MV, IV, SV>), grid, block, 0, s, b, N, partials, eps)
#define SBL_QMP8(BV)                        \
  if (N == 8) SBL_QMP(BV, 8, false, 3);     \
  else if (N == 7) SBL_QMP(BV, 8, false, 1); \
  else if (N == 6) SBL_QMP(BV, 8, false, 2); \
  else if (N == 5) SBL_QMP(BV, 8, false, 6); \
  else if (N == 3) SBL_QMP(BV, 8, false, 5); \
  else if (N == 4) SBL_QMP(BV, 8, false, 7); \
  else SBL_QMP(BV, 8, false, 0)
  if (bf16) {
    if (index_form(N, M)) { if (M == 4) SBL_QMP(true, 4, true, 0); else SBL_QMP(true, 8, true, 4); }
    else if (M == 4) SBL_QMP(true, 4, false, 0);
    else SBL_QMP8(true);
  } else {
    if (index_form(N, M)) { if (M == 4) SBL_QMP(false, 4, true, 0); else SBL_QMP(false, 8, true, 4); }
    else if (M == 4) SBL_QMP(false, 4, false, 0);
    else SBL_QMP8(false);
  }
#undef SBL_QMP8
#undef SBL_QMP
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool any_flips = false;
  for (int i = 0; i < count; ++i) any_flips |= items[i].flips != nullptr;
  if (any_flips) hipLaunchKernelGGL(k_mask_flips, dim3(count * kFlipBlocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone pack / unpack, one thread per 32-wide chunk of a row record.
// ---------------------------------------------------------------------------
template <bool IDX>
__global__ __launch_bounds__(256) void k_pack(bool with_mask, const int8_t* __restrict__ w_eff,
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
    if (with_mask) *(uint32_t*)(rec + mask_off + 4 * c) = keep;   // 2:8: the mask itself
    if (k0 >= K) keep = 0x33333333u;            // padding groups keep slots (0, 1)
    else if (K - k0 < 32) keep |= 0x33333333u & ~((1u << (K - k0)) - 1u);
    uint32_t cw = 0, iw = 0;
    for (int q = 0; q < 8; ++q) {
      const uint32_t kb = select2(keep >> (4 * q));     // (2:4 groups already hold two)
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
__global__ __launch_bounds__(256) void k_unpack(bool with_mask, const uint8_t* __restrict__ packed, int64_t O,
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
    if (with_mask) keep = *(const uint32_t*)(rec + mask_off + 4 * c);   // 2:8
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
  const bool with_mask = index_form(N, M) && M == 8;
  if (index_form(N, M))
    hipLaunchKernelGGL((k_pack<true>), grid, block, 0, s, with_mask, w_eff, mask, O, K, C,
                       (uint8_t*)packed, row_pitch(K, N, M), dense_code_bytes(K) / 8,
                       mask_area_offset(K, N, M));
  else
    hipLaunchKernelGGL((k_pack<false>), grid, block, 0, s, false, w_eff, mask, O, K, C,
                       (uint8_t*)packed, row_pitch(K, N, M), dense_code_bytes(K) / 8,
                       mask_area_offset(K, N, M));
  return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, int64_t O, int64_t K, int N, int M, int8_t* w_eff,
                         uint8_t* mask, hipStream_t s) {
  const int64_t C = row_chunks(K);
  const dim3 grid((unsigned)cdiv(O * C, 256)), block(256);
  const bool with_mask = index_form(N, M) && M == 8;
  if (index_form(N, M))
    hipLaunchKernelGGL((k_unpack<true>), grid, block, 0, s, with_mask, (const uint8_t*)packed, O,
                       K, C, row_pitch(K, N, M), mask_area_offset(K, N, M), w_eff, mask);
  else
    hipLaunchKernelGGL((k_unpack<false>), grid, block, 0, s, false, (const uint8_t*)packed, O, K,
                       C, row_pitch(K, N, M), mask_area_offset(K, N, M), w_eff, mask);
  return hipGetLastError();
}

}  // namespace sbl
