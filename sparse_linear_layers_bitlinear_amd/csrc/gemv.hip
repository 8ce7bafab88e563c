// a5 + a6 (and a1, fused) for decode-sized batches of at most 16 tokens: a
// streaming GEMV on the matrix cores.
//
// Sparse-BitNet summary, section 3.4 "Activation quantization" and "The Full
// Sparse-BitLinear Layer" (Eq. 4): per token x~ = Clip(x * 127 / (max|x| +
// eps), -128, 127), and y = (W_eff x~) scaled by the token's and the weight's
// scale. BitNet b1.58 2B4T summary, section 3.4 (per-token absmax, nearest
// rounding).
//
// With T <= 16 each packed weight byte meets at most 16 tokens: the work is
// bound by the HBM reads of the packed W, and with so little arithmetic per
// workgroup the instructions a wavefront executes once (not in a loop) are
// what the latency is made of. So every phase is either a handful of
// instructions or a short loop:
//  - the tokens are split into groups and the 16-row tiles of W evenly into
//    slices, one workgroup of 8 wavefronts per (group, slice) and at most one
//    per compute unit; each workgroup quantizes only its group's rows (that
//    VALU work grows with tokens x K, so long rows take small groups when
//    there are few tiles) and the groups of one slice share its W through
//    their XCD's L2. A workgroup copies all of its packed W
//    straight into LDS with 16-byte LDS-DMA loads (one instruction moves 1 KB:
//    16 rows x two K-steps), issued at the start so the whole weight stream is
//    in flight at once;
//  - the T activation rows are quantized by the first XW wavefronts (a token
//    is shared by 64 XW / T' threads, T' = T rounded up to a power of two; with
//    one wavefront per token its maximum needs no barrier), into int8 rows in
//    LDS -- the same arithmetic as the stand-alone quantizer, so the codes are
//    identical -- or, when xq is given, copied by LDS-DMA. For T <= 8 (when a
//    row fits), XW = 4 and the other four wavefronts issue the weight copies:
//    a wave's loads complete in order, so the quantizing waves then wait for x
//    alone and quantize while the weights are in flight;
//  - the waves then split the K-steps of each tile (MFMA A operand = 8 bytes of
//    packed W per lane and K-step, the operand layout of the prefill kernel;
//    B = the int8 rows, columns t >= T read row T-1 and are never stored),
//    add their int32 partial sums into LDS (ds_add, exact), and the
//    workgroup dequantizes y = fp32(fp32(acc * s_x) * s_w).
#include "sbl_internal.h"
#include "device_util.h"

#include <cstdlib>

namespace sbl {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecMaxVec = 16;               // 16-byte activation vectors per thread
constexpr int kDecMaxLds = 150 * 1024;       // dynamic LDS limit of the decode kernel

struct DecodeArgs {
  const void* x;          // XM 0: xq int8 [T, K]; XM 1 / 2: x bf16 / fp32 [T, K]
  const float* sx;        // XM 0: per-token scales
  float eps;              // XM 1 / 2: activation epsilon
  const uint8_t* packed;  // packed rows, pitch bytes each
  int pitch;
  const float* sw;        // weight scale(s), element o at o * sw_inc
  int sw_inc;
  int T, O, K, R;         // R: most tiles of one workgroup
  int tq, trem;           // tiles per slice: tq, one more for the first trem
  int S, tg;              // row-tile slices; tokens per workgroup (token group)
  int lg;                 // log2 of the threads per token (dec_group)
  int xw;                 // wavefronts that quantize x (4 or 8; the rest copy W)
  void* y;                // [T, O] bf16 or fp32
  int32_t* acc;           // optional [T, O] int32
};

// LDS: W [R][np][1 KB] | xs [tg][xpitch] int8 | sxs [16] f32 | pmax [16] u32 (per half-wave) |
//      red [R][4][64] i32     (np = pairs of K-steps; value k of lane l at 64 k + l)
__host__ __device__ inline int dec_np(int K) { return ((K + 127) / 128 + 1) / 2; }
__host__ __device__ inline int dec_xpitch(int K) { return 128 * ((K + 127) / 128) + 16; }
__host__ __device__ inline int dec_off_x(int K, int R) { return R * dec_np(K) * 1024; }
__host__ __device__ inline int dec_off_sx(int T, int K, int R) {
  return dec_off_x(K, R) + ((T * dec_xpitch(K) + 15) & ~15);
}
__host__ __device__ inline int dec_lds(int T, int K, int R) {
  return dec_off_sx(T, K, R) + 64 + 64 + R * 1024;
}
// threads per token: (quantizing threads) / (T rounded up to a power of two)
__host__ __device__ inline int dec_group(int T, int threads = kDecThreads) {
  int tp = 1;
  while (tp < T) tp <<= 1;
  return threads / tp;
}

// max over each row of 16 lanes, left in the row's lane 15 (row_shr 1, 2, 4, 8;
// lanes without a source keep 0, the identity of an unsigned max)
__device__ __forceinline__ uint32_t row_max_dpp(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x111, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x112, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, false));
  return m;
}

__device__ __forceinline__ v4i expand4(uint32_t w) {
  return v4i{(int)expand_codes(w, 0), (int)expand_codes(w, 1), (int)expand_codes(w, 2),
             (int)expand_codes(w, 3)};
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Workgroup barrier that waits only for the wave's LDS operations. A
// workgroup-scope fence (so __syncthreads()) also waits for every outstanding
// global load -- here the weight copies still in flight into LDS. The
// wavefront-scope fences keep the compiler from moving memory operations
// across the barrier and emit no wait; the explicit lgkmcnt(0) completes the
// wave's LDS writes before it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The MMA phase of one wavefront when the workgroup has two or more tiles:
// K-steps s = wave + 8 (c0 + i), i < KU, of every tile, for chunks c0 = 0,
// KU, ... of its nsw K-steps. A K-step's activation fragments are the same
// for every tile, so they are read from LDS once per chunk, and each tile's W
// fragments are read while the tile before it is computed. Reads past the
// wave's last K-step repeat it (in bounds; never computed). The int32 sums go
// to the tile's LDS accumulator (red + 256 r; this lane's k-th at rl + 64 k) by
// ds_add.
template <bool SP, int KU>
__device__ __forceinline__ void mma_tiles(const uint8_t* wsm, const int8_t* xr, int aoff, int wave,
                                          int nsw, int np, int ntb, int g, int* rl) {
  for (int c0 = 0; c0 < nsw; c0 += KU) {
    const int nc = min(KU, nsw - c0);
    int woff[KU];
    v4i xa[KU], xb[KU];
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int s = wave + kDecWaves * (c0 + min(i, nc - 1));
      woff[i] = (s >> 1) * 1024 + 512 * (s & 1) + aoff;
      const int kb = 128 * s;
      xa[i] = *(const v4i*)(xr + kb + (SP ? 16 : 32) * g);
      xb[i] = *(const v4i*)(xr + kb + (SP ? 64 + 16 * g : 32 * g + 16));
    }
    uint2 wa[KU], wb[KU];
    // tile r from cur (read earlier) while tile r + 1 is read into nxt; two
    // tiles per trip, so the buffers swap roles without register copies
    auto tile = [&](int r, const uint2 (&cur)[KU], uint2 (&nxt)[KU]) {
      if (r + 1 < ntb) {
        const uint8_t* const wr = wsm + (r + 1) * np * 1024;
#pragma unroll
        for (int i = 0; i < KU; ++i) nxt[i] = *(const uint2*)(wr + woff[i]);
      }
      v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < KU; ++i) {
        if (i < nc) {                                    // (uniform)
          v4i& acc = (i & 1) ? acc1 : acc0;
          if constexpr (SP)
            acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(
                expand4(cur[i].x),
                v8i{xa[i][0], xa[i][1], xa[i][2], xa[i][3], xb[i][0], xb[i][1], xb[i][2], xb[i][3]},
                acc, (int)cur[i].y, 0, 0);
          else {
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand4(cur[i].x), xa[i], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand4(cur[i].y), xb[i], acc, 0, 0, 0);
          }
        }
      }
      acc0 += acc1;
      int* const rp = rl + r * 256;
      atomicAdd(rp + 0, acc0[0]);
      atomicAdd(rp + 64, acc0[1]);
      atomicAdd(rp + 128, acc0[2]);
      atomicAdd(rp + 192, acc0[3]);
    };
#pragma unroll
    for (int i = 0; i < KU; ++i) wa[i] = *(const uint2*)(wsm + woff[i]);
    for (int r = 0; r < ntb; r += 2) {
      tile(r, wa, wb);
      if (r + 1 < ntb) tile(r + 1, wb, wa);
    }
  }
}

// XM: 0 = xq given, 1 = bf16 x, 2 = fp32 x. NV: most activation vectors of
// one thread (the loads and codes are unrolled NV times; few is faster).
template <bool SP, int XM, bool YBF16, int NV>
__global__ __launch_bounds__(kDecThreads) void k_decode(const DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int O = a.O, K = a.K;
  const int ns = (K + 127) >> 7, np = (ns + 1) >> 1;   // K-steps, pairs of K-steps
  const int XP = dec_xpitch(K);
  uint8_t* const wsm = smem;
  int8_t* const xs = (int8_t*)(smem + dec_off_x(K, a.R));
  float* const sxs = (float*)(smem + dec_off_sx(a.tg, K, a.R));
  uint32_t* const pmax = (uint32_t*)(sxs + 16);
  int* const red = (int*)(pmax + 16);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  // workgroup b = (token group) * S + (slice): the slice's 16-row tiles
  // [tb, tb + ntb) of the (O + 15) / 16 (even split, quotient and remainder
  // from the host) for the group's tokens [t0, t0 + T). With S a multiple of
  // 8 the token groups of one slice run on one XCD and share its W in L2.
  const int bx = blockIdx.x;
  const int grp = bx / a.S, slice = bx - grp * a.S;
  const int t0 = grp * a.tg;
  const int T = min(a.tg, a.T - t0);                     // this workgroup's tokens
  const int tb = slice * a.tq + min(slice, a.trem);
  const int ntb = a.tq + (slice < a.trem ? 1 : 0);
  // the weight scales of this thread's first output item (loaded now, so the
  // epilogue does not wait for them)
  float swp[4];
  {
    const int o = (tb + (tid >> 6)) * 16 + 4 * ((tid >> 4) & 3);
#pragma unroll
    for (int r = 0; r < 4; ++r) swp[r] = a.sw[(int64_t)min(o + r, O - 1) * a.sw_inc];
  }

  // activations of the thread's token (XM 1 / 2), loaded first: waiting for
  // them then does not wait for the W copies issued after them
  constexpr bool BF = XM == 1;
  constexpr int EV = XM == 0 ? 16 : BF ? 8 : 4;         // elements per 16-byte vector
  const int nvr = K / EV;                                // vectors per row
  const int XW = XM == 0 ? kDecWaves : a.xw;             // quantizing wavefronts
  const bool xwave = wave < XW;                          // (wave-uniform)
  const int lg = a.lg, G = 1 << lg;                      // threads per token
  const int tt = min(tid >> lg, T - 1), col = tid & (G - 1);   // token and first vector
  const bool tok = (tid >> lg) < T;                      // thread has a token
  const int nvt = (nvr + G - 1) >> lg;                   // vectors per thread (uniform)
  static_assert(NV <= kDecMaxVec, "activation registers");
  uint4 v[NV];
  if constexpr (XM != 0) {
    if (xwave) {
      const uint4* const row = (const uint4*)a.x + (int64_t)(t0 + tt) * nvr;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i < nvt) v[i] = row[min(col + G * i, nvr - 1)];   // clamped duplicates are harmless
    }
  }

  // packed W -> LDS: job j = (tile j / np, pair j % np), one DMA per wave and
  // job. Lane l moves 16 bytes of row l % 16 at byte 64 p + 16 (l / 16); the
  // second step of a last odd pair re-reads the first (it is never computed).
  // (by the wavefronts that do not quantize, when XW = 4: a wave's loads
  // complete in order, so the quantizing waves then wait for x alone)
  const int dw0 = XW < kDecWaves ? XW : 0, ndw = kDecWaves - dw0;
  if (wave >= dw0)
  for (int j = wave - dw0, r = j / np, p = j - r * np; j < ntb * np; j += ndw) {
    const int ch = lane >> 4;
    const int chs = (2 * p + (ch >> 1) < ns) ? ch : ch - 2;
    const int o = min((tb + r) * 16 + r16, O - 1);
    dma16(a.packed + (int64_t)o * a.pitch + 64 * p + 16 * chs, wsm + j * 1024);
    for (p += ndw; p >= np; p -= np) ++r;                // (r, p) of job j + ndw
  }
  for (int i = tid; i < ntb * 256; i += kDecThreads) red[i] = 0;

  if constexpr (XM == 0) {
    // xq rows -> LDS by DMA (K % 16 == 0): job (token t, 1 KB piece q)
    const int nq = (K + 1023) >> 10;
    const int8_t* const xq = (const int8_t*)a.x;
    for (int j = wave; j < T * nq; j += kDecWaves) {
      const int t = j / nq, q = j - t * nq;
      if (1024 * q + 16 * lane < K)
        dma16(xq + (int64_t)(t0 + t) * K + 1024 * q + 16 * lane, (uint8_t*)xs + t * XP + 1024 * q);
    }
    if (tid < T) sxs[tid] = a.sx[t0 + tid];
  } else {
    // per-token max over the token's G threads: within each wave by DPP (lane
    // 31 holds the max of lanes 0-31, lane 63 that of 32-63 or of the whole
    // wave), then over the token's waves through LDS
    uint32_t m = 0;
    if constexpr (BF) {
      // bf16 pairs with the signs cleared, as packed u16 (magnitudes order as
      // integers): packed maxima, then the larger half, as an fp32 pattern
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      auto mag = [](uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu); };
      u16x2 pm = {0, 0};
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (xwave && i < nvt)
          pm = __builtin_elementwise_max(
              pm, __builtin_elementwise_max(
                      __builtin_elementwise_max(mag(v[i].x), mag(v[i].y)),
                      __builtin_elementwise_max(mag(v[i].z), mag(v[i].w))));
      m = (uint32_t)max(pm.x, pm.y) << 16;
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (xwave && i < nvt) m = max(m, absmax_vec<BF>(v[i]));
    }
    m = row_max_dpp(m);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x142, 0xA, 0xF, false));
    if (G >= 64) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x143, 0xC, 0xF, false));
    const uint32_t m_lo = __builtin_amdgcn_readlane(m, 31), m_hi = __builtin_amdgcn_readlane(m, 63);
    // a wavefront that holds whole tokens (G = 64: one; G = 32: one per half)
    // has their maxima in lanes 63 and 31: no barrier
    uint32_t mt = (G == 32 && lane < 32) ? m_lo : m_hi;
    if (G > 64) {                                        // (uniform over the workgroup)
      if (lane == 0 && xwave) {
        pmax[2 * wave] = G >= 64 ? m_hi : m_lo;
        pmax[2 * wave + 1] = m_hi;
      }
      lds_barrier();
      if (xwave) {
        // all 16 partial maxima at once (constant indices: no dependent reads;
        // only in the quantizing waves: a compiled LDS read after the W
        // copies waits for all of them)
        uint32_t pm[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 q4 = *(const uint4*)(pmax + 4 * k);
          pm[4 * k] = q4.x; pm[4 * k + 1] = q4.y; pm[4 * k + 2] = q4.z; pm[4 * k + 3] = q4.w;
        }
        mt = 0;
        const int w0 = tt << (lg - 6), w1 = (tt + 1) << (lg - 6);   // the token's waves
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w)
          if (w >= w0 && w < w1) mt = max(mt, pm[2 * w]);
      }
    }
    const ActScale sc = act_scale(mt, a.eps);
    if (col == 0 && tok && xwave) sxs[tt] = sc.s;
    int8_t* const xrow = xs + tt * XP;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = col + G * i;
      if (xwave && i < nvt && c < nvr && tok) {
        const uint2 q = act_codes_vec<BF>(v[i], sc.q);
        if constexpr (BF) *(uint2*)(xrow + c * EV) = q;
        else *(uint32_t*)(xrow + c * EV) = q.x;
      }
    }
  }
  // columns K .. 128 * ns of every row are zero (they meet the padding of the
  // last K-step's codes)
  const int tail = 128 * ns - K;
  if (tail > 0)
    for (int i = tid; i < T * tail; i += kDecThreads) xs[(i / tail) * XP + K + i % tail] = 0;
  __builtin_amdgcn_s_waitcnt(0);    // this wave's LDS-DMA copies have landed ...
  __syncthreads();                   // ... and every wave's

  // K-steps s = wave, wave + 8, ... of every tile, two accumulators
  const int8_t* const xr = xs + min(r16, T - 1) * XP;
  const int aoff = 16 * r16 + 8 * (g & 1) + 256 * (g >> 1);
  auto unit = [&](int r, int s, v4i& acc) {
    const uint2 w = *(const uint2*)(wsm + (r * np + (s >> 1)) * 1024 + 512 * (s & 1) + aoff);
    const int kb = 128 * s;
    if constexpr (SP) {
      const v4i lo = *(const v4i*)(xr + kb + 16 * g);
      const v4i hi = *(const v4i*)(xr + kb + 64 + 16 * g);
      acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(
          expand4(w.x), v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, acc, (int)w.y,
          0, 0);
    } else {
      const v4i b0 = *(const v4i*)(xr + kb + 32 * g);
      const v4i b1 = *(const v4i*)(xr + kb + 32 * g + 16);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand4(w.x), b0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand4(w.y), b1, acc, 0, 0, 0);
    }
  };
  // the wave's K-steps (uniform); several tiles with at most 4 K-steps per
  // wave (K <= 4096): activation fragments read once, W one tile ahead (with
  // more K-steps the reads issued up front cost more than the reuse saves)
  const int nsw = wave < ns ? (ns - 1 - wave) / kDecWaves + 1 : 0;
  if (ntb >= 2 && nsw <= 4) {
    int* const rl = red + lane;
    if (nsw <= 2) mma_tiles<SP, 2>(wsm, xr, aoff, wave, nsw, np, ntb, g, rl);
    else mma_tiles<SP, 4>(wsm, xr, aoff, wave, nsw, np, ntb, g, rl);
  } else {
    for (int r = 0; r < ntb; ++r) {
      v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
      int s = wave;
      for (; s + kDecWaves < ns; s += 2 * kDecWaves) {
        unit(r, s, acc0);
        unit(r, s + kDecWaves, acc1);
      }
      if (s < ns) unit(r, s, acc0);
      acc0 += acc1;
      if (wave < ns) {
        // (k-major: the 64 lanes of one add hit 64 consecutive words, no
        // bank conflicts; lane-major quads put 8 lanes on each bank)
        int* const rp = red + r * 256 + lane;
        atomicAdd(rp + 0, acc0[0]);
        atomicAdd(rp + 64, acc0[1]);
        atomicAdd(rp + 128, acc0[2]);
        atomicAdd(rp + 192, acc0[3]);
      }
    }
  }
  __syncthreads();

  // lane l of tile r: outputs o = 16 (tb + r) + 4 (l / 16) + 0..3 of token l % 16
  auto rsum = [&](int i) {
    const int* const p = red + (i >> 6) * 256 + (i & 63);
    return v4i{p[0], p[64], p[128], p[192]};
  };
  for (int i = tid; i < ntb * 64; i += kDecThreads) {
    const int t = i & 15, o = (tb + (i >> 6)) * 16 + 4 * ((i >> 4) & 3);
    if (i != tid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) swp[k] = a.sw[(int64_t)min(o + k, O - 1) * a.sw_inc];
    }
    if (t < T && o < O)
      store_tile_sw<YBF16>(a.y, a.acc, rsum(i), t0 + t, o, O, sxs[t], swp);
  }
}

// Launch plan: the T tokens are split into groups of tg (the last may be
// shorter) and the 16-row tiles into S slices; one workgroup per (group,
// slice), at most one per compute unit, the groups of a slice on one XCD so
// that W comes from HBM once and from that XCD's L2 for the others. Every
// workgroup quantizes its group's rows itself (a whole row's maximum sets a
// token's scale), work that grows with tg * K, while more groups leave fewer
// slices, so more tiles -- R * np KB of W to copy and multiply -- per
// workgroup. The plan takes the tg among T, T/2, T/4, ... (rounded up) with
// the least tg * K + kDecElemsPerKB * R * np whose LDS and per-thread
// activation vectors fit: measured on 2560- and 6912-wide rows, about 600
// activation elements per workgroup cost as much as one more KB of W.
constexpr int kDecElemsPerKB = 600;
struct DecPlan {
  int tg, ng, S, R, tq, trem, blocks;
};
DecPlan dec_plan_tg(int64_t T, int64_t ntiles, int cus, int64_t tg) {
  DecPlan p{};
  p.tg = (int)tg;
  p.ng = (int)cdiv(T, tg);
  const char* ev = std::getenv("SBL_DECODE_BLOCKS");  // tuning override: slices
  int64_t S = ev ? std::atoi(ev) : 0;
  if (S < 1) {
    S = cus / p.ng;
    if (S >= 8) S = S / 8 * 8;                        // token groups of a slice on one XCD
    if (S < 1) S = 1;
  }
  if (S > ntiles) S = ntiles;
  p.S = (int)S;
  p.R = (int)cdiv(ntiles, S);
  p.tq = (int)(ntiles / S);
  p.trem = (int)(ntiles % S);
  p.blocks = p.S * p.ng;
  return p;
}
bool dec_plan_fits(const DecPlan& p, int64_t K, int xmode) {
  const int64_t nvr = K / (xmode == 0 ? 16 : xmode == 1 ? 8 : 4);   // vectors per row
  if (xmode != 0 && cdiv(nvr, dec_group(p.tg)) > kDecMaxVec) return false;
  return dec_lds(p.tg, (int)K, p.R) <= kDecMaxLds;
}
DecPlan dec_plan(int64_t T, int64_t O, int64_t K, int xmode) {
  const int64_t ntiles = cdiv(O, 16);
  const int cus = device_info().cus;
  const char* et = std::getenv("SBL_DECODE_TG");      // tuning override
  if (et && std::atoi(et) >= 1) return dec_plan_tg(T, ntiles, cus, std::min<int64_t>(T, std::atoi(et)));
  DecPlan best = dec_plan_tg(T, ntiles, cus, T);
  if (xmode == 0) return best;                        // (xq given: nothing to quantize)
  bool have = dec_plan_fits(best, K, xmode);
  int64_t best_cost = T * K + (int64_t)kDecElemsPerKB * best.R * dec_np((int)K);
  for (int64_t tg = T; tg > 1;) {
    tg = (tg + 1) / 2;
    const DecPlan p = dec_plan_tg(T, ntiles, cus, tg);
    if (!dec_plan_fits(p, K, xmode)) continue;
    const int64_t cost = tg * K + (int64_t)kDecElemsPerKB * p.R * dec_np((int)K);
    if (!have || cost < best_cost) {
      best = p;
      best_cost = cost;
      have = true;
    }
  }
  return best;
}

template <bool SP, int XM, bool YBF16, int NV>
hipError_t run_decode(const DecodeArgs& a, int blocks, hipStream_t s) {
  auto kern = k_decode<SP, XM, YBF16, NV>;
  const int lds = dec_lds(a.tg, a.K, a.R);
  if (lds > 65536) {
    static int set = 0;   // the attribute is per kernel; raised as needed
    if (lds > set) {
      const hipError_t e =
          hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      set = lds;
    }
  }
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kDecThreads), lds, s, a);
  return hipGetLastError();
}

template <bool SP, bool YBF16>
hipError_t dispatch_x(int xmode, int nv, const DecodeArgs& a, int blocks, hipStream_t s) {
  if (xmode == 0) return run_decode<SP, 0, YBF16, 1>(a, blocks, s);
  if (xmode == 1) {
    if (nv <= 4) return run_decode<SP, 1, YBF16, 4>(a, blocks, s);
    if (nv <= 8) return run_decode<SP, 1, YBF16, 8>(a, blocks, s);
    return run_decode<SP, 1, YBF16, kDecMaxVec>(a, blocks, s);
  }
  if (nv <= 4) return run_decode<SP, 2, YBF16, 4>(a, blocks, s);
  if (nv <= 8) return run_decode<SP, 2, YBF16, 8>(a, blocks, s);
  return run_decode<SP, 2, YBF16, kDecMaxVec>(a, blocks, s);
}

}  // namespace

bool decode_fits(int64_t T, int64_t O, int64_t K, int N, int M, int xmode) {
  if (T < 1 || T > 16 || O < 1 || K < 1 || K % 16 != 0) return false;
  if (O * row_pitch(K, N, M) >= (int64_t(1) << 31)) return false;
  if (K > (1 << 20)) return false;                    // (LDS holds far less)
  return dec_plan_fits(dec_plan(T, O, K, xmode), K, xmode);
}

hipError_t launch_decode(const void* x, int xmode, const float* sx, float eps, const void* packed,
                         const float* sw, int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N,
                         int M, void* y, bool y_bf16, int32_t* acc, hipStream_t s) {
  if (!decode_fits(T, O, K, N, M, xmode)) return hipErrorInvalidValue;
  const DecPlan p = dec_plan(T, O, K, xmode);
  const int blocks = p.blocks;
  // four quantizing wavefronts when a token gets at least half of one of them
  // (tg <= 8) and its vectors fit their registers; else all eight
  const int64_t nvr = K / (xmode == 1 ? 8 : 4);
  const int xw = (xmode != 0 && p.tg <= 8 && cdiv(nvr, dec_group(p.tg, 256)) <= kDecMaxVec) ? 4 : 8;
  int lg = 0;                                  // log2 of the threads per token
  while ((1 << lg) < dec_group(p.tg, 64 * xw)) ++lg;
  const DecodeArgs a{x, sx, eps, (const uint8_t*)packed, (int)row_pitch(K, N, M), sw,
                     (int)sw_inc, (int)T, (int)O, (int)K, p.R, p.tq, p.trem, p.S, p.tg, lg,
                     xw, y, acc};
  const int nv = xmode == 0 ? 0 : (int)cdiv(nvr, (int64_t)1 << lg);   // vectors per thread
  if (index_form(N, M))
    return y_bf16 ? dispatch_x<true, true>(xmode, nv, a, blocks, s)
                  : dispatch_x<true, false>(xmode, nv, a, blocks, s);
  return y_bf16 ? dispatch_x<false, true>(xmode, nv, a, blocks, s)
                : dispatch_x<false, false>(xmode, nv, a, blocks, s);
}

}  // namespace sbl
