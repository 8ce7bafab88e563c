// Backward of the Sparse-BitLinear layer under the Dual straight-through
// estimator (Sparse-BitNet summary, section 3.4 "Gradient Estimation: The
// Dual Straight-Through Estimator" and the backward walk-through of
// Algorithm 1 / Algorithm 2): with the forward y = x~ W~^T, where
// x~ = sx * xq is the dequantized int8 activation and W~ = sw * W_eff the
// scaled ternary-and-masked weight,
//   dX = dY W~            (gradient at x~; identity through Q_a)
//   dW = dY^T x~          (gradient at W~, handed unchanged to every master
//                          weight: neither the mask nor RoundClip blocks it)
// Both are dense contractions, so they run on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   dX: rows t, columns k, reduction over o. dY rows are read as they lie;
//       W_eff is decoded from the packed record (either form) into bf16.
//   dW: rows o, columns k, reduction over t. Both operands lie with the
//       reduction index as their slow axis; they are staged as they lie and
//       read transposed from LDS with ds_read_b64_tr_b16.
// x~ enters dW in bf16: k_act_dequant rounds fp32(sx * q) to nearest even.
//
// Lane layouts (v_mfma_f32_16x16x32_bf16): lane l holds A[l%16][r(l/16, j)]
// and B[r(l/16, j)][l%16] for j = 0..7 and returns C[4(l/16)+i][l%16],
// i = 0..3. Any one-to-one r(g, j) works as long as A and B use the same:
// kPermBlk8 takes r = 8g + j, kPermHalf r = 4g + j (j < 4), 16 + 4g + j - 4.
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes 4j + i / 4 (j = 0..3); with
// lane 4j + q pointing at row base + j, column 4q, lane i gets column i of
// rows base..base+3.
#include "sbl_internal.h"
#include "device_util.h"

#include <algorithm>
#include <type_traits>
#include <cstdlib>

namespace sbl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 2 x 2 waves
constexpr int kBR = 64;         // reduction rows per LDS stage (two MFMA depths)
constexpr int kPadRM = 16;      // r-major tile row padding (elements)
constexpr int kPitchMM = kBR + 8;   // m-major tile row pitch (elements)

enum { kModeDxDense = 0, kModeDxIndex = 1, kModeDw = 2 };

struct BwdArgs {
  const uint16_t* dy;    // dY bf16 [T][ldy]
  int64_t ldy;
  const void* b;         // dX: packed W (concatenated rows); dW: x~ bf16 [T][ldb]
  int64_t ldb;           // dX: packed row pitch in bytes; dW: x~ row stride in elements
  const float* sw_rows;  // dX: sw of each packed row (one value per segment is read)
  void* out;             // dX [T][ldo] / dW [O][ldo]
  int64_t ldo;
  int32_t T, O, K;
  int32_t nseg;          // dX: reduction segments of constant sw; dW: 1
  int32_t seg_end[4];    // end row of each segment (the first starts at 0)
  int32_t ntm, ntn;      // tiles along the output rows / columns
  int32_t gm;            // tile rows per group of the tile order (see tile_of)
  int32_t out_bf16, accumulate;
  const uint32_t* keep;  // dW only: keep bits [O][keep_pitch] (gated ablation) or null
  int32_t keep_pitch;
};

// The gated-gradient ablation: dW is kept only where the mask keeps the
// weight (bit col % 32 of word col / 32 of the row's keep bits).
__device__ __forceinline__ float gate_keep(const BwdArgs& a, int row, int col, float v) {
  if (a.keep == nullptr) return v;
  const uint32_t w = a.keep[(int64_t)row * a.keep_pitch + (col >> 5)];
  return ((w >> (col & 31)) & 1u) ? v : 0.f;
}

__device__ __forceinline__ i16x4 lds_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Fragment of strip s (16 columns) and MFMA depth u (32 rows) of an r-major
// tile [kBR][pitch] (rows = reduction index).
template <bool HALF>
__device__ __forceinline__ bf16x8 frag_rm(const uint16_t* tile, int pitch, int u, int s, int lane) {
  const int g = lane >> 4, k = lane & 15;
  const int r0 = u * 32 + (HALF ? 4 * g : 8 * g) + (k >> 2);
  const int r1 = r0 + (HALF ? 16 : 4);
  const int c = 16 * s + 4 * (k & 3);
  return join(lds_tr(tile + r0 * pitch + c), lds_tr(tile + r1 * pitch + c));
}

// Fragment of strip s and depth u of an m-major tile [rows][kPitchMM]
// (reduction index contiguous): one 16-byte read (kPermBlk8).
__device__ __forceinline__ bf16x8 frag_mm(const uint16_t* tile, int u, int s, int lane) {
  const uint4 v = *(const uint4*)(tile + (16 * s + (lane & 15)) * kPitchMM + u * 32 + 8 * (lane >> 4));
  return __builtin_bit_cast(bf16x8, v);
}

// Four 2-bit codes (one per byte of e) -> four bf16 (+1 = 0x3F80, -1 =
// 0xBF80): the codes select from byte tables with v_perm.
__device__ __forceinline__ uint2 codes4_bf16(uint32_t e) {
  const uint32_t s01 = __builtin_amdgcn_perm(e, e, 0x01010000u) + 0x00040004u;
  const uint32_t s23 = __builtin_amdgcn_perm(e, e, 0x03030202u) + 0x00040004u;
  // selector 0-3: high byte from 0xBF003F00; 4-7: low byte from 0x80008000
  return make_uint2(__builtin_amdgcn_perm(0x80008000u, 0xBF003F00u, s01),
                    __builtin_amdgcn_perm(0x80008000u, 0xBF003F00u, s23));
}

// Dense-form code word (16 codes, k = 16c + u) -> 16 bf16 in k order.
__device__ __forceinline__ void decode_dense16(uint32_t w, uint4& lo, uint4& hi) {
  const uint2 a = codes4_bf16(w & 0x03030303u);
  const uint2 b = codes4_bf16((w >> 2) & 0x03030303u);
  const uint2 c = codes4_bf16((w >> 4) & 0x03030303u);
  const uint2 d = codes4_bf16((w >> 6) & 0x03030303u);
  lo = make_uint4(a.x, a.y, b.x, b.y);
  hi = make_uint4(c.x, c.y, d.x, d.y);
}

// Index-form chunk (code word cw, index word iw) -> 16 bf16 of groups
// 4h..4h+3 (k = 32c + 16h + 0..15).
__device__ __forceinline__ void decode_index16(uint32_t cw, uint32_t iw, int h, uint4& lo, uint4& hi) {
  // group q = 4h + qq: its index nibble is bits 4qq.. of iwh, its codes are
  // fields 2q and 2q + 1, i.e. bits field_shift(2qq) + 4h .. of cw
  const uint32_t iwh = iw >> (16 * h), cwh = cw >> (4 * h);
  uint32_t out[8];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    // the kept slots s0 < s1 times 8 (bit offsets of their bytes) and codes
    const uint32_t b0 = (qq == 0 ? iwh << 3 : iwh >> (4 * qq - 3)) & 0x18u;
    const uint32_t b1 = (qq == 0 ? iwh << 1 : iwh >> (4 * qq - 1)) & 0x18u;
    const uint32_t c0 = (cwh >> field_shift(2 * qq)) & 3u, c1 = (cwh >> field_shift(2 * qq + 1)) & 3u;
    const uint2 v = codes4_bf16((c0 << b0) | (c1 << b1));   // slot codes, one per byte
    out[2 * qq] = v.x;
    out[2 * qq + 1] = v.y;
  }
  lo = make_uint4(out[0], out[1], out[2], out[3]);
  hi = make_uint4(out[4], out[5], out[6], out[7]);
}

// Block b of nb -> position in the tile order, so that the blocks one XCD
// receives (b % 8) take a contiguous run of it.
__device__ __forceinline__ int xcd_tile(int b, int nb) {
  const int x = b & 7, i = b >> 3, q = nb >> 3, rem = nb & 7;
  return x * q + min(x, rem) + i;
}

// Position t of the tile order -> (tile row, tile column). Groups of gm tile
// rows are taken one after another; inside a group the row index runs
// fastest, so the workgroups an XCD runs at the same time cover gm rows and a
// few columns and share both operands' panels in its L2 (gm is chosen on the
// host from the panel sizes). A row-major order would re-read the whole of
// the row operand from HBM once per few columns.
__device__ __forceinline__ void tile_of(int t, int ntm, int ntn, int gm, int& tm, int& tn) {
  const int g = t / (gm * ntn), r = t - g * gm * ntn;
  const int rows = min(gm, ntm - g * gm);
  tm = g * gm + r % rows;
  tn = r / rows;
}

template <int MODE, int WMB, int WNB, bool MULTI>
__global__ __launch_bounds__(kThreads, (WMB * WNB > 16) ? 1 : 2) void k_bwd(const BwdArgs a) {
  constexpr int BM = 32 * WMB, BN = 32 * WNB;   // 2 x 2 waves of (16 WMB) x (16 WNB)
  constexpr bool DX = MODE != kModeDw;
  constexpr int PA = DX ? kPitchMM : BM + kPadRM;          // A tile pitch
  constexpr int PB = BN + kPadRM;                          // B tile pitch (r-major)
  constexpr int SA = DX ? BM * kPitchMM : kBR * PA;        // A tile elements
  constexpr int SB = kBR * PB;
  constexpr bool HALF = !DX;                               // r permutation (see header)
  extern __shared__ __align__(16) uint16_t lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = a.ntm * a.ntn;
  int tm, tn;
  tile_of(xcd_tile(blockIdx.x, nb), a.ntm, a.ntn, a.gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int Mrows = DX ? a.T : a.O;

  // ---- staging: global -> registers -> LDS --------------------------------
  constexpr int NVA = BM * kBR / 8 / kThreads;             // 16-byte vectors of A per thread
  constexpr int NWB = kBR * (BN / 16) / kThreads;          // 16-element B pieces per thread
  static_assert(NVA >= 1 && NWB >= 1, "tile too small for the block");
  // Two register stages: the loads of step s + 1 are issued two steps ahead,
  // so their latency is covered by two compute phases, not one.
  struct Stage {
    uint4 ra[NVA];
    uint4 rb[MODE == kModeDw ? 2 * NWB : NWB];             // dW: 8-element vectors
  };
  Stage S0, S1;

  // (Loads are guarded per lane. A branch-free form -- clamped addresses and
  // a select -- measured 7-28% slower: the address arithmetic costs more than
  // the exec-mask branches, which are almost never taken.)
  auto load = [&](Stage& g, int rs, int rend) {
#pragma unroll
    for (int i = 0; i < NVA; ++i) {
      const int v = threadIdx.x + i * kThreads;
      int row, col;                                        // in dY: (t, o)
      bool ok;
      if constexpr (DX) {
        const int mr = v / (kBR / 8), cv = v % (kBR / 8);
        row = m0 + mr; col = rs + 8 * cv;
        ok = row < a.T && col < rend;
      } else {
        const int rr = v / (BM / 8), cv = v % (BM / 8);
        row = rs + rr; col = m0 + 8 * cv;
        ok = row < rend && col < a.O;
      }
      g.ra[i] = ok ? *(const uint4*)(a.dy + (int64_t)row * a.ldy + col) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (MODE == kModeDw) {
#pragma unroll
      for (int i = 0; i < 2 * NWB; ++i) {
        const int v = threadIdx.x + i * kThreads;
        const int rr = v / (BN / 8), cv = v % (BN / 8);
        const int t = rs + rr, k = n0 + 8 * cv;
        const bool ok = t < rend && k < a.K;
        g.rb[i] = ok ? *(const uint4*)((const uint16_t*)a.b + (int64_t)t * a.ldb + k) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NWB; ++i) {
        const int v = threadIdx.x + i * kThreads;
        const int rr = v / (BN / 16), cw = v % (BN / 16);
        const int o = rs + rr, k = n0 + 16 * cw;
        const uint8_t* row = (const uint8_t*)a.b + (int64_t)o * a.ldb;
        if constexpr (MODE == kModeDxDense) {
          const bool ok = o < rend && k < a.K;              // word k/16 lies in the code area
          g.rb[i].x = ok ? *(const uint32_t*)(row + 4 * (k >> 4)) : 0u;
        } else {
          const bool ok = o < rend && (k & ~31) < a.K;      // chunk k/32 exists
          const uint2 d = ok ? *(const uint2*)(row + 8 * (k >> 5)) : make_uint2(0u, 0u);
          g.rb[i].x = d.x;
          g.rb[i].y = d.y;
        }
      }
    }
  };
  auto store = [&](const Stage& g, uint16_t* A, uint16_t* B) {
#pragma unroll
    for (int i = 0; i < NVA; ++i) {
      const int v = threadIdx.x + i * kThreads;
      if constexpr (DX) {
        const int mr = v / (kBR / 8), cv = v % (kBR / 8);
        *(uint4*)(A + mr * PA + 8 * cv) = g.ra[i];
      } else {
        const int rr = v / (BM / 8), cv = v % (BM / 8);
        *(uint4*)(A + rr * PA + 8 * cv) = g.ra[i];
      }
    }
    if constexpr (MODE == kModeDw) {
#pragma unroll
      for (int i = 0; i < 2 * NWB; ++i) {
        const int v = threadIdx.x + i * kThreads;
        const int rr = v / (BN / 8), cv = v % (BN / 8);
        *(uint4*)(B + rr * PB + 8 * cv) = g.rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NWB; ++i) {
        const int v = threadIdx.x + i * kThreads;
        const int rr = v / (BN / 16), cw = v % (BN / 16);
        uint4 lo, hi;
        if constexpr (MODE == kModeDxDense) decode_dense16(g.rb[i].x, lo, hi);
        else decode_index16(g.rb[i].x, g.rb[i].y, ((n0 + 16 * cw) >> 4) & 1, lo, hi);
        *(uint4*)(B + rr * PB + 16 * cw) = lo;
        *(uint4*)(B + rr * PB + 16 * cw + 8) = hi;
      }
    }
  };

  f32x4 acc[WMB][WNB], tot[MULTI ? WMB : 1][MULTI ? WNB : 1];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MULTI) {
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j) tot[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nseg = DX ? a.nseg : 1;
  int r_begin = 0;
  float sw = 1.f;
  for (int sg = 0; sg < nseg; ++sg) {
    const int r_end = DX ? a.seg_end[sg] : a.T;
    if constexpr (DX) sw = a.sw_rows[r_begin];
    const int steps = (r_end - r_begin + kBR - 1) / kBR;
    if (steps == 0) {                                   // empty reduction (dW, T = 0)
      r_begin = r_end;
      continue;
    }
    load(S0, r_begin, r_end);
    store(S0, lds, lds + SA);
    if (steps > 1) load(S1, r_begin + kBR, r_end);
    if (steps > 2) load(S0, r_begin + 2 * kBR, r_end);
    __syncthreads();
    // step st: compute from LDS buffer st & 1; g holds step st + 1, which goes
    // to the other buffer, and then takes the loads of step st + 3
    auto step = [&](int st, Stage& g) {
      const int buf = st & 1;
      const uint16_t* A = lds + buf * (SA + SB);
      const uint16_t* B = A + SA;
#pragma unroll
      for (int u = 0; u < kBR / 32; ++u) {
        bf16x8 fa[WMB], fb[WNB];
#pragma unroll
        for (int i = 0; i < WMB; ++i) {
          if constexpr (DX) fa[i] = frag_mm(A + wm * (16 * WMB) * PA, u, i, lane);
          else fa[i] = frag_rm<HALF>(A + wm * (16 * WMB), PA, u, i, lane);
        }
#pragma unroll
        for (int j = 0; j < WNB; ++j) fb[j] = frag_rm<HALF>(B + wn * (16 * WNB), PB, u, j, lane);
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
          for (int j = 0; j < WNB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (st + 1 < steps) {
        uint16_t* An = lds + (buf ^ 1) * (SA + SB);
        store(g, An, An + SA);
        if (st + 3 < steps) load(g, r_begin + (st + 3) * kBR, r_end);
      }
      __syncthreads();
    };
    for (int st = 0; st < steps; st += 2) {
      step(st, S1);
      if (st + 1 < steps) step(st + 1, S0);
    }
    if constexpr (MULTI) {
#pragma unroll
      for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            tot[i][j][e] += sw * acc[i][j][e];
            acc[i][j][e] = 0.f;
          }
    }
    r_begin = r_end;
  }

  // ---- epilogue: C[row][col] (dX: sw * acc; dW: acc) ---------------------
  const int rbase = m0 + wm * (16 * WMB) + 4 * (lane >> 4);
  const int cbase = n0 + wn * (16 * WNB) + (lane & 15);
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rbase + 16 * i + e, col = cbase + 16 * j;
        if (row >= Mrows || col >= a.K) continue;
        float v;
        if constexpr (MULTI) v = tot[i][j][e];
        else v = DX ? sw * acc[i][j][e] : gate_keep(a, row, col, acc[i][j][e]);
        const int64_t off = (int64_t)row * a.ldo + col;
        if (a.out_bf16) {
          uint16_t* o = (uint16_t*)a.out + off;
          if (a.accumulate) v += bf16_bits_to_f32(*o);
          *o = (uint16_t)f32_to_bf16_bits(v);
        } else {
          float* o = (float*)a.out + off;
          if (a.accumulate) v += *o;
          *o = v;
        }
      }
}

// ---------------------------------------------------------------------------
// dW with direct global-to-LDS loads. Staging through registers (load, wait,
// write LDS) costs about as much as the products themselves here; the LDS DMA
// (global_load_lds, 16 bytes per lane) lands the operands without the waves'
// instructions, so the ring can run several steps ahead.
//   Tile BM x 128 (2 x 2 waves of (BM / 2) x 64), steps of 32 rows of T:
//   BM = 128 with four ring stages, or BM = 256 with three (each wave's
//   transposed fragment reads then feed twice the products: the kernel is
//   bound by LDS traffic per product, not by HBM).
//   LDS: stages of {BM / 128 dY sub-tiles, x~ tile}, each 32 rows x 256
//   bytes, no padding (one DMA instruction fills 4 whole rows); bank conflicts
//   of the transposed reads are avoided by XOR-swizzling the 16-byte chunks
//   of a row: chunk c of row r sits at c ^ (2 (r mod 8)).
//   Rows past the tile edges are loaded from clamped (valid) addresses: they
//   only reach outputs that are not written. Rows past T in the last step
//   would reach real outputs, so that step's x~ rows past T are zeroed in
//   LDS after their loads land.
// ---------------------------------------------------------------------------
constexpr int kDmaBR = 32;
constexpr int kDmaSub = kDmaBR * 128;                      // one 32 x 128 sub-tile

__device__ __forceinline__ int swz(int r, int c) { return c ^ (2 * (r & 7)); }

__device__ __forceinline__ void dma16(const void* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until at most n DMAs of this wave are outstanding (and all its LDS
// operations are done), then barrier. n is a compile-time constant at every
// call (the waits are instruction immediates). The empty asm statements keep
// the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposed fragment (kPermHalf) of strip s from a swizzled 32 x 128 tile.
__device__ __forceinline__ bf16x8 frag_swz(const uint16_t* tile, int col0, int s, int lane) {
  const int g = lane >> 4, k = lane & 15;
  const int r0 = 4 * g + (k >> 2), r1 = r0 + 16;
  const int col = col0 + 16 * s + 4 * (k & 3);
  const int c = col >> 3, e = col & 7;
  return join(lds_tr(tile + r0 * 128 + 8 * swz(r0, c) + e), lds_tr(tile + r1 * 128 + 8 * swz(r1, c) + e));
}

// The ring slots are separate LDS objects, each named at compile time (the
// loop is unrolled by the stage count): the compiler then knows that a read
// of one slot does not depend on the DMAs still landing in the others, and
// does not drain them before every read. 128-row tiles: four slots of two
// sub-tiles; 256-row tiles: three slots of three.
__shared__ __align__(16) uint16_t dma_slot0[2 * kDmaSub];
__shared__ __align__(16) uint16_t dma_slot1[2 * kDmaSub];
__shared__ __align__(16) uint16_t dma_slot2[2 * kDmaSub];
__shared__ __align__(16) uint16_t dma_slot3[2 * kDmaSub];
__shared__ __align__(16) uint16_t dma_wslot0[3 * kDmaSub];
__shared__ __align__(16) uint16_t dma_wslot1[3 * kDmaSub];
__shared__ __align__(16) uint16_t dma_wslot2[3 * kDmaSub];

template <int BM, int I>
__device__ __forceinline__ uint16_t* dma_slot() {
  if constexpr (BM == 256) {
    if constexpr (I == 0) return dma_wslot0;
    else if constexpr (I == 1) return dma_wslot1;
    else return dma_wslot2;
  } else {
    if constexpr (I == 0) return dma_slot0;
    else if constexpr (I == 1) return dma_slot1;
    else if constexpr (I == 2) return dma_slot2;
    else return dma_slot3;
  }
}

template <int BM>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dw_dma(const BwdArgs a) {
  static_assert(BM == 128 || BM == 256, "tile rows");
  constexpr int NS = BM == 256 ? 3 : 4;                    // ring stages
  constexpr int NH = BM / 128;                             // dY sub-tiles per stage
  constexpr int WM = BM / 2, NI = WM / 16;                 // wave rows, row strips
  constexpr int D = 2 * NH + 2;                            // DMAs per wave and step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(xcd_tile(blockIdx.x, a.ntm * a.ntn), a.ntm, a.ntn, a.gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * 128;
  const int T = a.T, steps = (T + kDmaBR - 1) / kDmaBR;
  const uint16_t* __restrict__ xt = (const uint16_t*)a.b;

  // DMA i of the wave fills rows 4 (2 wave + i) .. + 3 of a sub-tile; lane l
  // takes row + l / 16, physical chunk l % 16 (logical chunk swz of it)
  auto issue = [&](uint16_t* slot, int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * (2 * wave + i) + (lane >> 4);
      const int c = swz(r, lane & 15);
      const int t = min(st * kDmaBR + r, T - 1);
      const int k = min(n0 + 8 * c, a.K - 8);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int o = min(m0 + 128 * h + 8 * c, a.O - 8);
        dma16(a.dy + (int64_t)t * a.ldy + o, slot + h * kDmaSub + 4 * (2 * wave + i) * 128);
      }
      dma16(xt + (int64_t)t * a.ldb + k, slot + NH * kDmaSub + 4 * (2 * wave + i) * 128);
    }
  };

  f32x4 acc[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step st (st % NS == I): wait for its slot, refill the slot of step st - 1
  // with step st + NS - 1, compute
  auto body = [&](auto I_, int st) {
    constexpr int I = decltype(I_)::value;
    if (st >= steps) return;
    // at most the DMAs of the later issued steps (D per step and wave) may
    // still be outstanding
    const int later = min(NS - 2, steps - 1 - st);
    if (later >= 2) dma_wait_barrier<2 * D>();
    else if (later == 1) dma_wait_barrier<D>();
    else dma_wait_barrier<0>();
    if (st + NS - 1 < steps) issue(dma_slot<BM, (I + NS - 1) % NS>(), st + NS - 1);
    uint16_t* slot = dma_slot<BM, I>();
    const int valid = T - st * kDmaBR;
    if (valid < kDmaBR) {                                    // last step: zero x~ rows >= T
      uint16_t* xs = slot + NH * kDmaSub;
      for (int v = threadIdx.x; v < (kDmaBR - valid) * 16; v += kThreads)
        *(uint4*)(xs + (valid + v / 16) * 128 + 8 * (v % 16)) = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
    // wave rows: sub-tile wm, all 128 columns (BM 256), or sub-tile 0,
    // columns 64 wm .. (BM 128)
    const uint16_t* ya = slot + (NH == 2 ? wm : 0) * kDmaSub;
    const int ycol = NH == 2 ? 0 : 64 * wm;
    bf16x8 fa[NI], fb[4];
#pragma unroll
    for (int i = 0; i < NI; ++i) fa[i] = frag_swz(ya, ycol, i, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag_swz(slot + NH * kDmaSub, wn * 64, j, lane);
    // issue priority raised for the matrix-core block (of two waves on a SIMD
    // the one with MFMAs ready goes first; 7-8% on the 1.5B dW products)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    if (p < steps) {
      if constexpr (NS == 3) issue(p == 0 ? dma_slot<BM, 0>() : dma_slot<BM, 1>(), p);
      else issue(p == 0 ? dma_slot<BM, 0>() : p == 1 ? dma_slot<BM, 1>() : dma_slot<BM, 2>(), p);
    }
  }
  for (int st = 0; st < steps; st += NS) {
    body(std::integral_constant<int, 0>{}, st);
    body(std::integral_constant<int, 1>{}, st + 1);
    body(std::integral_constant<int, 2>{}, st + 2);
    if constexpr (NS == 4) body(std::integral_constant<int, 3>{}, st + 3);
  }

  const int rbase = m0 + wm * WM + 4 * (lane >> 4);
  const int cbase = n0 + wn * 64 + (lane & 15);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rbase + 16 * i + e, col = cbase + 16 * j;
        if (row >= a.O || col >= a.K) continue;
        const int64_t off = (int64_t)row * a.ldo + col;
        const float v = gate_keep(a, row, col, acc[i][j][e]);
        if (a.out_bf16) ((uint16_t*)a.out)[off] = (uint16_t)f32_to_bf16_bits(v);
        else ((float*)a.out)[off] = v;
      }
}


// ---------------------------------------------------------------------------
// dX of a single weight tensor with dY landed by LDS DMA. Tile BM x 128 of
// [T, K] (2 x 2 waves of (BM / 2) x 64), steps of 32 rows of O (one MFMA
// depth) in a ring of NS slots: BM = 128 with four, BM = 256 with three.
//   A (dY [t][o], the reduction index o contiguous): BM rows x 64 bytes per
//   step, 16 rows per DMA instruction (4 lanes per row); the 16-byte chunk c
//   of row r sits at c ^ ((r >> 1) & 3), so a fragment read (16 rows, one
//   chunk each) touches every bank pair once.
//   B (W_eff [o][k] in bf16, decoded from the packed rows): the codes of step
//   st + NS - 1 are loaded before that step's DMAs are issued and decoded
//   into its slot after the current step's products, so waiting for them
//   never waits for a DMA; rows o >= O decode to zeros.
//   Rows t >= T load row T - 1 and reach no stored output; columns o >= O of
//   the last step load valid data that meets those zero rows.
// ---------------------------------------------------------------------------
constexpr int kDxPB = 128 + kPadRM;                        // decoded W row pitch (elements)

template <int BM>
constexpr int dx_slot_elems() { return BM * 32 + 32 * kDxPB; }

__shared__ __align__(16) uint16_t dx_slot0[dx_slot_elems<128>()];
__shared__ __align__(16) uint16_t dx_slot1[dx_slot_elems<128>()];
__shared__ __align__(16) uint16_t dx_slot2[dx_slot_elems<128>()];
__shared__ __align__(16) uint16_t dx_slot3[dx_slot_elems<128>()];
__shared__ __align__(16) uint16_t dx_wslot0[dx_slot_elems<256>()];
__shared__ __align__(16) uint16_t dx_wslot1[dx_slot_elems<256>()];
__shared__ __align__(16) uint16_t dx_wslot2[dx_slot_elems<256>()];

template <int BM, int I>
__device__ __forceinline__ uint16_t* dx_slot() {
  if constexpr (BM == 256) {
    if constexpr (I == 0) return dx_wslot0;
    else if constexpr (I == 1) return dx_wslot1;
    else return dx_wslot2;
  } else {
    if constexpr (I == 0) return dx_slot0;
    else if constexpr (I == 1) return dx_slot1;
    else if constexpr (I == 2) return dx_slot2;
    else return dx_slot3;
  }
}

template <int BM, bool IDX>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dx_dma(const BwdArgs a) {
  static_assert(BM == 128 || BM == 256, "tile rows");
  constexpr int NS = BM == 256 ? 3 : 4;                    // ring stages
  constexpr int WM = BM / 2, NI = WM / 16;                 // wave rows, row strips
  constexpr int DA = BM / 64;                              // A DMAs per wave and step
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(xcd_tile(blockIdx.x, a.ntm * a.ntn), a.ntm, a.ntn, a.gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * 128;
  const int O = a.O, steps = (O + 31) / 32;
  const uint8_t* __restrict__ packed = (const uint8_t*)a.b;

  // A: DMA q = DA wave + i fills rows 16 q .. 16 q + 15 of the step's tile
  auto issue = [&](uint16_t* slot, int st) {
#pragma unroll
    for (int i = 0; i < DA; ++i) {
      const int q = DA * wave + i;
      const int r = 16 * q + (lane >> 2), pc = lane & 3;
      const int c = pc ^ ((r >> 1) & 3);
      const int t = min(m0 + r, a.T - 1);
      const int o = min(32 * st + 8 * c, O - 8);
      dma16(a.dy + (int64_t)t * a.ldy + o, slot + 16 * q * 32);
    }
  };
  // B: thread v takes row v / 8 of the step and 16 columns n0 + 16 (v % 8)
  const int brow = threadIdx.x >> 3, bcol = 16 * (threadIdx.x & 7);
  const int kk = n0 + bcol;
  auto load_codes = [&](int st) -> uint2 {
    const int o = 32 * st + brow;
    const uint8_t* row = packed + (int64_t)o * a.ldb;
    if constexpr (IDX) {
      const bool ok = o < O && (kk & ~31) < a.K;           // chunk kk / 32 exists
      return ok ? *(const uint2*)(row + 8 * (kk >> 5)) : make_uint2(0u, 0u);
    } else {
      const bool ok = o < O && kk < a.K;                   // word kk / 16 lies in the code area
      return make_uint2(ok ? *(const uint32_t*)(row + 4 * (kk >> 4)) : 0u, 0u);
    }
  };
  auto write_b = [&](uint16_t* slot, uint2 w) {
    uint4 lo, hi;
    if constexpr (IDX) decode_index16(w.x, w.y, (kk >> 4) & 1, lo, hi);
    else decode_dense16(w.x, lo, hi);
    uint16_t* B = slot + BM * 32 + brow * kDxPB + bcol;
    *(uint4*)B = lo;
    *(uint4*)(B + 8) = hi;
  };

  f32x4 acc[NI][4];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto body = [&](auto I_, int st) {
    constexpr int I = decltype(I_)::value;
    if (st >= steps) return;
    // at most the A DMAs of the later issued steps may still be outstanding
    // (the codes loaded in earlier steps were consumed there)
    const int later = min(NS - 2, steps - 1 - st);
    if (later >= 2) dma_wait_barrier<2 * DA>();
    else if (later == 1) dma_wait_barrier<DA>();
    else dma_wait_barrier<0>();
    const bool refill = st + NS - 1 < steps;
    uint2 w = make_uint2(0u, 0u);
    if (refill) {
      w = load_codes(st + NS - 1);
      issue(dx_slot<BM, (I + NS - 1) % NS>(), st + NS - 1);
    }
    const uint16_t* A = dx_slot<BM, I>();
    const uint16_t* B = A + BM * 32;
    bf16x8 fa[NI], fb[4];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = wm * WM + 16 * i + (lane & 15), g = lane >> 4;
      fa[i] = __builtin_bit_cast(bf16x8, *(const uint4*)(A + r * 32 + 8 * (g ^ ((r >> 1) & 3))));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag_rm<false>(B + wn * 64, kDxPB, 0, j, lane);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    if (refill) write_b(dx_slot<BM, (I + NS - 1) % NS>(), w);
  };

  // prologue: steps 0 .. NS - 2 (their B decoded now; the first barrier
  // publishes them)
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    if (p < steps) {
      const uint2 w = load_codes(p);
      uint16_t* slot = p == 0 ? dx_slot<BM, 0>() : p == 1 ? dx_slot<BM, 1>() : dx_slot<BM, 2>();
      issue(slot, p);
      write_b(slot, w);
    }
  }
  for (int st = 0; st < steps; st += NS) {
    body(std::integral_constant<int, 0>{}, st);
    body(std::integral_constant<int, 1>{}, st + 1);
    body(std::integral_constant<int, 2>{}, st + 2);
    if constexpr (NS == 4) body(std::integral_constant<int, 3>{}, st + 3);
  }

  const float sw = a.sw_rows[0];
  const int rbase = m0 + wm * WM + 4 * (lane >> 4);
  const int cbase = n0 + wn * 64 + (lane & 15);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rbase + 16 * i + e, col = cbase + 16 * j;
        if (row >= a.T || col >= a.K) continue;
        float v = sw * acc[i][j][e];
        const int64_t off = (int64_t)row * a.ldo + col;
        if (a.out_bf16) {
          uint16_t* o = (uint16_t*)a.out + off;
          if (a.accumulate) v += bf16_bits_to_f32(*o);
          *o = (uint16_t)f32_to_bf16_bits(v);
        } else {
          float* o = (float*)a.out + off;
          if (a.accumulate) v += *o;
          *o = v;
        }
      }
}


// x~ = bf16_rne(fp32(q) * sx[t]); 8 codes per thread (K % 8 == 0).
__global__ __launch_bounds__(256) void k_act_dequant(const int8_t* __restrict__ xq,
                                                      const float* __restrict__ sx, int64_t T,
                                                      int64_t K, uint16_t* __restrict__ xt) {
  const int64_t per_row = K / 8;
  const int64_t n = T * per_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_row, c = i - t * per_row;
    const float s = sx[t];
    const uint2 q = *(const uint2*)(xq + t * K + 8 * c);
    const uint32_t w[2] = {q.x, q.y};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t b0 = (int32_t)(w[h] << 24) >> 24, b1 = (int32_t)(w[h] << 16) >> 24;
      const int32_t b2 = (int32_t)(w[h] << 8) >> 24, b3 = (int32_t)w[h] >> 24;
      o[2 * h] = f32_to_bf16_bits((float)b0 * s) | (f32_to_bf16_bits((float)b1 * s) << 16);
      o[2 * h + 1] = f32_to_bf16_bits((float)b2 * s) | (f32_to_bf16_bits((float)b3 * s) << 16);
    }
    *(uint4*)(xt + t * K + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Workgroup tiles (rows x columns of the output; 2 x 2 waves each):
//   0: 128x128, 1: 64x128, 2: 64x64, 3: 256x128, 4: 128x256.
// Measured on the FFN shapes (T = 2048 and 4096): 128x128 (three waves per
// SIMD) is fastest whenever it gives about three quarters of the compute
// units a workgroup; below that 64x64 (more workgroups) wins. The two large
// tiles need 384 registers per lane -- one wave per SIMD, too little to hide
// the staging loads -- and stay selectable for tuning only.
constexpr int kNumBwdCfg = 5;
int pick_cfg(int64_t rows, int64_t cols) {
  // tuning override (read on every call so tests can force each configuration)
  const char* ev = std::getenv("SBL_BWD_TILE");
  const int forced = ev ? std::atoi(ev) : -1;
  if (forced >= 0 && forced < kNumBwdCfg) return forced;
  const int64_t want = device_info().cus * 3 / 4;
  return cdiv(rows, 128) * cdiv(cols, 128) >= want ? 0 : 2;
}

void set_order(BwdArgs& a, int BM, int BN, bool DX) {
  a.ntm = (int32_t)cdiv(DX ? a.T : a.O, BM);
  a.ntn = (int32_t)cdiv(a.K, BN);
  // Tile-order group: about `conc` workgroups run at once on an XCD (two or
  // four per CU, 32 CUs); a group of gm rows lets them share gm row panels
  // and conc / gm column panels. Pick gm to minimize the panel bytes fetched
  // beyond L2: each row panel once per conc/gm columns, each column panel
  // once per group.
  {
    const int64_t R = DX ? a.O : a.T;
    const double rowp = (double)BM * R * 2;                          // dY panel
    const double colp = DX ? (double)BN * R / 4 : (double)BN * R * 2;  // W codes / x~ panel
    const int conc = 32 * (BM * BN >= 128 * 128 ? 2 : 4);
    double best = 0;
    for (int gm = 1; gm <= 64; gm *= 2) {
      const int g = (int)std::min<int64_t>(gm, a.ntm);
      const int gn = std::max(1, conc / g);
      const double cost = a.ntm * rowp * (double)cdiv(a.ntn, gn) + a.ntn * colp * (double)cdiv(a.ntm, g);
      if (gm == 1 || cost < best) { best = cost; a.gm = g; }
    }
    if (const char* ev = std::getenv("SBL_BWD_GROUP")) a.gm = std::max(1, std::min(std::atoi(ev), a.ntm));
  }
}

template <int MODE, int WMB, int WNB, bool MULTI>
hipError_t launch_cfg(BwdArgs a, hipStream_t s) {
  constexpr int BM = 32 * WMB, BN = 32 * WNB;
  constexpr bool DX = MODE != kModeDw;
  constexpr size_t SA = DX ? (size_t)BM * kPitchMM : (size_t)kBR * (BM + kPadRM);
  constexpr size_t SB = (size_t)kBR * (BN + kPadRM);
  constexpr size_t lds = 2 * (SA + SB) * sizeof(uint16_t);
  auto kern = k_bwd<MODE, WMB, WNB, MULTI>;
  if (lds > 65536) {
    static bool set = false;
    if (!set) {
      const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      set = true;
    }
  }
  set_order(a, BM, BN, DX);
  const int64_t nb = (int64_t)a.ntm * a.ntn;
  hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int MODE, bool MULTI>
hipError_t launch_mode(const BwdArgs& a, int cfg, hipStream_t s) {
  if constexpr (!MULTI) {   // (the large tiles with a second accumulator set would spill)
    if (cfg == 3) return launch_cfg<MODE, 8, 4, MULTI>(a, s);
    if (cfg == 4) return launch_cfg<MODE, 4, 8, MULTI>(a, s);
  }
  switch (cfg) {
    case 1: return launch_cfg<MODE, 2, 4, MULTI>(a, s);
    case 2: return launch_cfg<MODE, 2, 2, MULTI>(a, s);
    default: return launch_cfg<MODE, 4, 4, MULTI>(a, s);
  }
}

}  // namespace

hipError_t launch_act_dequant(const int8_t* xq, const float* sx, int64_t T, int64_t K,
                              uint16_t* xt, hipStream_t s) {
  const int64_t n = T * (K / 8);
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), (int64_t)device_info().cus * 8);
  hipLaunchKernelGGL(k_act_dequant, dim3((unsigned)blocks), dim3(256), 0, s, xq, sx, T, K, xt);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dy, int64_t ldy, const void* packed, const float* sw_rows,
                         int64_t T, int64_t O, int64_t K, int N, int M, const int64_t* seg_end,
                         int nseg, void* dx, bool dx_bf16, int64_t lddx, bool accumulate,
                         int cfg, hipStream_t s) {
  BwdArgs a{};
  a.dy = dy; a.ldy = ldy; a.b = packed; a.ldb = row_pitch(K, N, M); a.sw_rows = sw_rows;
  a.out = dx; a.ldo = lddx; a.T = (int32_t)T; a.O = (int32_t)O; a.K = (int32_t)K;
  a.nseg = nseg;
  for (int i = 0; i < nseg; ++i) a.seg_end[i] = (int32_t)seg_end[i];
  a.out_bf16 = dx_bf16; a.accumulate = accumulate;
  if (cfg < 0) cfg = pick_cfg(T, K);
  const bool idx = index_form(N, M);
  // The LDS-DMA kernel with 256-row tiles where it measured faster: at
  // least two tiles per CU and a reduction of 2048 rows or more (Qwen2.5-3B
  // up 445 -> 360 us, down 514 -> 480); with fewer tiles or shorter
  // reductions (the 0.5B and 1.5B projections) the register-staged 128x128
  // kernel is faster. SBL_BWD_DX_DMA=1 forces it (SBL_BWD_DX_WIDE=0 / 1
  // picks the tile rows), SBL_BWD_DMA=0 disables it (tuning and tests).
  const char* ev = std::getenv("SBL_BWD_DMA");
  const char* ed = std::getenv("SBL_BWD_DX_DMA");
  const bool dma = ed ? ed[0] == '1'
                      : cdiv(T, 256) * cdiv(K, 128) >= 2 * (int64_t)device_info().cus && O >= 2048;
  if (nseg == 1 && cfg == 0 && dma && !(ev && ev[0] == '0')) {
    const char* ew = std::getenv("SBL_BWD_DX_WIDE");
    const bool wide = ew ? ew[0] == '1' : true;
    set_order(a, wide ? 256 : 128, 128, true);
    const dim3 grid((unsigned)(a.ntm * a.ntn)), block(kThreads);
    if (wide) {
      if (idx) hipLaunchKernelGGL((k_bwd_dx_dma<256, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_bwd_dx_dma<256, false>), grid, block, 0, s, a);
    } else {
      if (idx) hipLaunchKernelGGL((k_bwd_dx_dma<128, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_bwd_dx_dma<128, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  }
  if (nseg > 1)
    return idx ? launch_mode<kModeDxIndex, true>(a, cfg, s) : launch_mode<kModeDxDense, true>(a, cfg, s);
  return idx ? launch_mode<kModeDxIndex, false>(a, cfg, s) : launch_mode<kModeDxDense, false>(a, cfg, s);
}

hipError_t launch_bwd_dw(const uint16_t* dy, int64_t ldy, const uint16_t* xt, int64_t ldxt,
                         int64_t T, int64_t O, int64_t K, const uint32_t* keep, void* dw,
                         bool dw_bf16, int64_t lddw, int cfg, hipStream_t s) {
  BwdArgs a{};
  a.keep = keep;
  a.keep_pitch = (int32_t)row_chunks(K);
  a.dy = dy; a.ldy = ldy; a.b = xt; a.ldb = ldxt; a.sw_rows = nullptr;
  a.out = dw; a.ldo = lddw; a.T = (int32_t)T; a.O = (int32_t)O; a.K = (int32_t)K;
  a.nseg = 1; a.seg_end[0] = (int32_t)T;
  a.out_bf16 = dw_bf16; a.accumulate = 0;
  if (cfg < 0) cfg = pick_cfg(O, K);
  const char* ev = std::getenv("SBL_BWD_DMA");   // tuning: 0 keeps the register-staged kernel
  if (cfg == 0 && !(ev && ev[0] == '0')) {
    // 256-row tiles when they still give every CU at least one (measured
    // 1.02-1.29x faster on the Qwen2.5 0.5B-3B projections that qualify;
    // 0.78x on the 0.5B down projection's 152 tiles, which does not)
    const char* ew = std::getenv("SBL_BWD_DW_WIDE");   // tuning: 0 / 1 forces the tile rows
    const bool wide = ew ? ew[0] == '1' : cdiv(O, 256) * cdiv(K, 128) >= (int64_t)device_info().cus;
    if (wide) {
      set_order(a, 256, 128, false);
      hipLaunchKernelGGL(k_bwd_dw_dma<256>, dim3((unsigned)(a.ntm * a.ntn)), dim3(kThreads), 0, s, a);
    } else {
      set_order(a, 128, 128, false);
      hipLaunchKernelGGL(k_bwd_dw_dma<128>, dim3((unsigned)(a.ntm * a.ntn)), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
  }
  return launch_mode<kModeDw, false>(a, cfg, s);
}

}  // namespace sbl
