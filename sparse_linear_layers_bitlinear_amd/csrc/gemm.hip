// a5 + a6: int8 x ternary N:M GEMM with an int32 accumulator, dequantized in
// the epilogue. Sparse-BitNet summary, section 3.4 "The Full Sparse-BitLinear
// Layer": y = s * (W_eff x~), the scales absorbed into one multiply per
// output (Eq. 4).
//
// Operand roles: A = W_eff (rows = output features o), B = xq^T (columns =
// tokens t), C[o][t]. With the gfx950 16x16 MFMA output layout a lane holds
// C rows 4*(lane/16) + r, r = 0..3, of column lane%16 -- four consecutive
// outputs of one token, i.e. one 8/16-byte store into y[T, O].
//
// Dense form (any N:M except 2:4): W codes (2 bits/weight) are read from the
// packed record, expanded to int8 with one byte-permute per 4 weights while
// being staged into LDS, and multiplied with v_mfma_i32_16x16x64_i8.
// Operand A lane l holds row l%16, k = 16*(l/16) + [0,16); operand B the
// same k for column l%16 (any k order shared by A and B gives the same sum).
//
// Index form (2:4): the packed chunk already is the sparse-MFMA operand:
// 16 kept codes + one index word per 32 dense k. v_smfmac_i32_16x16x128_i8
// takes A lane l = row l%16 with the compressed values of dense
// k in [32g, 32g+32), g = l/16 (value v's slot in bits [2v+1:2v] of the
// index word), and B lane l = column l%16 with dense k in [16g, 16g+16) and
// [64+16g, 64+16g+16).
//
// Tiles: 4 or 8 wavefronts per workgroup, each owning a block of 16x16 MFMA
// tiles; K advances BK = 64 (dense) or 128 (2:4) per step; LDS is
// double-buffered so global loads of step s+1 overlap the MFMAs of step s.
// Staged rows have pitches of 80 / 144 bytes so that the 16-byte fragment
// reads of 16 consecutive rows fall in distinct banks.
#include "sbl_internal.h"
#include "device_util.h"

#include <cmath>
#include <cstdlib>

namespace sbl {

constexpr int kPitchA = 80;    // bytes per staged W row (64 values + 16 pad / index)
constexpr int kPitchBd = 80;   // bytes per staged xq row, dense (64 k)
constexpr int kPitchBs = 144;  // bytes per staged xq row, 2:4 (128 k)


template <bool KA16>
__device__ __forceinline__ uint4 load_x16(const int8_t* __restrict__ row, int64_t k, int64_t K) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if constexpr (KA16) {
    if (k < K) v = *(const uint4*)(row + k);
  } else {  // rows are only 4-byte aligned; K % 4 == 0
    const uint32_t* p = (const uint32_t*)(row + k);
    if (k < K) v.x = p[0];
    if (k + 4 < K) v.y = p[1];
    if (k + 8 < K) v.z = p[2];
    if (k + 12 < K) v.w = p[3];
  }
  return v;
}

template <bool YBF16>
__device__ __forceinline__ void store_out(void* __restrict__ y, int32_t* __restrict__ acc_out,
                                          const v4i& c, int64_t t, int64_t o, int64_t T,
                                          int64_t O, const float* __restrict__ sx,
                                          const float* __restrict__ sw, int64_t sw_inc) {
  if (t >= T || o >= O) return;
  const float s_t = sx[t];
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = (float)c[r] * s_t;
    v[r] = a * sw[(o + r < O ? o + r : o) * sw_inc];
  }
  const int64_t base = t * O + o;
  if (o + 3 < O && (O & 3) == 0) {
    if constexpr (YBF16) {
      const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *(uint2*)((uint16_t*)y + base) = make_uint2(lo, hi);
    } else {
      *(float4*)((float*)y + base) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (acc_out) *(int4*)(acc_out + base) = make_int4(c[0], c[1], c[2], c[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (o + r >= O) break;
      if constexpr (YBF16) ((uint16_t*)y)[base + r] = (uint16_t)f32_to_bf16_bits(v[r]);
      else ((float*)y)[base + r] = v[r];
      if (acc_out) acc_out[base + r] = c[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, each with
// its own L2. Block b runs on XCD b % 8; renumber so every XCD owns one
// contiguous range of tile ids, and walk tiles in groups of kGroupM O-tiles so
// neighbouring ids share W panels (A) and token panels (B).
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(int64_t bid, int64_t nb, int64_t ntm, int64_t ntn,
                                        int64_t& tm, int64_t& tn) {
  const int64_t xcd = bid % kXcds, local = bid / kXcds;
  const int64_t per = nb / kXcds, rem = nb % kXcds;
  const int64_t pid = xcd < rem ? xcd * (per + 1) + local
                                : rem * (per + 1) + (xcd - rem) * per + local;
  const int64_t gsz = (int64_t)kGroupM * ntn;
  const int64_t g = pid / gsz, first = g * kGroupM;
  const int64_t rows = (ntm - first) < kGroupM ? (ntm - first) : kGroupM;
  const int64_t in = pid % gsz;
  tm = first + in % rows;
  tn = in / rows;
}

// 32-bit form of tile_of (tile counts below 2^31).
__device__ __forceinline__ void tile_of32(uint32_t bid, uint32_t nb, uint32_t ntm, uint32_t ntn,
                                          int& tm, int& tn) {
  const uint32_t xcd = bid % kXcds, local = bid / kXcds;
  const uint32_t per = nb / kXcds, rem = nb % kXcds;
  const uint32_t pid = xcd < rem ? xcd * (per + 1) + local
                                 : rem * (per + 1) + (xcd - rem) * per + local;
  const uint32_t gsz = (uint32_t)kGroupM * ntn;
  const uint32_t g = pid / gsz, first = g * kGroupM;
  const uint32_t rows = (ntm - first) < (uint32_t)kGroupM ? (ntm - first) : (uint32_t)kGroupM;
  const uint32_t in = pid - g * gsz;
  tn = (int)(in / rows);
  tm = (int)(first + (in - (uint32_t)tn * rows));
}

// Two fp32 values -> packed bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32; finite inputs).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// One kernel for both forms. SP = false: dense form, BK = 64,
// v_mfma_i32_16x16x64_i8. SP = true: 2:4 index form, BK = 128,
// v_smfmac_i32_16x16x128_i8. Waves are arranged WAVES_M (along O) x WAVES_N
// (along T); each owns a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 tiles.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool KA16, bool YBF16,
          int MAXW = ((BM / WAVES_M) * (BN / WAVES_N) >= 128 * 128 ? 1 : 2)>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(1, MAXW)))
void k_gemm(const int8_t* __restrict__ xq, const float* __restrict__ sx,
            const uint8_t* __restrict__ packed, int64_t pitch, const float* __restrict__ sw,
            int64_t sw_inc, int64_t T, int64_t O, int64_t K, void* __restrict__ y,
            int32_t* __restrict__ acc_out) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FI = WM / 16, FJ = WN / 16;
  constexpr int BK = SP ? 128 : 64;
  constexpr int PB = SP ? kPitchBs : kPitchBd;
  constexpr int AROW = SP ? 32 : 16;          // packed bytes per W row per K-step
  constexpr int APT = BM * AROW / NT;          // packed bytes per thread per K-step
  constexpr int TPR = AROW / APT;              // threads per W row
  constexpr int SEGR = BK / 16;                // 16-byte xq segments per row per K-step
  constexpr int SEG = BN * SEGR;
  constexpr int NSEG = (SEG + NT - 1) / NT;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
  static_assert(APT >= (SP ? 8 : 4) && APT <= 32 && AROW % APT == 0, "A staging");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* As = smem;                          // [2][BM][kPitchA]
  uint8_t* Bs = smem + 2 * BM * kPitchA;       // [2][BN][PB]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int64_t ntm = cdiv(O, BM), ntn = cdiv(T, BN);
  int64_t tm, tn;
  tile_of(blockIdx.x, ntm * ntn, ntm, ntn, tm, tn);
  const int o0 = (int)(tm * BM), t0 = (int)(tn * BN);
  const int Oi = (int)O, Ti = (int)T, Ki = (int)K;
  const int nkf = Ki / BK;                     // full K-steps
  const int nk = (Ki + BK - 1) / BK;           // plus a masked tail step if K % BK != 0

  // Staging sources: consecutive lanes read consecutive 16-byte segments of a
  // row. Rows past O / T are clamped to the last valid row: they stay in
  // bounds and only feed accumulators that are never stored.
  const int ra = tid / TPR, pa = tid % TPR;
  const uint8_t* ap = packed + (int64_t)min(o0 + ra, Oi - 1) * pitch + APT * pa;
  const int8_t* bp[NSEG];
  int boff[NSEG];
#pragma unroll
  for (int q = 0; q < NSEG; ++q) {
    const int seg = min(tid + NT * q, SEG - 1);
    const int rb = seg / SEGR, cb = seg % SEGR;
    bp[q] = xq + (int64_t)min(t0 + rb, Ti - 1) * K + 16 * cb;
    boff[q] = rb * PB + 16 * cb;
  }
  const int aoff = ra * kPitchA;

  uint32_t ga[APT / 4];
  uint4 gb[NSEG];
  auto gload = [&](int ks) {
    const uint8_t* p = ap + (int64_t)ks * AROW;
    if constexpr (APT == 32) {
      const uint4 v0 = *(const uint4*)p, v1 = *(const uint4*)(p + 16);
      ga[0] = v0.x; ga[1] = v0.y; ga[2] = v0.z; ga[3] = v0.w;
      ga[4] = v1.x; ga[5] = v1.y; ga[6] = v1.z; ga[7] = v1.w;
    } else if constexpr (APT == 16) {
      const uint4 v = *(const uint4*)p;
      ga[0] = v.x; ga[1] = v.y; ga[2] = v.z; ga[3] = v.w;
    } else if constexpr (APT == 8) {
      const uint2 v = *(const uint2*)p;
      ga[0] = v.x; ga[1] = v.y;
    } else {
      ga[0] = *(const uint32_t*)p;
    }
    const int kb = ks * BK;
    if (KA16 && ks < nkf) {
#pragma unroll
      for (int q = 0; q < NSEG; ++q) gb[q] = *(const uint4*)(bp[q] + kb);
    } else {  // tail step, or rows only 4-byte aligned
#pragma unroll
      for (int q = 0; q < NSEG; ++q) {
        const int cb = min(tid + NT * q, SEG - 1) % SEGR;
        gb[q] = load_x16<KA16>(bp[q] - 16 * cb, kb + 16 * cb, K);
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* a = As + buf * BM * kPitchA + aoff;
    if constexpr (SP) {
#pragma unroll
      for (int c = 0; c < APT / 8; ++c) {
        const int ch = (APT / 8) * pa + c;
        const uint32_t cw = ga[2 * c], iw = ga[2 * c + 1];
        *(uint4*)(a + 16 * ch) = make_uint4(expand_codes(cw, 0), expand_codes(cw, 1),
                                            expand_codes(cw, 2), expand_codes(cw, 3));
        *(uint32_t*)(a + 64 + 4 * ch) = iw;
      }
    } else {
#pragma unroll
      for (int w = 0; w < APT / 4; ++w) {
        *(uint4*)(a + 16 * ((APT / 4) * pa + w)) =
            make_uint4(expand_codes(ga[w], 0), expand_codes(ga[w], 1), expand_codes(ga[w], 2),
                       expand_codes(ga[w], 3));
      }
    }
    uint8_t* b = Bs + buf * BN * PB;
#pragma unroll
    for (int q = 0; q < NSEG; ++q)
      if (NSEG * NT == SEG || tid + NT * q < SEG) *(uint4*)(b + boff[q]) = gb[q];
  };

  v4i acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  gload(0);
  sstore(0);
  __syncthreads();
  const int g = lane >> 4, r16 = lane & 15;
  const int afrag = (wm * WM + r16) * kPitchA, bfrag = (wn * WN + r16) * PB;
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* a = As + buf * BM * kPitchA + afrag;
    const uint8_t* b = Bs + buf * BN * PB + bfrag;
    // all fragments of this K-step are requested before the first MFMA
    if constexpr (SP) {
      v8i bf[FJ];
      v4i af[FI];
      int ai[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        af[i] = *(const v4i*)(a + 16 * i * kPitchA + 16 * g);
        ai[i] = *(const int*)(a + 16 * i * kPitchA + 64 + 4 * g);
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const v4i lo = *(const v4i*)(b + 16 * j * PB + 16 * g);
        const v4i hi = *(const v4i*)(b + 16 * j * PB + 64 + 16 * g);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(af[i], bf[j], acc[i][j], ai[i], 0, 0);
    } else {
      v4i bf[FJ], af[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) af[i] = *(const v4i*)(a + 16 * i * kPitchA + 16 * g);
#pragma unroll
      for (int j = 0; j < FJ; ++j) bf[j] = *(const v4i*)(b + 16 * j * PB + 16 * g);
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: one token column per lane and j; four consecutive outputs per tile
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int t = t0 + wn * WN + 16 * j + r16;
    if (t >= Ti) continue;
    const float s_t = sx[t];
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int o = o0 + wm * WM + 16 * i + 4 * g;
      if (o >= Oi) continue;
      store_tile<YBF16>(y, acc_out, acc[i][j], t, o, Oi, s_t, sw, (int)sw_inc);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel with LDS DMA (global_load_lds): used when K is a multiple of
// BK. Operand tiles go straight from global memory into an S-slot LDS ring in
// fragment-major order -- xq as 16-byte lane slots, packed W as 4-byte code
// (and, for 2:4, index) words -- without passing through registers, so S-2
// K-steps of MFMA work cover the global latency. One K-step ahead, the
// workgroup expands the next stage's 2-bit codes into an int8 A buffer.
// Every stage issues the same DMA instructions per wave (stages past the end
// reload the last stage into a free slot), so the wait count is a constant.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int waitcnt_vmcnt(int n) {
  // gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14]; lgkmcnt and
  // expcnt at their maxima (not waited on)
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Workgroup barrier for the DMA pipeline: wait until this wave has at most n
// vector-memory operations (LDS DMAs) outstanding and all its LDS operations
// are done, then s_barrier. Unlike __syncthreads() this does not drain the
// DMAs still in flight for later stages. The empty asm statements only stop
// the compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename P>
__device__ __forceinline__ void dma16(const P* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
template <typename P>
__device__ __forceinline__ void dma4(const P* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool YBF16, int S>
struct DmaCfg {
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int FA = BM / 16, FB = BN / 16;
  static constexpr int BFB = SP ? 2048 : 1024;
  static constexpr int SLOT_B = FB * BFB, SLOT_AC = FA * 256, SLOT_AI = SP ? FA * 256 : 0;
  static constexpr int SLOT = SLOT_B + SLOT_AC + SLOT_AI;
  static constexpr int AEXP = FA * 1024;
  static constexpr size_t LDS = (size_t)S * SLOT + 2 * AEXP;
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool YBF16, int S>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_gemm_dma(const int8_t* __restrict__ xq, const float* __restrict__ sx,
                const uint8_t* __restrict__ packed, int64_t pitch, const float* __restrict__ sw,
                int64_t sw_inc, int64_t T, int64_t O, int64_t K, void* __restrict__ y,
                int32_t* __restrict__ acc_out) {
  using C = DmaCfg<BM, BN, WAVES_M, WAVES_N, SP, YBF16, S>;
  constexpr int NW = C::NW, NT = C::NT;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FI = WM / 16, FJ = WN / 16;
  constexpr int BK = SP ? 128 : 64;
  constexpr int AROW = SP ? 32 : 16;
  constexpr int NBI = C::FB * (SP ? 2 : 1), NAI = C::FA * (SP ? 2 : 1), NI = NBI + NAI;
  constexpr int IPW = NI / NW;                 // DMA instructions per wave per stage
  constexpr int NEXP = C::FA * 64 / NT;        // A lane slots expanded per thread
  static_assert(NI % NW == 0 && (C::FA * 64) % NT == 0 && NEXP >= 1, "staging split");
  static_assert(S >= 3 && IPW * (S - 3) < 64, "pipeline depth");
  // Each ring slot is its own LDS object and the K-loop is unrolled by S, so
  // every LDS access names a compile-time slot: the compiler then only waits
  // for the DMAs that target the slot being read. The expanded-A buffer is a
  // separate object (no DMA ever targets it).
  constexpr int SL = C::SLOT;
  __shared__ __attribute__((aligned(16))) uint8_t rs0[SL], rs1[SL], rs2[SL];
  __shared__ __attribute__((aligned(16))) uint8_t rs3[S > 3 ? SL : 16], rs4[S > 4 ? SL : 16];
  __shared__ __attribute__((aligned(16))) uint8_t aexp[2 * C::AEXP];
  uint8_t* const slots[5] = {rs0, rs1, rs2, rs3, rs4};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int64_t ntm = cdiv(O, BM), ntn = cdiv(T, BN);
  int64_t tm, tn;
  tile_of(blockIdx.x, ntm * ntn, ntm, ntn, tm, tn);
  const int o0 = (int)(tm * BM), t0 = (int)(tn * BN);
  const int Oi = (int)O, Ti = (int)T;
  const int nk = (int)(K / BK);

  // this wave's DMA sources (stage 0) and slot-relative LDS destinations;
  // rows past O / T are clamped to the last valid row (never stored)
  const uint8_t* src[IPW];
  int dst[IPW];
  // Slot order inside a 16-row block: DMA lane l fills slot l with row l/4,
  // k-block (l%4) ^ ((l/16)%4), so four consecutive lanes fetch one row's 64
  // contiguous bytes; MFMA lane (row r, k-block g) reads slot
  // 4r + (g ^ (r/4)%4), which keeps each 16-lane group in distinct banks.
  const int drow = lane >> 2, dkb = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int idx = wave * IPW + u;
    if (idx < NBI) {
      const int f = SP ? idx >> 1 : idx, h = SP ? idx & 1 : 0;
      const int row = 16 * f + drow, seg = 4 * h + dkb;
      src[u] = (const uint8_t*)(xq + (int64_t)min(t0 + row, Ti - 1) * K + 16 * seg);
      dst[u] = f * C::BFB + h * 1024;
    } else {
      const int a = idx - NBI;
      const int f = SP ? a >> 1 : a, part = SP ? a & 1 : 0;
      const int row = 16 * f + drow, kb = dkb;
      src[u] = packed + (int64_t)min(o0 + row, Oi - 1) * pitch + (SP ? 8 * kb + 4 * part : 4 * kb);
      dst[u] = C::SLOT_B + part * C::SLOT_AC + f * 256;
    }
  }
  auto issue = [&](int ks, uint8_t* base) {
    const int kc = min(ks, nk - 1);
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const int idx = wave * IPW + u;          // uniform across the wave
      if (idx < NBI) dma16(src[u] + (int64_t)kc * BK, base + dst[u]);
      else dma4(src[u] + (int64_t)kc * AROW, base + dst[u]);
    }
  };
  auto expand = [&](const uint8_t* slot, int ebuf) {
    const uint8_t* codes = slot + C::SLOT_B;
    uint8_t* out = aexp + ebuf * C::AEXP;
#pragma unroll
    for (int q = 0; q < NEXP; ++q) {
      const int p = tid + NT * q, f = p >> 6, l = p & 63;
      const uint32_t cw = *(const uint32_t*)(codes + f * 256 + l * 4);
      *(uint4*)(out + f * 1024 + l * 16) =
          make_uint4(expand_codes(cw, 0), expand_codes(cw, 1), expand_codes(cw, 2), expand_codes(cw, 3));
    }
  };

  v4i acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int rs = 4 * (lane & 15) + ((lane >> 4) ^ ((lane >> 2) & 3));   // this lane's slot
  auto compute = [&](const uint8_t* slot, int ebuf) {
    const uint8_t* b = slot + (wn * FJ) * C::BFB + rs * 16;
    const uint8_t* a = aexp + ebuf * C::AEXP + (wm * FI) * 1024 + rs * 16;
    if constexpr (SP) {
      const uint8_t* ai_base = slot + C::SLOT_B + C::SLOT_AC + (wm * FI) * 256 + rs * 4;
      v8i bf[FJ];
      v4i af[FI];
      int ai[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        af[i] = *(const v4i*)(a + i * 1024);
        ai[i] = *(const int*)(ai_base + i * 256);
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const v4i lo = *(const v4i*)(b + j * C::BFB);
        const v4i hi = *(const v4i*)(b + j * C::BFB + 1024);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(af[i], bf[j], acc[i][j], ai[i], 0, 0);
    } else {
      v4i bf[FJ], af[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) af[i] = *(const v4i*)(a + i * 1024);
#pragma unroll
      for (int j = 0; j < FJ; ++j) bf[j] = *(const v4i*)(b + j * C::BFB);
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, slots[st]);
  dma_barrier<IPW * (S - 2)>();        // every wave's stage-0 DMAs landed
  expand(slots[0], 0);
  for (int ks0 = 0; ks0 < nk; ks0 += S) {
#pragma unroll
    for (int I = 0; I < S; ++I) {
      const int ks = ks0 + I;                 // stage ks lives in slot I
      if (ks < nk) {
        // stage ks+1 landed and visible; expand(ks) and compute(ks-1) done everywhere
        dma_barrier<IPW * (S - 3)>();
        issue(ks + S - 1, slots[(I + S - 1) % S]);   // into the slot of stage ks-1
        expand(slots[(I + 1) % S], (ks + 1) & 1);
        compute(slots[I], ks & 1);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));   // no DMA may still target LDS at exit

  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int t = t0 + wn * WN + 16 * j + r16;
    if (t >= Ti) continue;
    const float s_t = sx[t];
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int o = o0 + wm * WM + 16 * i + 4 * g;
      if (o >= Oi) continue;
      store_tile<YBF16>(y, acc_out, acc[i][j], t, o, Oi, s_t, sw, (int)sw_inc);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel with register-resident W fragments.
//
// LDS bandwidth, not the matrix cores, limits a kernel that stages both
// operands through LDS: a 64x64 wave tile reads 8 KB of fragments per 16
// MFMAs. Here only xq goes through LDS; the packed W rows go from global
// memory straight into VGPRs in MFMA layout (8 bytes of 2-bit codes, or one
// 2:4 chunk, per lane and K-step) and are expanded in registers. The waves of
// a K-group split the tile along O only, so each staged xq fragment is read
// by all of them, and no W byte is shared between waves.
//
// A K-step covers 128 dense k. Lane (r, g) of fragment i loads 8 bytes at
// byte 32*s + 8*g of W row o0 + 16*i + r:
//   dense form: code words 8s+2g and 8s+2g+1, i.e. k in [128s+32g, +32);
//     sub-step j in {0, 1} feeds k [128s + 32g + 16j, +16) to lane group g of
//     v_mfma_i32_16x16x64_i8, so B lane (t, g) reads xq[t][128s+32g+16j, +16);
//   2:4 index form: chunk 4s+g (codes word, index word), exactly the sparse
//     operand of v_smfmac_i32_16x16x128_i8; B lane (t, g) reads k [16g, +16)
//     and [64+16g, +16) of the step.
// W loads are issued NA-1 K-steps ahead into a ring of NA register slots;
// xq for step s+3 is loaded into registers at the end of step s and stored to
// a double-buffered LDS tile two steps later.
//
// KS > 1 splits the K-steps of one output tile between KS groups of WO waves
// (each group with its own xq tiles); their int32 accumulators are summed
// through LDS before the epilogue. Integer sums are exact, so the split does
// not change any result.
//
// The grid is persistent: workgroup b takes tiles b, b + G, b + 2G, ... The
// loads of a tile's first K-steps are issued before the previous tile's
// epilogue, so their latency hides behind it. The bf16 epilogue stages the
// dequantized tile in LDS and writes each output row segment with contiguous
// 16-byte lanes; the stores are non-temporal (y is not read again here, so it
// should not push the re-read W and xq panels out of the caches).
// ---------------------------------------------------------------------------
constexpr int kPitchR = 144;   // LDS bytes per staged xq row (128 k + 16 pad)

template <int WO, int KS, int FI, int FJ, int NA>
struct RaCfg {
  static constexpr int NTQ = 64 * WO, NT = NTQ * KS, NW = WO * KS;
  static constexpr int BM = WO * 16 * FI, BN = 16 * FJ;
  static constexpr int BUF = BN * kPitchR;
  static constexpr int PO = BM * 2 + 16;         // LDS bytes per staged output row
  static constexpr size_t LDS_B = (size_t)KS * 2 * BUF;
  static constexpr size_t LDS_RED = KS > 1 ? (size_t)WO * FI * FJ * 64 * 16 : 0;
  static constexpr size_t LDS_OUT = (size_t)BN * PO;
  static constexpr size_t M1 = LDS_B > LDS_RED ? LDS_B : LDS_RED;
  static constexpr size_t SCALES = M1 > LDS_OUT ? M1 : LDS_OUT;   // offset of sx / sw
  static constexpr int NSC = (BM + BN + NT - 1) / NT;            // scales per thread
  static constexpr size_t LDS = SCALES + (size_t)(BM + BN) * 4;
};

// largest divisor of n that is at most 8 (1 for n <= 0)
__host__ __device__ constexpr int largest_divisor_upto8(int n) {
  return n <= 0 ? 1 : n % 8 == 0 ? 8 : n % 7 == 0 ? 7 : n % 6 == 0 ? 6 : n % 5 == 0 ? 5 :
         n % 4 == 0 ? 4 : n % 3 == 0 ? 3 : n % 2 == 0 ? 2 : 1;
}

template <int WO, int KS, int FI, int FJ, int NA, bool SP, bool YBF16>
__global__ __launch_bounds__(64 * WO * KS) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_ra(const int8_t* __restrict__ xq, const float* __restrict__ sx,
               const uint8_t* __restrict__ packed, int64_t pitch, const float* __restrict__ sw,
               int64_t sw_inc, int64_t T, int64_t O, int64_t K, void* __restrict__ y,
               int32_t* __restrict__ acc_out) {
  using C = RaCfg<WO, KS, FI, FJ, NA>;
  constexpr int NT = C::NT, NTQ = C::NTQ, NW = C::NW, BM = C::BM, BN = C::BN;
  constexpr int SEGS = BN * 8;                       // 16-byte xq segments per step
  constexpr int NSB = (SEGS + NTQ - 1) / NTQ;
  constexpr int U = NA == 3 ? 6 : 4;                 // K-loop unroll (static slots)
  static_assert(NA >= 2 && NA <= 4, "W register ring");
  static_assert(NTQ % 8 == 0, "staging layout");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* const sxs = (float*)(smem + C::SCALES);     // [BN] sx of the tile's tokens
  float* const sws = sxs + BN;                       // [BM] sw of the tile's rows

  // Every global load below is unconditional and in bounds (row and step
  // indices are clamped), so no lane-divergent branch stands between a
  // prefetch and its use and the compiler's wait counts stay exact.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wo = wave % WO, q = wave / WO, tq = tid - q * NTQ;
  const int g = lane >> 4, r16 = lane & 15;
  const uint32_t ntm = (uint32_t)cdiv(O, BM), ntn = (uint32_t)cdiv(T, BN), ntiles = ntm * ntn;
  const int Oi = (int)O, Ti = (int)T, Ki = (int)K, pitchi = (int)pitch;
  const int ns = (Ki + 127) >> 7;                    // K-steps of 128 (ns >= 1)
  const int nsq = (ns + KS - 1) / KS;
  const int sb = q * nsq, se = min(ns, sb + nsq);    // this group's steps
  const int slast = max(se - 1, 0);                  // clamp for loads
  const int cb16 = 16 * (tq & 7);                    // xq segment column of this thread
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(packed), rbx = buffer_rsrc(xq);

  int o0 = 0, t0 = 0;
  uint32_t avo[FI];                                  // W row offsets (+ 8g)
  uint32_t bvo[NSB];                                 // xq row offsets (+ segment column)
  int bdst[NSB];
  float scr[C::NSC];
  // W rows past O and xq rows past T are clamped to the last valid row: they
  // only feed accumulators that are never stored. For s < ns the 8 bytes at
  // 32s + 8g lie inside the row record; in the dense form units past the code
  // words hold mask bits, which meet xq columns k >= K (zero in LDS).
  auto setup = [&](uint32_t tile) {
    int tm, tn;
    tile_of32(tile, ntiles, ntm, ntn, tm, tn);
    o0 = tm * BM;
    t0 = tn * BN;
#pragma unroll
    for (int i = 0; i < FI; ++i)
      avo[i] = (uint32_t)min(o0 + wo * 16 * FI + 16 * i + r16, Oi - 1) * (uint32_t)pitchi + 8 * g;
#pragma unroll
    for (int u = 0; u < NSB; ++u) {
      const int rb = min((tq >> 3) + (NTQ / 8) * u, BN - 1);
      bvo[u] = (uint32_t)min(t0 + rb, Ti - 1) * (uint32_t)Ki + cb16;
      bdst[u] = rb * kPitchR + cb16;
    }
#pragma unroll
    for (int c = 0; c < C::NSC; ++c) {
      const int e = min(tid + NT * c, BM + BN - 1);
      scr[c] = e < BN ? sx[min(t0 + e, Ti - 1)] : sw[(int64_t)min(o0 + e - BN, Oi - 1) * sw_inc];
    }
  };
  auto aload = [&](int s, uint2 (&d)[FI]) {
    const int soff = 32 * min(s, slast);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ra, avo[i], soff, 0);
      d[i] = make_uint2(v.x, v.y);
    }
  };
  // xq of step s: 16 bytes per segment. Only the final K-step can reach past
  // K; there the column is clamped (the data is zeroed at the store).
  auto bload = [&](int s, uint4 (&r)[NSB]) {
    const int sc = min(s, slast);
    const int kb = 128 * sc;
    if (kb + 128 <= Ki) {
#pragma unroll
      for (int u = 0; u < NSB; ++u) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rbx, bvo[u], kb, 0);
        r[u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    } else {
      const int over = max(kb + cb16 - (Ki - 16), 0);   // lanes whose segment passes K
#pragma unroll
      for (int u = 0; u < NSB; ++u) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rbx, bvo[u] - over, kb, 0);
        r[u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
  };
  uint8_t* const bq = smem + (size_t)q * 2 * C::BUF;
  // store the xq of step s; columns k >= K become zero (final step only)
  auto bstore = [&](int s, int buf, const uint4 (&r)[NSB]) {
    uint8_t* b = bq + buf * C::BUF;
    if (128 * s + 128 <= Ki) {
#pragma unroll
      for (int u = 0; u < NSB; ++u)
        if (NSB * NTQ == SEGS || tq + NTQ * u < SEGS) *(uint4*)(b + bdst[u]) = r[u];
    } else {
      const uint32_t m = (uint32_t)((128 * s + cb16 - Ki) >> 31);   // all ones if k < K
#pragma unroll
      for (int u = 0; u < NSB; ++u)
        if (NSB * NTQ == SEGS || tq + NTQ * u < SEGS)
          *(uint4*)(b + bdst[u]) = make_uint4(r[u].x & m, r[u].y & m, r[u].z & m, r[u].w & m);
    }
  };

  auto expand = [](uint32_t w) -> v4i {
    return v4i{(int)expand_codes(w, 0), (int)expand_codes(w, 1), (int)expand_codes(w, 2),
               (int)expand_codes(w, 3)};
  };
  v4i acc[FI][FJ];
  // exc: the expanded W fragment the next MFMAs consume. Each fragment is
  // expanded while the MFMAs of the previous one run (the last fragment of a
  // step expands the first of the next step), so the VALU work issues under
  // the matrix-core work instead of in front of it.
  v4i exc;

  // One K-step from LDS buffer buf with W slot a (an: the next step's slot).
  // (the wave's issue priority is raised while it issues its matrix-core
  // block, so that of two waves on a SIMD the one with MFMAs ready goes first:
  // 2-4% on the dense N:M shapes)
  auto compute = [&](int buf, const uint2 (&a)[FI], const uint2 (&an)[FI]) {
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* b = bq + buf * C::BUF + r16 * kPitchR;
    if constexpr (SP) {
      v8i bf[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const v4i lo = *(const v4i*)(b + 16 * j * kPitchR + 16 * g);
        const v4i hi = *(const v4i*)(b + 16 * j * kPitchR + 64 + 16 * g);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const v4i exn = expand(i + 1 < FI ? a[i + 1].x : an[0].x);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(exc, bf[j], acc[i][j], (int)a[i].y,
                                                               0, 0);
        exc = exn;
      }
#pragma unroll
      for (int m = 0; m < FI * FJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, (11 + FJ - 1) / FJ, 0);  // VALU share
      }
    } else {
      v4i bf[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) bf[j] = *(const v4i*)(b + 16 * j * kPitchR + 32 * g);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const uint32_t wn = i + 1 < FI ? (h ? a[i + 1].y : a[i + 1].x) : (h ? an[0].x : a[0].y);
          const v4i exn = expand(wn);
#pragma unroll
          for (int j = 0; j < FJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(exc, bf[j], acc[i][j], 0, 0, 0);
          exc = exn;
        }
        if (h == 0) {
          // xq fragments of sub-step 1 (the registers free up as the MFMAs
          // issue; wide wave tiles keep the loads behind this point so that
          // the two sub-steps' fragments never hold registers at once)
          if constexpr (FJ >= 8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < FJ; ++j) bf[j] = *(const v4i*)(b + 16 * j * kPitchR + 32 * g + 16);
        }
      }
#pragma unroll
      for (int m = 0; m < 2 * FI * FJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (11 + FJ - 1) / FJ, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // W for steps sb..sb+NA-2 in the ring. xq: with two register sets (small
  // wave tiles) step s+3 is loaded at the end of step s and stored two steps
  // later; with one set, step s+1 is loaded at the start of step s.
  constexpr int NBS = FI * FJ >= 32 ? 1 : 2;
  uint2 ar[NA][FI];
  uint4 rb[NBS][NSB];
  auto prologue = [&]() {
#pragma unroll
    for (int p = 0; p < NA - 1; ++p) aload(sb + p, ar[p]);
    bload(sb, rb[0]);
    if constexpr (NBS == 2) bload(sb + 1, rb[1]);
  };

  uint32_t tile = blockIdx.x;
  setup(tile);
  prologue();
  for (;;) {
    bstore(sb, 0, rb[0]);                             // xq of step sb into LDS
    if constexpr (NBS == 2) bload(sb + 2, rb[0]);
    exc = expand(ar[0][0].x);                         // first W fragment
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    __syncthreads();
    // this tile's scales to LDS (loaded with the tile's first operands, so
    // waiting for them here costs nothing; read after the loop's barriers)
#pragma unroll
    for (int c = 0; c < C::NSC; ++c) {
      const int e = tid + NT * c;
      if (e < BM + BN) sxs[e] = scr[c];              // sws follows sxs
    }

    for (int it = 0; it < nsq; it += U) {
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int s = sb + it + t;
        // (xq first: waiting for it before its LDS store then leaves the W
        // loads behind it in flight)
        if constexpr (NBS == 1) bload(s + 1, rb[0]);
        aload(s + NA - 1, ar[(t + NA - 1) % NA]);      // into the slot of step s-1
        if (s < se) compute(t & 1, ar[t % NA], ar[(t + 1) % NA]);
        if constexpr (NBS == 1) {
          bstore(s + 1, (t + 1) & 1, rb[0]);
        } else {
          // xq of step s+1 is in the register set of parity (t+1)&1
          bstore(s + 1, (t + 1) & 1, rb[(t + 1) & 1]);
          bload(s + 3, rb[(t + 1) & 1]);
        }
        // LDS-only barrier: the global loads of later steps stay in flight
        // (__syncthreads() would wait for all of them)
        dma_barrier<63>();
      }
    }

    // the next tile's first loads go out before this tile's epilogue
    const int eo0 = o0, et0 = t0;
    const uint32_t next = tile + gridDim.x;
    const bool more = next < ntiles;
    if (more) {
      setup(next);
      prologue();
    }

    if constexpr (KS > 1) {
      // sum the K-groups' accumulators into group 0 (through the xq area)
      v4i* red = (v4i*)smem;
#pragma unroll 1
      for (int r = 1; r < KS; ++r) {
        if (q == r) {
#pragma unroll
          for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) red[((wo * FI + i) * FJ + j) * 64 + lane] = acc[i][j];
        }
        __syncthreads();
        if (q == 0) {
#pragma unroll
          for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) acc[i][j] += red[((wo * FI + i) * FJ + j) * 64 + lane];
        }
        __syncthreads();
      }
    }

    if (YBF16 && acc_out == nullptr) {
      // dequantize into the LDS output tile (bf16), then write whole row segments
      uint8_t* const ot = smem;
      if (q == 0) {
        float4 w4[FI];
        float st[FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i) w4[i] = *(const float4*)(sws + wo * 16 * FI + 16 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < FJ; ++j) st[j] = sxs[16 * j + r16];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          const int tl = 16 * j + r16;
#pragma unroll
          for (int i = 0; i < FI; ++i) {
            const int ol = wo * 16 * FI + 16 * i + 4 * g;
            const float v0 = ((float)acc[i][j][0] * st[j]) * w4[i].x;
            const float v1 = ((float)acc[i][j][1] * st[j]) * w4[i].y;
            const float v2 = ((float)acc[i][j][2] * st[j]) * w4[i].z;
            const float v3 = ((float)acc[i][j][3] * st[j]) * w4[i].w;
            *(uint2*)(ot + tl * C::PO + 2 * ol) = make_uint2(pack_bf16x2(v0, v1),
                                                             pack_bf16x2(v2, v3));
          }
        }
      }
      __syncthreads();
      constexpr int RW = (BN + NW - 1) / NW;          // rows per wave
      constexpr int RC = RW < 8 ? RW : 8;             // rows in flight per wave
      constexpr int CPR = BM / 4;                     // 8-byte chunks per row
      constexpr int CL = (CPR + 63) / 64;             // chunks per lane and row
      constexpr int CP16 = BM / 8;                    // 16-byte chunks per row (full-tile path)
      constexpr int LPR = CP16 < 64 ? CP16 : 64;      // lanes per row
      constexpr int RPI = 64 / LPR;                   // rows per wave instruction
      constexpr int RWF = BN / (NW * RPI);            // row groups per wave
      constexpr int RF = largest_divisor_upto8(RWF);          // row groups in flight
      constexpr bool FULL_OK = CP16 % LPR == 0 && BN % (NW * RPI) == 0 && RWF % RF == 0 && RWF > 0;
      if (FULL_OK && (Oi & 7) == 0 && eo0 + BM <= Oi && et0 + BN <= Ti) {
        // whole tile inside y: straight-line reads and 16-byte stores
        constexpr int CF = CP16 / LPR;
        const int lr = lane / LPR, lc = lane % LPR;
#pragma unroll
        for (int m0 = 0; m0 < RWF; m0 += RF) {
          v4u v[RF][CF];
#pragma unroll
          for (int m = 0; m < RF; ++m)
#pragma unroll
            for (int c = 0; c < CF; ++c)
              v[m][c] = *(const v4u*)(ot + ((wave + NW * (m0 + m)) * RPI + lr) * C::PO +
                                      16 * (lc + LPR * c));
#pragma unroll
          for (int m = 0; m < RF; ++m) {
            uint16_t* yr = (uint16_t*)y +
                           (int64_t)(et0 + (wave + NW * (m0 + m)) * RPI + lr) * Oi + eo0;
#pragma unroll
            for (int c = 0; c < CF; ++c)
              __builtin_nontemporal_store(v[m][c], (v4u*)(yr + 8 * (lc + LPR * c)));
          }
        }
      } else {
        const bool fast = (Oi & 3) == 0 && eo0 + BM <= Oi;
#pragma unroll 1
        for (int m0 = 0; m0 < RW; m0 += RC) {
          uint2 v[RC][CL];
#pragma unroll
          for (int m = 0; m < RC; ++m)
#pragma unroll
            for (int c = 0; c < CL; ++c) {
              const int tl = min(wave + NW * (m0 + m), BN - 1), ch = min(lane + 64 * c, CPR - 1);
              v[m][c] = *(const uint2*)(ot + tl * C::PO + 8 * ch);
            }
#pragma unroll
          for (int m = 0; m < RC; ++m) {
            const int tl = wave + NW * (m0 + m), t = et0 + tl;
            if (m0 + m >= RW || tl >= BN || t >= Ti) continue;
            uint16_t* yr = (uint16_t*)y + (int64_t)t * Oi + eo0;
#pragma unroll
            for (int c = 0; c < CL; ++c) {
              const int ch = lane + 64 * c;
              if (ch >= CPR) continue;
              if (fast) {
                *(uint2*)(yr + 4 * ch) = v[m][c];
              } else {
                const uint16_t h[4] = {(uint16_t)(v[m][c].x & 0xFFFF), (uint16_t)(v[m][c].x >> 16),
                                       (uint16_t)(v[m][c].y & 0xFFFF), (uint16_t)(v[m][c].y >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (eo0 + 4 * ch + r < Oi) yr[4 * ch + r] = h[r];
              }
            }
          }
        }
      }
      __syncthreads();                                // output tile area free again
    } else {
      if (q == 0) {
        // fp32 output or int32 accumulators requested: store from registers
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          const int t = et0 + 16 * j + r16;
          if (t >= Ti) continue;
          const float s_t = sxs[16 * j + r16];
#pragma unroll
          for (int i = 0; i < FI; ++i) {
            const int o = eo0 + wo * 16 * FI + 16 * i + 4 * g;
            if (o >= Oi) continue;
            store_tile<YBF16>(y, acc_out, acc[i][j], t, o, Oi, s_t, sw, (int)sw_inc);
          }
        }
      }
      __syncthreads();
    }
    if (!more) break;
    tile = next;
  }
}

// ---------------------------------------------------------------------------
// Tile configurations and the per-shape choice.
// ---------------------------------------------------------------------------
enum TileCfg { kT256x256 = 0, kT256x128 = 1, kT128x256 = 2, kT128x128 = 3, kT256x32 = 4,
               kT128x32 = 5, kT256x256w8 = 6, kT128x256w8 = 7, kT256x128w8 = 8,
               kT256x256w8t = 9, kDma128x256 = 10, kDma256x128 = 11, kDma128x128 = 12,
               kDma256x256 = 13, kT64x128 = 14,
               // register-W kernel: WO x KS waves, wave tile (16 FI) x (16 FJ), ring NA
               kR256x64 = 15,      // WO 4, KS 1, FI 4, FJ 4
               kR256x128 = 16,     // WO 4, KS 1, FI 4, FJ 8 (NA 2)
               kR512x64 = 17,      // WO 4, KS 1, FI 8, FJ 4 (NA 2)
               kR128x128 = 18,     // WO 2, KS 1, FI 4, FJ 8 (NA 2)
               kR256x64k2 = 19,    // WO 4, KS 2, FI 4, FJ 4
               kR128x64k2 = 20,    // WO 2, KS 2, FI 4, FJ 4
               kR128x64k4 = 21,    // WO 2, KS 4, FI 4, FJ 4
               kR128x128k2 = 22,   // WO 2, KS 2, FI 4, FJ 8 (NA 2)
               kR512x64w8 = 23,    // WO 8, KS 1, FI 4, FJ 4
               kR256x80 = 24,      // WO 4, KS 1, FI 4, FJ 5
               kR256x96 = 25,      // WO 4, KS 1, FI 4, FJ 6 (NA 2)
               kR512x128w8 = 26,   // WO 8, KS 1, FI 4, FJ 8 (NA 2)
               kR384x64 = 27,      // WO 6, KS 1, FI 4, FJ 4
               kNumCfg = 28 };

struct Args {
  const int8_t* xq; const float* sx; const uint8_t* packed; int64_t pitch; const float* sw;
  int64_t sw_inc, T, O, K; void* y; int32_t* acc;
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool KA16, bool YBF16>
static hipError_t launch_cfg(const Args& a, hipStream_t s) {
  const size_t lds = 2 * (size_t)BM * kPitchA + 2 * (size_t)BN * (SP ? kPitchBs : kPitchBd);
  auto kern = k_gemm<BM, BN, WAVES_M, WAVES_N, SP, KA16, YBF16>;
  if (lds > 65536) {
    static bool set = false;  // attribute is per kernel; setting it twice is harmless
    if (!set) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      set = true;
    }
  }
  const int64_t nb = cdiv(a.O, BM) * cdiv(a.T, BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(64 * WAVES_M * WAVES_N), lds, s, a.xq, a.sx,
                     a.packed, a.pitch, a.sw, a.sw_inc, a.T, a.O, a.K, a.y, a.acc);
  return hipGetLastError();
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool YBF16, int S>
static hipError_t launch_dma(const Args& a, hipStream_t s) {
  auto kern = k_gemm_dma<BM, BN, WAVES_M, WAVES_N, SP, YBF16, S>;  // static LDS
  const int64_t nb = cdiv(a.O, BM) * cdiv(a.T, BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(64 * WAVES_M * WAVES_N), 0, s, a.xq, a.sx,
                     a.packed, a.pitch, a.sw, a.sw_inc, a.T, a.O, a.K, a.y, a.acc);
  return hipGetLastError();
}

template <int WO, int KS, int FI, int FJ, int NA, bool SP, bool KA16, bool YBF16>
static hipError_t launch_ra(const Args& a, hipStream_t s) {
  using C = RaCfg<WO, KS, FI, FJ, NA>;
  // 16-byte xq segments and 32-bit buffer offsets
  if (!KA16 || a.T * a.K >= (int64_t(1) << 31) || a.O * a.pitch >= (int64_t(1) << 31))
    return launch_cfg<128, 128, 2, 2, SP, KA16, YBF16>(a, s);
  auto kern = k_gemm_ra<WO, KS, FI, FJ, NA, SP, YBF16>;
  if (C::LDS > 65536) {
    static bool set = false;
    if (!set) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
      if (e != hipSuccess) return e;
      set = true;
    }
  }
  // persistent grid: as many workgroups as fit on the chip at once (a
  // multiple of the 8 XCDs, so each workgroup's tiles stay on one XCD's range)
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)kern, C::NT,
                                                                C::LDS);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
  }
  const int64_t ntiles = cdiv(a.O, C::BM) * cdiv(a.T, C::BN);
  int64_t nb = (int64_t)per_cu * device_info().cus;
  if (nb >= ntiles) nb = ntiles;
  else nb = nb / kXcds * kXcds;
  hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(C::NT), C::LDS, s, a.xq, a.sx, a.packed,
                     a.pitch, a.sw, a.sw_inc, a.T, a.O, a.K, a.y, a.acc);
  return hipGetLastError();
}

template <bool SP, bool KA16, bool YBF16>
static hipError_t launch_sel(int cfg, const Args& a, hipStream_t s) {
  switch (cfg) {
    case kR256x64: return launch_ra<4, 1, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kR256x128: return launch_ra<4, 1, 4, 8, 2, SP, KA16, YBF16>(a, s);
    case kR512x64: return launch_ra<4, 1, 8, 4, 2, SP, KA16, YBF16>(a, s);
    case kR128x128: return launch_ra<2, 1, 4, 8, 2, SP, KA16, YBF16>(a, s);
    case kR256x64k2: return launch_ra<4, 2, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kR128x64k2: return launch_ra<2, 2, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kR128x64k4: return launch_ra<2, 4, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kR128x128k2: return launch_ra<2, 2, 4, 8, 2, SP, KA16, YBF16>(a, s);
    case kR512x64w8: return launch_ra<8, 1, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kR256x80: return launch_ra<4, 1, 4, 5, 4, SP, KA16, YBF16>(a, s);
    case kR256x96: return launch_ra<4, 1, 4, 6, 2, SP, KA16, YBF16>(a, s);
    case kR512x128w8: return launch_ra<8, 1, 4, 8, 2, SP, KA16, YBF16>(a, s);
    case kR384x64: return launch_ra<6, 1, 4, 4, 4, SP, KA16, YBF16>(a, s);
    case kT64x128: return launch_cfg<64, 128, 2, 2, SP, KA16, YBF16>(a, s);
    case kDma128x256: return launch_dma<128, 256, 2, 4, SP, YBF16, SP ? 3 : 4>(a, s);
    case kDma256x128: return launch_dma<256, 128, 4, 2, SP, YBF16, SP ? 4 : 5>(a, s);
    case kDma128x128: return launch_dma<128, 128, 2, 2, SP, YBF16, SP ? 4 : 5>(a, s);
    case kDma256x256: return launch_dma<256, 256, 2, 4, SP, YBF16, SP ? 3 : 4>(a, s);
    case kT256x256: return launch_cfg<256, 256, 2, 2, SP, KA16, YBF16>(a, s);
    case kT256x128: return launch_cfg<256, 128, 2, 2, SP, KA16, YBF16>(a, s);
    case kT128x256: return launch_cfg<128, 256, 2, 2, SP, KA16, YBF16>(a, s);
    case kT256x32: return launch_cfg<256, 32, 4, 1, SP, KA16, YBF16>(a, s);
    case kT128x32: return launch_cfg<128, 32, 4, 1, SP, KA16, YBF16>(a, s);
    case kT256x256w8: return launch_cfg<256, 256, 2, 4, SP, KA16, YBF16>(a, s);
    case kT128x256w8: return launch_cfg<128, 256, 2, 4, SP, KA16, YBF16>(a, s);
    case kT256x128w8: return launch_cfg<256, 128, 4, 2, SP, KA16, YBF16>(a, s);
    case kT256x256w8t: return launch_cfg<256, 256, 4, 2, SP, KA16, YBF16>(a, s);
    default: return launch_cfg<128, 128, 2, 2, SP, KA16, YBF16>(a, s);
  }
}

// Tile choice for T > 32, from measured sweeps over the Qwen2.5-shaped FFN
// projections on MI355X (2048-8192 tokens, K 896-11008):
//  - too few 256x64 tiles to give every CU one: 128x64 tiles with the K-steps
//    split between two wave groups (register-W kernel);
//  - dense N:M, K >= 2048 and at least two 256x128 tiles per CU: 256x128
//    (wave tile 64x128, half the code-expansion work per MFMA);
//  - dense N:M otherwise: 256x96 (the 0.5B gate+up projection: 29.8 us
//    against 33.7 with 256x64);
//  - 2:4 and 2:8 (sparse MFMA): 256x96 (wave tile 64x96) below K = 4096; above,
//    256x128 when there are at least two such tiles per CU, else 512x64 (8 waves)
//    or 384x64 (6 waves), whichever leaves fewer CUs idle.
static int choose_cfg(int64_t T, int64_t O, int64_t K, bool sp) {
  // tuning override (read on every call so tests can force each configuration)
  const char* ev = std::getenv("SBL_GEMM_TILE");
  const int forced = ev ? std::atoi(ev) : -1;
  if (forced >= 0 && forced < kNumCfg) return forced;
  if (T <= 32) return O >= 8192 ? kT256x32 : kT128x32;
  const int cus = device_info().cus;
  const int64_t t64 = cdiv(O, 256) * cdiv(T, 64);
  const int64_t t128 = cdiv(O, 256) * cdiv(T, 128);
  if (t64 < cus) return kR128x64k2;
  // long rows with a 512x128 tile for every CU: one 8-wave workgroup per CU
  // stages each xq tile once for eight waves instead of four (Qwen2.5-3B down
  // projections, K = 11008: 2:4 123 -> 117 us, 2:8 116 -> 112, 6:8 equal)
  if (K >= 4096 && cdiv(O, 512) * cdiv(T, 128) >= cus) return kR512x128w8;
  if (sp) {
    if (K < 4096) return kR256x96;
    if (t128 >= 2 * cus) return kR256x128;
    // one workgroup per CU: 512x64 tiles (8 waves) unless they leave CUs idle
    // in the last round and 384x64 tiles (6 waves, measured 0.87x the rate
    // per CU) fill more of them (Qwen2.5-1.5B down, O = 1536: 192 tiles of
    // 512x64 against 256 of 384x64, 77 -> 66 us)
    const int64_t n512 = cdiv(O, 512) * cdiv(T, 64), n384 = cdiv(O, 384) * cdiv(T, 64);
    const double f512 = (double)n512 / (double)(cdiv(n512, cus) * cus);
    const double f384 = 0.87 * (double)n384 / (double)(cdiv(n384, cus) * cus);
    return f384 > f512 ? kR384x64 : kR512x64w8;
  }
  if (K >= 2048 && t128 >= 2 * cus) return kR256x128;
  return kR256x96;
}

hipError_t launch_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                       int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                       bool y_bf16, int32_t* acc, hipStream_t s) {
  if (T == 0 || O == 0) return hipSuccess;
  const bool sp = index_form(N, M);
  const Args a{xq, sx, (const uint8_t*)packed, row_pitch(K, N, M), sw, sw_inc, T, O, K, y, acc};
  const bool ka16 = (K % 16) == 0;
  const char* ev = std::getenv("SBL_GEMM_TILE");
  if (T <= 16 && !(ev && std::atoi(ev) >= 0) && decode_fits(T, O, K, N, M, 0))
    return launch_decode(xq, 0, sx, 0.0f, packed, sw, sw_inc, T, O, K, N, M, y, y_bf16, acc, s);
  int cfg = choose_cfg(T, O, K, sp);
  if (cfg >= kDma128x256 && K % (sp ? 128 : 64) != 0) cfg = kT128x128;  // DMA path needs whole K-steps
#define SBL_DISPATCH(SPV, KAV, YV) return launch_sel<SPV, KAV, YV>(cfg, a, s)
  if (sp) {
    if (ka16) { if (y_bf16) SBL_DISPATCH(true, true, true); else SBL_DISPATCH(true, true, false); }
    else { if (y_bf16) SBL_DISPATCH(true, false, true); else SBL_DISPATCH(true, false, false); }
  } else {
    if (ka16) { if (y_bf16) SBL_DISPATCH(false, true, true); else SBL_DISPATCH(false, true, false); }
    else { if (y_bf16) SBL_DISPATCH(false, false, true); else SBL_DISPATCH(false, false, false); }
  }
#undef SBL_DISPATCH
}

}  // namespace sbl
