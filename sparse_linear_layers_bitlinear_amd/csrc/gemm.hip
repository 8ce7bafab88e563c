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
// Tiles: 4 wavefronts per workgroup in a 2 (o) x 2 (t) grid, each wave a
// WM x WN block of 16x16 MFMA tiles; K advances BK = 64 (dense) or 128
// (2:4) per step; LDS is double-buffered so global loads of step s+1 overlap
// the MFMAs of step s. Row pitches of 80 / 144 bytes make the 16-byte
// fragment reads bank-conflict free.
#include "sbl_internal.h"
#include "device_util.cuh"

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

// ---------------------------------------------------------------------------
// One kernel for both forms. SP = false: dense form, BK = 64,
// v_mfma_i32_16x16x64_i8. SP = true: 2:4 index form, BK = 128,
// v_smfmac_i32_16x16x128_i8. Waves are arranged WAVES_M (along O) x WAVES_N
// (along T); each owns a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 tiles.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool KA16, bool YBF16>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((amdgpu_waves_per_eu(1, 2)))
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
  constexpr int SEG = BN * BK / 16;            // 16-byte xq segments per K-step
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
  const int64_t o0 = tm * BM, t0 = tn * BN;
  const int64_t nk = cdiv(K, BK);

  const int ra = tid / TPR, pa = tid % TPR;
  const bool va = o0 + ra < O;
  const uint8_t* arow = packed + (o0 + ra) * pitch + APT * pa;

  uint32_t ga[APT / 4];
  uint4 gb[NSEG];
  auto gload = [&](int64_t ks) {
    const uint8_t* p = arow + ks * AROW;
    if constexpr (APT == 32) {
      uint4 v0 = va ? *(const uint4*)p : make_uint4(0, SP ? 0x44444444u : 0, 0, SP ? 0x44444444u : 0);
      uint4 v1 = va ? *(const uint4*)(p + 16) : v0;
      ga[0] = v0.x; ga[1] = v0.y; ga[2] = v0.z; ga[3] = v0.w;
      ga[4] = v1.x; ga[5] = v1.y; ga[6] = v1.z; ga[7] = v1.w;
    } else if constexpr (APT == 16) {
      uint4 v = va ? *(const uint4*)p : make_uint4(0, SP ? 0x44444444u : 0, 0, SP ? 0x44444444u : 0);
      ga[0] = v.x; ga[1] = v.y; ga[2] = v.z; ga[3] = v.w;
    } else if constexpr (APT == 8) {
      uint2 v = va ? *(const uint2*)p : make_uint2(0, SP ? 0x44444444u : 0);
      ga[0] = v.x; ga[1] = v.y;
    } else {
      ga[0] = va ? *(const uint32_t*)p : 0u;
    }
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + NT * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      gb[q] = (seg < SEG && t0 + rb < T)
                  ? load_x16<KA16>(xq + (t0 + rb) * K, ks * BK + 16 * cb, K)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* a = As + (buf * BM + ra) * kPitchA;
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
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + NT * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      if (seg < SEG) *(uint4*)(Bs + (buf * BN + rb) * PB + 16 * cb) = gb[q];
    }
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
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* a = As + (buf * BM + wm * WM + r16) * kPitchA;
    const uint8_t* b = Bs + (buf * BN + wn * WN + r16) * PB;
    if constexpr (SP) {
      v8i bf[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const v4i lo = *(const v4i*)(b + 16 * j * PB + 16 * g);
        const v4i hi = *(const v4i*)(b + 16 * j * PB + 64 + 16 * g);
        bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const v4i af = *(const v4i*)(a + 16 * i * kPitchA + 16 * g);
        const int ai = *(const int*)(a + 16 * i * kPitchA + 64 + 4 * g);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(af, bf[j], acc[i][j], ai, 0, 0);
      }
    } else {
      v4i bf[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) bf[j] = *(const v4i*)(b + 16 * j * PB + 16 * g);
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const v4i af = *(const v4i*)(a + 16 * i * kPitchA + 16 * g);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = t0 + wn * WN + 16 * j + r16;
      const int64_t o = o0 + wm * WM + 16 * i + 4 * g;
      store_out<YBF16>(y, acc_out, acc[i][j], t, o, T, O, sx, sw, sw_inc);
    }
}

// ---------------------------------------------------------------------------
// Tile configurations and the per-shape choice.
// ---------------------------------------------------------------------------
enum TileCfg { kT256x256 = 0, kT256x128 = 1, kT128x256 = 2, kT128x128 = 3, kT256x32 = 4,
               kT128x32 = 5, kT256x256w8 = 6, kT128x256w8 = 7, kT256x128w8 = 8,
               kT256x256w8t = 9, kNumCfg = 10 };

struct Args {
  const int8_t* xq; const float* sx; const uint8_t* packed; int64_t pitch; const float* sw;
  int64_t sw_inc, T, O, K; void* y; int32_t* acc;
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool SP, bool KA16, bool YBF16>
static hipError_t launch_cfg(const Args& a, hipStream_t s) {
  constexpr int PB = SP ? kPitchBs : kPitchBd;
  const size_t lds = 2 * (size_t)BM * kPitchA + 2 * (size_t)BN * PB;
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

template <bool SP, bool KA16, bool YBF16>
static hipError_t launch_sel(int cfg, const Args& a, hipStream_t s) {
  switch (cfg) {
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

// Estimated time of a configuration: rounds of workgroups over the CUs times
// the per-workgroup MFMA work, scaled by the relative efficiency of the tile.
static int choose_cfg(int64_t T, int64_t O, int64_t K) {
  // tuning override (read on every call so tests can force each configuration)
  const char* ev = std::getenv("SBL_GEMM_TILE");
  const int forced = ev ? std::atoi(ev) : -1;
  if (forced >= 0 && forced < kNumCfg) return forced;
  if (T <= 32) return O >= 8192 ? kT256x32 : kT128x32;
  const int cus = device_info().cus;
  struct C { int cfg, bm, bn, per_cu; double eff; };
  const C cs[] = {{kT256x256, 256, 256, 1, 1.0}, {kT256x128, 256, 128, 2, 0.85},
                  {kT128x256, 128, 256, 2, 0.85}, {kT128x128, 128, 128, 2, 0.6}};
  int best = kT128x128;
  double best_t = 1e30;
  for (const C& c : cs) {
    const double nb = (double)cdiv(O, c.bm) * (double)cdiv(T, c.bn);
    const double rounds = std::ceil(nb / (double)(cus * c.per_cu));
    const double t = rounds * c.per_cu * (double)c.bm * c.bn * (double)K / c.eff;
    if (t < best_t) { best_t = t; best = c.cfg; }
  }
  return best;
}

hipError_t launch_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                       int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                       bool y_bf16, int32_t* acc, hipStream_t s) {
  if (T == 0 || O == 0) return hipSuccess;
  const bool sp = index_form(N, M);
  const Args a{xq, sx, (const uint8_t*)packed, row_pitch(K, N, M), sw, sw_inc, T, O, K, y, acc};
  const int cfg = choose_cfg(T, O, K);
  const bool ka16 = (K % 16) == 0;
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
