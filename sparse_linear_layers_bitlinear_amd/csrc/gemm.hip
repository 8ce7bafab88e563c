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
// Dense form: v_mfma_i32_16x16x64_i8
// ---------------------------------------------------------------------------
template <int WM, int WN, bool KA16, bool YBF16>
__global__ __launch_bounds__(256) void k_gemm_dense(const int8_t* __restrict__ xq,
                                                    const float* __restrict__ sx,
                                                    const uint8_t* __restrict__ packed,
                                                    int64_t pitch, const float* __restrict__ sw,
                                                    int64_t sw_inc, int64_t T, int64_t O,
                                                    int64_t K, void* __restrict__ y,
                                                    int32_t* __restrict__ acc_out) {
  constexpr int BM = 2 * WM, BN = 2 * WN, BK = 64;
  constexpr int FI = WM / 16, FJ = WN / 16;
  constexpr int TPR_A = 256 / BM;        // threads per staged W row
  constexpr int WPT_A = 4 / TPR_A;       // code words (16 k each) per thread
  constexpr int SEG_B = BN * BK / 16;    // 16-byte xq segments per K-step
  constexpr int NSEG = (SEG_B + 255) / 256;
  static_assert(TPR_A >= 1 && WPT_A >= 1 && BM <= 256, "tile");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* As = smem;                          // [2][BM][kPitchA]
  uint8_t* Bs = smem + 2 * BM * kPitchA;       // [2][BN][kPitchBd]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave & 1, wt = wave >> 1;
  const int64_t o0 = (int64_t)blockIdx.y * BM, t0 = (int64_t)blockIdx.x * BN;
  const int64_t nk = cdiv(K, BK);

  // this thread's staging slots
  const int ra = tid / TPR_A, pa = tid % TPR_A;
  const bool va = o0 + ra < O;
  const uint8_t* arow = packed + (o0 + ra) * pitch + 4 * WPT_A * pa;

  uint32_t ga[WPT_A];
  uint4 gb[NSEG];
  auto gload = [&](int64_t ks) {
#pragma unroll
    for (int w = 0; w < WPT_A; ++w) ga[w] = 0;
    if (va) {
      const uint8_t* p = arow + ks * 16;
      if constexpr (WPT_A == 4) { uint4 v = *(const uint4*)p; ga[0] = v.x; ga[1] = v.y; ga[2] = v.z; ga[3] = v.w; }
      else if constexpr (WPT_A == 2) { uint2 v = *(const uint2*)p; ga[0] = v.x; ga[1] = v.y; }
      else { ga[0] = *(const uint32_t*)p; }
    }
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + 256 * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      gb[q] = (seg < SEG_B && t0 + rb < T)
                  ? load_x16<KA16>(xq + (t0 + rb) * K, ks * BK + 16 * cb, K)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* a = As + (buf * BM + ra) * kPitchA + 16 * WPT_A * pa;
#pragma unroll
    for (int w = 0; w < WPT_A; ++w) {
      uint4 v = make_uint4(expand_codes(ga[w], 0), expand_codes(ga[w], 1),
                           expand_codes(ga[w], 2), expand_codes(ga[w], 3));
      *(uint4*)(a + 16 * w) = v;
    }
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + 256 * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      if (seg < SEG_B) *(uint4*)(Bs + (buf * BN + rb) * kPitchBd + 16 * cb) = gb[q];
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
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* a = As + buf * BM * kPitchA;
    const uint8_t* b = Bs + buf * BN * kPitchBd;
    const int koff = 16 * (lane >> 4);
    v4i af[FI], bf[FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
      af[i] = *(const v4i*)(a + (wo * WM + 16 * i + (lane & 15)) * kPitchA + koff);
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      bf[j] = *(const v4i*)(b + (wt * WN + 16 * j + (lane & 15)) * kPitchBd + koff);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = t0 + wt * WN + 16 * j + (lane & 15);
      const int64_t o = o0 + wo * WM + 16 * i + 4 * (lane >> 4);
      store_out<YBF16>(y, acc_out, acc[i][j], t, o, T, O, sx, sw, sw_inc);
    }
}

// ---------------------------------------------------------------------------
// 2:4 index form: v_smfmac_i32_16x16x128_i8
// ---------------------------------------------------------------------------
template <int WM, int WN, bool KA16, bool YBF16>
__global__ __launch_bounds__(256) void k_gemm_sparse24(const int8_t* __restrict__ xq,
                                                       const float* __restrict__ sx,
                                                       const uint8_t* __restrict__ packed,
                                                       int64_t pitch, const float* __restrict__ sw,
                                                       int64_t sw_inc, int64_t T, int64_t O,
                                                       int64_t K, void* __restrict__ y,
                                                       int32_t* __restrict__ acc_out) {
  constexpr int BM = 2 * WM, BN = 2 * WN, BK = 128;
  constexpr int FI = WM / 16, FJ = WN / 16;
  constexpr int TPR_A = 256 / BM;        // threads per staged W row
  constexpr int CPT_A = 4 / TPR_A;       // 32-k chunks (8 bytes each) per thread
  constexpr int SEG_B = BN * BK / 16;
  constexpr int NSEG = (SEG_B + 255) / 256;
  static_assert(TPR_A >= 1 && CPT_A >= 1 && BM <= 256, "tile");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* As = smem;                          // [2][BM][kPitchA]: 64 B values, 16 B idx
  uint8_t* Bs = smem + 2 * BM * kPitchA;       // [2][BN][kPitchBs]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave & 1, wt = wave >> 1;
  const int64_t o0 = (int64_t)blockIdx.y * BM, t0 = (int64_t)blockIdx.x * BN;
  const int64_t nk = cdiv(K, BK);

  const int ra = tid / TPR_A, pa = tid % TPR_A;
  const bool va = o0 + ra < O;
  const uint8_t* arow = packed + (o0 + ra) * pitch + 8 * CPT_A * pa;

  uint2 ga[CPT_A];
  uint4 gb[NSEG];
  auto gload = [&](int64_t ks) {
#pragma unroll
    for (int c = 0; c < CPT_A; ++c) ga[c] = make_uint2(0, 0x44444444u);
    if (va) {
      const uint8_t* p = arow + ks * 32;
      if constexpr (CPT_A == 4) {
        uint4 v0 = *(const uint4*)p, v1 = *(const uint4*)(p + 16);
        ga[0] = make_uint2(v0.x, v0.y); ga[1] = make_uint2(v0.z, v0.w);
        ga[2] = make_uint2(v1.x, v1.y); ga[3] = make_uint2(v1.z, v1.w);
      } else if constexpr (CPT_A == 2) {
        uint4 v0 = *(const uint4*)p;
        ga[0] = make_uint2(v0.x, v0.y); ga[1] = make_uint2(v0.z, v0.w);
      } else {
        ga[0] = *(const uint2*)p;
      }
    }
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + 256 * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      gb[q] = (seg < SEG_B && t0 + rb < T)
                  ? load_x16<KA16>(xq + (t0 + rb) * K, ks * BK + 16 * cb, K)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* a = As + (buf * BM + ra) * kPitchA;
#pragma unroll
    for (int c = 0; c < CPT_A; ++c) {
      const int ch = CPT_A * pa + c;
      uint4 v = make_uint4(expand_codes(ga[c].x, 0), expand_codes(ga[c].x, 1),
                           expand_codes(ga[c].x, 2), expand_codes(ga[c].x, 3));
      *(uint4*)(a + 16 * ch) = v;
      *(uint32_t*)(a + 64 + 4 * ch) = ga[c].y;
    }
#pragma unroll
    for (int q = 0; q < NSEG; ++q) {
      const int seg = tid + 256 * q, rb = seg / (BK / 16), cb = seg % (BK / 16);
      if (seg < SEG_B) *(uint4*)(Bs + (buf * BN + rb) * kPitchBs + 16 * cb) = gb[q];
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
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* a = As + buf * BM * kPitchA;
    const uint8_t* b = Bs + buf * BN * kPitchBs;
    const int g = lane >> 4;
    v4i af[FI];
    int ai[FI];
    v8i bf[FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const uint8_t* r = a + (wo * WM + 16 * i + (lane & 15)) * kPitchA;
      af[i] = *(const v4i*)(r + 16 * g);
      ai[i] = *(const int*)(r + 64 + 4 * g);
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const uint8_t* r = b + (wt * WN + 16 * j + (lane & 15)) * kPitchBs;
      const v4i lo = *(const v4i*)(r + 16 * g), hi = *(const v4i*)(r + 64 + 16 * g);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(af[i], bf[j], acc[i][j], ai[i], 0, 0);
    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = t0 + wt * WN + 16 * j + (lane & 15);
      const int64_t o = o0 + wo * WM + 16 * i + 4 * (lane >> 4);
      store_out<YBF16>(y, acc_out, acc[i][j], t, o, T, O, sx, sw, sw_inc);
    }
}

// ---------------------------------------------------------------------------
template <int WM, int WN, bool KA16, bool YBF16>
static hipError_t launch_tiles(bool idx, const int8_t* xq, const float* sx, const uint8_t* packed,
                               int64_t pitch, const float* sw, int64_t sw_inc, int64_t T,
                               int64_t O, int64_t K, void* y, int32_t* acc, hipStream_t s) {
  constexpr int BM = 2 * WM, BN = 2 * WN;
  const dim3 grid((unsigned)cdiv(T, BN), (unsigned)cdiv(O, BM)), block(256);
  if (idx) {
    const size_t lds = 2 * (size_t)BM * kPitchA + 2 * (size_t)BN * kPitchBs;
    hipLaunchKernelGGL((k_gemm_sparse24<WM, WN, KA16, YBF16>), grid, block, lds, s, xq, sx,
                       packed, pitch, sw, sw_inc, T, O, K, y, acc);
  } else {
    const size_t lds = 2 * (size_t)BM * kPitchA + 2 * (size_t)BN * kPitchBd;
    hipLaunchKernelGGL((k_gemm_dense<WM, WN, KA16, YBF16>), grid, block, lds, s, xq, sx, packed,
                       pitch, sw, sw_inc, T, O, K, y, acc);
  }
  return hipGetLastError();
}

template <bool KA16, bool YBF16>
static hipError_t launch_gemm_k(bool idx, const int8_t* xq, const float* sx, const uint8_t* packed,
                                int64_t pitch, const float* sw, int64_t sw_inc, int64_t T,
                                int64_t O, int64_t K, void* y, int32_t* acc, hipStream_t s) {
  if (T <= 32)
    return launch_tiles<64, 16, KA16, YBF16>(idx, xq, sx, packed, pitch, sw, sw_inc, T, O, K, y, acc, s);
  return launch_tiles<64, 64, KA16, YBF16>(idx, xq, sx, packed, pitch, sw, sw_inc, T, O, K, y, acc, s);
}

hipError_t launch_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                       int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                       bool y_bf16, int32_t* acc, hipStream_t s) {
  if (T == 0 || O == 0) return hipSuccess;
  const bool idx = index_form(N, M);
  const int64_t pitch = row_pitch(K, N, M);
  const uint8_t* p = (const uint8_t*)packed;
  const bool ka16 = (K % 16) == 0;
  if (ka16) {
    return y_bf16 ? launch_gemm_k<true, true>(idx, xq, sx, p, pitch, sw, sw_inc, T, O, K, y, acc, s)
                  : launch_gemm_k<true, false>(idx, xq, sx, p, pitch, sw, sw_inc, T, O, K, y, acc, s);
  }
  return y_bf16 ? launch_gemm_k<false, true>(idx, xq, sx, p, pitch, sw, sw_inc, T, O, K, y, acc, s)
                : launch_gemm_k<false, false>(idx, xq, sx, p, pitch, sw, sw_inc, T, O, K, y, acc, s);
}

}  // namespace sbl
