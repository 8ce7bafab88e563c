// Internal declarations shared by the library's translation units.
// Nothing here is part of the public ABI (include/sbl.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sbl.h"
#include <stddef.h>

namespace sbl {

// ---- packed-format geometry (see include/sbl.h) ---------------------------
// 2:4 and 2:8 use the index form (the 2:4 sparse MFMA operand; every 2:8
// pattern is also a 2:4 pattern); 2:8 records add the mask words.
__host__ __device__ inline bool index_form(int N, int M) { return N == 2 && (M == 4 || M == 8); }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
// bytes of the code area of a dense-form row (ceil(K/64) * 16)
__host__ __device__ inline int64_t dense_code_bytes(int64_t K) { return cdiv(K, 64) * 16; }
// bytes of the mask area of a dense-form row (ceil(K/128) * 16)
__host__ __device__ inline int64_t dense_mask_bytes(int64_t K) { return cdiv(K, 128) * 16; }
__host__ __device__ inline int64_t row_pitch(int64_t K, int N, int M) {
  return index_form(N, M) ? cdiv(K, 128) * 32 + (M == 8 ? dense_mask_bytes(K) : 0)
                          : dense_code_bytes(K) + dense_mask_bytes(K);
}
// byte offset of the mask words in a record (dense form, or 2:8 index form)
__host__ __device__ inline int64_t mask_area_offset(int64_t K, int N, int M) {
  return index_form(N, M) ? cdiv(K, 128) * 32 : dense_code_bytes(K);
}
// 32-wide chunks per packed row record (both forms cover ceil(K/128)*4 chunks)
__host__ __device__ inline int64_t row_chunks(int64_t K) { return cdiv(K, 128) * 4; }

// Max workgroups of the absmean partial pass (over a whole batch of
// weights); fixes the workspace size.
constexpr int kAbsmeanMaxBlocks = 256;
// Most weight tensors one batched preparation handles.
constexpr int kMaxPrepBatch = 8;
// Workspace of the weight-prep path: the 16 partial exponent bins of every
// workgroup of the partial pass, then a 4-word compact record of each (any
// batch size).
inline size_t prep_workspace_bytes(int count = 1) {
  (void)count;
  return (size_t)kAbsmeanMaxBlocks * 20 * sizeof(unsigned long long);
}

// One weight tensor of a (batched) preparation, as the library's launcher
// receives it.
struct PrepTensor {
  const void* w;
  int64_t O, K;
  int8_t* w_eff;      // optional
  uint8_t* mask;      // optional
  void* packed;       // optional
  float* gamma_sw;    // required, device float[2]
  float* sw_rows;     // optional
  uint32_t* mask_bits = nullptr;             // optional diagnostics (see sbl.h)
  const uint32_t* prev_mask_bits = nullptr;
  unsigned long long* flips = nullptr;
  float* group_thr = nullptr;
  int variant = 0;                           // 0: method; 1: mask ranked on |W_q|
};

struct DeviceInfo {
  int cus = 256;
};
const DeviceInfo& device_info();  // cached per device

// Host validation of sbl_quant_mask_weight's arguments apart from the
// workspace.
sbl_status check_quant_mask_weight(const void* w, int wdt, int64_t O, int64_t K, int N, int M,
                                   float eps_w, const void* w_eff, const void* mask,
                                   const void* packed, const void* gamma_sw, const void* sw_rows);

// ---- launchers (return hipGetLastError() of the launch) -------------------
hipError_t launch_quant_act(const void* x, bool bf16, int64_t T, int64_t K, int64_t ldx,
                            float eps, int8_t* xq, float* sx, hipStream_t s);

// x [T,K] with 16-byte aligned rows and K a multiple of the vector width
hipError_t launch_rmsnorm_quant_act(const void* x, bool bf16, const float* gain, int64_t T,
                                    int64_t K, int64_t ldx, float eps_n, float eps, int8_t* xq,
                                    float* sx, hipStream_t s);

// count in [1, kMaxPrepBatch]; every tensor of the batch shares dtype and N:M
hipError_t launch_quant_mask_weight(const PrepTensor* items, int count, bool bf16, int N, int M,
                                    float eps, void* ws, hipStream_t s);

hipError_t launch_pack(const int8_t* w_eff, const uint8_t* mask, int64_t O, int64_t K, int N,
                       int M, void* packed, hipStream_t s);
hipError_t launch_unpack(const void* packed, int64_t O, int64_t K, int N, int M, int8_t* w_eff,
                         uint8_t* mask, hipStream_t s);

// Decode path (1 <= T <= 16). xmode 0: xq int8 [T,K] and sx given; 1 / 2:
// x bf16 / fp32 [T,K], quantized per token inside the kernel with eps.
// decode_fits() tells whether a shape takes it (else the tiled GEMM runs).
// Backward (Dual STE). x~ bf16 [T,K] from xq, sx (K % 8 == 0).
hipError_t launch_act_dequant(const int8_t* xq, const float* sx, int64_t T, int64_t K,
                              uint16_t* xt, hipStream_t s);
// dX [T,K] (+)= sum over segments of sw(seg) * dY[:, seg] W_eff[seg, :];
// seg_end: end row of each of nseg (<= 4) segments; cfg < 0 picks the tile.
hipError_t launch_bwd_dx(const uint16_t* dy, int64_t ldy, const void* packed, const float* sw_rows,
                         int64_t T, int64_t O, int64_t K, int N, int M, const int64_t* seg_end,
                         int nseg, void* dx, bool dx_bf16, int64_t lddx, bool accumulate,
                         int cfg, hipStream_t s);
// dW [O,K] = dY^T x~ (dY [T, ldy] bf16, x~ [T, ldxt] bf16); keep: optional
// keep bits [O][row_chunks(K)] gating dW (the ablated estimator).
hipError_t launch_bwd_dw(const uint16_t* dy, int64_t ldy, const uint16_t* xt, int64_t ldxt,
                         int64_t T, int64_t O, int64_t K, const uint32_t* keep, void* dw,
                         bool dw_bf16, int64_t lddw, int cfg, hipStream_t s);

bool decode_fits(int64_t T, int64_t O, int64_t K, int N, int M, int xmode);
hipError_t launch_decode(const void* x, int xmode, const float* sx, float eps, const void* packed,
                         const float* sw, int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N,
                         int M, void* y, bool y_bf16, int32_t* acc, hipStream_t s);

hipError_t launch_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                       int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                       bool y_bf16, int32_t* acc, hipStream_t s);

}  // namespace sbl
