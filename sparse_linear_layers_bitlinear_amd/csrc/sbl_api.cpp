// C ABI of the Sparse-BitLinear library: argument validation (on the host,
// before anything is enqueued), workspace sizing and dispatch to the kernels.
#include "sbl.h"
#include "sbl_internal.h"

#include <cmath>
#include <cfloat>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <mutex>

static_assert(sbl::kMaxPrepBatch == SBL_MAX_PREP_BATCH, "batch limit of the ABI");

namespace sbl {

static bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("SBL_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

const DeviceInfo& device_info() {
  static DeviceInfo infos[64];
  static std::once_flag flags[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::call_once(flags[dev], [dev] {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      infos[dev].cus = cus;
  });
  return infos[dev];
}

}  // namespace sbl

using namespace sbl;

namespace {

constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kLim31 = int64_t(1) << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int d) { return d == SBL_BF16 || d == SBL_FP32; }
bool nm_ok(int N, int M) { return (M == 4 || M == 8) && N >= 1 && N <= M; }
bool eps_ok(float e) { return std::isfinite(e) && e >= FLT_MIN; }

sbl_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SBL_OK;
  if (log_enabled()) std::fprintf(stderr, "sbl: %s failed: %s\n", what, hipGetErrorString(e));
  return SBL_ERR_HIP;
}

// Shape check shared by the weight-side calls.
sbl_status check_wshape(int64_t O, int64_t K, int N, int M) {
  if (!nm_ok(N, M)) return SBL_ERR_NM;
  if (O < 0 || K < 1 || K > kMaxK || K % M != 0) return SBL_ERR_SHAPE;
  if (O >= kLim31) return SBL_ERR_SHAPE;
  return SBL_OK;
}

// Sizes one GEMM call can address: the kernels index every operand with
// 32-bit offsets (xq [T,K] bytes, packed [O, pitch] bytes, y / acc [T,O]
// elements), so each must stay below 2^31.
sbl_status check_gemm_extent(int64_t T, int64_t O, int64_t K, int N, int M) {
  if (T < 0 || T >= kLim31 || O >= kLim31) return SBL_ERR_SHAPE;
  if (T * K >= kLim31 || O * row_pitch(K, N, M) >= kLim31 || T * O >= kLim31) return SBL_ERR_SHAPE;
  return SBL_OK;
}

// Shapes shared by the two gradient products.
sbl_status check_bwd_shape(int64_t ldy, int64_t T, int64_t O, int64_t K) {
  if (T < 0 || T > INT32_MAX || O < 8 || O > INT32_MAX || O % 8 != 0) return SBL_ERR_SHAPE;
  if (K < 8 || K > kMaxK || K % 8 != 0) return SBL_ERR_SHAPE;
  if (ldy < O || ldy % 8 != 0) return SBL_ERR_SHAPE;
  return SBL_OK;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct LinearWs {
  size_t xq, sx, gsw, prep, packed, total;
};
LinearWs linear_ws_layout(int64_t T, int64_t O, int64_t K, int N, int M, bool prepacked) {
  LinearWs L{};
  size_t off = 0;
  L.xq = off; off += align256((size_t)(T * K));
  L.sx = off; off += align256((size_t)T * 4);
  L.gsw = off; off += 256;
  L.prep = off; off += prepacked ? 0 : align256(prep_workspace_bytes());
  L.packed = off; off += prepacked ? 0 : align256((size_t)(O * row_pitch(K, N, M)));
  L.total = off;
  return L;
}

}  // namespace

namespace sbl {
sbl_status check_quant_mask_weight(const void* w, int wdt, int64_t O, int64_t K, int N, int M,
                                   float eps_w, const void* w_eff, const void* mask,
                                   const void* packed, const void* gamma_sw, const void* sw_rows) {
  if (!dtype_ok(wdt)) return SBL_ERR_DTYPE;
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (O < 1 || O * K >= (int64_t(1) << 31)) return SBL_ERR_SHAPE;
  if (!eps_ok(eps_w)) return SBL_ERR_VALUE;
  if (!w || !gamma_sw) return SBL_ERR_NULL;
  for (const void* p : {w, w_eff, mask, packed, gamma_sw, sw_rows})
    if (p && !aligned16(p)) return SBL_ERR_ALIGN;
  return SBL_OK;
}
}  // namespace sbl

extern "C" {

const char* sbl_status_string(int s) {
  switch (s) {
    case SBL_OK: return "SBL_OK";
    case SBL_ERR_NULL: return "SBL_ERR_NULL: required pointer is NULL";
    case SBL_ERR_SHAPE: return "SBL_ERR_SHAPE: invalid size (K % M, bounds, ldx)";
    case SBL_ERR_NM: return "SBL_ERR_NM: unsupported N:M (M in {4,8}, 1 <= N <= M)";
    case SBL_ERR_DTYPE: return "SBL_ERR_DTYPE: dtype must be SBL_BF16 or SBL_FP32";
    case SBL_ERR_ALIGN: return "SBL_ERR_ALIGN: device pointer not 16-byte aligned";
    case SBL_ERR_WORKSPACE: return "SBL_ERR_WORKSPACE: workspace too small";
    case SBL_ERR_HIP: return "SBL_ERR_HIP: HIP runtime or launch failure";
    case SBL_ERR_VALUE: return "SBL_ERR_VALUE: eps must be a positive normal finite float";
    default: return "SBL: unknown status";
  }
}

const char* sbl_version(void) { return "sbl 0.1 gfx950"; }

sbl_status sbl_quant_act(const void* x, sbl_dtype xdt, int64_t T, int64_t K, int64_t ldx,
                         float eps_a, int8_t* xq, float* sx, hipStream_t stream) {
  if (!dtype_ok(xdt)) return SBL_ERR_DTYPE;
  if (T < 0 || K < 1 || K > kMaxK || ldx < K) return SBL_ERR_SHAPE;
  if (!eps_ok(eps_a)) return SBL_ERR_VALUE;
  if (T == 0) return SBL_OK;
  if (!x || !xq || !sx) return SBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(sx)) return SBL_ERR_ALIGN;
  return hip_status(launch_quant_act(x, xdt == SBL_BF16, T, K, ldx, eps_a, xq, sx, stream),
                    "quant_act");
}

sbl_status sbl_rmsnorm_quant_act(const void* x, sbl_dtype xdt, const float* gain, int64_t T,
                                 int64_t K, int64_t ldx, float eps_n, float eps_a, int8_t* xq,
                                 float* sx, hipStream_t stream) {
  if (!dtype_ok(xdt)) return SBL_ERR_DTYPE;
  if (T < 0 || K < 1 || K > kMaxK || ldx < K) return SBL_ERR_SHAPE;
  const int64_t es = xdt == SBL_BF16 ? 2 : 4, V = 16 / es;
  if (K % V != 0 || (ldx * es) % 16 != 0) return SBL_ERR_SHAPE;
  if (!eps_ok(eps_a) || !eps_ok(eps_n)) return SBL_ERR_VALUE;
  if (T == 0) return SBL_OK;
  if (!x || !xq || !sx) return SBL_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(sx) || (gain && !aligned16(gain)))
    return SBL_ERR_ALIGN;
  return hip_status(launch_rmsnorm_quant_act(x, xdt == SBL_BF16, gain, T, K, ldx, eps_n, eps_a,
                                             xq, sx, stream),
                    "rmsnorm_quant_act");
}

sbl_status sbl_quant_mask_weight_workspace(int64_t O, int64_t K, size_t* bytes) {
  if (!bytes) return SBL_ERR_NULL;
  if (O < 1 || K < 1 || O * K >= (int64_t(1) << 31)) return SBL_ERR_SHAPE;
  *bytes = prep_workspace_bytes();
  return SBL_OK;
}

sbl_status sbl_quant_mask_weight(const void* w, sbl_dtype wdt, int64_t O, int64_t K, int N, int M,
                                 float eps_w, int8_t* w_eff, uint8_t* mask, void* packed,
                                 float* gamma_sw, float* sw_rows, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  sbl_status st = sbl::check_quant_mask_weight(w, wdt, O, K, N, M, eps_w, w_eff, mask, packed,
                                               gamma_sw, sw_rows);
  if (st != SBL_OK) return st;
  if (!ws) return SBL_ERR_WORKSPACE;
  if (ws_bytes < prep_workspace_bytes()) return SBL_ERR_WORKSPACE;
  if (!aligned16(ws)) return SBL_ERR_ALIGN;
  const PrepTensor t{w, O, K, w_eff, mask, packed, gamma_sw, sw_rows};
  return hip_status(launch_quant_mask_weight(&t, 1, wdt == SBL_BF16, N, M, eps_w, ws, stream),
                    "quant_mask_weight");
}

sbl_status sbl_quant_mask_weight_batch_workspace(int count, size_t* bytes) {
  if (!bytes) return SBL_ERR_NULL;
  if (count < 1 || count > SBL_MAX_PREP_BATCH) return SBL_ERR_SHAPE;
  *bytes = prep_workspace_bytes(count);
  return SBL_OK;
}

sbl_status sbl_quant_mask_weight_batch(const sbl_weight_prep* items, int count, sbl_dtype wdt,
                                       int N, int M, float eps_w, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (!items) return SBL_ERR_NULL;
  if (count < 1 || count > SBL_MAX_PREP_BATCH) return SBL_ERR_SHAPE;
  if (!dtype_ok(wdt)) return SBL_ERR_DTYPE;
  if (!eps_ok(eps_w)) return SBL_ERR_VALUE;
  PrepTensor t[SBL_MAX_PREP_BATCH];
  for (int i = 0; i < count; ++i) {
    const sbl_weight_prep& it = items[i];
    sbl_status st = check_wshape(it.O, it.K, N, M);
    if (st != SBL_OK) return st;
    if (it.O < 1 || it.O * it.K >= (int64_t(1) << 31)) return SBL_ERR_SHAPE;
    if (!it.w || !it.gamma_sw) return SBL_ERR_NULL;
    if ((it.prev_mask_bits == nullptr) != (it.flips == nullptr)) return SBL_ERR_NULL;
    if (it.flips && !it.mask_bits) return SBL_ERR_NULL;   // flips compare the new mask bits
    for (const void* p : {it.w, (const void*)it.w_eff, (const void*)it.mask,
                          (const void*)it.packed, (const void*)it.gamma_sw,
                          (const void*)it.sw_rows, (const void*)it.mask_bits,
                          (const void*)it.prev_mask_bits, (const void*)it.flips,
                          (const void*)it.group_thr})
      if (p && !aligned16(p)) return SBL_ERR_ALIGN;
    t[i] = PrepTensor{it.w, it.O, it.K, it.w_eff, it.mask, it.packed, it.gamma_sw, it.sw_rows};
    t[i].mask_bits = it.mask_bits;
    t[i].prev_mask_bits = it.prev_mask_bits;
    t[i].flips = it.flips;
    t[i].group_thr = it.group_thr;
    if (it.variant != SBL_PREP_METHOD && it.variant != SBL_PREP_MASK_FROM_TERNARY &&
        it.variant != SBL_PREP_MASK_THEN_QUANT)
      return SBL_ERR_VALUE;
    // mask-then-quant changes the partial pass for the whole batch
    if ((it.variant == SBL_PREP_MASK_THEN_QUANT) != (items[0].variant == SBL_PREP_MASK_THEN_QUANT))
      return SBL_ERR_VALUE;
    t[i].variant = it.variant;
  }
  if (!ws) return SBL_ERR_WORKSPACE;
  if (ws_bytes < prep_workspace_bytes(count)) return SBL_ERR_WORKSPACE;
  if (!aligned16(ws)) return SBL_ERR_ALIGN;
  return hip_status(launch_quant_mask_weight(t, count, wdt == SBL_BF16, N, M, eps_w, ws, stream),
                    "quant_mask_weight_batch");
}

sbl_status sbl_packed_bytes(int64_t O, int64_t K, int N, int M, size_t* bytes) {
  if (!bytes) return SBL_ERR_NULL;
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  *bytes = (size_t)(O * row_pitch(K, N, M));
  return SBL_OK;
}

sbl_status sbl_pack(const int8_t* w_eff, const uint8_t* mask, int64_t O, int64_t K, int N, int M,
                    void* packed, hipStream_t stream) {
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (O == 0) return SBL_OK;
  if (!w_eff || !mask || !packed) return SBL_ERR_NULL;
  if (!aligned16(w_eff) || !aligned16(mask) || !aligned16(packed)) return SBL_ERR_ALIGN;
  return hip_status(launch_pack(w_eff, mask, O, K, N, M, packed, stream), "pack");
}

sbl_status sbl_unpack(const void* packed, int64_t O, int64_t K, int N, int M, int8_t* w_eff,
                      uint8_t* mask, hipStream_t stream) {
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (O == 0) return SBL_OK;
  if (!w_eff || !mask || !packed) return SBL_ERR_NULL;
  if (!aligned16(w_eff) || !aligned16(mask) || !aligned16(packed)) return SBL_ERR_ALIGN;
  return hip_status(launch_unpack(packed, O, K, N, M, w_eff, mask, stream), "unpack");
}

sbl_status sbl_gemm(const int8_t* xq, const float* sx, const void* packed, const float* sw,
                    int64_t sw_inc, int64_t T, int64_t O, int64_t K, int N, int M, void* y,
                    sbl_dtype ydt, int32_t* acc, hipStream_t stream) {
  if (!dtype_ok(ydt)) return SBL_ERR_DTYPE;
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (T < 0 || (sw_inc != 0 && sw_inc != 1)) return SBL_ERR_SHAPE;
  st = check_gemm_extent(T, O, K, N, M);
  if (st != SBL_OK) return st;
  if (T == 0 || O == 0) return SBL_OK;
  if (!xq || !sx || !packed || !sw || !y) return SBL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(sx) || !aligned16(packed) || !aligned16(y) ||
      (acc && !aligned16(acc)) || ((uintptr_t)sw & 3u))
    return SBL_ERR_ALIGN;
  return hip_status(launch_gemm(xq, sx, packed, sw, sw_inc, T, O, K, N, M, y, ydt == SBL_BF16,
                                acc, stream),
                    "gemm");
}

sbl_status sbl_linear_fwd_workspace(int64_t T, int64_t O, int64_t K, int N, int M, int prepacked,
                                    size_t* bytes) {
  if (!bytes) return SBL_ERR_NULL;
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (T < 0) return SBL_ERR_SHAPE;
  *bytes = linear_ws_layout(T, O, K, N, M, prepacked != 0).total;
  return SBL_OK;
}

sbl_status sbl_linear_fwd(const void* x, sbl_dtype xdt, const void* w_master, sbl_dtype wdt,
                          const void* prepacked, const float* sw_prepacked, int64_t sw_inc,
                          int64_t T, int64_t O, int64_t K, int N, int M, float eps_a, float eps_w,
                          void* y, sbl_dtype ydt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(xdt) || !dtype_ok(ydt) || (w_master && !dtype_ok(wdt))) return SBL_ERR_DTYPE;
  sbl_status st = check_wshape(O, K, N, M);
  if (st != SBL_OK) return st;
  if (T < 0) return SBL_ERR_SHAPE;
  st = check_gemm_extent(T, O, K, N, M);
  if (st != SBL_OK) return st;
  const bool pre = prepacked != nullptr;
  if (pre == (w_master != nullptr)) return SBL_ERR_NULL;  // exactly one weight source
  if (pre && sw_inc != 0 && sw_inc != 1) return SBL_ERR_SHAPE;
  if (!pre && (O < 1 || O * K >= (int64_t(1) << 31))) return SBL_ERR_SHAPE;
  if (!eps_ok(eps_a) || (!pre && !eps_ok(eps_w))) return SBL_ERR_VALUE;
  if (T == 0 || O == 0) return SBL_OK;
  if (!x || !y || (pre && !sw_prepacked)) return SBL_ERR_NULL;
  const LinearWs L = linear_ws_layout(T, O, K, N, M, pre);
  if (!ws || ws_bytes < L.total) return SBL_ERR_WORKSPACE;
  for (const void* p : {x, w_master, prepacked, (const void*)y, (const void*)ws})
    if (p && !aligned16(p)) return SBL_ERR_ALIGN;
  if (pre && ((uintptr_t)sw_prepacked & 3u)) return SBL_ERR_ALIGN;

  char* base = (char*)ws;
  int8_t* xq = (int8_t*)(base + L.xq);
  float* sx = (float*)(base + L.sx);
  float* gsw = (float*)(base + L.gsw);
  const void* packed = prepacked;
  const float* sw = sw_prepacked;
  int64_t inc = sw_inc;
  hipError_t e;
  if (!pre) {
    void* pk = base + L.packed;
    const PrepTensor t{w_master, O, K, nullptr, nullptr, pk, gsw, nullptr};
    e = launch_quant_mask_weight(&t, 1, wdt == SBL_BF16, N, M, eps_w, base + L.prep, stream);
    if (e != hipSuccess) return hip_status(e, "linear_fwd/quant_mask_weight");
    packed = pk;
    sw = gsw + 1;
    inc = 0;
  }
  // decode-sized batches: activation quantization fused into the GEMV
  const int xmode = xdt == SBL_BF16 ? 1 : 2;
  const char* ev = std::getenv("SBL_GEMM_TILE");   // a forced tile configuration takes the GEMM
  if (T <= 16 && !(ev && std::atoi(ev) >= 0) && decode_fits(T, O, K, N, M, xmode))
    return hip_status(launch_decode(x, xmode, nullptr, eps_a, packed, sw, inc, T, O, K, N, M, y,
                                    ydt == SBL_BF16, nullptr, stream),
                      "linear_fwd/decode");
  e = launch_quant_act(x, xdt == SBL_BF16, T, K, K, eps_a, xq, sx, stream);
  if (e != hipSuccess) return hip_status(e, "linear_fwd/quant_act");
  return hip_status(launch_gemm(xq, sx, packed, sw, inc, T, O, K, N, M, y, ydt == SBL_BF16,
                                nullptr, stream),
                    "linear_fwd/gemm");
}

// ---- backward (Dual STE) ------------------------------------------------
sbl_status sbl_act_dequant(const int8_t* xq, const float* sx, int64_t T, int64_t K, void* xt,
                           hipStream_t stream) {
  if (T < 0 || T > INT32_MAX || K < 8 || K > kMaxK || K % 8 != 0) return SBL_ERR_SHAPE;
  if (T == 0) return SBL_OK;
  if (!xq || !sx || !xt) return SBL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(sx) || !aligned16(xt)) return SBL_ERR_ALIGN;
  return hip_status(launch_act_dequant(xq, sx, T, K, (uint16_t*)xt, stream), "sbl_act_dequant");
}

sbl_status sbl_linear_bwd_dx(const void* dy, int64_t ldy, const void* packed, const float* sw_rows,
                             int64_t T, int64_t O, int64_t K, int N, int M, const int64_t* seg_rows,
                             int nseg, void* dx, sbl_dtype dxdt, int64_t lddx, int accumulate,
                             hipStream_t stream) {
  if (!dtype_ok(dxdt)) return SBL_ERR_DTYPE;
  if (!nm_ok(N, M)) return SBL_ERR_NM;
  sbl_status st = check_bwd_shape(ldy, T, O, K);
  if (st != SBL_OK) return st;
  if (K % M != 0 || lddx < K) return SBL_ERR_SHAPE;
  if (nseg < 1 || nseg > 4) return SBL_ERR_SHAPE;
  if (nseg > 1 && !seg_rows) return SBL_ERR_NULL;
  int64_t ends[4];
  int64_t sum = 0;
  for (int i = 0; i < nseg; ++i) {
    const int64_t r = seg_rows ? seg_rows[i] : O;
    if (r < 8 || r % 8 != 0) return SBL_ERR_SHAPE;
    sum += r;
    ends[i] = sum;
  }
  if (sum != O) return SBL_ERR_SHAPE;
  if (T == 0) return SBL_OK;
  if (!dy || !packed || !sw_rows || !dx) return SBL_ERR_NULL;
  if (!aligned16(dy) || !aligned16(packed) || !aligned16(sw_rows) || !aligned16(dx))
    return SBL_ERR_ALIGN;
  return hip_status(launch_bwd_dx((const uint16_t*)dy, ldy, packed, sw_rows, T, O, K, N, M, ends,
                                  nseg, dx, dxdt == SBL_BF16, lddx, accumulate != 0, -1, stream),
                    "sbl_linear_bwd_dx");
}

sbl_status sbl_linear_bwd_dw(const void* dy, int64_t ldy, const void* xt, int64_t T, int64_t O,
                             int64_t K, const uint32_t* keep_bits, void* dw, sbl_dtype dwdt,
                             hipStream_t stream) {
  if (!dtype_ok(dwdt)) return SBL_ERR_DTYPE;
  sbl_status st = check_bwd_shape(ldy, T, O, K);
  if (st != SBL_OK) return st;
  if (!dw || (T > 0 && (!dy || !xt))) return SBL_ERR_NULL;
  if ((dy && !aligned16(dy)) || (xt && !aligned16(xt)) || !aligned16(dw) ||
      (keep_bits && !aligned16(keep_bits)))
    return SBL_ERR_ALIGN;
  return hip_status(launch_bwd_dw((const uint16_t*)dy, ldy, (const uint16_t*)xt, K, T, O, K,
                                  keep_bits, dw, dwdt == SBL_BF16, K, -1, stream),
                    "sbl_linear_bwd_dw");
}

}  // extern "C"
