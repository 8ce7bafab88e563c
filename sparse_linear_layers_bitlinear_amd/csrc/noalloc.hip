// Weight preparation for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): sbl_quant_mask_weight with its workspace -- the absmean
// partial bins and compact records -- taken from a fixed array in device
// memory owned by the library instead of a caller-provided buffer.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy until the process ends. Host code never passes the
// array's name to a kernel (on the host it only stands in for the symbol);
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address is used.
#include "sbl.h"
#include "sbl_internal.h"

#include <mutex>

namespace sbl {
namespace {

// Largest workspace the allocation-free entry point can serve. The weight
// preparation needs prep_workspace_bytes() (40 KiB) for any shape.
constexpr size_t kScratchBytes = 64 * 1024;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's scratch array (nullptr on failure).
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace sbl

extern "C" sbl_status sbl_quant_mask_weight_noalloc(const void* w, sbl_dtype wdt, int64_t O,
                                                    int64_t K, int N, int M, float eps_w,
                                                    int8_t* w_eff, uint8_t* mask, void* packed,
                                                    float* gamma_sw, float* sw_rows,
                                                    hipStream_t stream) {
  // the same argument checks as the workspace entry point, first
  const sbl_status st = sbl::check_quant_mask_weight(w, wdt, O, K, N, M, eps_w, w_eff, mask,
                                                     packed, gamma_sw, sw_rows);
  if (st != SBL_OK) return st;
  if (sbl::prep_workspace_bytes() > sbl::kScratchBytes) return SBL_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* const ws = sbl::scratch_ptr(&e);
  if (!ws) return SBL_ERR_HIP;
  // the workspace entry point's kernels, given the scratch array's device
  // address as their workspace
  const sbl::PrepTensor t{w, O, K, w_eff, mask, packed, gamma_sw, sw_rows};
  e = sbl::launch_quant_mask_weight(&t, 1, wdt == SBL_BF16, N, M, eps_w, ws, stream);
  return e == hipSuccess ? SBL_OK : SBL_ERR_HIP;
}
