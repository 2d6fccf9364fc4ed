// noalloc.hip -- rmsnorm_bwd for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the backward's partial rows go to a fixed scratch array of the
// library instead of a caller's workspace.
//
// The array lives in device memory for as long as the library is loaded, one
// copy per GPU.  In host code its name only stands in for the symbol: the
// device address of this GPU's copy comes from hipGetSymbolAddress, taken
// once per device (with that device current) on the first call there and
// kept; that address, never the name, is what the kernels get.
#include <mutex>

#include "../../include/normrope.h"
#include "nr_internal.hpp"

static __device__ __align__(256) unsigned char scratch[NR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // this GPU's copy of `scratch`, once looked up

// Device address of the current GPU's scratch array, or null (and the HIP
// error in *err) when the lookup fails.
void* scratch_on_current_device(hipError_t* err) {
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((*err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

nr_status_t rmsnorm_bwd_noalloc(nr_dtype_t dt, const void* dy, const void* x, const void* w,
                                const float* inv_rms, void* dx, float* dw, int64_t rows,
                                int64_t n, int gemma_offset, void* stream) {
  // the same checks as rmsnorm_bwd run there; only the scratch size is
  // checked here, before the (one-time) symbol lookup
  const bool long_rows = n >= nr::kLongRowMin;  // may take two passes, which need it without dw
  const bool needs = dw != nullptr || long_rows;
  const size_t need = needs ? nr_bwd_workspace_bytes(rows, n, 0) : 0;
  if (need > NR_NOALLOC_SCRATCH_BYTES) return NR_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = scratch_on_current_device(&e);
    if (ws == nullptr) return static_cast<nr_status_t>(nr::record_hip_error(e));
  }
  return rmsnorm_bwd(dt, dy, x, w, inv_rms, dx, dw, rows, n, gemma_offset, ws,
                     ws != nullptr ? static_cast<size_t>(NR_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

}  // extern "C"
