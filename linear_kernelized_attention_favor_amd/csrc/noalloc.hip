// favor_fwd_attn_noalloc: the forward pass with no workspace argument and no
// allocation, for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The kernels' workspace (split partials or segment states, references and
// the query side's operand copies) lives in one file-scope device array,
// `scratch`, of FAVOR_NOALLOC_SCRATCH_BYTES per GPU, held from the library's
// load until the process ends.  Its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; host
// code passes only that address to the kernels, never the array's name.
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (several streams, or several host threads) race on it.  The forward
// kernels need no cleared workspace (every byte they read was written
// earlier in the same call), so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "favor.h"
#include "favor_internal.h"

namespace favor {
namespace {

static_assert(FAVOR_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size in 256-byte units");

__device__ __align__(256) unsigned char scratch[FAVOR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (looked up on the
// first call on that device), or nullptr with *e set.
void* scratch_of_current_device(int dev, hipError_t* e) {
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_err[dev] = r;
    g_ptr[dev] = (r == hipSuccess) ? p : nullptr;
  });
  *e = g_err[dev];
  return g_ptr[dev];
}

}  // namespace
}  // namespace favor

extern "C" int favor_fwd_attn_noalloc(int32_t B, int32_t H, int32_t L, int32_t d, int32_t m,
                                      int32_t dtype, int32_t causal, int32_t attn_kernel,
                                      const void* Q, const void* K, const void* V, const float* W,
                                      void* O, void* stream) {
  size_t need = 0;
  const int st = favor_workspace_bytes(B, H, L, d, m, dtype, causal ? 1 : 0, &need);
  if (st != FAVOR_OK) return st;
  if (need > static_cast<size_t>(FAVOR_NOALLOC_SCRATCH_BYTES)) return FAVOR_ERR_SCRATCH;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return favor::record_hip_error(e);
  if (dev < 0 || dev >= favor::kMaxDevices) return FAVOR_ERR_SCRATCH;
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return favor::record_hip_error(e);
    if (sdev != dev) return FAVOR_ERR_SCRATCH;
  }
  void* ws = favor::scratch_of_current_device(dev, &e);
  if (!ws) return favor::record_hip_error(e);
  return favor::forward_call(B, H, L, d, m, dtype, causal ? 1 : 0, attn_kernel, Q, K, V, W, O, ws,
                             static_cast<size_t>(FAVOR_NOALLOC_SCRATCH_BYTES), stream);
}
