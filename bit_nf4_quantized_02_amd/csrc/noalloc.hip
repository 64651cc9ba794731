// The layer forward without any allocation: qlora_linear_fwd with its
// workspace taken from a fixed device array the library owns, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ symbol. Each device that loads the
// library holds its own copy at its own address until the process ends; on
// the first call that needs it on a device, that address is looked up once
// with hipGetSymbolAddress (with the device current) and kept per device. The
// host-side name of the symbol is never used as a device address.
//
// Nothing here allocates or frees: the call carves the same regions
// qlora_linear_fwd carves from a caller's workspace, and launches the same
// kernels. No region needs to start at zero (every value a kernel reads
// from it is written earlier in the same call), so the array is never
// cleared. Calls that overlap on one device (two streams, or two threads)
// share the array and race; serialize them.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "qlora.h"

namespace {

static __device__ __align__(256) char scratch[QLORA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up yet)

// Address of the array on the device `stream` belongs to.
qlora_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return QLORA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return QLORA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return QLORA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return QLORA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" qlora_status qlora_linear_fwd_scratch(const qlora_nf4_weight* w, const void* X, int64_t M, const void* A,
                                                 const void* B, int r, float scale, void* Y, float* T_save,
                                                 void* stream) {
  if (w == nullptr) return QLORA_ERR_INVALID_ARG;
  if (M < 0 || r < 0 || r > QLORA_MAX_RANK || w->n < 1 || w->k < 1 || w->k % QLORA_BLOCK) return QLORA_ERR_SHAPE;
  const size_t need = M > 0 ? qlora::linear_fwd_ws_bytes(M, w->n, w->k, r, T_save != nullptr) : 0;
  if (need > (size_t)QLORA_SCRATCH_BYTES) return QLORA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const qlora_status s = scratch_for(static_cast<hipStream_t>(stream), &ws);
    if (s != QLORA_OK) return s;
  }
  return qlora::linear_fwd_impl(w, X, M, A, B, r, scale, nullptr, 1.0f, Y, T_save, ws,
                                need > 0 ? (size_t)QLORA_SCRATCH_BYTES : 0, stream);
}
