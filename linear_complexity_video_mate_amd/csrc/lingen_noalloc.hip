// The mixer forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its workspace is a file-scope device array of fixed size,
// one copy per GPU, alive until the process ends; nothing here allocates.
//
// The array's name is a host-side stand-in in host code: its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and that address, never the name, is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lingen_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[LINGEN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return LINGEN_ERR_HIP;
  }
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return LINGEN_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LINGEN_OK;
}

}  // namespace

extern "C" int lingen_mate_fwd_noalloc(const void* x, const float* dt, const float* A, const void* B,
                                       const void* C, const float* D, const void* q, const void* k, const void* v,
                                       int32_t layer_idx, const lingen_mate_shape* shape, void* y,
                                       hipStream_t stream) {
  if (int rc = lingen::validate_shape(shape)) return rc;
  // Everything the mixer keeps in its workspace (chunk states, chunk decays,
  // review-token buffers) is written before it is read within one call, so
  // nothing in the array needs clearing between calls.
  if (lingen::ws_layout(shape).total > size_t(LINGEN_NOALLOC_SCRATCH_BYTES)) return LINGEN_ERR_SCRATCH;
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return lingen_mate_fwd(x, dt, A, B, C, D, q, k, v, layer_idx, shape, y, ws,
                         size_t(LINGEN_NOALLOC_SCRATCH_BYTES), stream);
}
