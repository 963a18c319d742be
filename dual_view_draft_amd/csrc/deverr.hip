// The device error word: one 32-bit word per GPU that kernels OR
// ORTHRUS_DEVERR_* bits into when a device-side precondition they cannot
// check on the host is violated (a sequence length, a page id, an emitted
// count), at the point where they clamp the value to stay in bounds.  It
// starts at zero when the library is loaded on a device and is read (and
// optionally cleared) by orthrus_device_errors, in stream order.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "check.h"
#include "launch.h"

namespace orthrus {
namespace {

__device__ unsigned int g_device_errors = 0u;

constexpr int kMaxErrorDevices = 64;
std::mutex g_err_mu;
unsigned int* g_err_ptr[kMaxErrorDevices] = {};

__global__ void device_errors_kernel(unsigned int* word, uint32_t* out, int clear) {
  const unsigned int v = clear ? atomicExch(word, 0u) : atomicOr(word, 0u);
  *out = v;
}

}  // namespace

hipError_t device_error_word(unsigned int** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxErrorDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_err_mu);
  if (!g_err_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_errors));
    if (e != hipSuccess) return e;
    g_err_ptr[dev] = static_cast<unsigned int*>(p);
  }
  *ptr = g_err_ptr[dev];
  return hipSuccess;
}

hipError_t launch_device_errors(uint32_t* out, int clear, hipStream_t stream) {
  unsigned int* word = nullptr;
  hipError_t e = device_error_word(&word);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(device_errors_kernel, dim3(1), dim3(1), 0, stream, word, out, clear);
  return hipGetLastError();
}

}  // namespace orthrus
