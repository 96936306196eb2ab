// noalloc.hip - the device scratch behind pa_decode_noalloc: a file-scope array that
// stands in for the caller's decode workspace, so that the call allocates nothing.
//
// Each GPU the library runs on holds its own copy of the array (kStaticScratchBytes)
// from the first use until the process ends.  Host code never passes the array's name
// to a kernel (in host code that name is only a stand-in, not a device address): once
// per device, with that device current, its device address is looked up with
// hipGetSymbolAddress and kept; every later use goes through that pointer.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "kernels.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// zero n16 16-byte words from p (grid-stride)
__global__ void clear_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_clear(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 || reinterpret_cast<uintptr_t>(p) % 16) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int grid = (int)std::min<int64_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(clear_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace pa
