// The library's fixed scratch buffer: device memory the no-allocation GEMM
// entry point uses in place of a caller-supplied workspace (arrival counters,
// split-K partials, prefill INT4 offsets). It is a file-scope device array,
// so every GPU the library runs on holds one copy, at its own address, for
// the life of the process; nothing here allocates or frees device memory.
//
// Host code never passes the array's name to a kernel or a copy (on the host
// the name is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// is kept per device.
#include <mutex>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;
  bool counters_cleared = false;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// Zero n 16-byte words (the arrival counters at the start of the scratch).
__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t stream_device(hipStream_t st, int* dev) {
  if (st != nullptr) return hipStreamGetDevice(st, dev);
  return hipGetDevice(dev);
}

}  // namespace

hipError_t scratch_for_stream(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = stream_device(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (d.ptr == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    d.ptr = p;
  }
  if (!d.counters_cleared) {
    // The counters must start at zero; every kernel that counts arrivals
    // returns them to zero before it ends, so one clear per device suffices.
    // A fill kernel, not a memset node: the first call may be under capture.
    constexpr int words = (int)(kCounterBytes / 16);
    zero_words_kernel<<<dim3((words + 255) / 256), 256, 0, st>>>(static_cast<uint4*>(d.ptr), words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    d.counters_cleared = true;
  }
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace qg
