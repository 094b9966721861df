// Read-stream probe: a measurement aid, not a step of the method. It reads a
// buffer once with 16-byte vector loads and discards the data, so the time of
// a launch over a buffer that the 256 MB Infinity Cache cannot hold is the
// rate at which this GPU streams that many bytes from HBM in one launch. The
// HBM-bound kernels of the library are reported against it beside the 8 TB/s
// figure.
//
// Each thread walks the buffer with a grid stride, four nontemporal loads in
// flight (a wavefront's load covers 1 KiB of consecutive bytes; the streaming
// hint measured ~10% faster than plain loads on 256 MiB reads and the same on
// 25 MB), XORs what it reads, and stores one word only if the XOR equals a
// fixed constant, which keeps the loads from being optimised away and lets a
// test see that the last word of the buffer is read.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kReadProbeMark) sink[0] = v;
}

}  // namespace

hipError_t launch_read_stream(const void* src, int64_t bytes, int workgroups, void* sink,
                              hipStream_t st) {
  read_stream_kernel<<<workgroups, 256, 0, st>>>(static_cast<const u32x4*>(src), bytes / 16,
                                                 static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace qg
