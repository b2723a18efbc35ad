// A plain streaming read of device memory: the measured read ceiling that the
// row-statistics pass is compared with, beside the published HBM peak.
//
// Not part of the verify sampler.  Built into its own library so that the
// sampler's ABI stays the sampler's; only the throughput measurement loads it.
//
// Each 256-thread workgroup walks the buffer grid-stride, one 16-byte load per
// thread per step, and folds what it read into one float that is stored only if
// it equals one particular value (so the loads are not dead code and, in
// practice, the kernel writes nothing).  One load per step beat four loads a
// grid-stride apart on MI355X (6.5-6.8 against 5.1-6.1 TB/s over 1 GiB): four
// far-apart streams per wave spread over more DRAM pages at once.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                               float* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const uint4 x = src[i];
    acc += __uint_as_float(x.x) + __uint_as_float(x.y) + __uint_as_float(x.z) + __uint_as_float(x.w);
  }
  if (acc == 1.2345f) sink[0] = acc;
}

}  // namespace

// Reads `bytes` bytes at device address `src` once, on `stream` (asynchronous).
//   src    device memory, 16-byte aligned; bytes a multiple of 16 (0 launches nothing)
//   grid   workgroups of 256 threads, 1 .. 1048576
//   sink   one device float (written only if the folded sum hits one particular value)
// Returns 0, 1 for a bad argument, 2 if the launch failed.
extern "C" int dspark_stream_read(const void* src, size_t bytes, int grid, float* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || (bytes % 16) != 0 || ((uintptr_t)src % 16) != 0 || grid < 1 ||
      grid > (1 << 20))
    return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, stream, (const uint4*)src, bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
