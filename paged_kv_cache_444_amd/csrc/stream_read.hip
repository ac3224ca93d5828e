// A plain streaming read, the measured ceiling that the decode kernel's HBM rate is compared
// against: every byte of a buffer read once, in order, with 16-byte non-temporal loads, four in
// flight per thread.  The XOR of what a workgroup read goes to one sink word, so no load is
// dropped.

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* src, size_t n16,
                                                               uint32_t* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t x = 0;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_nontemporal_load((const u32x4*)(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(src + i));
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

int stream_read_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // Two workgroups of 256 threads per CU: with four 16-byte non-temporal loads in flight per
  // thread, the fastest of the launch shapes and load kinds measured (2 to 32 workgroups per CU,
  // temporal or non-temporal, 2 to 8 loads in flight): 7.0 TB/s over 4 GiB.
  return 2 * cus;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream) {
  TraceScope t("stream_read", stream);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pa
