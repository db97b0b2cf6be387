// Final state of an empty sequence (L = 0): a copy of the initial state, or zeros, written by a
// kernel rather than a memory-set or copy node, so that a caller capturing a graph records only
// kernels.
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

__global__ __launch_bounds__(256) void state_fill_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_state_fill(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(state_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace ssm
