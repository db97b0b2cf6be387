// Vector-ALU rate probe for gfx950 (measurement support, not part of the selective-scan path).
//
// Three kernels, each a fixed number of independent dependency chains per lane so that issue
// throughput, not latency, bounds them, launched over enough waves to fill every SIMD:
//   kind 0: fp32 FMA chains                    -> lane-FMAs per second
//   kind 1: v_exp_f32 chains                   -> lane-exps per second
//   kind 2: the scan's per-state-step mix: Delta a (mul), 2^t (v_exp_f32), (Abar - 1) / a (fma),
//           B x (mul), their product (mul), h = Abar h + u (fma), y += C h (fma)
//                                              -> lane state-steps per second
// Packed FP32 is disabled at compile time like the library, so these are single-lane rates.
// The C entry point only enqueues; the caller times the launch on its stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void fma_kernel(const float* in, float* out, int iters) {
  float a[kChains];
  const float m = in[0], c = in[1];
#pragma unroll
  for (int k = 0; k < kChains; ++k) a[k] = in[2 + k] + threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int k = 0; k < kChains; ++k) a[k] = fmaf(a[k], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += a[k];
  if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void exp_kernel(const float* in, float* out, int iters) {
  float a[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) a[k] = in[2 + k] * (1.0f + threadIdx.x * 1e-6f);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int k = 0; k < kChains; ++k) a[k] = __builtin_amdgcn_exp2f(-a[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += a[k];
  if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mix_kernel(const float* in, float* out, int iters) {
  // 16 tokens (step size, input) per round in registers, 8 states per lane, readout into two
  // partial sums (as a lane holding two states of a channel does); the token values shift by a
  // per-round amount so nothing can be hoisted out of the loop (2 adds per token, 0.25 per
  // state-step, on top of the mix)
  float h[kChains], a2[kChains], ia[kChains], bk[kChains], ck[kChains], dv[16], xv[16];
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    h[k] = 0.f;
    a2[k] = -(k + 1) * 1.4426950408889634f * (1.0f + threadIdx.x * 1e-7f);
    ia[k] = -1.0f / (k + 1);
    bk[k] = in[2 + k];
    ck[k] = in[2 + (k + 3) % kChains];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    dv[r] = 0.01f + 0.001f * r * in[0];
    xv[r] = in[1] + 0.1f * r;
  }
  float y0 = 0.f, y1 = 0.f;
  for (int i = 0; i < iters; ++i) {
    const float fi = (float)i * 1e-9f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float dr = dv[r] + fi, xr = xv[r] - fi;
#pragma unroll
      for (int k = 0; k < kChains; ++k) {
        const float e = __builtin_amdgcn_exp2f(dr * a2[k]);
        const float u = fmaf(e, ia[k], -ia[k]) * (bk[k] * xr);
        h[k] = fmaf(e, h[k], u);
        if (k & 1) y1 = fmaf(ck[k], h[k], y1);
        else y0 = fmaf(ck[k], h[k], y0);
      }
    }
  }
  if (y0 + y1 == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = y0;
}

}  // namespace

extern "C" {

// Enqueue `blocks` workgroups of 256 threads of probe `kind` (0 FMA, 1 exp, 2 scan mix), each lane
// running iters x 16 x 8 operations of that kind. in: >= 12 floats on the device (any finite
// values); out: blocks x 256 floats (written only in a case that does not occur). Returns the
// launch's hipError_t.
int probe_valu_rates(int kind, int blocks, int iters, const float* in, float* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(256);
  if (kind == 0) hipLaunchKernelGGL(fma_kernel, grid, block, 0, st, in, out, iters);
  else if (kind == 1) hipLaunchKernelGGL(exp_kernel, grid, block, 0, st, in, out, iters);
  else if (kind == 2) hipLaunchKernelGGL(mix_kernel, grid, block, 0, st, in, out, iters);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // extern "C"
