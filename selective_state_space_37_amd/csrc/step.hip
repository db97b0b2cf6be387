// One-token decode step (ssm_state_update) on gfx950.
//
// Page "Mamba and state space models", section "fixed-size state": generation keeps, per
// channel, the N-number SSM state and a short convolution holding the last few inputs, so each
// new token costs the same work. Per (b, d): shift the conv register and take the depthwise
// causal convolution u of the raw inputs, then one scan step on u (Abar = exp(Delta A),
// h = Abar h + expm1(Delta A)/A B u, y = C . h + D u), then the gate.
//
// The step is a single streaming pass bound by the state traffic (h read and written, 128 B
// per channel at N = 16). One lane owns one channel and all N of its states, so every byte is
// loaded once and in wide pieces: h and A as 16-byte vectors, the width-4 bf16 conv register as
// one 8-byte load, the conv weights as one 16-byte load. A wave covers 64 consecutive channels,
// i.e. 4 KiB of contiguous state at N = 16.
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kMaxW = 8;

template <int N>
struct Vec {
  // N floats loaded/stored as 16-byte pieces when N % 4 == 0.
  __device__ __forceinline__ static void load(const float* p, float out[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int k = 0; k < N / 4; ++k) {
        const float4 v = reinterpret_cast<const float4*>(p)[k];
        out[4 * k] = v.x; out[4 * k + 1] = v.y; out[4 * k + 2] = v.z; out[4 * k + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < N; ++k) out[k] = p[k];
    }
  }
  __device__ __forceinline__ static void store(float* p, const float in[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int k = 0; k < N / 4; ++k)
        reinterpret_cast<float4*>(p)[k] = make_float4(in[4 * k], in[4 * k + 1], in[4 * k + 2], in[4 * k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < N; ++k) p[k] = in[k];
    }
  }
};

template <typename io_t, int N>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  using Io = IoTraits<io_t>;
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // b * D + d
  if (ch >= p.B * p.D) return;
  const int64_t d = ch % p.D;
  const int64_t b = ch / p.D;

  // ---- conv register: shift, insert x, depthwise causal convolution
  float u = Io::load(static_cast<const io_t*>(p.x), ch);
  if (p.conv_state) {
    io_t* cs = static_cast<io_t*>(p.conv_state) + ch * p.W;
    float reg[kMaxW];
    if (p.W == 4) {
      float old[4], wv[4];
      Io::load4(cs, 0, old);
      const float4 w4 = *reinterpret_cast<const float4*>(p.conv_w + d * 4);
      reg[0] = old[1]; reg[1] = old[2]; reg[2] = old[3]; reg[3] = u;
      wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
      float acc = p.conv_b ? p.conv_b[d] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = fmaf(wv[k], reg[k], acc);
      Io::store4(cs, 0, reg);
      u = acc;
    } else {
#pragma unroll
      for (int k = 0; k < kMaxW; ++k) {
        if (k + 1 < p.W) reg[k] = Io::load(cs, k + 1);
        else if (k + 1 == p.W) reg[k] = u;
      }
      float acc = p.conv_b ? p.conv_b[d] : 0.f;
#pragma unroll
      for (int k = 0; k < kMaxW; ++k)
        if (k < p.W) acc = fmaf(p.conv_w[d * p.W + k], reg[k], acc);
#pragma unroll
      for (int k = 0; k < kMaxW; ++k)
        if (k < p.W) Io::store(cs, k, reg[k]);
      u = acc;
    }
  }

  float dt = Io::load(static_cast<const io_t*>(p.delta), ch) + (p.delta_bias ? p.delta_bias[d] : 0.f);
  if (p.delta_softplus) dt = softplus_f32(dt);

  // ---- one scan step on u for the N states of the channel
  const io_t* Bg = static_cast<const io_t*>(p.Bm) + b * N;
  const io_t* Cg = static_cast<const io_t*>(p.Cm) + b * N;
  float* hp = p.h + ch * N;
  float h[N], A[N], Bv[N], Cv[N];
  Vec<N>::load(hp, h);
  Vec<N>::load(p.A + d * N, A);
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      Io::load4(Bg, 4 * k, &Bv[4 * k]);
      Io::load4(Cg, 4 * k, &Cv[4 * k]);
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bv[n] = Io::load(Bg, n);
      Cv[n] = Io::load(Cg, n);
    }
  }
  float yv = 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float ia = 1.0f / A[n];
    const float abar = exp2_fast(dt * A[n] * kLog2e);
    const float coef = fmaf(abar, ia, -ia);
    h[n] = fmaf(abar, h[n], coef * (Bv[n] * u));
    yv = fmaf(Cv[n], h[n], yv);
  }
  Vec<N>::store(hp, h);
  if (p.Dskip) yv = fmaf(p.Dskip[d], u, yv);
  if (p.z) yv *= silu(Io::load(static_cast<const io_t*>(p.z), ch));
  Io::store(static_cast<io_t*>(p.y), ch, yv);
}

template <typename io_t>
hipError_t launch_io(const StepParams& p, hipStream_t stream) {
  const int64_t total = p.B * p.D;
  const dim3 grid((unsigned)((total + 255) / 256));
  switch (p.N) {
    case 1: hipLaunchKernelGGL((step_kernel<io_t, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((step_kernel<io_t, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((step_kernel<io_t, 4>), grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((step_kernel<io_t, 8>), grid, dim3(256), 0, stream, p); break;
    case 16: hipLaunchKernelGGL((step_kernel<io_t, 16>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const StepParams& p, hipStream_t stream) {
  return p.io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ssm
