// One-token decode step (ssm_state_update) on gfx950.
//
// Page "Mamba and state space models", section "fixed-size state": generation keeps, per
// channel, the N-number SSM state and a short convolution holding the last few inputs, so each
// new token costs the same work. Per (b, d): shift the conv register and take the depthwise
// causal convolution u of the raw inputs, then one scan step on u (Abar = exp(Delta A),
// h = Abar h + expm1(Delta A)/A B u, y = C . h + D u), then the gate.
//
// The step is a single streaming pass bound by the state traffic (h read and written, 128 B
// per channel at N = 16). LPC = N / NS lanes share one channel, each owning NS consecutive
// states, so that every h load/store is one 16-byte access and a wave covers 1 KiB of
// contiguous state; the readout is reduced with a butterfly (identical result in every lane).
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kMaxW = 8;

template <typename io_t, int NS, int LPC>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  using Io = IoTraits<io_t>;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = p.B * p.D * LPC;
  if (i >= total) return;  // LPC divides 64 and total: a channel's lanes leave together
  const int64_t ch = i / LPC;  // b * D + d
  const int s = (int)(i % LPC);
  const int64_t d = ch % p.D;
  const int64_t b = ch / p.D;
  constexpr int N = NS * LPC;

  const io_t* xg = static_cast<const io_t*>(p.x);
  float u = Io::load(xg, ch);
  if (p.conv_state) {
    io_t* cs = static_cast<io_t*>(p.conv_state) + ch * p.W;
    float reg[kMaxW];
#pragma unroll
    for (int k = 0; k < kMaxW; ++k) {
      if (k + 1 < p.W) reg[k] = Io::load(cs, k + 1);
      else if (k + 1 == p.W) reg[k] = u;
    }
    float acc = p.conv_b ? p.conv_b[d] : 0.f;
#pragma unroll
    for (int k = 0; k < kMaxW; ++k)
      if (k < p.W) acc = fmaf(p.conv_w[d * p.W + k], reg[k], acc);
    if (s == 0) {
#pragma unroll
      for (int k = 0; k < kMaxW; ++k)
        if (k < p.W) Io::store(cs, k, reg[k]);
    }
    u = acc;
  }

  float dt = Io::load(static_cast<const io_t*>(p.delta), ch) + (p.delta_bias ? p.delta_bias[d] : 0.f);
  if (p.delta_softplus) dt = softplus_f32(dt);

  const io_t* Bg = static_cast<const io_t*>(p.Bm) + b * N + s * NS;
  const io_t* Cg = static_cast<const io_t*>(p.Cm) + b * N + s * NS;
  const float* Ad = p.A + d * N + s * NS;
  float* hp = p.h + ch * N + s * NS;
  float h[NS];
  if constexpr (NS == 4) {
    const float4 v = *reinterpret_cast<const float4*>(hp);
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) h[j] = hp[j];
  }
  float yp = 0.f;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float a = Ad[j];
    const float ia = 1.0f / a;
    const float abar = exp2_fast(dt * a * kLog2e);
    const float coef = fmaf(abar, ia, -ia);
    h[j] = fmaf(abar, h[j], coef * (Io::load(Bg, j) * u));
    yp = fmaf(Io::load(Cg, j), h[j], yp);
  }
  if constexpr (NS == 4) {
    *reinterpret_cast<float4*>(hp) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) hp[j] = h[j];
  }
#pragma unroll
  for (int off = 1; off < LPC; off <<= 1) yp += __shfl_xor(yp, off, 64);
  if (s == 0) {
    float yv = yp + (p.Dskip ? p.Dskip[d] * u : 0.f);
    if (p.z) yv *= silu(Io::load(static_cast<const io_t*>(p.z), ch));
    Io::store(static_cast<io_t*>(p.y), ch, yv);
  }
}

template <typename io_t>
hipError_t launch_io(const StepParams& p, hipStream_t stream) {
  auto go = [&](auto kern, int lpc) {
    const int64_t total = p.B * p.D * lpc;
    hipLaunchKernelGGL(kern, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
  };
  switch (p.N) {
    case 1: return go(step_kernel<io_t, 1, 1>, 1);
    case 2: return go(step_kernel<io_t, 2, 1>, 1);
    case 4: return go(step_kernel<io_t, 4, 1>, 1);
    case 8: return go(step_kernel<io_t, 4, 2>, 2);
    case 16: return go(step_kernel<io_t, 4, 4>, 4);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_update(const StepParams& p, hipStream_t stream) {
  return p.io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ssm
