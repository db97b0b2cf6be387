// One-token decode step (ssm_state_update) on gfx950.
//
// Page "Mamba and state space models", section "fixed-size state": generation keeps, per
// channel, the N-number SSM state and a short convolution holding the last few inputs, so each
// new token costs the same work. Per (b, d): shift the conv register and take the depthwise
// causal convolution u of the raw inputs, then one scan step on u (Abar = exp(Delta A),
// h = Abar h + expm1(Delta A)/A B u, y = C . h + D u), then the gate.
//
// The step is a single streaming pass bound by the state traffic (h read and written, 128 B
// per channel at N = 16). The state of a channel is split over N / 4 lanes (4 states each, one
// 16-byte load), so consecutive lanes hold consecutive 16-byte pieces of h and A and a wave's
// load covers 1 KiB of contiguous state. The lanes of a channel share x, Delta, z and the conv
// register (same addresses, one fetch), each forms its part of C . h, and the parts are added
// across the lanes with DPP quad permutes. At N < 4 one lane owns the whole channel.
#include <type_traits>

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

// CONV: 0 = no conv register, 4 = width 4 (vector loads), -1 = any width 1..8.
// R: batch rows per thread. The thread handles channel d, state slice q of rows bq R .. bq R +
// R - 1; the per-channel operands (A, conv weights, bias, D) are loaded once for the R rows.
// All loads of a lane are issued before any arithmetic, so a wave pays one memory round trip.
template <typename io_t, int N, int CONV, int R>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  using Io = IoTraits<io_t>;
  using raw4 = typename Io::raw4;
  constexpr int SPL = N >= 4 ? 4 : N;   // states per lane
  constexpr int LPC = N / SPL;          // lanes per channel
  const int64_t nbq = (p.B + R - 1) / R;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (bq * D + d) * LPC + q
  // the grid is whole channels: LPC divides the block size, so a channel's lanes are all
  // present or all absent and the DPP sums below only combine lanes of one channel
  if (gid >= nbq * p.D * LPC) return;
  const int64_t cq = gid / LPC;   // bq * D + d
  const int q = (int)(gid % LPC);
  int64_t bq, d;
  if (nbq * p.D <= 0x7fffffff) {   // uniform: 32-bit division when the channel count allows
    const uint32_t c32 = (uint32_t)cq, D32 = (uint32_t)p.D;
    const uint32_t b32 = c32 / D32;
    bq = b32;
    d = c32 - b32 * D32;
  } else {
    bq = cq / p.D;
    d = cq - bq * p.D;
  }
  const int n0 = q * SPL;
  // rows past B repeat the last row's loads and skip every store
  int64_t ch[R], brow[R];
  bool live[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = bq * R + r;
    live[r] = b < p.B;
    brow[r] = live[r] ? b : p.B - 1;
    ch[r] = brow[r] * p.D + d;
  }

  // ---- loads: per-channel operands once, per-row operands for each of the R rows
  const io_t* xg = static_cast<const io_t*>(p.x);
  const io_t* dg = static_cast<const io_t*>(p.delta);
  const io_t* zg = static_cast<const io_t*>(p.z);
  // optional tensors are read through a valid stand-in address when absent and the value is
  // dropped afterwards: no branch around a load, so no wait is forced before the join
  const float* fstand = p.A;   // any float array with at least D entries
  const float bias_v = (p.delta_bias ? p.delta_bias : fstand)[d];
  const float dsk_v = (p.Dskip ? p.Dskip : fstand)[d];
  float A[SPL];
  Vec<SPL>::load(p.A + d * N + n0, A);
  float4 cw4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float cb = 0.f;
  if constexpr (CONV == 4) cw4 = *reinterpret_cast<const float4*>(p.conv_w + d * 4);
  if constexpr (CONV != 0) cb = (p.conv_b ? p.conv_b : fstand)[d];
  uint32_t x_bits[R], d_bits[R], z_bits[R];
  raw4 creg[R];
  float h[R][SPL], Bv[R][SPL], Cv[R][SPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    x_bits[r] = Io::load_bits(xg, ch[r]);
    d_bits[r] = Io::load_bits(dg, ch[r]);
    z_bits[r] = Io::load_bits(zg ? zg : xg, ch[r]);
    creg[r] = Io::zero4();
    if constexpr (CONV == 4) creg[r] = Io::load4_raw(static_cast<const io_t*>(p.conv_state) + ch[r] * 4, 0);
    Vec<SPL>::load(p.h + ch[r] * N + n0, h[r]);
    const io_t* Bg = static_cast<const io_t*>(p.Bm) + brow[r] * N + n0;
    const io_t* Cg = static_cast<const io_t*>(p.Cm) + brow[r] * N + n0;
    if constexpr (SPL == 4) {
      const raw4 br = Io::load4_raw(Bg, 0), cr = Io::load4_raw(Cg, 0);
      Io::unpack4(br, Bv[r]);
      Io::unpack4(cr, Cv[r]);
    } else {
#pragma unroll
      for (int n = 0; n < SPL; ++n) {
        Bv[r][n] = Io::load(Bg, n);
        Cv[r][n] = Io::load(Cg, n);
      }
    }
  }

  const float bias = p.delta_bias ? bias_v : 0.f;
  const float dsk = p.Dskip ? dsk_v : 0.f;
  if constexpr (CONV != 0) cb = p.conv_b ? cb : 0.f;
  float ia[SPL], a2[SPL];
#pragma unroll
  for (int n = 0; n < SPL; ++n) {
    ia[n] = 1.0f / A[n];
    a2[n] = A[n] * kLog2e;
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    // ---- conv register: shift, insert x, depthwise causal convolution (every lane of the
    //      channel computes u; lane 0 writes the register back)
    float u = Io::from_bits(x_bits[r]);
    if constexpr (CONV == 4) {
      float old[4];
      Io::unpack4(creg[r], old);
      const float reg[4] = {old[1], old[2], old[3], u};
      float acc = cb;
      acc = fmaf(cw4.x, reg[0], acc);
      acc = fmaf(cw4.y, reg[1], acc);
      acc = fmaf(cw4.z, reg[2], acc);
      acc = fmaf(cw4.w, reg[3], acc);
      if (q == 0 && live[r]) Io::store4(static_cast<io_t*>(p.conv_state) + ch[r] * 4, 0, reg);
      u = acc;
    } else if constexpr (CONV == -1) {
      io_t* cs = static_cast<io_t*>(p.conv_state) + ch[r] * p.W;
      float reg[kMaxW];
#pragma unroll
      for (int k = 0; k < kMaxW; ++k) {
        if (k + 1 < p.W) reg[k] = Io::load(cs, k + 1);
        else if (k + 1 == p.W) reg[k] = u;
      }
      float acc = cb;
#pragma unroll
      for (int k = 0; k < kMaxW; ++k)
        if (k < p.W) acc = fmaf(p.conv_w[d * p.W + k], reg[k], acc);
      if (q == 0 && live[r]) {
#pragma unroll
        for (int k = 0; k < kMaxW; ++k)
          if (k < p.W) Io::store(cs, k, reg[k]);
      }
      u = acc;
    }

    float dt = Io::from_bits(d_bits[r]) + bias;
    if (p.delta_softplus) dt = softplus_f32(dt);

    // ---- one scan step on u for this lane's SPL states (n = q SPL ..)
    float yv = 0.f;
#pragma unroll
    for (int n = 0; n < SPL; ++n) {
      const float tx = dt * a2[n];
      const float abar = exp2_fast(tx);
      const float coef = zoh_input_scale<std::is_same<io_t, float>::value>(abar, tx, dt, ia[n]);
      h[r][n] = fmaf(abar, h[r][n], coef * (Bv[r][n] * u));
      yv = fmaf(Cv[r][n], h[r][n], yv);
    }
    if (live[r]) Vec<SPL>::store(p.h + ch[r] * N + n0, h[r]);
    yv = sum_channel_lanes<LPC>(yv);
    if (q == 0 && live[r]) {
      yv = fmaf(dsk, u, yv);
      if (zg) yv *= silu(Io::from_bits(z_bits[r]));
      Io::store(static_cast<io_t*>(p.y), ch[r], yv);
    }
  }
}

// Rows per thread: 2 when the batch allows (each wave has twice the independent loads in
// flight and loads the per-channel operands once for both rows), else 1. Measured at batch 128:
// 1 row 22.0 us, 2 rows 19.1 us, 4 rows 20.3 us, 8 rows 22.7 us per step.
template <typename io_t, int N, int R>
void launch_nr(const StepParams& p, hipStream_t stream) {
  constexpr int LPC = N >= 4 ? N / 4 : 1;
  const int64_t total = (p.B + R - 1) / R * p.D * LPC;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (!p.conv_state)
    hipLaunchKernelGGL((step_kernel<io_t, N, 0, R>), grid, dim3(256), 0, stream, p);
  else if (p.W == 4)
    hipLaunchKernelGGL((step_kernel<io_t, N, 4, R>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((step_kernel<io_t, N, -1, R>), grid, dim3(256), 0, stream, p);
}

template <typename io_t, int N>
void launch_n(const StepParams& p, hipStream_t stream) {
  if (p.B >= 2) launch_nr<io_t, N, 2>(p, stream);
  else launch_nr<io_t, N, 1>(p, stream);
}

template <typename io_t>
hipError_t launch_io(const StepParams& p, hipStream_t stream) {
  switch (p.N) {
    case 1: launch_n<io_t, 1>(p, stream); break;
    case 2: launch_n<io_t, 2>(p, stream); break;
    case 4: launch_n<io_t, 4>(p, stream); break;
    case 8: launch_n<io_t, 8>(p, stream); break;
    case 16: launch_n<io_t, 16>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const StepParams& p, hipStream_t stream) {
  return p.io_bf16 ? launch_io<bf16_t>(p, stream) : launch_io<float>(p, stream);
}

}  // namespace ssm
