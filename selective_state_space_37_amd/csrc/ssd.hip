// Mamba-2 (SSD) chunked forward on gfx950: MFMA for the within-chunk contractions.
//
// Page "Mamba and state space models", section "Mamba-2: two algorithms": with A a scalar times
// the identity per head, the layer multiplies the input by a lower-triangular matrix whose
// entry (i, j) is C_i . B_j times all decay between steps j and i. The sequence is cut into
// chunks of Q tokens; inside a chunk that masked product runs on the matrix cores, and only the
// state passes between chunks. With zero-order hold the input of step j enters with the scale
// phi_j = expm1(a Delta_j) / a, and with S the inclusive cumulative sum of Delta in the chunk:
//   state kernel : s_c[p, n] = sum_j exp(a (S_last - S_j)) phi_j x_j[p] B_j[n]     (MFMA, K = Q)
//   pass kernel  : h_c = exp(a S_last,c) h_{c-1} + s_c, in float32, over the chunks of a head
//   output kernel: y_i = sum_{j<=i} (C_i . B_j) exp(a (S_i - S_j)) phi_j x_j        (MFMA, K = N, Q)
//                      + exp(a S_i) C_i . h_{c-1}                                    (MFMA, K = N)
//                      (+ D x_i, gate)
// Decays are always formed from differences of cumulative sums inside one chunk, so no
// intermediate exponential can overflow. Operands are bf16, accumulation float32.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (lane l, g = l / 16):
//   A (16 x 32, M x K): row l % 16, k = 8g .. 8g+7;  B (32 x 16, K x N): col l % 16, k = 8g .. 8g+7;
//   D (16 x 16): col l % 16, rows 4g .. 4g+3.
// The K order inside one product is free as long as A and B agree; the output kernel uses that
// to feed a G^T tile pair straight from the D layout into the A operand of the next product.
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_frag() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
  return v;
}

__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

constexpr int kP = 64;  // head dim supported

// Step sizes, inclusive cumulative sums and ZOH input scales of one chunk (Q <= 256 tokens),
// for 256 threads. Tokens past L get Delta = 0 (identity).
template <int Q>
__device__ void chunk_prologue(const SsdParams& p, int64_t b, int64_t c, int64_t h, float a,
                               float* sS, float* sPhi, float* sTot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t t = c * Q + tid;
  float dt = 0.f;
  if (tid < Q && t < p.L) {
    dt = bf16_to_f32(static_cast<const bf16_t*>(p.delta)[(b * p.L + t) * p.H + h].bits) +
         (p.delta_bias ? p.delta_bias[h] : 0.f);
    if (p.delta_softplus) dt = softplus_f32(dt);
  }
  float v = dt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) sTot[w] = v;
  __syncthreads();
  float pre = 0.f;
  for (int k = 0; k < w; ++k) pre += sTot[k];
  if (tid < Q) {
    sS[tid] = v + pre;
    sPhi[tid] = expm1f(a * dt) / a;
  }
  __syncthreads();
}

// Stage x[b, chunk, h, :] transposed into LDS as bf16 Xt[p][j] (row stride Q + 8), optionally
// scaled per token by sScale[j].
template <int Q>
__device__ void stage_x_transposed(const SsdParams& p, int64_t b, int64_t c, int64_t h,
                                   __bf16* Xt, const float* sScale) {
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  for (int g = threadIdx.x; g < Q * (kP / 8); g += blockDim.x) {
    const int j = g / (kP / 8), pg = g % (kP / 8);
    const int64_t t = c * Q + j;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (t < p.L) raw = *reinterpret_cast<const uint4*>(xg + ((b * p.L + t) * p.H + h) * kP + pg * 8);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
    const float sc = sScale ? sScale[j] : 1.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = (q & 1) ? bf16_hi(wv[q >> 1]) : bf16_lo(wv[q >> 1]);
      Xt[(pg * 8 + q) * (Q + 8) + j] = (__bf16)(f * sc);
    }
  }
}

// ---------------------------------------------------------------------------- chunk states
template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_state_kernel(SsdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 Xt[kP * (Q + 8)];
  __shared__ __attribute__((aligned(16))) __bf16 Bt[N * (Q + 8)];
  __shared__ float sS[Q], sPhi[Q], sW[Q], sTot[4];
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  const float a = p.A[h];
  const float a2 = a * kLog2e;
  chunk_prologue<Q>(p, b, c, h, a, sS, sPhi, sTot);
  const int tid = threadIdx.x;
  const float s_last = sS[Q - 1];
  if (tid < Q) sW[tid] = exp2_fast(a2 * (s_last - sS[tid])) * sPhi[tid];
  if (tid == 0) p.ws_sum[(b * nch + c) * p.H + h] = s_last;
  __syncthreads();
  stage_x_transposed<Q>(p, b, c, h, Xt, sW);
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm);
  for (int g = tid; g < Q * (N / 8); g += 256) {
    const int j = g / (N / 8), ng = g % (N / 8);
    const int64_t t = c * Q + j;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (t < p.L) raw = *reinterpret_cast<const uint4*>(Bg + (b * p.L + t) * N + ng * 8);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint16_t bits = (q & 1) ? (uint16_t)(wv[q >> 1] >> 16) : (uint16_t)(wv[q >> 1] & 0xffff);
      Bt[(ng * 8 + q) * (Q + 8) + j] = __builtin_bit_cast(__bf16, bits);
    }
  }
  __syncthreads();

  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  constexpr int NT = N / 16;           // n tiles
  constexpr int NTW = NT / 4;          // n tiles per wave
  f32x4 acc[4][NTW];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int k = 0; k < NTW; ++k) acc[pt][k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < Q; k0 += 32) {
    bf16x8 av[4], bv[NTW];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      av[pt] = *reinterpret_cast<const bf16x8*>(&Xt[(pt * 16 + r16) * (Q + 8) + k0 + 8 * g]);
#pragma unroll
    for (int k = 0; k < NTW; ++k)
      bv[k] = *reinterpret_cast<const bf16x8*>(&Bt[((w * NTW + k) * 16 + r16) * (Q + 8) + k0 + 8 * g]);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int k = 0; k < NTW; ++k) acc[pt][k] = mfma16(av[pt], bv[k], acc[pt][k]);
  }
  float* out = p.ws_state + ((b * nch + c) * p.H + h) * (int64_t)(kP * N);
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int k = 0; k < NTW; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(pt * 16 + 4 * g + r) * N + (w * NTW + k) * 16 + r16] = acc[pt][k][r];
}

// ---------------------------------------------------------------------------- state pass
// One thread per (b, h, p, n): h_in[c] = state entering chunk c (written over s_c).
__global__ __launch_bounds__(256) void ssd_pass_kernel(SsdParams p, int64_t nch) {
  const int64_t PN = kP * p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.B * p.H * PN) return;
  const int64_t e = i % PN;
  const int64_t h = (i / PN) % p.H;
  const int64_t b = i / (PN * p.H);
  const float a2 = p.A[h] * kLog2e;
  float st = p.h0 ? p.h0[(b * p.H + h) * PN + e] : 0.f;
  for (int64_t c = 0; c < nch; ++c) {
    float* slot = p.ws_state + ((b * nch + c) * p.H + h) * PN + e;
    const float sc = *slot;
    *slot = st;
    st = fmaf(exp2_fast(a2 * p.ws_sum[(b * nch + c) * p.H + h]), st, sc);
  }
  if (p.h_last) p.h_last[(b * p.H + h) * PN + e] = st;
}

// ---------------------------------------------------------------------------- outputs
template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_out_kernel(SsdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 Xt[kP * (Q + 8)];
  __shared__ float sS[Q], sPhi[Q], sTot[4];
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  const float a = p.A[h];
  const float a2 = a * kLog2e;
  chunk_prologue<Q>(p, b, c, h, a, sS, sPhi, sTot);
  stage_x_transposed<Q>(p, b, c, h, Xt, nullptr);
  __syncthreads();

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  constexpr int NIB = Q / 16;   // 16-row blocks of the chunk
  constexpr int KS = N / 32;    // K steps over the state dimension
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm);
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm);
  const float* hin = p.ws_state + ((b * nch + c) * p.H + h) * (int64_t)(kP * N);
  const float dsk = p.Dskip ? p.Dskip[h] : 0.f;
  const bf16_t* zg = static_cast<const bf16_t*>(p.z);
  bf16_t* yg = static_cast<bf16_t*>(p.y);

  // Balanced triangle: block x and block NIB-1-x hold NIB+1 tiles together.
  constexpr int kBlocksPerWave = NIB >= 8 ? NIB / 4 : 1;
  for (int kb = 0; kb < kBlocksPerWave; ++kb) {
    int ib;
    if (NIB >= 8) {
      const int pair = w + 4 * (kb >> 1);
      ib = (kb & 1) ? (NIB - 1 - pair) : pair;
    } else {
      ib = w;
      if (ib >= NIB) break;
    }
    const int i0 = ib * 16;
    const int il = i0 + r16;                  // this lane's row (A operand / G^T column)
    const int64_t ti = c * Q + il;
    const bool ti_ok = ti < p.L;
    const float Si = sS[il];
    bf16x8 cf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      cf[ks] = ti_ok ? load_frag(Cg + (b * p.L + ti) * N + ks * 32 + 8 * g) : zero_frag();

    f32x4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // carried state: exp(a S_i) C_i . h_in[p, :]
    const float eSi = exp2_fast(a2 * Si);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 av;
#pragma unroll
      for (int q = 0; q < 8; ++q) av[q] = (__bf16)((float)cf[ks][q] * eSi);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float* hp = hin + (pt * 16 + r16) * N + ks * 32 + 8 * g;
        const float4 h0v = *reinterpret_cast<const float4*>(hp);
        const float4 h1v = *reinterpret_cast<const float4*>(hp + 4);
        bf16x8 bv;
        bv[0] = (__bf16)h0v.x; bv[1] = (__bf16)h0v.y; bv[2] = (__bf16)h0v.z; bv[3] = (__bf16)h0v.w;
        bv[4] = (__bf16)h1v.x; bv[5] = (__bf16)h1v.y; bv[6] = (__bf16)h1v.z; bv[7] = (__bf16)h1v.w;
        acc[pt] = mfma16(av, bv, acc[pt]);
      }
    }

    // within the chunk: masked (C_i . B_j) decay phi_j times x_j, two 16-token j tiles per product
    for (int jp = 0; 2 * jp <= ib; ++jp) {
      float m[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jt = 2 * jp + half;
        if (jt > ib) {
#pragma unroll
          for (int r = 0; r < 4; ++r) m[half * 4 + r] = 0.f;
          continue;
        }
        const int64_t tj = c * Q + jt * 16 + r16;
        const bool tj_ok = tj < p.L;
        f32x4 gacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 bfr = tj_ok ? load_frag(Bg + (b * p.L + tj) * N + ks * 32 + 8 * g) : zero_frag();
          gacc = mfma16(bfr, cf[ks], gacc);   // G^T[j][i]
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jt * 16 + 4 * g + r;
          m[half * 4 + r] = (j <= il) ? gacc[r] * exp2_fast(a2 * (Si - sS[j])) * sPhi[j] : 0.f;
        }
      }
      bf16x8 av;
#pragma unroll
      for (int q = 0; q < 8; ++q) av[q] = (__bf16)m[q];
      const int jb = jp * 32;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const __bf16* xr = &Xt[(pt * 16 + r16) * (Q + 8) + jb + 4 * g];
        bf16x8 bv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bv[q] = xr[q];
          bv[4 + q] = xr[16 + q];
        }
        acc[pt] = mfma16(av, bv, acc[pt]);
      }
    }

    // epilogue: D term, gate, store y[b, t, h, p]
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * g + r;
        const int pp = pt * 16 + r16;
        const int64_t t = c * Q + i;
        if (t < p.L) {
          float v = acc[pt][r];
          v = fmaf(dsk, (float)Xt[pp * (Q + 8) + i], v);
          const int64_t o = ((b * p.L + t) * p.H + h) * kP + pp;
          if (zg) v *= silu(bf16_to_f32(zg[o].bits));
          yg[o].bits = f32_to_bf16(v);
        }
      }
    }
  }
}

template <int Q, int N>
hipError_t launch_qn(const SsdParams& p, hipStream_t stream) {
  const int64_t nch = (p.L + Q - 1) / Q;
  const dim3 grid((unsigned)p.H, (unsigned)nch, (unsigned)p.B);
  hipLaunchKernelGGL((ssd_state_kernel<Q, N>), grid, dim3(256), 0, stream, p);
  const int64_t chains = p.B * p.H * kP * p.N;
  hipLaunchKernelGGL(ssd_pass_kernel, dim3((unsigned)((chains + 255) / 256)), dim3(256), 0, stream, p, nch);
  hipLaunchKernelGGL((ssd_out_kernel<Q, N>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t ssd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t Q) {
  const int64_t nch = (L + Q - 1) / Q;
  return (size_t)(B * nch * H * P * N) * sizeof(float) + (size_t)(B * nch * H) * sizeof(float) + 256;
}

hipError_t launch_ssd(const SsdParams& p, hipStream_t stream) {
  if (p.N == 128) {
    if (p.Q == 64) return launch_qn<64, 128>(p, stream);
    if (p.Q == 128) return launch_qn<128, 128>(p, stream);
    if (p.Q == 256) return launch_qn<256, 128>(p, stream);
  } else if (p.N == 64) {
    if (p.Q == 64) return launch_qn<64, 64>(p, stream);
    if (p.Q == 128) return launch_qn<128, 64>(p, stream);
    if (p.Q == 256) return launch_qn<256, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
