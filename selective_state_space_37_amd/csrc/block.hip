// One decode token through a Mamba block, for the generation workload: LayerNorm, the input
// projections, the short causal convolution with SiLU, the projections to Delta, B and C, the
// selective state update, the output projection and the residual. Launches per block step:
// LayerNorm; the input projection with conv + SiLU and the x projection's per-slice partials in
// its epilogue; their reduction; the Delta projection fused with the state update
// (block_ssm_kernel); the output projection with the residual (+ its reduction).
//
// The block follows the pages as read for this workload: the pre-norm residual block with
// LayerNorm of the code overview on "Beyond attention: exploring Mamba and state space models";
// the gated block of the news write-up's "architecture" section (an SSM branch and a gate branch
// from one input projection, multiplied, then an output projection); the convolution over the
// last 4 inputs of "Mamba and state space models", section "fixed-size state"; Delta, B and C as
// small linear projections of the token (same page, "decided by the token").
//
// At decode time every projection is a product of the batch's token rows (M <= 128) with a
// weight matrix that is read once per step: the kernel streams the weights from HBM and keeps
// the activations in L2. MFMA v_mfma_f32_16x16x32_bf16, lane layout as in the SSD kernels:
//   A (16 x 32): row l % 16, k = 8g .. 8g+7;  B (32 x 16): col l % 16, k = 8g .. 8g+7;
//   D (16 x 16): col l % 16, rows 4g .. 4g+3  (g = l / 16).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
  return v;
}

// Four floats rounded to bf16 (nearest even) as two words: one v_cvt_pk_bf16_f32 per pair.
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){c, d}, bf16x2_t)));
}

// ---------------------------------------------------------------------------- LayerNorm
// One workgroup (256 threads) per row of D <= 8192 bf16 values (D % 8 == 0): each thread keeps up
// to four 8-element pieces in registers; mean, then variance of the centred values, both summed
// in float32 through a fixed tree (deterministic). The row, w and b are all loaded before the
// first sum (pieces past D read the last piece and are dropped: no branch around a load), so the
// kernel pays one memory round trip.
__global__ __launch_bounds__(256) void layernorm_kernel(int64_t D, const bf16_t* x, const float* w, const float* b,
                                                        float eps, bf16_t* y) {
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bf16_t* xr = x + row * D;
  uint4 xw[4];
  float wt[4][8], bt[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t c = std::min<int64_t>((int64_t)(tid + 256 * k) * 8, D - 8);
    xw[k] = *reinterpret_cast<const uint4*>(xr + c);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      wt[k][q] = w[c + q];
      bt[k][q] = b[c + q];
    }
  }
  float v[4][8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool in = (int64_t)(tid + 256 * k) * 8 < D;
    const uint32_t wd[4] = {xw[k].x, xw[k].y, xw[k].z, xw[k].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[k][2 * q] = in ? bf16_lo(wd[q]) : 0.f;
      v[k][2 * q + 1] = in ? bf16_hi(wd[q]) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[k][q];
  }
  auto block_sum = [&](float t, int slot) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
    if (lane == 0) red[slot * 4 + wv] = t;
    __syncthreads();
    return (red[slot * 4] + red[slot * 4 + 1]) + (red[slot * 4 + 2] + red[slot * 4 + 3]);
  };
  const float mean = block_sum(s, 0) / (float)D;
  float s2 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((int64_t)(tid + 256 * k) * 8 < D) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float d = v[k][q] - mean;
        s2 += d * d;
      }
    }
  }
  const float rstd = rsqrtf(block_sum(s2, 1) / (float)D + eps);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t c = (int64_t)(tid + 256 * k) * 8;
    if (c < D) {
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = (v[k][q] - mean) * rstd * wt[k][q] + bt[k][q];
      const uint2 lo = pack4(o[0], o[1], o[2], o[3]), hi = pack4(o[4], o[5], o[6], o[7]);
      *reinterpret_cast<uint4*>(y + row * D + c) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

// ---------------------------------------------------------------------------- skinny GEMM
// Y[m][n] = sum_k X[m][k] W[n][k] (+ R[m][n]) for M <= 128 token rows: every weight is read once
// per step, so both kernels are built to keep enough weight bytes in flight. The products are
// computed transposed (D[n][m]: A = W rows, B = X rows), so a lane ends with four consecutive
// outputs of one row (one 8-byte store). With one K split the epilogue (residual, bf16) is applied
// in place; otherwise float32 partials [S, M, Nout] go to gemm_reduce_kernel, which adds them in
// split order.
//
// gemm_xwt_kernel (chunked): grid (ceil(Nout / 128), row blocks, S), 8 waves, wave w owns the
// 16-column tile w. The row block's X slice goes through LDS in 128-wide K chunks (double-buffered,
// one barrier per chunk, loaded two chunks ahead) and is shared by the waves; each wave streams
// its own W rows two chunks ahead in a register ring (the loop is unrolled by 2 so the ring is
// indexed statically). Used where the column tiles alone fill the GPU (the LM head).
// The conv + SiLU epilogue for channels n .. n + 3 of row m, given their product values v: per
// channel the register of the last W inputs (oldest first) is shifted, the new input (rounded to
// bf16, the register's type) appended, and u = SiLU(sum_k w[k] reg[k] + bias), the newest input
// multiplied by w[W - 1]. At width 4 the caller has loaded the 32 register bytes (r0, r1).
// (cwq, cbq: the width-4 weights of the four channels and their biases when the caller loaded
// them ahead, else NULL)
__device__ __forceinline__ float4 conv_silu4(const GemmParams& p, int64_t m, int64_t n, float4 v, uint4 r0, uint4 r1,
                                             const float4* cwq = nullptr, const float4* cbq = nullptr) {
  const int64_t W = p.conv_W;
  bf16_t* reg = static_cast<bf16_t*>(p.conv_state) + (m * p.conv_D + n) * W;
  const float xv[4] = {v.x, v.y, v.z, v.w};
  float uo[4];
  if (W == 4) {
    // 4 channels x 4 taps: 32 contiguous bytes of the register
    const uint32_t wd[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xb = f32_to_bf16(xv[j]);
      // taps oldest first: (lo, hi) of word 2j, then of word 2j + 1; shift by one and append x
      const float t1 = bf16_hi(wd[2 * j]), t2 = bf16_lo(wd[2 * j + 1]), t3 = bf16_hi(wd[2 * j + 1]);
      const float t4 = bf16_to_f32(xb);
      const float* cwg = p.conv_w + (n + j) * 4;
      const float4 cw = cwq ? cwq[j] : make_float4(cwg[0], cwg[1], cwg[2], cwg[3]);
      const float cbv[4] = {cbq ? cbq->x : 0.f, cbq ? cbq->y : 0.f, cbq ? cbq->z : 0.f, cbq ? cbq->w : 0.f};
      float acc = cbq ? cbv[j] : (p.conv_b ? p.conv_b[n + j] : 0.f);
      acc += cw.x * t1;
      acc += cw.y * t2;
      acc += cw.z * t3;
      acc += cw.w * t4;
      uo[j] = silu(acc);
      out[2 * j] = (wd[2 * j] >> 16) | (wd[2 * j + 1] << 16);
      out[2 * j + 1] = (wd[2 * j + 1] >> 16) | (xb << 16);
    }
    reinterpret_cast<uint4*>(reg)[0] = make_uint4(out[0], out[1], out[2], out[3]);
    reinterpret_cast<uint4*>(reg)[1] = make_uint4(out[4], out[5], out[6], out[7]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16_t* r = reg + j * W;
      const float* cw = p.conv_w + (n + j) * W;
      float acc = p.conv_b ? p.conv_b[n + j] : 0.f;
      for (int64_t k = 0; k + 1 < W; ++k) {
        const bf16_t t = r[k + 1];
        r[k] = t;
        acc += cw[k] * bf16_to_f32(t.bits);
      }
      bf16_t xb;
      xb.bits = f32_to_bf16(xv[j]);
      r[W - 1] = xb;
      acc += cw[W - 1] * bf16_to_f32(xb.bits);
      uo[j] = silu(acc);
    }
  }
  *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.u) + m * p.conv_D + n) = pack4(uo[0], uo[1], uo[2], uo[3]);
  return make_float4(uo[0], uo[1], uo[2], uo[3]);
}

constexpr int kGemmKC = 128;  // K chunk
constexpr int kGemmXS = kGemmKC + 8;   // LDS row stride (bf16) of an X chunk
constexpr int kGemmNW = 8;    // waves per workgroup: 16 output columns each

template <int MT, bool XRES = false>
__global__ __launch_bounds__(64 * kGemmNW) void gemm_xwt_kernel(GemmParams p) {
  // W chunks in flight per wave (the loop is unrolled by this); with the X slice resident the
  // loop has no barrier, so a deeper ring keeps more of the weight stream in flight
  constexpr int kGemmPD = XRES ? 4 : 2;
  constexpr int NT = 64 * kGemmNW;
  constexpr int ROWS = MT * 16;
  constexpr int KS = kGemmKC / 32;                         // 32-wide steps per chunk
  constexpr int XPIECES = ROWS * (kGemmKC / 8);            // 16-byte pieces of an X chunk
  constexpr int XPER = (XPIECES + NT - 1) / NT;            // per thread
  __shared__ __attribute__((aligned(16))) __bf16 xs_st[XRES ? 1 : 2][XRES ? 8 : ROWS * kGemmXS];
  // resident X: the row block's whole K slice, rows kslice + 8 elements apart (dynamic LDS)
  extern __shared__ __attribute__((aligned(16))) __bf16 xs_dyn[];
  __bf16* const xs0 = XRES ? xs_dyn : &xs_st[0][0];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t col0 = (int64_t)blockIdx.x * 16 * kGemmNW;
  const int64_t m0 = (int64_t)blockIdx.y * ROWS;
  const int64_t ks = blockIdx.z;
  const int64_t kbeg = ks * p.kslice;
  const int64_t nchunks = p.kslice / kGemmKC;
  const bf16_t* W = static_cast<const bf16_t*>(p.w);
  const bf16_t* X = static_cast<const bf16_t*>(p.x);

  // this wave's W rows and the row block's X rows through buffer descriptors: a row past Nout (or
  // past M) lies beyond the descriptor's size and reads as zero, so no load is conditional and the
  // compiler's count of loads in flight stays exact (a branch around a load makes it wait for
  // every load at the join). Sizes are counted from the slice start kbeg; a valid row's slice ends
  // at or before K, so it stays inside.
  const int64_t wrow0 = col0 + w * 16;
  const int64_t wrows = std::max<int64_t>(0, std::min<int64_t>(16, p.Nout - wrow0));
  const Rsrc wr_rs = make_rsrc(W + std::min<int64_t>(wrow0, p.Nout - 1) * p.K + kbeg,
                               (int)(wrow0 < p.Nout ? wrows * p.K * 2 - kbeg * 2 : 0));
  const uint32_t wlane = (uint32_t)((r16 * p.K + 8 * g) * 2);
  // a chunk past the end loads from an offset past every descriptor's size: it reads zeros
  // (unused) and moves no data
  constexpr uint32_t kPastEnd = 0x80000000u;
  auto load_w = [&](int64_t c, bf16x8 out[KS]) __attribute__((always_inline)) {
    const uint32_t o = c < nchunks ? wlane + (uint32_t)(c * kGemmKC * 2) : kPastEnd;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      uint4 v;
      buf_load(wr_rs, o + (uint32_t)(s2 * 64), v);
      out[s2] = __builtin_bit_cast(bf16x8, v);
    }
  };
  // this thread's pieces of an X chunk: row e / (KC / 8), 8-element column group e % (KC / 8)
  // (threads past the pieces read past the size, and their values are never stored)
  constexpr int PPR = kGemmKC / 8;
  const int64_t xrows = std::max<int64_t>(0, std::min<int64_t>(ROWS, p.M - m0));
  const Rsrc x_rs = make_rsrc(X + std::min<int64_t>(m0, p.M - 1) * p.ldx + kbeg,
                              (int)(m0 < p.M ? (xrows - 1) * p.ldx * 2 + (p.K - kbeg) * 2 : 0));
  auto load_x = [&](int64_t c, uint4 out[XPER]) __attribute__((always_inline)) {
    const uint32_t o = c < nchunks ? (uint32_t)(c * kGemmKC * 2) : kPastEnd;
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
      const int e = tid + NT * k;
      buf_load(x_rs, o + (uint32_t)(((e / PPR) * p.ldx + (e % PPR) * 8) * 2), out[k]);
    }
  };
  auto store_x = [&](int buf, const uint4 in[XPER]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
      const int e = tid + NT * k;
      if (e < XPIECES) *reinterpret_cast<uint4*>(&xs0[buf * (ROWS * kGemmXS) + (e / PPR) * kGemmXS + (e % PPR) * 8]) = in[k];
    }
  };

  // conv epilogue (no split of K, width 4): the register words of this lane's outputs, loaded
  // before the stream when the tile is small (a lane past conv_D or past M reads a valid
  // stand-in and drops it), else in the epilogue
  constexpr bool kRegEarly = MT <= 2;
  const int64_t ne = col0 + w * 16 + 4 * g;
  auto reg_words = [&](int mt, uint4& r0, uint4& r1) __attribute__((always_inline)) {
    const int64_t me = std::min<int64_t>(m0 + mt * 16 + r16, p.M - 1);
    const uint4* rp = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(p.conv_state) +
                                                     (me * p.conv_D + std::min<int64_t>(ne, p.conv_D - 4)) * 4);
    r0 = rp[0];
    r1 = rp[1];
  };
  uint4 rg[kRegEarly ? MT : 1][2];
#pragma unroll
  for (int mt = 0; mt < (kRegEarly ? MT : 1); ++mt) rg[mt][0] = rg[mt][1] = make_uint4(0, 0, 0, 0);
  // and the width-4 weights and biases of the lane's four channels (a workgroup past conv_D
  // reads channel conv_D - 4 as a stand-in)
  float4 cwq[kRegEarly ? 4 : 1], cbq = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < (kRegEarly ? 4 : 1); ++j) cwq[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (kRegEarly) {
    if (p.conv_state && p.conv_W == 4) {   // uniform
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) reg_words(mt, rg[mt][0], rg[mt][1]);
      // (element loads: the block step does not require these tensors to be 16-byte aligned)
      const int64_t nc = std::min<int64_t>(ne, p.conv_D - 4);
      const float* cw = p.conv_w + nc * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) cwq[j] = make_float4(cw[4 * j], cw[4 * j + 1], cw[4 * j + 2], cw[4 * j + 3]);
      if (p.conv_b) cbq = make_float4(p.conv_b[nc], p.conv_b[nc + 1], p.conv_b[nc + 2], p.conv_b[nc + 3]);
    }
  }
  // x-projection epilogue: this wave's W_xp fragments (output fragments w + 8 i, i < kXpF, of the
  // (xp_n / 16) x MT grid), loaded before the stream as well (rows past xp_n repeat the last)
  constexpr int kXpF = MT <= 2 ? 3 : 1;
  const bool xp_on = MT <= 2 && p.xp_w && p.conv_state && p.S == 1 && col0 < p.conv_D;   // per workgroup
  const int xp_rt = (int)((p.xp_n + 15) / 16);
  bf16x8 xpa[kXpF][4];
  if constexpr (MT <= 2) {
    if (xp_on) {   // uniform
#pragma unroll
      for (int i = 0; i < kXpF; ++i) {
        const int f = std::min(w + 8 * i, xp_rt * MT - 1);
        const bf16_t* wxr = static_cast<const bf16_t*>(p.xp_w) +
                            std::min<int64_t>(16 * (f / MT) + r16, p.xp_n - 1) * p.conv_D + col0 + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) xpa[i][s2] = *reinterpret_cast<const bf16x8*>(wxr + 32 * s2);
      }
    }
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 wr[kGemmPD][KS];
  int64_t c = 0;
  if constexpr (XRES) {
    // The row block's X slice goes straight to LDS once (each wave load moves 1 KB: 512 elements
    // of one row, lane l's 16 bytes landing 16 l bytes after the load's base); rows past M read
    // as zero. Then the weight ring is issued, and the wait for all but the ring's loads retires
    // the X loads. No barrier interrupts the stream after that.
    const int64_t XSTR = p.kslice + 8;
    const int per_row = (int)(p.kslice / 512);
    for (int q = w; q < ROWS * per_row; q += kGemmNW) {   // uniform per wave
      const int r = q / per_row, part = q % per_row;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x_rs, (__attribute__((address_space(3))) void*)(xs0 + r * XSTR + part * 512), 16,
          (uint32_t)((r * p.ldx + part * 512 + lane * 8) * 2), 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kGemmPD; ++k) load_w(k, wr[k]);
    constexpr int kRing = kGemmPD * KS;   // loads of the ring, issued after the X loads
    static_assert(kRing < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((kRing & 15) | ((kRing >> 4) << 14) | 0x0F70);
    __syncthreads();
    const __bf16* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrow[mt] = xs0 + (mt * 16 + r16) * XSTR + 8 * g;
    // chunk c: X from the resident rows, W from ring slot c % PD
    auto step = [&](int64_t cc, int slot) __attribute__((always_inline)) {
      const int kc = (int)(cc * kGemmKC);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 xf = *reinterpret_cast<const bf16x8*>(xrow[mt] + kc + s2 * 32);
          acc[mt] = mfma16(wr[slot][s2], xf, acc[mt]);
        }
      }
      load_w(cc + kGemmPD, wr[slot]);   // refill the slot just used
    };
    for (; c + kGemmPD <= nchunks; c += kGemmPD) {
#pragma unroll
      for (int k = 0; k < kGemmPD; ++k) step(c + k, k);
    }
#pragma unroll
    for (int k = 0; k < kGemmPD; ++k)
      if (c + k < nchunks) step(c + k, k);
    // every wave is done with X before the epilogue parks its u tile over it
    if (xp_on) __syncthreads();   // uniform
  } else {
#pragma unroll
    for (int k = 0; k < kGemmPD; ++k) load_w(k, wr[k]);
    // X chunks two ahead in registers: xr[(c + 1) % 2] holds chunk c + 1 when chunk c is used
    uint4 xr[2][XPER];
    load_x(0, xr[0]);
    store_x(0, xr[0]);
    load_x(1, xr[1]);
    load_x(2, xr[0]);
    __syncthreads();

    // chunk c: X from LDS buffer c % 2, W from ring slot c % PD (PD even, so slot parity = c parity)
    auto step = [&](int64_t cc, int slot) __attribute__((always_inline)) {
      const int buf = (int)(cc & 1);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 xf = *reinterpret_cast<const bf16x8*>(&xs0[buf * (ROWS * kGemmXS) + (mt * 16 + r16) * kGemmXS + s2 * 32 + 8 * g]);
          acc[mt] = mfma16(wr[slot][s2], xf, acc[mt]);
        }
      }
      load_w(cc + kGemmPD, wr[slot]);        // refill the slot just used
      store_x(buf ^ 1, xr[(slot + 1) & 1]);  // chunk c + 1 (its buffer held chunk c - 1)
      load_x(cc + 3, xr[(slot + 1) & 1]);
      __syncthreads();
    };
    for (; c + kGemmPD <= nchunks; c += kGemmPD) {
#pragma unroll
      for (int k = 0; k < kGemmPD; ++k) step(c + k, k);
    }
#pragma unroll
    for (int k = 0; k < kGemmPD; ++k)
      if (c + k < nchunks) step(c + k, k);
  }

  // epilogue: the lane holds n = col0 + w 16 + 4 g + r, m = m0 + mt 16 + r16. With the
  // x-projection epilogue the u values of this workgroup (all in the conv range, as conv_D is a
  // multiple of 128) are also parked in LDS as a [ROWS][kGemmXS] bf16 tile (the X buffers are free
  // after the last chunk's barrier); rows past M are left as they are and only feed rows that are
  // never stored.
  __bf16* ut = xs0;
  const int64_t n = col0 + w * 16 + 4 * g;
  if (n < p.Nout) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m0 + mt * 16 + r16;
      if (m >= p.M) continue;
      float4 sv = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
      if (p.S > 1) {
        *reinterpret_cast<float4*>(p.partial + (ks * p.M + m) * p.Nout + n) = sv;
      } else if (p.conv_state && n < p.conv_D) {
        float4 uv;
        if constexpr (kRegEarly) {
          uv = p.conv_W == 4 ? conv_silu4(p, m, n, sv, rg[mt][0], rg[mt][1], cwq, &cbq)
                             : conv_silu4(p, m, n, sv, rg[mt][0], rg[mt][1]);
        } else {
          if (p.conv_W == 4) reg_words(mt, rg[0][0], rg[0][1]);
          uv = conv_silu4(p, m, n, sv, rg[0][0], rg[0][1]);
        }
        if (xp_on)
          *reinterpret_cast<uint2*>(&ut[(mt * 16 + r16) * kGemmXS + w * 16 + 4 * g]) = pack4(uv.x, uv.y, uv.z, uv.w);
      } else {
        if (p.residual) {
          const uint2 rr = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p.residual) + m * p.ldy + n);
          sv.x += bf16_lo(rr.x); sv.y += bf16_hi(rr.x); sv.z += bf16_lo(rr.y); sv.w += bf16_hi(rr.y);
        }
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.y) + m * p.ldy + n) = pack4(sv.x, sv.y, sv.z, sv.w);
      }
    }
  }

  // x-projection partial of this 128-channel slice: D[r][m] = sum_k W_xp[r][col0 + k] u[m][k]
  // (A = W_xp rows, rows past xp_n repeating the last; B = u rows from LDS), wave w taking the
  // output fragments w, w + 8, ... of the (xp_n / 16) x MT grid: the first kXpF with the W_xp
  // fragments loaded at the start, any further ones (xp_n > 192) loading theirs here
  if constexpr (MT <= 2) {
    if (xp_on) {   // uniform per workgroup
      __syncthreads();
      const int64_t slice = col0 / 128;
      const int nf = xp_rt * MT;
      auto frag = [&](int f, const bf16x8 (&a)[4]) __attribute__((always_inline)) {
        const int rt = f / MT, mt = f % MT;
        bf16x8 b[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          b[s2] = *reinterpret_cast<const bf16x8*>(&ut[(mt * 16 + r16) * kGemmXS + 32 * s2 + 8 * g]);
        f32x4 acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc4 = mfma16(a[s2], b[s2], acc4);
        const int64_t ro = 16 * rt + 4 * g, m = m0 + mt * 16 + r16;
        if (ro < p.xp_n && m < p.M)
          *reinterpret_cast<float4*>(p.xp_partial + (slice * p.M + m) * p.xp_n + ro) =
              make_float4(acc4[0], acc4[1], acc4[2], acc4[3]);
      };
#pragma unroll
      for (int i = 0; i < kXpF; ++i)
        if (w + 8 * i < nf) frag(w + 8 * i, xpa[i]);   // uniform per wave
      for (int f = w + 8 * kXpF; f < nf; f += 8) {
        const bf16_t* wxr = static_cast<const bf16_t*>(p.xp_w) +
                            std::min<int64_t>(16 * (f / MT) + r16, p.xp_n - 1) * p.conv_D + col0 + 8 * g;
        bf16x8 a[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) a[s2] = *reinterpret_cast<const bf16x8*>(wxr + 32 * s2);
        frag(f, a);
      }
    }
  }
}

// gemm_res_kernel (resident): grid (column blocks, S), 8 waves. A workgroup owns NC * CT * 16
// output columns, every row (MT tiles) and the K slice blockIdx.y of length KR = KH * KW. Its X
// slice is loaded into LDS once; wave w = (cg, kh) = (w % NC, w / NC) owns
// CT column tiles of the column group cg and the KW-long part kh of the slice, and issues all of its
// weight loads (CT * KW / 2 bytes per lane) right after the X loads, before the first product: the
// workgroup's whole weight slice is in flight at once and no barrier interrupts the stream. Each X
// fragment read from LDS feeds CT products. The KH part sums of each output fragment are added
// through LDS in the order kh = 0, 1, ..., so the sum over K has a fixed order.
template <int MT, int CT, int KH, int KW>
struct ResShape {
  static constexpr int NC = 8 / KH, KR = KH * KW, ROWS = MT * 16, XS = KR + 8, KSTEPS = KW / 32;
  static constexpr int COLS = NC * CT * 16;
  static constexpr int X_BYTES = ROWS * XS * 2;                      // row stride KR + 8: conflict-free reads
  static constexpr int RED_BYTES = KH > 1 ? KH * NC * CT * MT * 64 * 16 : 0;
  static constexpr int LDS = X_BYTES > RED_BYTES ? X_BYTES : RED_BYTES;
};

template <int MT, int CT, int KH, int KW>
__global__ __launch_bounds__(512) void gemm_res_kernel(GemmParams p) {
  using SH = ResShape<MT, CT, KH, KW>;
  constexpr int NC = SH::NC, KR = SH::KR, ROWS = SH::ROWS, XS = SH::XS, KSTEPS = SH::KSTEPS;
  static_assert(8 % KH == 0 && KW % 32 == 0 && CT * KW <= 512 && SH::LDS <= 160 * 1024, "resident GEMM shape");
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::LDS];
  __bf16* xs = reinterpret_cast<__bf16*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = w % NC, kh = w / NC;
  const int64_t col0 = (int64_t)blockIdx.x * SH::COLS + cg * CT * 16;
  const int64_t ks = blockIdx.y;
  const int64_t kbeg = ks * KR;
  const bf16_t* W = static_cast<const bf16_t*>(p.w);
  const bf16_t* X = static_cast<const bf16_t*>(p.x);

  // Every load is unconditional (a branch around a load makes the compiler wait for all loads in
  // flight at the join): X rows past M read row M - 1 and W rows past Nout read row Nout - 1; they
  // only feed outputs that are never stored. Threads past the last X piece repeat it.
  // The X slice: 16-byte pieces, row e / (KR / 8), 8-element column group e % (KR / 8).
  constexpr int PPR = KR / 8, XPIECES = ROWS * PPR, XPER = (XPIECES + 511) / 512;
  uint4 xr[XPER];
#pragma unroll
  for (int k = 0; k < XPER; ++k) {
    const int e = std::min(tid + 512 * k, XPIECES - 1);
    const int64_t m = std::min<int64_t>(e / PPR, p.M - 1);
    xr[k] = *reinterpret_cast<const uint4*>(X + m * p.ldx + kbeg + (e % PPR) * 8);
  }
  // this wave's weights: row n = col0 + 16 ct + r16, k = kh KW + 32 s + 8 g
  bf16x8 wr[CT][KSTEPS];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int64_t n = std::min<int64_t>(col0 + ct * 16 + r16, p.Nout - 1);
    const bf16_t* wrow = W + n * p.K + kbeg + kh * KW + 8 * g;
#pragma unroll
    for (int s2 = 0; s2 < KSTEPS; ++s2) wr[ct][s2] = *reinterpret_cast<const bf16x8*>(wrow + s2 * 32);
  }
#pragma unroll
  for (int k = 0; k < XPER; ++k) {
    const int e = std::min(tid + 512 * k, XPIECES - 1);
    *reinterpret_cast<uint4*>(&xs[(e / PPR) * XS + (e % PPR) * 8]) = xr[k];
  }
  __syncthreads();

  f32x4 acc[CT][MT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < KSTEPS; ++s2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 xf = *reinterpret_cast<const bf16x8*>(&xs[(mt * 16 + r16) * XS + kh * KW + s2 * 32 + 8 * g]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct][mt] = mfma16(wr[ct][s2], xf, acc[ct][mt]);
    }
  }

  // epilogue for one 16 x 16 output fragment: the lane holds n = c0 + 4 g + r (r = 0..3), m = 16 mt + r16
  auto store = [&](int64_t c0, int mt, f32x4 v) __attribute__((always_inline)) {
    const int64_t n = c0 + 4 * g, m = mt * 16 + r16;
    if (n >= p.Nout || m >= p.M) return;
    float4 sv = make_float4(v[0], v[1], v[2], v[3]);
    if (p.S > 1) {
      *reinterpret_cast<float4*>(p.partial + (ks * p.M + m) * p.Nout + n) = sv;
    } else {
      if (p.residual) {
        const uint2 rr = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p.residual) + m * p.ldy + n);
        sv.x += bf16_lo(rr.x); sv.y += bf16_hi(rr.x); sv.z += bf16_lo(rr.y); sv.w += bf16_hi(rr.y);
      }
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.y) + m * p.ldy + n) = pack4(sv.x, sv.y, sv.z, sv.w);
    }
  };
  if constexpr (KH == 1) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store(col0 + ct * 16, mt, acc[ct][mt]);
  } else {
    // every wave parks its part sums in LDS (the X slice is no longer read), then the NC * CT * MT
    // fragments are shared out over the 8 waves, each adding the KH parts of its fragments in order
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(((kh * NC + cg) * CT + ct) * MT + mt) * 64 + lane] = acc[ct][mt];
    __syncthreads();
    constexpr int F = NC * CT * MT;
#pragma unroll 1
    for (int f = w; f < F; f += 8) {
      const int fcg = f / (CT * MT), fct = (f / MT) % CT, fmt = f % MT;
      f32x4 v = red[((fcg * CT + fct) * MT + fmt) * 64 + lane];
#pragma unroll
      for (int part = 1; part < KH; ++part) v += red[(((part * NC + fcg) * CT + fct) * MT + fmt) * 64 + lane];
      store((int64_t)blockIdx.x * SH::COLS + (fcg * CT + fct) * 16, fmt, v);
    }
  }
}

// Y = sum over the S partials in order (+ R), four outputs per thread. A thread issues its
// residual and eight partials before any arithmetic (without a residual it reads a valid
// stand-in and drops it; partials past S are masked by value), so no load sits behind a branch.
// KB partials are loaded per batch before they are added (8, or 32 for long split lists such as
// the x projection's 32 slices, which would otherwise take 4 round trips).
template <int KB>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmParams p) {
  const int64_t total = p.M * (p.Nout / 4);
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t m = e / (p.Nout / 4), n = (e % (p.Nout / 4)) * 4;
    const float* src = p.partial + m * p.Nout + n;
    const int64_t stride = p.M * p.Nout;
    const bf16_t* rsrc = p.residual ? static_cast<const bf16_t*>(p.residual) + m * p.ldy + n
                                    : reinterpret_cast<const bf16_t*>(src);
    const uint2 rr = *reinterpret_cast<const uint2*>(rsrc);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t k0 = 0; k0 < p.S; k0 += KB) {
      float4 t[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) t[k] = *reinterpret_cast<const float4*>(src + std::min<int64_t>(k0 + k, p.S - 1) * stride);
      __builtin_amdgcn_sched_barrier(0);   // all KB loads leave before the first add waits
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const bool in = k0 + k < p.S;   // a select on the values, not a branch
        s.x += in ? t[k].x : 0.f; s.y += in ? t[k].y : 0.f; s.z += in ? t[k].z : 0.f; s.w += in ? t[k].w : 0.f;
      }
    }
    if (p.residual) {
      s.x += bf16_lo(rr.x); s.y += bf16_hi(rr.x); s.z += bf16_lo(rr.y); s.w += bf16_hi(rr.y);
    }
    *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.y) + m * p.ldy + n) = pack4(s.x, s.y, s.z, s.w);
  }
}

// ---------------------------------------------------------------------------- Delta + state update
// The block's SSM step with the Delta projection folded in. Grid (Di / 16, ceil(B / 32)), 4 waves:
// a workgroup owns channels d0 .. d0 + 15 and batch rows b0 .. b0 + 31. Thread (b_off, c, q)
// owns states 4q .. 4q + 3 of channel d0 + c for the rows b0 + b_off + BPP j, j < U (for one row
// the 16 channels' states are 16 N contiguous floats, covered by consecutive threads). Waves 0
// and 1 compute the pre-activation of Delta for the 16 channels and rows b0 + 16 w .. b0 + 16 w +
// 15 as one MFMA tile per 32-wide step of the rank (A = rows of W_dt, B = rows of the rank slice
// of xp), add the bias, apply the softplus and park Delta in LDS. Every thread issues the Delta
// operands (the first 128 of the rank) first, then all of its state, B, C, u and gate loads, so
// the Delta products wait only for their own operands and overlap the state loads. Rows past B
// repeat row B - 1 and store nothing. The state update is the decode kernel's arithmetic.
struct BlockSsmParams {
  int64_t B, Di, R, XP, z_stride;
  const bf16_t* u;      // [B, Di]
  const bf16_t* xp;     // [B, XP]: Delta rank part [0, R), B [R, R + N), C [R + N, R + 2N)
  const bf16_t* z;      // gate, row stride z_stride
  const bf16_t* W_dt;   // [Di, R]
  const float* b_dt;    // [Di]
  const float* A;       // [Di, N]
  const float* Dskip;   // [Di] or NULL
  float* h;             // [B, Di, N], in place
  bf16_t* y;            // [B, Di]
};

template <int N>
__global__ __launch_bounds__(256) void block_ssm_kernel(BlockSsmParams p) {
  constexpr int LPC = N / 4;          // lanes per channel, 4 states each
  constexpr int BPP = 16 / LPC;       // batch rows per pass of the 256 threads
  constexpr int U = 32 / BPP;         // passes per workgroup (32 rows)
  constexpr int DS = 17;              // LDS row stride of Delta (floats)
  __shared__ float dts[32 * DS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int64_t d0 = (int64_t)blockIdx.x * 16, b0 = (int64_t)blockIdx.y * 32;
  const int q = tid % LPC, c = (tid / LPC) % 16, boff = tid / (16 * LPC);
  const int64_t d = d0 + c;
  const int n0 = 4 * q;

  // the first 128 of the rank for the Delta tile, issued before the state loads so that the
  // Delta products wait only for these (loads complete in issue order); every wave loads them
  // (waves 2 and 3 for the tiles of waves 0 and 1) so the loads sit behind no branch
  const int dw = w & 1;
  const bf16_t* wrow = p.W_dt + (d0 + r16) * p.R + 8 * g;
  const bf16_t* xrow = p.xp + std::min<int64_t>(b0 + 16 * dw + r16, p.B - 1) * p.XP + 8 * g;
  bf16x8 da[4], db[4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    da[s2] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s2);
    db[s2] = *reinterpret_cast<const bf16x8*>(xrow + 32 * s2);
  }

  float4 hv[U];
  uint2 bv[U], cv[U];
  float uv[U], zv[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t b = std::min<int64_t>(b0 + boff + BPP * j, p.B - 1);
    hv[j] = *reinterpret_cast<const float4*>(p.h + (b * p.Di + d) * N + n0);
    bv[j] = *reinterpret_cast<const uint2*>(p.xp + b * p.XP + p.R + n0);
    cv[j] = *reinterpret_cast<const uint2*>(p.xp + b * p.XP + p.R + N + n0);
    uv[j] = bf16_to_f32(p.u[b * p.Di + d].bits);
    zv[j] = bf16_to_f32(p.z[b * p.z_stride + d].bits);
  }
  const float4 Av = *reinterpret_cast<const float4*>(p.A + d * N + n0);
  const float dsk = p.Dskip ? p.Dskip[d] : 0.f;

  if (w < 2) {   // wave-uniform
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) acc = mfma16(da[s2], db[s2], acc);
    for (int64_t k = 128; k < p.R; k += 128) {   // ranks past 128
      bf16x8 a[4], b[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        a[s2] = *reinterpret_cast<const bf16x8*>(wrow + k + 32 * s2);
        b[s2] = *reinterpret_cast<const bf16x8*>(xrow + k + 32 * s2);
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc = mfma16(a[s2], b[s2], acc);
    }
    // the lane holds channels 4 g .. 4 g + 3 of row b0 + 16 w + r16
#pragma unroll
    for (int i = 0; i < 4; ++i) dts[(16 * w + r16) * DS + 4 * g + i] = softplus_f32(acc[i] + p.b_dt[d0 + 4 * g + i]);
  }
  const float a2[4] = {Av.x * kLog2e, Av.y * kLog2e, Av.z * kLog2e, Av.w * kLog2e};
  const float ia[4] = {1.0f / Av.x, 1.0f / Av.y, 1.0f / Av.z, 1.0f / Av.w};
  __syncthreads();

#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t b = b0 + boff + BPP * j;
    const bool live = b < p.B;
    const float dt = dts[(boff + BPP * j) * DS + c];
    const float Bq[4] = {bf16_lo(bv[j].x), bf16_hi(bv[j].x), bf16_lo(bv[j].y), bf16_hi(bv[j].y)};
    const float Cq[4] = {bf16_lo(cv[j].x), bf16_hi(cv[j].x), bf16_lo(cv[j].y), bf16_hi(cv[j].y)};
    float hq[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w};
    float yv = 0.f;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float abar = exp2_fast(dt * a2[n]);
      const float coef = fmaf(abar, ia[n], -ia[n]);
      hq[n] = fmaf(abar, hq[n], coef * (Bq[n] * uv[j]));
      yv = fmaf(Cq[n], hq[n], yv);
    }
    if (live) *reinterpret_cast<float4*>(p.h + (b * p.Di + d) * N + n0) = make_float4(hq[0], hq[1], hq[2], hq[3]);
    yv = sum_channel_lanes<LPC>(yv);
    if (q == 0 && live) {
      yv = fmaf(dsk, uv[j], yv);
      yv *= silu(zv[j]);
      p.y[b * p.Di + d].bits = f32_to_bf16(yv);
    }
  }
}

}  // namespace

// Configurations of gemm_res_kernel: (CT, KH, KW) -> NC * CT * 16 columns, a K slice of KH * KW.
struct ResCfg {
  int ct, kh, kw;
};
constexpr ResCfg kResCfgs[] = {{2, 2, 256}, {2, 4, 128}, {2, 8, 64}, {2, 4, 32}, {1, 4, 32}};

static int row_tiles(int64_t M) {
  int mt = 1;
  while (mt * 16 < M) mt *= 2;  // 1, 2, 4, 8
  return mt;
}

// Plan of a product (M <= 128 rows, all in one row block). When the 128-column blocks alone
// number 256 or more (the LM head), the chunked kernel streams the activations with no split of
// K: split partials would cost as much traffic as the weights. Otherwise the resident kernel,
// with K slices of 512 where K allows (else 128) and the widest column block whose grid still
// reaches 256 workgroups (else the narrowest). Measured at 128 rows (kernel + reduction, weights
// rotated through more than the last-level cache): 2048 -> 8192 20.7 us (chunked, rows in 4
// blocks: 22.5), 4096 -> 2048 15.3 us (17.4), 4096 -> 160 8.6 us (10.1), 128 -> 4096 4.3 us
// (4.7), 2048 -> 50288 chunked 74 us (resident with K in 4: 111).
GemmChoice gemm_plan(int64_t M, int64_t K, int64_t Nout) {
  const int mt = row_tiles(M);
  // the column blocks alone fill the GPU: stream the activations, no split of K
  if ((Nout + 16 * kGemmNW - 1) / (16 * kGemmNW) >= 256) return GemmChoice{0, mt, 0, 1};
  const int order512[] = {0, 1, 2}, order128[] = {3, 4};
  const bool k512 = K % 512 == 0;
  const int* order = k512 ? order512 : order128;
  const int n = k512 ? 3 : 2;
  int i = 0;
  for (; i < n - 1; ++i) {
    const ResCfg& c = kResCfgs[order[i]];
    const int64_t cols = (8 / c.kh) * c.ct * 16;
    if ((Nout + cols - 1) / cols * (K / (c.kh * c.kw)) >= 256) break;
  }
  const ResCfg& c = kResCfgs[order[i]];
  return GemmChoice{1, mt, order[i], K / (c.kh * c.kw)};
}

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t Nout) {
  const GemmChoice c = gemm_plan(M, K, Nout);
  return c.S > 1 ? (size_t)(c.S * M * Nout) * 4 : 0;
}

template <int MT, int CT, int KH, int KW>
static void launch_res(const GemmParams& p, hipStream_t stream) {
  constexpr int COLS = ResShape<MT, CT, KH, KW>::COLS;
  const dim3 grid((unsigned)((p.Nout + COLS - 1) / COLS), (unsigned)p.S);
  hipLaunchKernelGGL((gemm_res_kernel<MT, CT, KH, KW>), grid, dim3(512), 0, stream, p);
}

template <int CT, int KH, int KW>
static void launch_res_mt(const GemmParams& p, int mt, hipStream_t stream) {
  switch (mt) {
    case 1: launch_res<1, CT, KH, KW>(p, stream); break;
    case 2: launch_res<2, CT, KH, KW>(p, stream); break;
    case 4: launch_res<4, CT, KH, KW>(p, stream); break;
    default: launch_res<8, CT, KH, KW>(p, stream); break;
  }
}

static void launch_reduce(const GemmParams& p, hipStream_t stream) {
  const int64_t total = p.M * (p.Nout / 4);
  const dim3 grid((unsigned)std::min<int64_t>((total + 255) / 256, 4096));
  if (p.S > 8) hipLaunchKernelGGL(gemm_reduce_kernel<32>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(gemm_reduce_kernel<8>, grid, dim3(256), 0, stream, p);
}

// The chunked kernel with the row block's X slice resident in LDS (kind 2): its dynamic LDS limit
// is raised once per process to what a workgroup may hold.
constexpr size_t kXresMaxLds = 160 * 1024 - 1024;
size_t gemm_xres_lds_bytes(int mt, int64_t kslice) { return (size_t)mt * 16 * (size_t)(kslice + 8) * 2; }
bool gemm_xres_fits(int mt, int64_t kslice) {
  return mt <= 2 && kslice % 512 == 0 && gemm_xres_lds_bytes(mt, kslice) <= kXresMaxLds;
}
template <int MT>
static hipError_t launch_xres(const GemmParams& p, dim3 grid, dim3 block, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_xwt_kernel<MT, true>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXresMaxLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_xwt_kernel<MT, true>), grid, block, gemm_xres_lds_bytes(MT, p.kslice), stream, p);
  return hipSuccess;
}

hipError_t launch_gemm_with(GemmParams p, const GemmChoice& c, hipStream_t stream) {
  p.S = c.S;
  p.kslice = p.K / p.S;
  if (c.kind == 2) {
    if (!gemm_xres_fits(c.mt, p.kslice)) return hipErrorInvalidValue;
    const int64_t blocks = (p.M + c.mt * 16 - 1) / (c.mt * 16);
    const dim3 grid((unsigned)((p.Nout + 16 * kGemmNW - 1) / (16 * kGemmNW)), (unsigned)blocks, (unsigned)p.S);
    const dim3 block(64 * kGemmNW);
    const hipError_t e = c.mt == 1 ? launch_xres<1>(p, grid, block, stream) : launch_xres<2>(p, grid, block, stream);
    if (e != hipSuccess) return e;
  } else if (c.kind == 0) {
    const int64_t blocks = (p.M + c.mt * 16 - 1) / (c.mt * 16);
    const dim3 grid((unsigned)((p.Nout + 16 * kGemmNW - 1) / (16 * kGemmNW)), (unsigned)blocks, (unsigned)p.S);
    const dim3 block(64 * kGemmNW);
    switch (c.mt) {
      case 1: hipLaunchKernelGGL(gemm_xwt_kernel<1>, grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL(gemm_xwt_kernel<2>, grid, block, 0, stream, p); break;
      case 4: hipLaunchKernelGGL(gemm_xwt_kernel<4>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(gemm_xwt_kernel<8>, grid, block, 0, stream, p); break;
    }
  } else {
    switch (c.cfg) {
      case 0: launch_res_mt<2, 2, 256>(p, c.mt, stream); break;
      case 1: launch_res_mt<2, 4, 128>(p, c.mt, stream); break;
      case 2: launch_res_mt<2, 8, 64>(p, c.mt, stream); break;
      case 3: launch_res_mt<2, 4, 32>(p, c.mt, stream); break;
      default: launch_res_mt<1, 4, 32>(p, c.mt, stream); break;
    }
  }
  if (p.S > 1) {
    launch_reduce(p, stream);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(GemmParams p, hipStream_t stream) {
  return launch_gemm_with(p, gemm_plan(p.M, p.K, p.Nout), stream);
}

hipError_t launch_layernorm(int64_t M, int64_t D, const void* x, const float* w, const float* b, float eps, void* y,
                            hipStream_t stream) {
  hipLaunchKernelGGL(layernorm_kernel, dim3((unsigned)M), dim3(256), 0, stream, D, static_cast<const bf16_t*>(x), w,
                     b, eps, static_cast<bf16_t*>(y));
  return hipGetLastError();
}

// Workspace of one block step: xn [B, Dm], xz [B, 2 Di] (SSM branch and gate), u, y [B, Di],
// xp [B, R + 2 N] (Delta rank part, B, C) (bf16, each 256-byte aligned) and the largest product's
// partial sums.
static size_t blk_align(size_t n) { return (n + 255) & ~(size_t)255; }

size_t block_workspace_bytes(int64_t B, int64_t Dm, int64_t Di, int64_t N, int64_t R) {
  const size_t acts = blk_align(B * Dm * 2) + blk_align(B * 2 * Di * 2) + 2 * blk_align(B * Di * 2) +
                      blk_align(B * (R + 2 * N) * 2);
  // the input projection runs with K whole; its x-projection epilogue leaves one partial per
  // 128-channel slice; the output projection splits K
  size_t part = (size_t)(Di / 128) * B * (R + 2 * N) * 4;
  part = std::max(part, gemm_workspace_bytes(B, Di, Dm));
  return acts + blk_align(part);
}

hipError_t launch_block_step(const BlockParams& bp, void* ws, hipStream_t st) {
  const int64_t B = bp.B, Dm = bp.Dm, Di = bp.Di, N = bp.N, R = bp.R, XP = R + 2 * N;
  char* base = static_cast<char*>(ws);
  auto take = [&](size_t n) { void* q = base; base += blk_align(n); return q; };
  bf16_t* xn = static_cast<bf16_t*>(take(B * Dm * 2));
  bf16_t* xz = static_cast<bf16_t*>(take(B * 2 * Di * 2));
  bf16_t* u = static_cast<bf16_t*>(take(B * Di * 2));
  bf16_t* y = static_cast<bf16_t*>(take(B * Di * 2));
  bf16_t* xp = static_cast<bf16_t*>(take(B * XP * 2));
  float* partial = reinterpret_cast<float*>(base);
  auto gemm = [&](const void* x, int64_t ldx, int64_t K, const void* w, int64_t Nout, void* out, const void* res) {
    GemmParams g{};
    g.M = B; g.K = K; g.Nout = Nout; g.x = x; g.ldx = ldx; g.w = w; g.y = out; g.ldy = Nout; g.residual = res;
    g.partial = partial;
    return launch_gemm(g, st);
  };
  hipError_t e = launch_layernorm(B, Dm, bp.hidden, bp.ln_w, bp.ln_b, bp.eps, xn, st);
  // [x | z] with conv + SiLU applied to the x half in the product's epilogue (the chunked kernel
  // with K whole, rows in blocks of 32), which also multiplies each 128-channel slice of u by the
  // matching columns of W_xp
  if (e == hipSuccess) {
    GemmParams g{};
    g.M = B; g.K = Dm; g.Nout = 2 * Di; g.x = xn; g.ldx = Dm; g.w = bp.W_in; g.y = xz; g.ldy = 2 * Di;
    g.conv_state = bp.conv_state; g.conv_w = bp.conv_w; g.conv_b = bp.conv_b; g.u = u;
    g.conv_D = Di; g.conv_W = bp.W;
    g.xp_w = bp.W_xp; g.xp_n = XP; g.xp_partial = partial;   // [Delta rank | B | C] per 128-channel slice
    // (the X slice resident in LDS where a 32-row block of it fits)
    const int mt = std::min(row_tiles(B), 2);
    e = launch_gemm_with(g, GemmChoice{gemm_xres_fits(mt, Dm) ? 2 : 0, mt, 0, 1}, st);
  }
  if (e == hipSuccess) {   // xp = the sum of the Di / 128 slice partials
    GemmParams r{};
    r.M = B; r.Nout = XP; r.S = Di / 128; r.partial = partial; r.y = xp; r.ldy = XP;
    launch_reduce(r, st);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    BlockSsmParams sp{};
    sp.B = B; sp.Di = Di; sp.R = R; sp.XP = XP; sp.z_stride = 2 * Di;
    sp.u = u; sp.xp = xp; sp.z = xz + Di; sp.W_dt = static_cast<const bf16_t*>(bp.W_dt); sp.b_dt = bp.b_dt;
    sp.A = bp.A; sp.Dskip = bp.Dskip; sp.h = bp.h; sp.y = y;
    const dim3 grid((unsigned)(Di / 16), (unsigned)((B + 31) / 32));
    switch (N) {
      case 4: hipLaunchKernelGGL(block_ssm_kernel<4>, grid, dim3(256), 0, st, sp); break;
      case 8: hipLaunchKernelGGL(block_ssm_kernel<8>, grid, dim3(256), 0, st, sp); break;
      default: hipLaunchKernelGGL(block_ssm_kernel<16>, grid, dim3(256), 0, st, sp); break;
    }
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = gemm(y, Di, Di, bp.W_out, Dm, bp.hidden, bp.hidden);
  return e;
}

}  // namespace ssm
