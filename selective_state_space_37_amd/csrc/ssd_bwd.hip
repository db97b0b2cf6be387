// Gradients of the Mamba-2 (SSD) layer on gfx950: MFMA for every contraction inside a chunk.
//
// Page "Mamba and state space models", section "Mamba-2: two algorithms": the layer is a
// lower-triangular matrix applied chunk by chunk, and only the state passes between chunks. The
// backward keeps that split. Per chunk of Q = 64 tokens, with S the inclusive cumulative sum of
// Delta in the chunk, phi_j = expm1(a Delta_j) / a, ybar = dy times the gate factor z sigmoid(z),
// H_c the state entering the chunk and Gc the adjoint of the state leaving it:
//   h_t     = exp(a S_t) H_c + sum_{j<=t} exp(a (S_t - S_j)) phi_j x_j B_j^T
//   dL/dh_t = exp(a (S_Q - S_t)) Gc + sum_{i>=t} exp(a (S_i - S_t)) ybar_i C_i^T
// Both are needed only through contractions, never per token:
//   U_ij  = ybar_i . x_j,  W_ij = exp(a (S_i - S_j)) phi_j U_ij (i >= j),  K_ij = (C_i . B_j) W_ij
//   dC_i  = sum_j W_ij B_j + exp(a S_i) H_c^T ybar_i                   (summed over the group)
//   dB_j  = sum_i W_ij C_i + exp(a (S_Q - S_j)) phi_j Gc^T x_j
//   w_j   = sum_{i>=j} (C_i . B_j) exp(a (S_i - S_j)) ybar_i + exp(a (S_Q - S_j)) Gc B_j
//   dx_j  = phi_j w_j + D ybar_j
//   dDelta_t = a <dL/dh_t, h_t> + x_t . w_t     (derivative of exp(a Delta) and phi together)
//   <dL/dh_t, h_t> = exp(a S_Q) <Gc, H_c> + sum_{i>=t} ybar_i . Yoff_i
//                    + sum_{j<=t} phi_j x_j . (exp(a (S_Q - S_j)) Gc B_j) + sum_{j<=t<=i} K_ij
//   dA    = sum_t Delta_t <dL/dh_t, h_t> + (Delta_t - phi_t) / a  x_t . w_t
// with Yoff_i = exp(a S_i) H_c C_i (the carried-state part of y_i), and dz from the recomputed
// pre-gate output. The passes:
//   cumsum, prep (G = C B^T, B^T, C^T per chunk and group), the forward state
//   pass (H_c for every chunk, bf16), the adjoint state pass (Gc for every chunk, bf16, and dh0),
//   the main kernel below, and two reductions in a fixed order (dB and dC over heads, the
//   parameter gradients over batch rows and chunks).
#include <algorithm>

#include "ssd_device.h"

namespace ssm {
namespace {

constexpr int kQb = (int)kSsdBwdQ;
static_assert(kQb == 64, "the main kernel's wave layout assumes 64-token chunks");

__device__ __forceinline__ bf16x8 pack8(const float v[8]) {
  bf16x8 o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = (__bf16)v[q];
  return o;
}

__device__ __forceinline__ bf16x8 frag_from_pieces(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ void unpack8(uint4 v, float out[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = bf16_lo(w[k]);
    out[2 * k + 1] = bf16_hi(w[k]);
  }
}

// grid (H / hb, chunks, B), 512 threads. Token tile tt = w % 4 (tokens 16 tt .. 16 tt + 15 of the
// chunk) belongs to waves tt and tt + 4, which split the work by halves (hf = w / 4): of the
// states n for dB and dC, of the channels p for y, dz, dx. Each of the two computes the U tiles
// its products need itself (a few MFMAs) rather than passing them through LDS. A tile is used in
// both roles: as the rows i of dC, y and dz and as the columns j of dB, dx and w. The MFMA
// products are oriented so that the outputs come out with four consecutive states or channels
// per lane (one 8- or 16-byte store), and a product that feeds another (W) comes out in the
// operand layout of the next one: two 16-token tiles per K = 32 step, four tokens of each per
// lane, the same K order on both operands. dB and dC are summed over the workgroup's hb heads
// (consecutive heads of one group) in registers; B^T and C^T, shared by those heads, are staged
// in LDS once.
template <int N, bool GATE>
__global__ __launch_bounds__(512) void ssd_bwd_main_kernel(SsdBwdParams bp) {
  constexpr int Q = kQb;
  constexpr int NT = N / 16;   // 16-state tiles
  constexpr int NTH = NT / 2;  // per half
  constexpr int KSN = N / 32;  // K steps over the states
  constexpr int RS = Q + 8;    // row stride (bf16) of the token tiles
  constexpr int RSP = kP + 8;  // row stride (bf16) of the transposed states
  // row stride (float) of G: rows stay 16-byte aligned for float4 reads of a row, and a wave's
  // column reads (16 columns x 4 row groups) fall on 64 different banks
  constexpr int GST = Q + 4;
  __shared__ __attribute__((aligned(16))) __bf16 Xn[Q * RS];     // x [j][p]
  __shared__ __attribute__((aligned(16))) __bf16 Yhi[Q * RS];    // ybar [i][p], bf16 rounded
  // ybar - Yhi, bf16 rounded (with a gate; without one ybar = dy is exactly bf16)
  __shared__ __attribute__((aligned(16))) __bf16 Ylo[GATE ? Q * RS : 8];
  __shared__ __attribute__((aligned(16))) __bf16 YT[kP * RS];    // ybar^T [p][i]
  __shared__ __attribute__((aligned(16))) __bf16 XT[kP * RS];    // (phi x)^T [p][j] (gate only)
  __shared__ __attribute__((aligned(16))) __bf16 HT[N * RSP];    // H_c^T [n][p]
  __shared__ __attribute__((aligned(16))) __bf16 GcT[N * RSP];   // Gc^T [n][p]
  __shared__ __attribute__((aligned(16))) __bf16 BtS[N * RS];    // B^T [n][j] of the chunk (all heads)
  __shared__ __attribute__((aligned(16))) __bf16 CtS[N * RS];    // C^T [n][i]
  __shared__ __attribute__((aligned(16))) float GS[Q * GST];     // G [i][j], float32 (all heads)
  __shared__ float sS[Q], sPhi[Q];
  // the per-wave parts of <Gc, H_c>, by head parity: wave 0 reads those of head kh in the per-token
  // phase while the other waves may already stage head kh + 1
  __shared__ float sRed[2][8];
  __shared__ float sKr[Q], sKc[Q];   // row and column sums of K (see the dDelta phase)
  __shared__ float sQv[2][Q], sRv[2][Q], sVv[2][Q];
  __shared__ float sDD[4][kP];

  const SsdParams& p = bp.f;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the tile loops over it) in scalar registers, so branches on it are not divergent
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tt = w & 3, hf = w >> 2;
  const int64_t hblk = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  const int64_t L = p.L, H = p.H;
  const int64_t grp = hblk * bp.hb / (H / p.G);
  const int64_t bg = b * p.G + grp;
  const int64_t rs = p.G * N;   // token row stride of B and C
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm) + b * L * rs + grp * N;
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * L * rs + grp * N;
  // G = C B^T of the chunk, float32 (only tiles on / below the diagonal are written and read)
  const float* Gm = static_cast<const float*>(p.ws_G) + (bg * nch + c) * (int64_t)(Q * Q);
  const bf16_t* Btm = static_cast<const bf16_t*>(p.ws_Bt) + (bg * nch + c) * (int64_t)(N * Q);
  const bf16_t* Ctm = static_cast<const bf16_t*>(p.ws_Ct) + (bg * nch + c) * (int64_t)(N * Q);
  const int64_t tc0 = c * Q;      // first token of the chunk
  const int il = tt * 16 + r16;   // this lane's token in the chunk (column role)
  const int64_t tl = tc0 + il;
  const bool lane_valid = tl < L;
  const int64_t tstride = H * kP;  // token stride of x, dy, z

  // fragments of the staged tiles: token row t of the chunk, channels p0 .. p0 + 7. ybar is held
  // as hi + lo (hi = ybar rounded to bf16, lo = the rounding error rounded), so products with x
  // (exactly bf16) lose nothing to the operand rounding.
  auto x8 = [&](int t, int p0) { return *reinterpret_cast<const bf16x8*>(&Xn[t * RS + p0]); };
  auto yhi8 = [&](int t, int p0) { return *reinterpret_cast<const bf16x8*>(&Yhi[t * RS + p0]); };
  auto ylo8 = [&](int t, int p0) { return *reinterpret_cast<const bf16x8*>(&Ylo[t * RS + p0]); };

  f32x4 dC[NTH], dB[NTH];
#pragma unroll
  for (int k = 0; k < NTH; ++k) dC[k] = dB[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B^T, C^T and G of the chunk are the same for the workgroup's heads: staged once (visible
  // after the first head's staging barrier)
  for (int e = tid; e < Q * Q / 4; e += 512) {
    const int i = e / (Q / 4), j4 = (e % (Q / 4)) * 4;
    *reinterpret_cast<float4*>(&GS[i * GST + j4]) = *reinterpret_cast<const float4*>(Gm + i * Q + j4);
  }
  // G[i][j .. j + 3] (a row piece) and G[i .. i + 3][j] (a column piece, G^T[j][i .. i + 3])
  auto grow4 = [&](int i, int j) { return *reinterpret_cast<const float4*>(&GS[i * GST + j]); };
  auto gcol4 = [&](int i, int j) {
    return make_float4(GS[i * GST + j], GS[(i + 1) * GST + j], GS[(i + 2) * GST + j], GS[(i + 3) * GST + j]);
  };
  for (int e = tid; e < N * Q / 8; e += 512) {
    const int n = e / (Q / 8), j8 = (e % (Q / 8)) * 8;
    *reinterpret_cast<uint4*>(&BtS[n * RS + j8]) = *reinterpret_cast<const uint4*>(Btm + n * Q + j8);
    *reinterpret_cast<uint4*>(&CtS[n * RS + j8]) = *reinterpret_cast<const uint4*>(Ctm + n * Q + j8);
  }

  // Per-head global operands, loaded into registers one head ahead: the loads of head kh + 1 are
  // issued in the last phase of head kh (per-token sums, few live registers) and used at the
  // start of head kh + 1. Staging roles: threads 0..255 take x, threads 256..511 dy (and z);
  // item (token pair sip, channels 8 spg .. 8 spg + 7). Thread tid < 32 (N / 8) also takes the
  // H_c and Gc rows of channel pair hpp, states 8 hng .. 8 hng + 7. Every lane also takes the
  // operands of its Gc B_j product (the rows of Gc of this half's channel tiles and B_j of its
  // token, over the states), which is formed before the staging barrier.
  constexpr bool gate = GATE;   // z given (one instantiation each way)
  const int srole = w >> 2;   // wave-uniform
  constexpr int NHG = 32 * (N / 8);
  static_assert(NHG <= 512, "one H_c / Gc item per thread at most");
  uint4 pv[4];     // x pair (role 0), or dy pair and z pair (role 1)
  uint4 phg[4];    // H_c rows 2 hpp, 2 hpp + 1, then Gc rows 2 hpp, 2 hpp + 1
  float4 pphi;     // (S, phi) of tokens 2 sip, 2 sip + 1 (role 0, with a gate)
  float2 psp;      // (S, phi) of token tid (tid < Q)
  uint32_t pdl;    // Delta bits of token tid of the chunk (wave 0)
  bf16x8 pgc[2][KSN], pbj[KSN];
  // Addresses are a wave-uniform base (scalar registers) plus a 32-bit per-lane byte offset, and
  // the per-lane parts are formed from `tv`, the thread index passed through an empty asm in each
  // head: neither 64-bit per-lane pointers nor per-lane LDS addresses are then carried across
  // the head loop, where they would take registers from the products.
  // the operands of the Gc B_j product: one head ahead without a gate; with one (more live
  // registers in the gate's products) at the start of the head
  constexpr bool kEarlyGcB = !GATE;
  auto load_gcb = [&](int64_t kh, int tv) __attribute__((always_inline)) {
    const int lane = tv & 63, g = lane >> 4, r16 = lane & 15;
    const int64_t h = hblk * bp.hb + kh;
    const bf16_t* gs = static_cast<const bf16_t*>(p.ws_gout) + ((b * nch + c) * H + h) * (int64_t)(kP * N);
    const uint32_t foff = (uint32_t)(r16 * N + 8 * g) * 2u;
    const uint32_t boff = (uint32_t)(r16 * rs + 8 * g) * 2u;
    const bf16_t* bj0 = Bg + (tc0 + tt * 16) * rs;
    const bool valid = tc0 + tt * 16 + r16 < L;
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks) {
#pragma unroll
      for (int k = 0; k < 2; ++k) pgc[k][ks] = ld_at<bf16x8>(gs + (2 * hf + k) * 16 * N + 32 * ks, foff);
      pbj[ks] = valid ? ld_at<bf16x8>(bj0 + 32 * ks, boff) : zero_frag();
    }
  };
  auto prefetch = [&](int64_t kh, int tv) __attribute__((always_inline)) {
    const int lane = tv & 63, g = lane >> 4, r16 = lane & 15;
    const int sip = tv & 31, spg = (tv >> 5) & 7, hpp = tv & 31, hng = tv >> 5;
    const int64_t h = hblk * bp.hb + kh;
    const int64_t t = tc0 + 2 * sip;
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    const int64_t row0 = ((b * L + tc0) * H + h) * kP;   // element of (token tc0, head h, channel 0)
    const uint32_t toff = (uint32_t)((2 * sip) * tstride + 8 * spg) * 2u;
    const bf16_t* src = static_cast<const bf16_t*>(srole == 0 ? p.x : p.dy) + row0;
    pv[0] = t < L ? ld_at<uint4>(src, toff) : zero4;
    pv[1] = t + 1 < L ? ld_at<uint4>(src + tstride, toff) : zero4;
    const float2* sp = p.ws_sphi + ((b * nch + c) * H + h) * Q;
    if constexpr (gate) {
      if (srole == 1) {
        const bf16_t* zs = static_cast<const bf16_t*>(p.z) + row0;
        pv[2] = t < L ? ld_at<uint4>(zs, toff) : zero4;
        pv[3] = t + 1 < L ? ld_at<uint4>(zs + tstride, toff) : zero4;
      } else {
        pphi = ld_at<float4>(sp, (uint32_t)sip * 16u);
      }
    }
    const int64_t so = ((b * nch + c) * H + h) * (int64_t)(kP * N);
    const bf16_t* hs = static_cast<const bf16_t*>(p.ws_hin) + so;
    const bf16_t* gs = static_cast<const bf16_t*>(p.ws_gout) + so;
    if (tv < NHG) {
      const uint32_t hoff = (uint32_t)((2 * hpp) * N + 8 * hng) * 2u;
      phg[0] = ld_at<uint4>(hs, hoff);
      phg[1] = ld_at<uint4>(hs + N, hoff);
      phg[2] = ld_at<uint4>(gs, hoff);
      phg[3] = ld_at<uint4>(gs + N, hoff);
    }
    if (tv < Q) psp = ld_at<float2>(sp, (uint32_t)tv * 8u);
    if (w == 0) {
      const bf16_t* dl0 = static_cast<const bf16_t*>(p.delta) + (b * L + tc0) * H + h;
      // (an unconditional load of a row inside the sequence, then a select: a load under a branch
      // leaves the compiler unsure of the loads in flight, and it then waits for all of them)
      const int lr = (int)std::min<int64_t>(lane, L - 1 - tc0);
      pdl = ld_at<uint16_t>(dl0, (uint32_t)(lr * H) * 2u);   // rows past L: zeroed at use
    }
    if constexpr (kEarlyGcB) load_gcb(kh, tv);
  };
  prefetch(0, tid);

  for (int64_t kh = 0; kh < bp.hb; ++kh) {
    int tv = tid;
    asm volatile("" : "+v"(tv));
    const int lane = tv & 63, g = lane >> 4, r16 = lane & 15;
    const int il = tt * 16 + r16;
    const int64_t tl = tc0 + il;
    const bool lane_valid = tl < L;
    const int sip = tv & 31, spg = (tv >> 5) & 7, hpp = tv & 31, hng = tv >> 5;
    const bool has_hg = tv < NHG;
    const int64_t h = hblk * bp.hb + kh;
    const float a = p.A[h], a2 = a * kLog2e;
    // the step-size bias of the head, loaded here with the head's other scalars (a stand-in
    // address and a select when there is none: see the Delta bits in the prefetch)
    const float dbias_v = *(p.delta_bias ? p.delta_bias + h : p.A + h);
    const float dbias = p.delta_bias ? dbias_v : 0.f;
    // (first token of this wave's tile, head h, channel 0), and this lane's token and channel
    // group 4 g relative to it
    const int64_t trow = ((b * L + tc0 + tt * 16) * H + h) * kP;
    const uint32_t toff = (uint32_t)(r16 * tstride + 4 * g) * 2u;
    const bf16_t* hin = static_cast<const bf16_t*>(p.ws_hin) + ((b * nch + c) * H + h) * (int64_t)(kP * N);
    const bool dpc = p.Dskip && p.dskip_per_channel;
    const float dhead = p.Dskip && !p.dskip_per_channel ? p.Dskip[h] : 0.f;
    auto dskip = [&](int ch) { return dpc ? p.Dskip[h * kP + ch] : dhead; };
    if constexpr (!kEarlyGcB) load_gcb(kh, tv);
    // ------------------------------------------------------------------ staging
    float dot = 0.f;   // <Gc, H_c> over this thread's pieces
    if (srole == 0) {
      // x (natural), and (phi x)^T with a gate for the recomputed within-chunk output. Lanes
      // 0..31 of a wave write 32 consecutive words of a transposed row, lanes 32..63 the rows 8
      // further (288 words on): the 64 writes fall on 64 banks.
      *reinterpret_cast<uint4*>(&Xn[(2 * sip) * RS + 8 * spg]) = pv[0];
      *reinterpret_cast<uint4*>(&Xn[(2 * sip + 1) * RS + 8 * spg]) = pv[1];
      if constexpr (gate) {
        float xv0[8], xv1[8];
        unpack8(pv[0], xv0);
        unpack8(pv[1], xv1);
        uint32_t* X32 = reinterpret_cast<uint32_t*>(XT);
#pragma unroll
        for (int k = 0; k < 8; ++k) X32[(8 * spg + k) * (RS / 2) + sip] = pack_bf16x2(pphi.y * xv0[k], pphi.w * xv1[k]);
      }
    } else {
      // ybar (natural, as bf16 hi + lo) and ybar^T
      float y0[8], y1[8];
      unpack8(pv[0], y0);
      unpack8(pv[1], y1);
      if constexpr (gate) {
        float zv0[8], zv1[8];
        unpack8(pv[2], zv0);
        unpack8(pv[3], zv1);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          y0[k] *= silu(zv0[k]);
          y1[k] *= silu(zv1[k]);
        }
      }
      uint32_t* Y32 = reinterpret_cast<uint32_t*>(YT);
#pragma unroll
      for (int k = 0; k < 8; ++k) Y32[(8 * spg + k) * (RS / 2) + sip] = pack_bf16x2(y0[k], y1[k]);
      if constexpr (gate) {
        float h0[8], h1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          h0[k] = (float)(__bf16)y0[k];
          h1[k] = (float)(__bf16)y1[k];
          y0[k] -= h0[k];
          y1[k] -= h1[k];
        }
        *reinterpret_cast<bf16x8*>(&Yhi[(2 * sip) * RS + 8 * spg]) = pack8(h0);
        *reinterpret_cast<bf16x8*>(&Yhi[(2 * sip + 1) * RS + 8 * spg]) = pack8(h1);
        *reinterpret_cast<bf16x8*>(&Ylo[(2 * sip) * RS + 8 * spg]) = pack8(y0);
        *reinterpret_cast<bf16x8*>(&Ylo[(2 * sip + 1) * RS + 8 * spg]) = pack8(y1);
      } else {
        *reinterpret_cast<uint4*>(&Yhi[(2 * sip) * RS + 8 * spg]) = pv[0];
        *reinterpret_cast<uint4*>(&Yhi[(2 * sip + 1) * RS + 8 * spg]) = pv[1];
      }
    }
    if (has_hg) {
      // channels (2 hpp, 2 hpp + 1), states 8 hng .. 8 hng + 7 of H_c and Gc, written transposed
      float h0v[8], h1v[8], g0v[8], g1v[8];
      unpack8(phg[0], h0v);
      unpack8(phg[1], h1v);
      unpack8(phg[2], g0v);
      unpack8(phg[3], g1v);
      uint32_t* H32 = reinterpret_cast<uint32_t*>(HT);
      uint32_t* G32 = reinterpret_cast<uint32_t*>(GcT);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        H32[(8 * hng + k) * (RSP / 2) + hpp] = pack_bf16x2(h0v[k], h1v[k]);
        G32[(8 * hng + k) * (RSP / 2) + hpp] = pack_bf16x2(g0v[k], g1v[k]);
        dot += h0v[k] * g0v[k] + h1v[k] * g1v[k];
      }
    }
    if (tid < Q) {
      sS[tid] = psp.x;
      sPhi[tid] = psp.y;
    }
    const uint32_t dl = pdl;
    // vo[p][j] = sum_n Gc[p][n] B_j[n] (this half's channel tiles, own token j)
    f32x4 vo[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks)
#pragma unroll
      for (int k = 0; k < 2; ++k) vo[k] = mfma16(pgc[k][ks], pbj[ks], vo[k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) sRed[kh & 1][w] = dot;
    __syncthreads();

    const float Sq = sS[Q - 1];
    const float Sl = sS[il], phil = sPhi[il];   // this lane's token (column role)
    // this lane's token: ybar and x fragments over the 64 channels (two K steps)
    bf16x8 yb_own[2], yb_lo[2] = {zero_frag(), zero_frag()}, x_own[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      yb_own[kk] = yhi8(il, 32 * kk + 8 * g);
      if constexpr (gate) yb_lo[kk] = ylo8(il, 32 * kk + 8 * g);
      x_own[kk] = x8(il, 32 * kk + 8 * g);
    }

    // ------------------------------------------------------------------ dC (rows i = own tile)
    float qpart = 0.f;   // this lane's part of ybar_i . Yoff_i (token il, this half's states)
    // this lane's parts of the row sum (token il as row i) and the column sum (token il as
    // column j) of K_ij = (C_i . B_j) W_ij, kept by the first half
    float krow = 0.f, kcol = 0.f;
    {
      // U^T tiles (j tile jt <= tt, i = own): D[j][i] = sum_p x_j[p] ybar_i[p]; the lane holds
      // U[il][jt 16 + 4 g + r]. W (as the B operand of the next product) and the row sum of K.
      bf16x8 wmA[2] = {zero_frag(), zero_frag()};
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt > tt) continue;
        f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 xa = x8(jt * 16 + r16, 32 * kk + 8 * g);
          u = mfma16(xa, yb_own[kk], u);
          if constexpr (gate) u = mfma16(xa, yb_lo[kk], u);
        }
        const float4 g4 = grow4(il, jt * 16 + 4 * g);
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jt * 16 + 4 * g + r;
          const float wm = j <= il ? exp2_fast(a2 * (Sl - sS[j])) * sPhi[j] * u[r] : 0.f;
          krow += gv[r] * wm;
          wmA[jt >> 1][(jt & 1) * 4 + r] = (__bf16)wm;
        }
      }
      // ybar of the own token scaled by exp(a S_i) for the carried-state term
      const float eSi = exp2_fast(a2 * Sl);
      bf16x8 yb_sc[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int q = 0; q < 8; ++q) yb_sc[kk][q] = (__bf16)(((float)yb_own[kk][q] + (float)yb_lo[kk][q]) * eSi);
#pragma unroll
      for (int k = 0; k < NTH; ++k) {
        f32x4 acc = dC[k];
        const int n = (hf * NTH + k) * 16 + r16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (2 * kk > tt) break;   // the pair holds no tile j <= i
          const uint2 lo = *reinterpret_cast<const uint2*>(&BtS[n * RS + 32 * kk + 4 * g]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&BtS[n * RS + 32 * kk + 16 + 4 * g]);
          acc = mfma16(frag_from_pieces(lo, hi), wmA[kk], acc);   // D[n][i] = sum_j B_j[n] W_ij
        }
        // the carried-state part M[n][i] = exp(a S_i) sum_p H_c[p][n] ybar_i[p], kept apart
        // first: sum_n C_i[n] M[n][i] is ybar_i . Yoff_i (this lane: states
        // (hf NTH + k) 16 + 4 g + r of token il)
        f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          m = mfma16(*reinterpret_cast<const bf16x8*>(&HT[n * RSP + 32 * kk + 8 * g]), yb_sc[kk], m);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          qpart += (float)CtS[((hf * NTH + k) * 16 + 4 * g + r) * RS + il] * m[r];
          acc[r] += m[r];
        }
        dC[k] = acc;
      }
    }

    // ------------------------------------------------------------------ dB (columns j = own tile)
    // vin: this lane's part of x_j . sum_{i>=j} (C_i . B_j) exp(a (S_i - S_j)) ybar_i, formed in
    // float32 from U (the within-chunk part of x_j . w_j, for dDelta; kept by the first half)
    float vin = 0.f;
    {
      // U tiles (i tile it >= tt, j = own): D[i][j] = sum_p ybar_i[p] x_j[p]; the lane holds
      // U[it 16 + 4 g + r][il].
      bf16x8 wmB[2] = {zero_frag(), zero_frag()};
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (it < tt) continue;
        f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u = mfma16(yhi8(it * 16 + r16, 32 * kk + 8 * g), x_own[kk], u);
          if constexpr (gate) u = mfma16(ylo8(it * 16 + r16, 32 * kk + 8 * g), x_own[kk], u);
        }
        const float4 g4 = gcol4(it * 16 + 4 * g, il);   // G[i][il]
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = it * 16 + 4 * g + r;
          const float e = i >= il ? exp2_fast(a2 * (sS[i] - Sl)) : 0.f;
          vin += gv[r] * e * u[r];
          wmB[it >> 1][(it & 1) * 4 + r] = (__bf16)(e * phil * u[r]);
        }
      }
      if (hf != 0) vin = 0.f;
      kcol = vin * phil;   // sum_i K_ij = phi_j sum_i (C_i . B_j) exp(a (S_i - S_j)) U_ij
      const float eq = exp2_fast(a2 * (Sq - Sl)) * phil;
      bf16x8 x_sc[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int q = 0; q < 8; ++q) x_sc[kk][q] = (__bf16)((float)x_own[kk][q] * eq);
#pragma unroll
      for (int k = 0; k < NTH; ++k) {
        f32x4 acc = dB[k];
        const int n = (hf * NTH + k) * 16 + r16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (2 * kk + 1 < tt) continue;   // the pair holds no tile i >= j
          const uint2 lo = *reinterpret_cast<const uint2*>(&CtS[n * RS + 32 * kk + 4 * g]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&CtS[n * RS + 32 * kk + 16 + 4 * g]);
          acc = mfma16(frag_from_pieces(lo, hi), wmB[kk], acc);   // D[n][j] = sum_i C_i[n] W_ij
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          acc = mfma16(*reinterpret_cast<const bf16x8*>(&GcT[n * RSP + 32 * kk + 8 * g]), x_sc[kk], acc);
        dB[k] = acc;
      }
    }

    // ------------------------------------------------------------------ y (rows i = own tile)
    // With a gate, the pre-gate output per channel: Yoff[p][i] = exp(a S_i) sum_n H_c[p][n] C_i[n]
    // and the within-chunk part Ydiag[p][i] = sum_{j<=i} (C_i . B_j) exp(a (S_i - S_j)) phi_j x_j[p].
    // This half's channel tiles: pt = 2 hf, 2 hf + 1.
    f32x4 yo[2], yd[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) yo[k] = yd[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (gate) {
      const float eSi = exp2_fast(a2 * Sl);
#pragma unroll
      for (int ks = 0; ks < KSN; ++ks) {
        bf16x8 cf = lane_valid ? ld_at<bf16x8>(Cg + (tc0 + tt * 16) * rs + 32 * ks, (uint32_t)(r16 * rs + 8 * g) * 2u)
                               : zero_frag();
#pragma unroll
        for (int q = 0; q < 8; ++q) cf[q] = (__bf16)((float)cf[q] * eSi);
#pragma unroll
        for (int k = 0; k < 2; ++k)
          yo[k] = mfma16(ld_at<bf16x8>(hin + (2 * hf + k) * 16 * N + 32 * ks, (uint32_t)(r16 * N + 8 * g) * 2u), cf, yo[k]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (2 * kk > tt) break;
        float gl[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int jt = 2 * kk + half;
          if (jt <= tt) {
            const float4 g4 = grow4(il, jt * 16 + 4 * g);
            const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = jt * 16 + 4 * g + r;
              gl[half * 4 + r] = j <= il ? gv[r] * exp2_fast(a2 * (Sl - sS[j])) : 0.f;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) gl[half * 4 + r] = 0.f;
          }
        }
        const bf16x8 glf = pack8(gl);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int row = ((2 * hf + k) * 16 + r16) * RS;
          const uint2 lo = *reinterpret_cast<const uint2*>(&XT[row + 32 * kk + 4 * g]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&XT[row + 32 * kk + 16 + 4 * g]);
          yd[k] = mfma16(frag_from_pieces(lo, hi), glf, yd[k]);
        }
      }
    }
    // epilogue: the lane holds channels pt 16 + 4 g + r (pt = 2 hf + k) of token il
    float ybv[2][4], xv[2][4];
    {
      float dd[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pt = 2 * hf + k;
        const int lo = il * RS + pt * 16 + 4 * g;
        const uint2 xr = *reinterpret_cast<const uint2*>(&Xn[lo]);
        const uint2 yhr = *reinterpret_cast<const uint2*>(&Yhi[lo]);
        const uint2 ylr = gate ? *reinterpret_cast<const uint2*>(&Ylo[lo]) : make_uint2(0u, 0u);
        const float xx[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
        const float ybr[4] = {bf16_lo(yhr.x) + bf16_lo(ylr.x), bf16_hi(yhr.x) + bf16_hi(ylr.x),
                              bf16_lo(yhr.y) + bf16_lo(ylr.y), bf16_hi(yhr.y) + bf16_hi(ylr.y)};
        float dv[4] = {0.f, 0.f, 0.f, 0.f}, zv[4] = {0.f, 0.f, 0.f, 0.f};
        if (gate && lane_valid) {
          const uint2 dr = ld_at<uint2>(static_cast<const bf16_t*>(p.dy) + trow + pt * 16, toff);
          const uint2 zr = ld_at<uint2>(static_cast<const bf16_t*>(p.z) + trow + pt * 16, toff);
          dv[0] = bf16_lo(dr.x); dv[1] = bf16_hi(dr.x); dv[2] = bf16_lo(dr.y); dv[3] = bf16_hi(dr.y);
          zv[0] = bf16_lo(zr.x); zv[1] = bf16_hi(zr.x); zv[2] = bf16_lo(zr.y); zv[3] = bf16_hi(zr.y);
        }
        float dzv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ch = pt * 16 + 4 * g + r;
          xv[k][r] = xx[r];
          const float yb = ybr[r];
          ybv[k][r] = yb;
          dd[k][r] = yb * xx[r];
          if constexpr (gate) {
            const float ypre = yo[k][r] + yd[k][r] + dskip(ch) * xx[r];
            const float sg = sigmoid_fast(zv[r]);
            dzv[r] = dv[r] * ypre * sg * (1.f + zv[r] * (1.f - sg));
          }
        }
        if (gate && lane_valid) {
          uint2 out;
          out.x = pack_bf16x2(dzv[0], dzv[1]);
          out.y = pack_bf16x2(dzv[2], dzv[3]);
          st_at(static_cast<bf16_t*>(bp.dz) + trow + pt * 16, toff, out);
        }
      }
      // dD per channel: sum over the 16 tokens of the tile (lanes with the same g)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = dd[k][r];
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
          if (r16 == 0) sDD[tt][(2 * hf + k) * 16 + 4 * g + r] = v;
        }
    }

    // ------------------------------------------------------------------ dx (columns j = own tile)
    // w_j[p] = sum_{i>=j} (C_i . B_j) exp(a (S_i - S_j)) ybar_i[p]   +   exp(a (S_Q - S_j)) (Gc B_j)[p]
    f32x4 wi[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) wi[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (2 * kk + 1 < tt) continue;
      float gl[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int it = 2 * kk + half;
        if (it >= tt) {
          const float4 g4 = gcol4(it * 16 + 4 * g, il);   // G[i][j], i = it 16 + 4 g ..
          const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = it * 16 + 4 * g + r;
            gl[half * 4 + r] = i >= il ? gv[r] * exp2_fast(a2 * (sS[i] - Sl)) : 0.f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) gl[half * 4 + r] = 0.f;
        }
      }
      const bf16x8 glf = pack8(gl);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int row = ((2 * hf + k) * 16 + r16) * RS;
        const uint2 lo = *reinterpret_cast<const uint2*>(&YT[row + 32 * kk + 4 * g]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&YT[row + 32 * kk + 16 + 4 * g]);
        wi[k] = mfma16(frag_from_pieces(lo, hi), glf, wi[k]);   // D[p][j] = sum_i ybar_i[p] GL_ij
      }
    }
    float vvp = vin, rp = 0.f;
    {
      const float eq = exp2_fast(a2 * (Sq - Sl));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pt = 2 * hf + k;
        float dxv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = eq * vo[k][r];
          const float wv = wi[k][r] + v;
          dxv[r] = phil * wv + dskip(pt * 16 + 4 * g + r) * ybv[k][r];
          rp += xv[k][r] * v;
        }
        if (lane_valid) {
          uint2 out;
          out.x = pack_bf16x2(dxv[0], dxv[1]);
          out.y = pack_bf16x2(dxv[2], dxv[3]);
          st_at(static_cast<bf16_t*>(bp.dx) + trow + pt * 16, toff, out);
        }
      }
      vvp += rp;   // x_j . (exp(a (S_Q - S_j)) Gc B_j)
      rp *= phil;
    }
    // per-token sums over this half's channels: lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same token
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      qpart += __shfl_xor(qpart, off, 64);
      vvp += __shfl_xor(vvp, off, 64);
      rp += __shfl_xor(rp, off, 64);
      if (hf == 0) {
        krow += __shfl_xor(krow, off, 64);
        kcol += __shfl_xor(kcol, off, 64);
      }
    }
    if (g == 0) {
      sQv[hf][il] = qpart;
      sVv[hf][il] = vvp;
      sRv[hf][il] = rp;
      if (hf == 0) {
        sKr[il] = krow;
        sKc[il] = kcol;
      }
    }
    if (kh + 1 < bp.hb) prefetch(kh + 1, tv);
    __syncthreads();

    // ------------------------------------------------------------------ per-token: dDelta
    if (w == 0) {
      const int t = lane;
      // sq: suffix sum over i >= t of ybar_i . Yoff_i. pv: prefix sum over s <= t of the
      // Gc B_j input term plus (column sum - row sum) of K: sum_{j<=t<=i} K_ij is the sum over
      // the columns up to t less the rows before t (K_ij = 0 for j > i), the row sum of t itself
      // added back below. The two scans run interleaved.
      float sq = sQv[0][t] + sQv[1][t];
      const float krt = sKr[t];
      float pv = sRv[0][t] + sRv[1][t] + sKc[t] - krt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float os = __shfl_down(sq, off, 64);
        const float op = __shfl_up(pv, off, 64);
        if (t + off < 64) sq += os;
        if (t >= off) pv += op;
      }
      float red = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) red += sRed[kh & 1][k];
      const float t1 = exp2_fast(a2 * Sq) * red;
      const float u = t1 + sq + pv + krt;
      const float vv = sVv[0][t] + sVv[1][t];
      const float ddt = a * u + vv;
      const int64_t tt2 = tc0 + t;
      // (no branch on the token: rows past L compute from a zero step and are selected away, and
      // their dDelta store falls outside the descriptor, so the stores in flight are the same on
      // every path)
      const float raw = (tt2 < L ? bf16_to_f32((uint16_t)dl) : 0.f) + dbias;
      const float dt = p.delta_softplus ? softplus_f32(raw) : raw;
      const float gu = p.delta_softplus ? ddt * sigmoid_fast(raw) : ddt;
      const int64_t rows_in = std::min<int64_t>(64, L - tc0);
      buf_store(make_rsrc(static_cast<bf16_t*>(bp.ddelta) + (b * L + tc0) * H + h, (int)(((rows_in - 1) * H + 1) * 2)),
                (uint32_t)(t * H) * 2u, gu, (bf16_t*)nullptr);
      // (Delta - phi) / a = (a Delta - expm1(a Delta)) / a^2
      const float xa = a * dt;
      float pa = dt * u + (xa - expm1f(xa)) / (a * a) * vv;
      float pb = gu;
      if (!(tt2 < L)) pa = pb = 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        pa += __shfl_xor(pa, off, 64);
        pb += __shfl_xor(pb, off, 64);
      }
      const int64_t pidx = (b * nch + c) * H + h;
      // (every lane holds the sums: all store the same value, with no branch)
      bp.ws_pA[pidx] = pa;
      bp.ws_pb[pidx] = pb;
      bp.ws_pD[pidx * kP + t] = sDD[0][t] + sDD[1][t] + sDD[2][t] + sDD[3][t];
    }
    // (no barrier here: the next head's staging writes none of what wave 0 reads above, and the
    // arrays it reads are written again only after the next staging barrier, which wave 0 joins
    // when done)
  }

  // dB and dC of this workgroup's heads: the lane holds states n .. n + 3 of token il
  if (lane_valid) {
    const int64_t orow = ((b * (H / bp.hb) + hblk) * L + tl) * N + 4 * g;
#pragma unroll
    for (int k = 0; k < NTH; ++k) {
      const int n0 = (hf * NTH + k) * 16;
      *reinterpret_cast<float4*>(bp.ws_dCp + orow + n0) = make_float4(dC[k][0], dC[k][1], dC[k][2], dC[k][3]);
      *reinterpret_cast<float4*>(bp.ws_dBp + orow + n0) = make_float4(dB[k][0], dB[k][1], dB[k][2], dB[k][3]);
    }
  }
}

// dB, dC [B, L, G, N] = sums over each group's head blocks, in block order; 4 states per thread.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_bc_kernel(SsdBwdParams bp) {
  const SsdParams& p = bp.f;
  const int64_t nblk = p.H / bp.hb, per = nblk / p.G;   // head blocks, per group
  const int64_t total = p.B * p.L * p.G * (p.N / 4);
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n4 = e % (p.N / 4);
    int64_t rest = e / (p.N / 4);
    const int64_t grp = rest % p.G;
    rest /= p.G;
    const int64_t t = rest % p.L, b = rest / p.L;
    float4 sb = make_float4(0.f, 0.f, 0.f, 0.f), sc = sb;
    for (int64_t k = 0; k < per; ++k) {
      const int64_t src = ((b * nblk + grp * per + k) * p.L + t) * p.N + 4 * n4;
      const float4 vb = *reinterpret_cast<const float4*>(bp.ws_dBp + src);
      const float4 vc = *reinterpret_cast<const float4*>(bp.ws_dCp + src);
      sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
      sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
    }
    const int64_t dst = ((b * p.L + t) * p.G + grp) * p.N + 4 * n4;
    *reinterpret_cast<float4*>(bp.dBm + dst) = sb;
    *reinterpret_cast<float4*>(bp.dCm + dst) = sc;
  }
}

// dA, ddelta_bias [H] and dD ([H] or [H, P]): sums over the B x chunks partials of each head, in
// a fixed order: thread t of the 256 takes entries t, t + 256, ... (dA, ddelta_bias) or, per
// channel, entries t / 64, t / 64 + 4, ... (dD); the per-thread sums are combined by a fixed tree.
__global__ __launch_bounds__(256) void ssd_bwd_reduce_param_kernel(SsdBwdParams bp, int64_t nch) {
  __shared__ float sA[256], sB[256], sD[256];
  const SsdParams& p = bp.f;
  const int64_t h = blockIdx.x, nbc = p.B * nch;
  const int tid = threadIdx.x, ch = tid & 63, q = tid >> 6;
  float a = 0.f, b = 0.f, d = 0.f;
  for (int64_t k = tid; k < nbc; k += 256) {
    a += bp.ws_pA[k * p.H + h];
    b += bp.ws_pb[k * p.H + h];
  }
  // eight loads in flight per step, added in the same order as one at a time
  int64_t k = q;
  for (; k + 28 < nbc; k += 32) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = bp.ws_pD[((k + 4 * u) * p.H + h) * kP + ch];
#pragma unroll
    for (int u = 0; u < 8; ++u) d += v[u];
  }
  for (; k < nbc; k += 4) d += bp.ws_pD[(k * p.H + h) * kP + ch];
  sA[tid] = a;
  sB[tid] = b;
  sD[tid] = d;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (tid < off) {
      sA[tid] += sA[tid + off];
      sB[tid] += sB[tid + off];
      if (off >= 64) sD[tid] += sD[tid + off];   // the four partials of each channel
    }
    __syncthreads();
  }
  // sD[0 .. 63] now hold the per-channel sums
  if (bp.dDskip && p.dskip_per_channel && tid < 64) bp.dDskip[h * kP + tid] = sD[tid];
  __syncthreads();
  for (int off = 32; off >= 1; off >>= 1) {
    if (tid < off) sD[tid] += sD[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    bp.dA[h] = sA[0];
    if (bp.ddelta_bias) bp.ddelta_bias[h] = sB[0];
    if (bp.dDskip && !p.dskip_per_channel) bp.dDskip[h] = sD[0];
  }
}

template <int N>
hipError_t launch_n(const SsdBwdParams& bp, hipStream_t stream) {
  constexpr int Q = kQb;
  const SsdParams& p = bp.f;
  const int64_t nch = (p.L + Q - 1) / Q;
  hipLaunchKernelGGL((ssd_cumsum_kernel<Q>), dim3((unsigned)((p.H + kCumHeads - 1) / kCumHeads), (unsigned)nch, (unsigned)p.B),
                     dim3(256), 0, stream, p);
  hipLaunchKernelGGL((ssd_prep_kernel<Q, N, true>), dim3(prep_parts<Q>(), (unsigned)nch, (unsigned)(p.B * p.G)), dim3(256), 0,
                     stream, p);
  // the two state passes take the chunks four at a time (one 256-token step), storing the state
  // at every chunk boundary
  hipLaunchKernelGGL((ssd_chunk_state_kernel<4 * Q, Q, N, false>), dim3((unsigned)p.H, (unsigned)p.B),
                     dim3(64 * (N / 32)), 0, stream, p);
  hipLaunchKernelGGL((ssd_chunk_state_kernel<4 * Q, Q, N, true>), dim3((unsigned)p.H, (unsigned)p.B),
                     dim3(64 * (N / 32)), 0, stream, p);
  const dim3 grid((unsigned)(p.H / bp.hb), (unsigned)nch, (unsigned)p.B);
  if (p.z)
    hipLaunchKernelGGL((ssd_bwd_main_kernel<N, true>), grid, dim3(512), 0, stream, bp);
  else
    hipLaunchKernelGGL((ssd_bwd_main_kernel<N, false>), grid, dim3(512), 0, stream, bp);
  const int64_t total = p.B * p.L * p.G * (p.N / 4);
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(ssd_bwd_reduce_bc_kernel, dim3(blocks), dim3(256), 0, stream, bp);
  hipLaunchKernelGGL(ssd_bwd_reduce_param_kernel, dim3((unsigned)p.H), dim3(256), 0, stream, bp, nch);
  return hipGetLastError();
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t hb) {
  const int64_t Q = kQb, nch = (L + Q - 1) / Q;
  const size_t st = align256((size_t)(B * nch * H * P * N) * 2);
  const size_t gg = align256((size_t)(B * G * nch * Q * Q) * 4);
  const size_t bt = align256((size_t)(B * G * nch * N * Q) * 2);
  const size_t sp = align256((size_t)(B * nch * H * Q) * 8);
  const size_t part = align256((size_t)(B * (H / hb) * L * N) * 4);
  const size_t ph = align256((size_t)(B * nch * H) * 4);
  const size_t pd = align256((size_t)(B * nch * H * P) * 4);
  return 2 * st + gg + 4 * bt + sp + 2 * part + 2 * ph + pd;
}

void ssd_bwd_workspace_carve(SsdBwdParams& bp, void* ws) {
  SsdParams& p = bp.f;
  const int64_t Q = kQb, nch = (p.L + Q - 1) / Q;
  const size_t st = align256((size_t)(p.B * nch * p.H * p.P * p.N) * 2);
  const size_t gg = align256((size_t)(p.B * p.G * nch * Q * Q) * 4);
  const size_t bt = align256((size_t)(p.B * p.G * nch * p.N * Q) * 2);
  const size_t sp = align256((size_t)(p.B * nch * p.H * Q) * 8);
  const size_t part = align256((size_t)(p.B * (p.H / bp.hb) * p.L * p.N) * 4);
  const size_t ph = align256((size_t)(p.B * nch * p.H) * 4);
  char* base = static_cast<char*>(ws);
  p.ws_hin = base; base += st;
  p.ws_gout = base; base += st;
  p.ws_G = base; base += gg;
  p.ws_Bt = base; base += bt;
  p.ws_Ct = base; base += bt;
  p.ws_Btf = base; base += bt;
  p.ws_Ctf = base; base += bt;
  p.ws_sphi = reinterpret_cast<float2*>(base); base += sp;
  bp.ws_dBp = reinterpret_cast<float*>(base); base += part;
  bp.ws_dCp = reinterpret_cast<float*>(base); base += part;
  bp.ws_pA = reinterpret_cast<float*>(base); base += ph;
  bp.ws_pb = reinterpret_cast<float*>(base); base += ph;
  bp.ws_pD = reinterpret_cast<float*>(base);
}

hipError_t launch_ssd_bwd(const SsdBwdParams& bp, hipStream_t stream) {
  if (bp.f.N == 128) return launch_n<128>(bp, stream);
  if (bp.f.N == 64) return launch_n<64>(bp, stream);
  return hipErrorInvalidValue;
}

}  // namespace ssm
