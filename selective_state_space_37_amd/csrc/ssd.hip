// Mamba-2 (SSD) chunked forward on gfx950: MFMA for the within-chunk contractions.
//
// Page "Mamba and state space models", section "Mamba-2: two algorithms": with A a scalar times
// the identity per head, the layer multiplies the input by a lower-triangular matrix whose
// entry (i, j) is C_i . B_j times all decay between steps j and i. The sequence is cut into
// chunks of Q tokens; inside a chunk that masked product runs on the matrix cores, and only the
// state passes between chunks. With zero-order hold the input of step j enters with the scale
// phi_j = expm1(a Delta_j) / a, and with S the inclusive cumulative sum of Delta in the chunk:
//   prep kernel  : per (batch, chunk, group), G = C B^T (Q x Q, MFMA, shared by the group's
//                  heads) and a transposed copy of B for the state kernel's operand layout
//   state kernel : per (batch, head), sequential over the chunks with the state
//                  in MFMA accumulators: store h_{c-1} (bf16, the carry the outputs need), then
//                  h_c = exp(a S_last) h_{c-1} + sum_j exp(a (S_last - S_j)) phi_j x_j B_j^T
//   output kernel: per (batch, chunk, head),
//                  y_i = sum_{j<=i} G_ij exp(a (S_i - S_j)) phi_j x_j                 (MFMA, K = Q)
//                      + exp(a S_i) C_i . h_{c-1}                                    (MFMA, K = N)
//                      (+ D x_i, gate)
// Decays are always formed from differences of cumulative sums inside one chunk, so no
// intermediate exponential can overflow. Operands are bf16, accumulation float32.
// B and C come in G groups ([B, L, G, N]); head h reads group h / (H / G) (G = 1: one B and C
// for all heads). The skip weight D is per head or per channel of a head.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (lane l, g = l / 16):
//   A (16 x 32, M x K): row l % 16, k = 8g .. 8g+7;  B (32 x 16, K x N): col l % 16, k = 8g .. 8g+7;
//   D (16 x 16): col l % 16, rows 4g .. 4g+3.
// The K order inside one product is free as long as A and B agree; the output kernel uses that
// to take two 16-token tiles of j (four tokens of each per lane) in one product. The A and B
// layouts mirror each other, so swapping the operands yields the transposed product.
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
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

// LDS layout of a transposed x tile (rows = channels p, columns = tokens j, row stride Q + 8
// bf16): the 4-byte word column of row p is XORed with 8 ((p >> 4) & 3) (kept inside the row).
// The staging writes (8 channel groups x 8 token pairs per wave) then fall on 64 different banks
// instead of 16, while a reader that takes 16 consecutive rows of one 16-row group sees a
// uniform XOR: its bank pattern and 8-byte alignment are those of the plain layout.
template <int Q>
__device__ __forceinline__ int xt_swizzle_words(int row) {
  return (8 * ((row >> 4) & 3)) & (Q / 2 - 1);
}

// Stage x[b, chunk, h, :] transposed into LDS (the layout above), each token's column scaled by
//   cp_j = exp(a (S_e - S_j)) phi_j,   e = the last token of j's 16-token tile (S_e >= S_j),
// computed from the chunk's (S, phi) table sp; a2 = a log2(e). Each thread takes two
// consecutive tokens, so every LDS write is one 32-bit word holding the pair (j, j + 1) of one
// channel; the scaled values are rounded to bf16 once. Tokens past L are staged as zeros.
template <int Q>
__device__ void stage_x_transposed_scaled(const SsdParams& p, int64_t b, int64_t c, int64_t h, __bf16* Xt,
                                          const float2* sp, float a2) {
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  uint32_t* X32 = reinterpret_cast<uint32_t*>(Xt);
  for (int g = threadIdx.x; g < (Q / 2) * (kP / 8); g += blockDim.x) {
    const int jp = g / (kP / 8), pg = g % (kP / 8);
    const int64_t t = c * Q + 2 * jp;
    uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0;
    if (t < p.L) r0 = *reinterpret_cast<const uint4*>(xg + ((b * p.L + t) * p.H + h) * kP + pg * 8);
    if (t + 1 < p.L) r1 = *reinterpret_cast<const uint4*>(xg + ((b * p.L + t + 1) * p.H + h) * kP + pg * 8);
    const float2 v0 = sp[2 * jp], v1 = sp[2 * jp + 1];
    const float se = sp[(2 * jp) | 15].x;
    const float cp0 = exp2_fast(a2 * (se - v0.x)) * v0.y, cp1 = exp2_fast(a2 * (se - v1.x)) * v1.y;
    const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // channels 2k (low halves) and 2k+1 (high halves) of the two tokens
      const int ra = pg * 8 + 2 * k, rb = ra + 1;
      X32[ra * ((Q + 8) / 2) + (jp ^ xt_swizzle_words<Q>(ra))] =
          (uint32_t)f32_to_bf16(bf16_lo(w0[k]) * cp0) | ((uint32_t)f32_to_bf16(bf16_lo(w1[k]) * cp1) << 16);
      X32[rb * ((Q + 8) / 2) + (jp ^ xt_swizzle_words<Q>(rb))] =
          (uint32_t)f32_to_bf16(bf16_hi(w0[k]) * cp0) | ((uint32_t)f32_to_bf16(bf16_hi(w1[k]) * cp1) << 16);
    }
  }
}

// ---------------------------------------------------------------------------- step sizes
// grid (H, chunks, B): per chunk and head, the inclusive cumulative sum S_j of the step sizes and
// the ZOH input scale phi_j = expm1(a Delta_j) / a, for the state and output kernels.
template <int Q>
__global__ __launch_bounds__(256) void ssd_cumsum_kernel(SsdParams p) {
  __shared__ float sS[Q], sPhi[Q], sTot[4];
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  chunk_prologue<Q>(p, b, c, h, p.A[h], sS, sPhi, sTot);
  const int tid = threadIdx.x;
  if (tid < Q) p.ws_sphi[((b * nch + c) * p.H + h) * Q + tid] = make_float2(sS[tid], sPhi[tid]);
}

// ---------------------------------------------------------------------------- prep
// grid (4, chunks, B G): part `part` transposes states [part N/4, (part+1) N/4) of one group's B
// and computes every fourth lower-triangular 16 x 16 tile of that group's G (row blocks ib,
// column tiles jt <= ib). Token t's row of the group starts at element (t G + grp) N.
template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdParams p) {
  const int part = blockIdx.x;
  const int64_t c = blockIdx.y, bg = blockIdx.z;   // bg = b G + grp
  const int64_t b = bg / p.G, grp = bg % p.G;
  const int64_t nch = gridDim.y;
  const int tid = threadIdx.x;
  const int64_t rs = p.G * N;                      // token row stride of B and C
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm) + b * p.L * rs + grp * N;
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * p.L * rs + grp * N;
  // transposed B: Bt[n][j], 8 tokens per 16-byte store
  bf16_t* Bt = static_cast<bf16_t*>(p.ws_Bt) + (bg * nch + c) * (int64_t)(N * Q);
  constexpr int NQ = N / 4;
  for (int it = tid; it < NQ * (Q / 8); it += 256) {
    const int n = part * NQ + it / (Q / 8);
    const int j0 = (it % (Q / 8)) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = 0, hi = 0;
      const int64_t t0 = c * Q + j0 + 2 * q;
      if (t0 < p.L) lo = Bg[t0 * rs + n].bits;
      if (t0 + 1 < p.L) hi = Bg[(t0 + 1) * rs + n].bits;
      wv[q] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(Bt + (int64_t)n * Q + j0) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  // G tiles
  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the row blocks derived from it) in scalar registers, so branches on it are not divergent
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, r16 = lane & 15;
  constexpr int NIB = Q / 16, KS = N / 32, NTILES = NIB * (NIB + 1) / 2;
  bf16_t* G = static_cast<bf16_t*>(p.ws_G) + (bg * nch + c) * (int64_t)(Q * Q);
  for (int k = part * 4 + w; k < NTILES; k += 16) {
    int ib = 0, rem = k;
    while (rem > ib) { rem -= ib + 1; ++ib; }
    const int jt = rem;
    const int64_t ti = c * Q + ib * 16 + r16, tj = c * Q + jt * 16 + r16;   // tokens in the row
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ca = ti < p.L ? load_frag(Cg + ti * rs + ks * 32 + 8 * g) : zero_frag();
      const bf16x8 bb = tj < p.L ? load_frag(Bg + tj * rs + ks * 32 + 8 * g) : zero_frag();
      acc = mfma16(ca, bb, acc);  // D[i][j] = sum_n C_i[n] B_j[n]
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) G[(int64_t)(ib * 16 + 4 * g + r) * Q + jt * 16 + r16].bits = f32_to_bf16(acc[r]);
  }
}

// ---------------------------------------------------------------------------- chunk states
// grid (H, B), 512 threads: one head, sequential over the chunks. Wave w owns the state block
// p in [16 pq, 16 pq + 16) x n in [NH w2, NH (w2 + 1)) with pq = w / 2, w2 = w % 2, NH = N / 2,
// as NTW = N / 32 MFMA tiles computed transposed (states x channels), so that
// acc[k][r] = h[p = 16 pq + lane % 16][n = (w2 NTW + k) 16 + 4 g + r]: four consecutive states
// per lane, stored as one 8-byte (bf16) or 16-byte (float) piece. Per chunk the transposed B
// (shared by the heads of a group) and the scaled, transposed x of the head are staged in LDS
// once for all eight waves.
//
// Inputs are loaded two chunks ahead into two register buffers used in turn (the loop is
// unrolled by two; no buffer is copied). Every global load and store of the loop is issued
// unconditionally -- rows past L are read from the last token, whose weight phi is 0 for padded
// tokens anyway, and the prefetch index is clamped -- so the compiler's count of outstanding
// memory operations stays exact and the waits for a buffer do not also wait for the loads of
// the other.
template <int Q, int N>
__global__ __launch_bounds__(512) void ssd_state_kernel(SsdParams p) {
  constexpr int KQ = Q / 32;                 // K steps over a chunk
  constexpr int NTW = N / 32;                // state tiles per wave
  constexpr int XPAIRS = Q / 2 * 4;          // (token pair, 16-channel group) items of x
  constexpr int BT16 = N * Q / 8;            // 16-byte pieces of B^T
  static_assert(BT16 % 512 == 0, "B^T pieces divide over the threads");
  static_assert(512 % XPAIRS == 0, "x items repeat evenly over the threads");
  constexpr int BT_PER = BT16 / 512;
  __shared__ __attribute__((aligned(16))) __bf16 Xs[kP * (Q + 8)];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[N * (Q + 8)];
  const int64_t h = blockIdx.x, b = blockIdx.y;
  const int64_t nch = (p.L + Q - 1) / Q;
  const int tid = threadIdx.x;
  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the row blocks derived from it) in scalar registers, so branches on it are not divergent
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, r16 = lane & 15;
  const int pq = w >> 1, w2 = w & 1;
  const float a2 = p.A[h] * kLog2e;
  const int64_t PN = (int64_t)kP * N;
  // first of the four consecutive states of tile k
  auto st_idx = [&](int k) { return (int64_t)(16 * pq + r16) * N + (w2 * NTW + k) * 16 + 4 * g; };

  f32x4 acc[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.h0) {
      const float4 v = *reinterpret_cast<const float4*>(p.h0 + (b * p.H + h) * PN + st_idx(k));
      acc[k] = f32x4{v.x, v.y, v.z, v.w};
    }
  }
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  bf16_t* hin_all = static_cast<bf16_t*>(p.ws_hin);
  const int64_t bg = b * p.G + h / (p.H / p.G);   // this head's (batch, group)
  const bf16_t* Bt_all = static_cast<const bf16_t*>(p.ws_Bt) + bg * nch * (int64_t)(N * Q);

  // x item of this thread: tokens (2 jp, 2 jp + 1), channels [16 pg, 16 pg + 16). With fewer
  // items than threads, threads tid and tid + XPAIRS take the same item and write the same
  // values to the same LDS words.
  const int item = tid % XPAIRS;
  const int jp = item >> 2, pg = item & 3;
  // native vector fields: plain register loads and stores (a struct-typed copy becomes a memcpy,
  // which keeps the buffer out of registers)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  struct ChunkIn {
    u32x4 x[2][2];      // two tokens x 16 channels
    f32x2 sphi[2];      // (S_j, phi_j) of the two tokens
    float s_last;
    u32x4 bt[BT_PER];   // pieces of the chunk's B^T
  };
  // (both lambdas are forced inline: the buffers they take by reference must stay in registers)
  auto load_chunk = [&](int64_t c, ChunkIn& in) __attribute__((always_inline)) {
    const float2* sp = p.ws_sphi + ((b * nch + c) * p.H + h) * Q;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * jp + u;
      const int64_t t = c * Q + j < p.L ? c * Q + j : p.L - 1;
      const u32x4* src = reinterpret_cast<const u32x4*>(xg + ((b * p.L + t) * p.H + h) * kP + 16 * pg);
      in.x[u][0] = src[0];
      in.x[u][1] = src[1];
      in.sphi[u] = reinterpret_cast<const f32x2*>(sp)[j];
    }
    in.s_last = sp[Q - 1].x;
    const u32x4* bt = reinterpret_cast<const u32x4*>(Bt_all + c * (int64_t)(N * Q));
#pragma unroll
    for (int k = 0; k < BT_PER; ++k) in.bt[k] = bt[tid + 512 * k];
  };

  auto process = [&](int64_t c, ChunkIn& cur) __attribute__((always_inline)) {
    // stage B^T and the decay-scaled x^T of chunk c
#pragma unroll
    for (int k = 0; k < BT_PER; ++k) {
      const int e = tid + 512 * k;
      const int n = e / (Q / 8), j8 = (e % (Q / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Bs[n * (Q + 8) + j8]) = cur.bt[k];
    }
    {
      float wj[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) wj[u] = exp2_fast(a2 * (cur.s_last - cur.sphi[u].x)) * cur.sphi[u].y;
      uint32_t* X32 = reinterpret_cast<uint32_t*>(Xs);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const u32x4 v0 = cur.x[0][q >> 3], v1 = cur.x[1][q >> 3];
        const uint32_t u0 = ((q & 7) >> 1) == 0 ? v0.x : ((q & 7) >> 1) == 1 ? v0.y : ((q & 7) >> 1) == 2 ? v0.z : v0.w;
        const uint32_t u1 = ((q & 7) >> 1) == 0 ? v1.x : ((q & 7) >> 1) == 1 ? v1.y : ((q & 7) >> 1) == 2 ? v1.z : v1.w;
        const float f0 = (q & 1) ? bf16_hi(u0) : bf16_lo(u0);
        const float f1 = (q & 1) ? bf16_hi(u1) : bf16_lo(u1);
        // word column XORed with 16 pg (inside the row): the four channel groups of a wave
        // write to four different 16-bank ranges
        X32[(16 * pg + q) * ((Q + 8) / 2) + (jp ^ ((16 * pg) & (Q / 2 - 1)))] =
            (uint32_t)f32_to_bf16(f0 * wj[0]) | ((uint32_t)f32_to_bf16(f1 * wj[1]) << 16);
      }
    }
    const float decay = exp2_fast(a2 * cur.s_last);
    load_chunk(c + 2 < nch ? c + 2 : nch - 1, cur);
    // the state entering chunk c, for the output kernel; then decay it over the chunk
    bf16_t* hin = hin_all + ((b * nch + c) * p.H + h) * PN;
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[k][0]) | ((uint32_t)f32_to_bf16(acc[k][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[k][2]) | ((uint32_t)f32_to_bf16(acc[k][3]) << 16);
      *reinterpret_cast<uint2*>(hin + st_idx(k)) = make_uint2(lo, hi);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[k][r] *= decay;
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(
          &Xs[(16 * pq + r16) * (Q + 8) + ((kq * 32 + 8 * g) ^ ((32 * pq) & (Q - 1)))]);
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const bf16x8 ba = *reinterpret_cast<const bf16x8*>(&Bs[((w2 * NTW + k) * 16 + r16) * (Q + 8) + kq * 32 + 8 * g]);
        acc[k] = mfma16(ba, xb, acc[k]);   // (states x tokens) . (tokens x channels)
      }
    }
    __syncthreads();
  };

  ChunkIn buf0, buf1;   // even chunks in buf0, odd chunks in buf1
  if (nch > 0) {
    load_chunk(0, buf0);
    load_chunk(nch > 1 ? 1 : 0, buf1);
  }
  int64_t c = 0;
  for (; c + 1 < nch; c += 2) {
    process(c, buf0);
    process(c + 1, buf1);
  }
  if (c < nch) process(c, buf0);

  if (p.h_last) {
#pragma unroll
    for (int k = 0; k < NTW; ++k)
      *reinterpret_cast<float4*>(p.h_last + (b * p.H + h) * PN + st_idx(k)) =
          make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
}

// ---------------------------------------------------------------------------- outputs
// Decay of a mask entry (i, j), j <= i: exp(a (S_i - S_j)) phi_j. It factors through the last
// token e of j's 16-token tile:
//   exp(a (S_i - S_e)) * [exp(a (S_e - S_j)) phi_j].
// The bracket depends on j only and is folded into x^T when it is staged (exponent <= 0). The
// first factor is one exp per lane and tile: <= 1 off the diagonal, and on the diagonal tile
// (S_i <= S_e, at most 15 steps apart) at most exp(15 |a| max Delta), far inside the range of
// float32 and bf16. So every mask entry is G_ij times a per-row factor, with the causal cut
// j <= i on the diagonal tile.
template <int Q, int N>
__global__ __launch_bounds__(256) void ssd_out_kernel(SsdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 Xt[kP * (Q + 8)];
  // the carried-in state h_{c-1} (P x N bf16), staged once for the four waves; rows padded by
  // 8 elements so a wave's 16-byte fragment reads (16 rows apart by one row) hit 64 banks
  __shared__ __attribute__((aligned(16))) __bf16 Hs[kP * (N + 8)];
  __shared__ float sS[Q];
  const int64_t h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  const float a2 = p.A[h] * kLog2e;
  const int tid = threadIdx.x;
  const float2* sp = p.ws_sphi + ((b * nch + c) * p.H + h) * Q;
  if (tid < Q) sS[tid] = sp[tid].x;
  stage_x_transposed_scaled<Q>(p, b, c, h, Xt, sp, a2);
  {
    const bf16_t* hin = static_cast<const bf16_t*>(p.ws_hin) + ((b * nch + c) * p.H + h) * (int64_t)(kP * N);
    for (int e = tid; e < kP * N / 8; e += blockDim.x) {   // 16-byte pieces
      const int row = e / (N / 8), c8 = (e % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(&Hs[row * (N + 8) + c8]) = *reinterpret_cast<const uint4*>(hin + row * N + c8);
    }
  }
  __syncthreads();

  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the row blocks derived from it) in scalar registers, so branches on it are not divergent
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, r16 = lane & 15;
  constexpr int NIB = Q / 16;   // 16-row blocks of the chunk
  constexpr int KS = N / 32;    // K steps over the state dimension
  const int64_t grp = h / (p.H / p.G), rs = p.G * N;   // this head's group, token row stride of C
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * p.L * rs + grp * N;
  const bf16_t* G = static_cast<const bf16_t*>(p.ws_G) + ((b * p.G + grp) * nch + c) * (int64_t)(Q * Q);
  const float dsk = p.Dskip && !p.dskip_per_channel ? p.Dskip[h] : 0.f;
  const bf16_t* zg = static_cast<const bf16_t*>(p.z);
  bf16_t* yg = static_cast<bf16_t*>(p.y);

  // Balanced triangle: block x and block NIB-1-x hold NIB+1 tiles together.
  constexpr int kBlocksPerWave = NIB >= 8 ? NIB / 4 : 1;
  auto block_of = [&](int kb) {
    if (NIB < 8) return w;
    const int pair = w + 4 * (kb >> 1);
    return (kb & 1) ? (NIB - 1 - pair) : pair;
  };
  // carried-state fragments (the A operand of the carried term), the same for every row block;
  // every product here is computed transposed (channels x tokens) so a lane ends up holding four
  // consecutive channels of one token
  bf16x8 hf[KS][4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      hf[ks][pt] = *reinterpret_cast<const bf16x8*>(&Hs[(pt * 16 + r16) * (N + 8) + ks * 32 + 8 * g]);
  auto load_c = [&](int ib, bf16x8 out[KS]) {
    const int64_t ti = c * Q + ib * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      out[ks] = ti < p.L ? load_frag(Cg + ti * rs + ks * 32 + 8 * g) : zero_frag();
  };
  bf16x8 cnext[KS];
  if (NIB >= 4 || w < NIB) load_c(block_of(0), cnext);
  // fully unrolled: the C fragments loaded one block ahead are then renamed, not copied (a copy
  // of registers with loads in flight would wait for them at the end of the previous block)
#pragma unroll
  for (int kb = 0; kb < kBlocksPerWave; ++kb) {
    const int ib = block_of(kb);
    if (ib >= NIB) break;
    bf16x8 cf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cf[ks] = cnext[ks];
    if (kb + 1 < kBlocksPerWave) load_c(block_of(kb + 1), cnext);
    const int i0 = ib * 16;
    const int il = i0 + r16;                  // this lane's token row of M (B operand)
    const float Si = sS[il];
    const bf16_t* Grow = G + (int64_t)il * Q;  // G[il][j]: the lane's four j of a tile are contiguous

    f32x4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // carried state: exp(a S_i) C_i . h_in[p, :]
    {
      const float eSi = exp2_fast(a2 * Si);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 av;
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = (__bf16)((float)cf[ks][q] * eSi);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma16(hf[ks][pt], av, acc[pt]);
      }
    }

    // within the chunk: masked G_ij decay phi_j times x_j, two 16-token j tiles per product;
    // the G tiles of the next pair are requested while the current pair is processed
    auto load_g = [&](int jt) {
      return jt <= ib ? *reinterpret_cast<const uint2*>(Grow + jt * 16 + 4 * g) : make_uint2(0, 0);
    };
    // fully unrolled (at most NIB / 2 pairs, leaving at the diagonal): the pair prefetched one
    // step ahead is renamed rather than copied, so its loads overlap the current pair's work
    uint2 gcur[2] = {load_g(0), load_g(1)}, gnext[2];
#pragma unroll
    for (int jp = 0; jp < (NIB + 1) / 2; ++jp) {
      if (2 * jp > ib) break;   // uniform (ib is a scalar)
      gnext[0] = load_g(2 * jp + 2);
      gnext[1] = load_g(2 * jp + 3);
      float m[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jt = 2 * jp + half;
        const uint2 gw = gcur[half];
        const float gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
        const int j0 = jt * 16 + 4 * g;
        if (jt < ib) {
          const float r = exp2_fast(a2 * (Si - sS[jt * 16 + 15]));
#pragma unroll
          for (int q = 0; q < 4; ++q) m[half * 4 + q] = gv[q] * r;
        } else if (jt == ib) {
          const float r = exp2_fast(a2 * (Si - sS[jt * 16 + 15]));
#pragma unroll
          for (int q = 0; q < 4; ++q) m[half * 4 + q] = (j0 + q <= il) ? gv[q] * r : 0.f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) m[half * 4 + r] = 0.f;
        }
      }
      bf16x8 av;
#pragma unroll
      for (int q = 0; q < 8; ++q) av[q] = (__bf16)m[q];
      const int jb = jp * 32;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int sw = 2 * xt_swizzle_words<Q>(pt * 16);   // in bf16 elements, uniform over the wave
        const uint2 lo = *reinterpret_cast<const uint2*>(&Xt[(pt * 16 + r16) * (Q + 8) + ((jb + 4 * g) ^ sw)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Xt[(pt * 16 + r16) * (Q + 8) + ((jb + 16 + 4 * g) ^ sw)]);
        const uint4 pk = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc[pt] = mfma16(__builtin_bit_cast(bf16x8, pk), av, acc[pt]);
      }
      gcur[0] = gnext[0];
      gcur[1] = gnext[1];
    }

    // epilogue: D term, gate, store. acc[pt][r] = y[i0 + r16][pt * 16 + 4 g + r], so each lane
    // finishes four consecutive channels of one token (8-byte loads of x and z, 8-byte store).
    const int64_t t = c * Q + i0 + r16;
    if (t < p.L) {
      const int64_t orow = ((b * p.L + t) * p.H + h) * kP + 4 * g;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int64_t o = orow + pt * 16;
        float v[4] = {acc[pt][0], acc[pt][1], acc[pt][2], acc[pt][3]};
        if (p.Dskip) {
          const uint2 xr = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p.x) + o);
          float d[4] = {dsk, dsk, dsk, dsk};
          if (p.dskip_per_channel) {   // channels pt 16 + 4 g .. + 3 of head h
            const float4 dv = *reinterpret_cast<const float4*>(p.Dskip + h * kP + pt * 16 + 4 * g);
            d[0] = dv.x; d[1] = dv.y; d[2] = dv.z; d[3] = dv.w;
          }
          v[0] = fmaf(d[0], bf16_lo(xr.x), v[0]);
          v[1] = fmaf(d[1], bf16_hi(xr.x), v[1]);
          v[2] = fmaf(d[2], bf16_lo(xr.y), v[2]);
          v[3] = fmaf(d[3], bf16_hi(xr.y), v[3]);
        }
        if (zg) {
          const uint2 zr = *reinterpret_cast<const uint2*>(zg + o);
          v[0] *= silu(bf16_lo(zr.x));
          v[1] *= silu(bf16_hi(zr.x));
          v[2] *= silu(bf16_lo(zr.y));
          v[3] *= silu(bf16_hi(zr.y));
        }
        uint2 out;
        out.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        out.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(yg + o) = out;
      }
    }
  }
}

template <int Q, int N>
hipError_t launch_qn(const SsdParams& p, hipStream_t stream) {
  const int64_t nch = (p.L + Q - 1) / Q;
  hipLaunchKernelGGL((ssd_cumsum_kernel<Q>), dim3((unsigned)p.H, (unsigned)nch, (unsigned)p.B), dim3(256), 0,
                     stream, p);
  hipLaunchKernelGGL((ssd_prep_kernel<Q, N>), dim3(4, (unsigned)nch, (unsigned)(p.B * p.G)), dim3(256), 0, stream,
                     p);
  hipLaunchKernelGGL((ssd_state_kernel<Q, N>), dim3((unsigned)p.H, (unsigned)p.B), dim3(512), 0, stream, p);
  hipLaunchKernelGGL((ssd_out_kernel<Q, N>), dim3((unsigned)p.H, (unsigned)nch, (unsigned)p.B), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// Workspace: carried states (bf16), G per chunk and group (bf16), transposed B per chunk and
// group (bf16), (S, phi) per chunk, head and token (float2), each 256-byte aligned.
static size_t ssd_align(size_t n) { return (n + 255) & ~(size_t)255; }

size_t ssd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q) {
  const int64_t nch = (L + Q - 1) / Q;
  return ssd_align((size_t)(B * nch * H * P * N) * 2) + ssd_align((size_t)(B * G * nch * Q * Q) * 2) +
         ssd_align((size_t)(B * G * nch * N * Q) * 2) + ssd_align((size_t)(B * nch * H * Q) * 8);
}

void ssd_workspace_carve(SsdParams& p, void* ws) {
  const int64_t nch = (p.L + p.Q - 1) / p.Q;
  char* base = static_cast<char*>(ws);
  p.ws_hin = base;
  base += ssd_align((size_t)(p.B * nch * p.H * p.P * p.N) * 2);
  p.ws_G = base;
  base += ssd_align((size_t)(p.B * p.G * nch * p.Q * p.Q) * 2);
  p.ws_Bt = base;
  base += ssd_align((size_t)(p.B * p.G * nch * p.N * p.Q) * 2);
  p.ws_sphi = reinterpret_cast<float2*>(base);
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
