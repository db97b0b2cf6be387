// Device code shared by the Mamba-2 (SSD) forward and backward: MFMA helpers, the per-chunk
// step-size prologue, the transposed x staging, and the cumsum, prep and chunk-state kernels.
// Page "Mamba and state space models", section "Mamba-2: two algorithms": the layer is a
// lower-triangular matrix applied chunk by chunk, with only the state passed between chunks.
#pragma once

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

// Two floats rounded to bf16 (nearest even) in one 32-bit word, lo in the low half: one
// v_cvt_pk_bf16_f32 for the pair.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// A load at a wave-uniform base plus a 32-bit per-lane byte offset (the scalar-base form of the
// global load: one offset register per lane rather than a 64-bit address)
template <class T, class E>
__device__ __forceinline__ T ld_at(const E* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <class T, class E>
__device__ __forceinline__ void st_at(E* base, uint32_t byte_off, const T& v) {
  *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off) = v;
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

// Floor of the base-2 exponent of the staged x scale (see below): 2^-64 keeps a scaled input far
// inside the normal range of bf16 and float32, and the diagonal tile's compensating factor at most
// 2^64.
constexpr float kSsdStageExpFloor = -64.0f;

// Stage x[b, chunk, h, :] transposed into LDS (the layout above), each token's column scaled by
//   cp_j = 2^max(a2 (S_e - S_j), -64) phi_j,   e = the last token of j's 16-token tile (S_e >= S_j),
// computed from the chunk's (S, phi) table sp; a2 = a log2(e). The floor matters only where the
// decay from j to the tile end is below 2^-64: rows after the tile then see the input at most
// 2^-64 |phi_j x_j| too large (far below bf16 rounding), and the diagonal tile divides the same
// floored factor out of each entry. Each thread takes two consecutive tokens, so every LDS write
// is one 32-bit word holding the pair (j, j + 1) of one channel; the scaled values are rounded to
// bf16 once. Tokens past L are staged as zeros.
template <int Q, int NT>
__device__ void stage_x_transposed_scaled(const SsdParams& p, int64_t b, int64_t c, int64_t h, __bf16* Xt,
                                          const float2* sp, float a2) {
  // NT threads; every thread's loads are issued before any is used (one memory latency per stage)
  constexpr int kItems = (Q / 2) * (kP / 8);
  constexpr int kPer = (kItems + NT - 1) / NT;
  static_assert(kItems % NT == 0 || kItems < NT, "the items divide over the threads");
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  uint32_t* X32 = reinterpret_cast<uint32_t*>(Xt);
  uint4 r0[kPer], r1[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int g = threadIdx.x + k * NT;
    const int jp = g / (kP / 8), pg = g % (kP / 8);
    const int64_t t = c * Q + 2 * jp;
    r0[k] = r1[k] = make_uint4(0, 0, 0, 0);
    if (g >= kItems) continue;
    if (t < p.L) r0[k] = *reinterpret_cast<const uint4*>(xg + ((b * p.L + t) * p.H + h) * kP + pg * 8);
    if (t + 1 < p.L) r1[k] = *reinterpret_cast<const uint4*>(xg + ((b * p.L + t + 1) * p.H + h) * kP + pg * 8);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int g = threadIdx.x + k * NT;
    if (g >= kItems) continue;
    const int jp = g / (kP / 8), pg = g % (kP / 8);
    const float2 v0 = sp[2 * jp], v1 = sp[2 * jp + 1];
    const float se = sp[(2 * jp) | 15].x;
    const float cp0 = exp2_fast(fmaxf(a2 * (se - v0.x), kSsdStageExpFloor)) * v0.y;
    const float cp1 = exp2_fast(fmaxf(a2 * (se - v1.x), kSsdStageExpFloor)) * v1.y;
    const uint32_t w0[4] = {r0[k].x, r0[k].y, r0[k].z, r0[k].w}, w1[4] = {r1[k].x, r1[k].y, r1[k].z, r1[k].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // channels 2q (low halves) and 2q+1 (high halves) of the two tokens
      const int ra = pg * 8 + 2 * q, rb = ra + 1;
      X32[ra * ((Q + 8) / 2) + (jp ^ xt_swizzle_words<Q>(ra))] =
          pack_bf16x2(bf16_lo(w0[q]) * cp0, bf16_lo(w1[q]) * cp1);
      X32[rb * ((Q + 8) / 2) + (jp ^ xt_swizzle_words<Q>(rb))] =
          pack_bf16x2(bf16_hi(w0[q]) * cp0, bf16_hi(w1[q]) * cp1);
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
// BWD: C is transposed as well (ws_Ct), and G is stored in float32 (ws_G, [Q][Q]) for the
// backward's elementwise use. Only the tiles on and below the diagonal of G are written; the
// forward packs them (bf16) in row-block order for the output kernel's LDS copy.
template <int Q, int N, bool BWD = false>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdParams p) {
  const int part = blockIdx.x;
  const int64_t c = blockIdx.y, bg = blockIdx.z;   // bg = b G + grp
  const int64_t b = bg / p.G, grp = bg % p.G;
  const int64_t nch = gridDim.y;
  const int tid = threadIdx.x;
  const int64_t rs = p.G * N;                      // token row stride of B and C
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm) + b * p.L * rs + grp * N;
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * p.L * rs + grp * N;
  // transposed B, 8 tokens per 16-byte store. Backward: Bt[n][j]. Forward: in the order the
  // forward's chunk-state kernel reads its MFMA operands (v_mfma_f32_32x32x16_bf16, A = B^T): the
  // piece (n, j0 .. j0 + 7) of 32-row tile nt = n / 32 and 16-token step s = j0 / 16 is lane
  // n % 32 + 32 ((j0 / 8) % 2) of the 1 KB fragment (nt, s), fragments in the order
  // nt Q / 16 + s, so that one fragment load of a wave is 1 KB of consecutive memory.
  bf16_t* Bt = static_cast<bf16_t*>(p.ws_Bt) + (bg * nch + c) * (int64_t)(N * Q);
  constexpr int NQ = N / 4;
  auto piece_off = [](int n, int j0) -> int64_t {
    if constexpr (BWD) return (int64_t)n * Q + j0;
    const int frag = (n / 32) * (Q / 16) + j0 / 16, ln = n % 32 + 32 * ((j0 / 8) % 2);
    return (int64_t)frag * 512 + ln * 8;
  };
  auto transpose = [&](const bf16_t* src, bf16_t* dst) {
    for (int it = tid; it < NQ * (Q / 8); it += 256) {
      const int n = part * NQ + it / (Q / 8);
      const int j0 = (it % (Q / 8)) * 8;
      uint32_t wv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = 0, hi = 0;
        const int64_t t0 = c * Q + j0 + 2 * q;
        if (t0 < p.L) lo = src[t0 * rs + n].bits;
        if (t0 + 1 < p.L) hi = src[(t0 + 1) * rs + n].bits;
        wv[q] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(dst + piece_off(n, j0)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  };
  transpose(Bg, Bt);
  if constexpr (BWD) transpose(Cg, static_cast<bf16_t*>(p.ws_Ct) + (bg * nch + c) * (int64_t)(N * Q));
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
    if constexpr (BWD) {
      float* G32 = static_cast<float*>(p.ws_G) + (bg * nch + c) * (int64_t)(Q * Q);
#pragma unroll
      for (int r = 0; r < 4; ++r) G32[(int64_t)(ib * 16 + 4 * g + r) * Q + jt * 16 + r16] = acc[r];
    } else {
      // forward: bf16, the lower-triangular tiles packed in row-block order (tile (ib, jt) is the
      // 256 elements at ib (ib + 1) / 2 + jt, row-major)
      bf16_t* Gt = G + (int64_t)(ib * (ib + 1) / 2 + jt) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) Gt[(4 * g + r) * 16 + r16].bits = f32_to_bf16(acc[r]);
    }
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
// unconditionally -- rows past L are read from the last token, whose weight is 0 for padded
// tokens, and the prefetch index is clamped -- so the compiler's count of outstanding
// memory operations stays exact and the waits for a buffer do not also wait for the loads of
// the other.
//
// ADJ: the same pass run backwards for the adjoint of the state (the backward's dL/dh). With
// ybar = dy sigmoid-gated (dy z sigmoid(z), or dy without a gate) it walks the chunks from the
// last, stores the adjoint of the state leaving chunk c (ws_gout), then
//   g_{c-1} = exp(a S_last) g_c + sum_i exp(a S_i) ybar_i C_i^T
// (C^T of the chunk from ws_Ct, tokens past L weighted 0), starting from dh_last and ending with
// dh0.
template <int Q, int N, bool ADJ = false>
__global__ __launch_bounds__(512) void ssd_state_kernel(SsdParams p) {
  constexpr int KQ = Q / 32;                 // K steps over a chunk
  constexpr int NTW = N / 32;                // state tiles per wave
  constexpr int XPAIRS = Q / 2 * 4;          // (token pair, 16-channel group) items of x
  constexpr int BT16 = N * Q / 8;            // 16-byte pieces of B^T
  static_assert(BT16 % 512 == 0, "B^T pieces divide over the threads");
  static_assert(512 % XPAIRS == 0, "x items repeat evenly over the threads");
  constexpr int BT_PER = BT16 / 512;
  // two buffers of each where they fit beside each other in LDS (chunks of up to 128 tokens)
  constexpr bool kDoubleLds = Q <= 128;
  __shared__ __attribute__((aligned(16))) __bf16 Xs[kDoubleLds ? 2 : 1][kP * (Q + 8)];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[kDoubleLds ? 2 : 1][N * (Q + 8)];
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

  const float* s_init = ADJ ? p.dh_last : p.h0;
  f32x4 acc[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s_init) {
      const float4 v = *reinterpret_cast<const float4*>(s_init + (b * p.H + h) * PN + st_idx(k));
      acc[k] = f32x4{v.x, v.y, v.z, v.w};
    }
  }
  // per-token input: x (forward) or dy (adjoint; z alongside for the gate)
  const bf16_t* xg = static_cast<const bf16_t*>(ADJ ? p.dy : p.x);
  const bf16_t* zg = ADJ ? static_cast<const bf16_t*>(p.z) : nullptr;
  bf16_t* hin_all = static_cast<bf16_t*>(ADJ ? p.ws_gout : p.ws_hin);
  const int64_t bg = b * p.G + h / (p.H / p.G);   // this head's (batch, group)
  const bf16_t* Bt_all = static_cast<const bf16_t*>(ADJ ? p.ws_Ct : p.ws_Bt) + bg * nch * (int64_t)(N * Q);

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
    u32x4 z[ADJ ? 2 : 1][ADJ ? 2 : 1];   // the gate of the same elements (adjoint with z)
    f32x2 sphi[2];      // (S_j, phi_j) of the two tokens
    float s_last;
    u32x4 bt[BT_PER];   // pieces of the chunk's B^T (C^T in the adjoint)
  };
  // (both lambdas are forced inline: the buffers they take by reference must stay in registers)
  auto load_chunk = [&](int64_t c, ChunkIn& in) __attribute__((always_inline)) {
    const float2* sp = p.ws_sphi + ((b * nch + c) * p.H + h) * Q;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * jp + u;
      const int64_t t = c * Q + j < p.L ? c * Q + j : p.L - 1;
      const int64_t off = ((b * p.L + t) * p.H + h) * kP + 16 * pg;
      const u32x4* src = reinterpret_cast<const u32x4*>(xg + off);
      in.x[u][0] = src[0];
      in.x[u][1] = src[1];
      if constexpr (ADJ) {
        if (zg) {
          const u32x4* zs = reinterpret_cast<const u32x4*>(zg + off);
          in.z[u][0] = zs[0];
          in.z[u][1] = zs[1];
        }
      }
      in.sphi[u] = reinterpret_cast<const f32x2*>(sp)[j];
    }
    in.s_last = sp[Q - 1].x;
    const u32x4* bt = reinterpret_cast<const u32x4*>(Bt_all + c * (int64_t)(N * Q));
#pragma unroll
    for (int k = 0; k < BT_PER; ++k) in.bt[k] = bt[tid + 512 * k];
  };

  auto pick = [](const u32x4& v, int q) { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; };
  // chunk of the k-th step: ascending in the forward, descending in the adjoint
  auto chunk_of = [&](int64_t k) { return ADJ ? nch - 1 - k : k; };

  // stage B^T (C^T) and the weighted, transposed x (ybar) of the chunk in `in` into the LDS
  // buffers xsb, bsb; returns the chunk's decay exp(a S_last)
  auto stage = [&](int64_t c, const ChunkIn& in, __bf16* xsb, __bf16* bsb) __attribute__((always_inline)) {
#pragma unroll
    for (int k2 = 0; k2 < BT_PER; ++k2) {
      const int e = tid + 512 * k2;
      const int n = e / (Q / 8), j8 = (e % (Q / 8)) * 8;
      *reinterpret_cast<u32x4*>(&bsb[n * (Q + 8) + j8]) = in.bt[k2];
    }
    float wj[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (ADJ)
        wj[u] = c * Q + 2 * jp + u < p.L ? exp2_fast(a2 * in.sphi[u].x) : 0.f;
      else
        wj[u] = exp2_fast(a2 * (in.s_last - in.sphi[u].x)) * in.sphi[u].y;
    }
    uint32_t* X32 = reinterpret_cast<uint32_t*>(xsb);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t u0 = pick(in.x[0][q >> 3], (q & 7) >> 1);
      const uint32_t u1 = pick(in.x[1][q >> 3], (q & 7) >> 1);
      float f0 = (q & 1) ? bf16_hi(u0) : bf16_lo(u0);
      float f1 = (q & 1) ? bf16_hi(u1) : bf16_lo(u1);
      if constexpr (ADJ) {
        if (zg) {
          const uint32_t v0 = pick(in.z[0][q >> 3], (q & 7) >> 1);
          const uint32_t v1 = pick(in.z[1][q >> 3], (q & 7) >> 1);
          f0 *= silu((q & 1) ? bf16_hi(v0) : bf16_lo(v0));
          f1 *= silu((q & 1) ? bf16_hi(v1) : bf16_lo(v1));
        }
      }
      // word column XORed with 16 pg (inside the row): the four channel groups of a wave
      // write to four different 16-bank ranges
      X32[(16 * pg + q) * ((Q + 8) / 2) + (jp ^ ((16 * pg) & (Q / 2 - 1)))] = pack_bf16x2(f0 * wj[0], f1 * wj[1]);
    }
    return exp2_fast(a2 * in.s_last);
  };
  // the state entering chunk c (the adjoint of the state leaving it), for the output kernel
  // (the backward); then decay it over the chunk
  auto store_and_decay = [&](int64_t c, float decay) __attribute__((always_inline)) {
    bf16_t* hin = hin_all + ((b * nch + c) * p.H + h) * PN;
#pragma unroll
    for (int k2 = 0; k2 < NTW; ++k2) {
      *reinterpret_cast<uint2*>(hin + st_idx(k2)) =
          make_uint2(pack_bf16x2(acc[k2][0], acc[k2][1]), pack_bf16x2(acc[k2][2], acc[k2][3]));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[k2][r] *= decay;
    }
  };
  // acc += (B^T of the chunk) (weighted x^T), operands read one K step ahead into a second
  // register set; the scheduling barriers keep the reads of step kq + 1 ahead of the products
  // of step kq (without them the compiler reuses one register set and waits for each read
  // before its product)
  auto products = [&](const __bf16* xsb, const __bf16* bsb) __attribute__((always_inline)) {
    auto frag_x = [&](int kq) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(&xsb[(16 * pq + r16) * (Q + 8) + ((kq * 32 + 8 * g) ^ ((32 * pq) & (Q - 1)))]);
    };
    auto frag_b = [&](int kq, int k2) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(&bsb[((w2 * NTW + k2) * 16 + r16) * (Q + 8) + kq * 32 + 8 * g]);
    };
    bf16x8 xf[2], bfr[2][NTW];
    xf[0] = frag_x(0);
#pragma unroll
    for (int k2 = 0; k2 < NTW; ++k2) bfr[0][k2] = frag_b(0, k2);
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const int cb = kq & 1;
      if (kq + 1 < KQ) {
        xf[cb ^ 1] = frag_x(kq + 1);
#pragma unroll
        for (int k2 = 0; k2 < NTW; ++k2) bfr[cb ^ 1][k2] = frag_b(kq + 1, k2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k2 = 0; k2 < NTW; ++k2) acc[k2] = mfma16(bfr[cb][k2], xf[cb], acc[k2]);   // (states x tokens) . (tokens x channels)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  ChunkIn buf0, buf1;   // even steps in buf0, odd steps in buf1
  if (nch > 0) {
    load_chunk(chunk_of(0), buf0);
    load_chunk(chunk_of(nch > 1 ? 1 : 0), buf1);
  }
  // wait for the entering state here, once: its loads are conditional, and a first use inside
  // the loop would put a wait for every outstanding load at the head of each step
#pragma unroll
  for (int k = 0; k < NTW; ++k) asm volatile("" : "+v"(acc[k]));
  if constexpr (!kDoubleLds) {
    // one LDS buffer: stage, barrier, products, barrier
    auto process = [&](int64_t k, ChunkIn& cur) __attribute__((always_inline)) {
      const int64_t c = chunk_of(k);
      const float decay = stage(c, cur, Xs[0], Bs[0]);
      load_chunk(chunk_of(k + 2 < nch ? k + 2 : nch - 1), cur);
      store_and_decay(c, decay);
      __syncthreads();
      products(Xs[0], Bs[0]);
      __syncthreads();
    };
    int64_t k = 0;
    for (; k + 1 < nch; k += 2) {
      process(k, buf0);
      process(k + 1, buf1);
    }
    if (k < nch) process(k, buf0);
  } else {
    // two LDS buffers: chunk k + 1 is staged while the products of chunk k run; one barrier
    // per chunk (after it, the next chunk's operands are complete and this chunk's buffer free)
    float dec = 0.f;
    if (nch > 0) {
      dec = stage(chunk_of(0), buf0, Xs[0], Bs[0]);
      load_chunk(chunk_of(nch > 2 ? 2 : nch - 1), buf0);
    }
    __syncthreads();
    // step k: the register buffer `nxt` holds chunk k + 1 (k + 1 < nch), refilled with k + 3
    auto step = [&](int64_t k, ChunkIn& nxt) __attribute__((always_inline)) {
      const int64_t c = chunk_of(k);
      store_and_decay(c, dec);
      if (k + 1 < nch) dec = stage(chunk_of(k + 1), nxt, Xs[(k + 1) & 1], Bs[(k + 1) & 1]);
      // (issued on the last step too, where it is not used: with every load of the loop
      // unconditional the compiler's count of outstanding operations at the loop head is exact)
      load_chunk(chunk_of(k + 3 < nch ? k + 3 : nch - 1), nxt);
      products(Xs[k & 1], Bs[k & 1]);
      __syncthreads();
    };
    int64_t k = 0;
    for (; k + 1 < nch; k += 2) {
      step(k, buf1);
      step(k + 1, buf0);
    }
    if (k < nch) step(k, buf1);
  }

  float* s_out = ADJ ? p.dh0 : p.h_last;
  if (s_out) {
#pragma unroll
    for (int k2 = 0; k2 < NTW; ++k2)
      *reinterpret_cast<float4*>(s_out + (b * p.H + h) * PN + st_idx(k2)) =
          make_float4(acc[k2][0], acc[k2][1], acc[k2][2], acc[k2][3]);
  }
}

}  // namespace
}  // namespace ssm
