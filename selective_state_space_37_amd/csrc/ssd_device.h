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

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

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
// grid (ceil(H / 4), chunks, B), 256 threads: per chunk and head the inclusive cumulative sum
// S_j of the step sizes (bias and softplus applied) and the ZOH input scale
// phi_j = expm1(a Delta_j) / a, for the state and output kernels. A workgroup takes 4 heads, so
// the step sizes of a token row come in as one contiguous run (8 bytes in bf16) rather than one
// element 2 H bytes from the next; they pass through LDS (rows padded to a word past the heads),
// and each wave then scans one head. Lane l owns tokens l, l + 64, ...: each 64-token block is one wave
// scan, the blocks are joined by their totals, and every store of the (S, phi) table is 512
// contiguous bytes. Tokens past L get Delta = 0 (identity).
constexpr int kCumHeads = 4;
template <int Q>
__global__ __launch_bounds__(256) void ssd_cumsum_kernel(SsdParams p) {
  static_assert(Q % 64 == 0 && Q <= 256, "chunks of 64, 128 or 256 tokens");
  constexpr int NB = Q / 64;                        // 64-token blocks
  constexpr int E = Q * kCumHeads / 256;            // loaded elements per thread
  constexpr int RS = kCumHeads + 1;                 // LDS row stride (words)
  __shared__ float sDt[Q * RS];
  const int64_t h0 = (int64_t)blockIdx.x * kCumHeads, c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y, H = p.H, L = p.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // every load issued before any is used
  float raw[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int idx = tid + k * 256, row = idx / kCumHeads, hh = idx % kCumHeads;
    const int64_t t = c * Q + row, h = h0 + hh;
    raw[k] = 0.f;
    if (t < L && h < H) {
      const int64_t i = (b * L + t) * H + h;
      raw[k] = p.delta_f32 ? static_cast<const float*>(p.delta)[i] : bf16_to_f32(static_cast<const bf16_t*>(p.delta)[i].bits);
    }
  }
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int idx = tid + k * 256, row = idx / kCumHeads, hh = idx % kCumHeads;
    const int64_t t = c * Q + row, h = h0 + hh;
    float dt = 0.f;
    if (t < L && h < H) {
      dt = raw[k] + (p.delta_bias ? p.delta_bias[h] : 0.f);
      if (p.delta_softplus) dt = softplus_f32(dt);
    }
    sDt[row * RS + hh] = dt;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCumHeads / 4; ++i) {
    const int hh = w * (kCumHeads / 4) + i;
    const int64_t h = h0 + hh;
    if (h >= H) break;   // uniform
    const float a = p.A[h];
    float dt[NB], v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = dt[u] = sDt[(lane + 64 * u) * RS + hh];
    // inclusive scans of the blocks over the wave, interleaved
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float o = __shfl_up(v[u], off, 64);
        if (lane >= off) v[u] += o;
      }
    }
    float2* dst = p.ws_sphi + ((b * nch + c) * H + h) * Q + lane;
    float carry = 0.f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      dst[64 * u] = make_float2(carry + v[u], expm1f(a * dt[u]) / a);
      carry += __shfl(v[u], 63, 64);
    }
  }
}

// ---------------------------------------------------------------------------- prep
// grid (prep_parts<Q>(), chunks, B G), 256 threads.
// (1) B^T (and C^T in the backward) of one group's chunk, written in the order the chunk-state
// kernel reads its MFMA operands (v_mfma_f32_32x32x16_bf16, A = B^T): the piece
// (n, j0 .. j0 + 7) of 32-row tile nt = n / 32 and 16-token step s = j0 / 16 is lane
// n % 32 + 32 ((j0 / 8) % 2) of the 1 KB fragment (nt, s), fragments in the order nt Q / 16 + s,
// so that one fragment load of a wave is 1 KB of consecutive memory. The backward's main kernel
// also gets plain [n][j] copies (ws_Bt, ws_Ct). Part k takes states [k N / parts, (k + 1) N / parts),
// a thread 8 tokens of one state per item (one 16-byte store); spreading the items over every part
// keeps each thread's work to one round trip (the items are few per chunk). Token t's row of the
// group starts at element (t G + grp) N.
// (2) The lower-triangular 16 x 16 tiles of G = C B^T (row blocks ib, column tiles jt <= ib),
// spread over the kPrepParts x 4 waves of a chunk; a wave issues the row loads of all its tiles
// before its first product. BWD: G is stored in float32 (ws_G, [Q][Q]) for the backward's
// elementwise use; the forward packs the tiles (bf16) in row-block order for the output kernel's
// LDS copy.
// Parts per chunk: Q / 16 (measured: 16 parts at 256-token chunks take 19 us against 22 us for
// 4; 64-token chunks take 13 us with 4 parts against 24 us with 16).
template <int Q>
constexpr int prep_parts() { return Q / 16; }
template <int Q, int N, bool BWD = false>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdParams p) {
  constexpr int kPrepParts = prep_parts<Q>();
  static_assert(N % kPrepParts == 0, "the states divide over the parts");
  const int part = blockIdx.x;
  const int64_t c = blockIdx.y, bg = blockIdx.z;   // bg = b G + grp
  const int64_t b = bg / p.G, grp = bg % p.G;
  const int64_t nch = gridDim.y;
  const int tid = threadIdx.x;
  const int64_t rs = p.G * N;                      // token row stride of B and C
  const bf16_t* Bg = static_cast<const bf16_t*>(p.Bm) + b * p.L * rs + grp * N;
  const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * p.L * rs + grp * N;
  const int64_t cbase = (bg * nch + c) * (int64_t)(N * Q);
  auto frag_off = [](int n, int j0) -> int64_t {
    const int frag = (n / 32) * (Q / 16) + j0 / 16, ln = n % 32 + 32 * ((j0 / 8) % 2);
    return (int64_t)frag * 512 + ln * 8;
  };
  // Workgroups go to the XCDs by linear id, and part is its lowest index: the tiles are dealt to
  // the parts rotated by chunk, so that the parts holding the most tiles do not all fall on the
  // same XCDs.
  const int rpart = (int)((part + c + bg) % kPrepParts);
  auto transpose = [&](const bf16_t* src, void* plain, void* frag) {
    constexpr int NQ = N / kPrepParts;
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
      const uint4 v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      *reinterpret_cast<uint4*>(static_cast<bf16_t*>(frag) + cbase + frag_off(n, j0)) = v;
      if constexpr (BWD) *reinterpret_cast<uint4*>(static_cast<bf16_t*>(plain) + cbase + (int64_t)n * Q + j0) = v;
    }
  };
  transpose(Bg, p.ws_Bt, p.ws_Btf);
  if constexpr (BWD) transpose(Cg, p.ws_Ct, p.ws_Ctf);
  // G tiles
  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the row blocks derived from it) in scalar registers, so branches on it are not divergent
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, r16 = lane & 15;
  constexpr int NIB = Q / 16, KS = N / 32, NTILES = NIB * (NIB + 1) / 2;
  constexpr int kWaves = kPrepParts * 4, kPerWave = (NTILES + kWaves - 1) / kWaves;
  bf16x8 ca[kPerWave][KS], bb[kPerWave][KS];
  int tib[kPerWave], tjt[kPerWave];
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int k = rpart * 4 + w + q * kWaves;
    int ib = 0, rem = k < NTILES ? k : 0;
    while (rem > ib) { rem -= ib + 1; ++ib; }
    tib[q] = ib;
    tjt[q] = rem;
    const int64_t ti = c * Q + ib * 16 + r16, tj = c * Q + rem * 16 + r16;   // tokens in the row
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ca[q][ks] = ti < p.L ? load_frag(Cg + ti * rs + ks * 32 + 8 * g) : zero_frag();
      bb[q][ks] = tj < p.L ? load_frag(Bg + tj * rs + ks * 32 + 8 * g) : zero_frag();
    }
  }
  bf16_t* G = static_cast<bf16_t*>(p.ws_G) + (bg * nch + c) * (int64_t)(Q * Q);
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    if (rpart * 4 + w + q * kWaves >= NTILES) break;   // uniform
    const int ib = tib[q], jt = tjt[q];
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16(ca[q][ks], bb[q][ks], acc);  // D[i][j] = sum_n C_i[n] B_j[n]
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
// grid (H, B, segments), N / 32 waves: one head, sequential over its chunks of QS tokens (those of
// one L-segment), with the P x N state in MFMA accumulators. Wave w owns the states n in
// [32 w, 32 w + 32) for every channel p, as two 32 x 32 tiles of D[n][p] (v_mfma_f32_32x32x16_bf16,
// computed transposed: states x channels; output layout: lane l, value v holds column l % 32,
// row 8 (v / 4) + 4 (l / 32) + v % 4).
// The tokens are taken Q at a time (one step): per step the x^T of its Q tokens is staged once,
// and the step's loads are issued at its start (the x of the step one or two ahead, the B^T
// fragments of the next step; see the loop). A step is one or more whole chunks (Q >= QS) or a
// part of one (Q < QS); per chunk,
// at its first part:
//   store h_{c-1} (bf16: the carried state of the output kernel), decay it by exp(a S_last),
// and per part h_c += sum_j B_j^T (w_j x_j), w_j = exp(a (S_last - S_j)) phi_j.
// The B^T operand comes straight from global memory in the prep kernel's fragment order (1 KB of
// consecutive memory per load, each wave reading only its own 32 rows).
//
// Segments (forward only): with several, segment s runs chunks [s nch / S, (s + 1) nch / S), the
// first from h0 and the others from zero; the carried states it stores are then those of the
// segment alone. It leaves its end state (ws_seg_h) and its total sum of step sizes (ws_seg_s),
// and per chunk the sum of the step sizes of the segment's earlier chunks (ws_dpre); the carry
// kernel composes the segments and the output kernel adds the decayed entering state.
//
// ADJ: the same pass run backwards for the adjoint of the state (the backward's dL/dh): with
// ybar = dy z sigmoid(z) (dy without a gate) it walks the chunks from the last, stores the
// adjoint of the state leaving chunk c (ws_gout), then
//   g_{c-1} = exp(a S_last) g_c + sum_i exp(a S_i) ybar_i C_i^T,
// starting from dh_last and ending with dh0.
typedef __attribute__((ext_vector_type(16))) float f32x16;
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int Q, int QS, int N, bool ADJ = false>
__global__ __launch_bounds__(64 * (N / 32)) void ssd_chunk_state_kernel(SsdParams p) {
  constexpr int NW = N / 32, NT = 64 * NW;
  constexpr int UT = Q < QS ? Q : QS;        // tokens of one unit: a chunk, or a part of one
  static_assert(Q % UT == 0 && QS % UT == 0 && UT % 16 == 0, "steps and chunks are whole units");
  constexpr int NU = Q / UT;                 // units per step
  constexpr int PPC = QS / UT;               // units (parts) per chunk
  constexpr int KU = UT / 16;                // 16-token MFMA steps per unit
  constexpr int KQ = Q / 16;                 // ... per step
  constexpr int XS = Q + 8;                  // LDS row stride (bf16) of x^T
  constexpr int kItems = (Q / 2) * (kP / 8); // (token pair, 8-channel group) items of a step's x
  static_assert(kItems % NT == 0 || kItems < NT, "the x items divide over the threads");
  constexpr int XPER = (kItems + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) __bf16 Xs[2][kP * XS];
  // Workgroups go to the 8 XCDs round-robin by linear id. In the segmented forward pass with H a
  // multiple of 8, XCD x takes the heads [x H/8, (x+1) H/8) of each (batch, segment), so heads
  // that sit side by side in every token row of x are read from one XCD at about the same time
  // (89.9 -> 87.9 us at the 80-head layer; the backward's unsegmented passes ran 1.5% slower with
  // it and keep the plain order).
  int64_t h = blockIdx.x;
  if (!ADJ && gridDim.z > 1 && gridDim.x % 8 == 0) {
    const int64_t per = gridDim.x / 8;
    h = (blockIdx.x % 8) * per + blockIdx.x / 8;
  }
  const int64_t b = blockIdx.y, seg = blockIdx.z, nseg = gridDim.z;
  const int64_t L = p.L, H = p.H;
  const int64_t nch = (L + QS - 1) / QS;       // chunks
  const int64_t c_begin = seg * nch / nseg, c_end = (seg + 1) * nch / nseg;
  const int64_t nun = (c_end - c_begin) * PPC; // units of the segment
  const int64_t nst = (nun + NU - 1) / NU;     // steps
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const float a2 = p.A[h] * kLog2e;
  const int64_t PN = (int64_t)kP * N;
  const int64_t bg = b * p.G + h / (H / p.G);   // this head's (batch, group)
  const bf16_t* Bt_all = static_cast<const bf16_t*>(ADJ ? p.ws_Ctf : p.ws_Btf) + bg * nch * (int64_t)(N * QS);
  // unit at position q of step k: its chunk and its first token inside the chunk (units past the
  // segment's end map to a chunk out of [c_begin, c_end) and are never processed)
  auto unit_at = [&](int64_t k, int q, int64_t& c, int& off) __attribute__((always_inline)) {
    const int64_t u = k * NU + q;
    const int64_t ur = ADJ ? nun - 1 - u : u;   // the adjoint takes the units in reverse
    const int64_t cc = ur >= 0 ? ur / PPC : -1;
    c = c_begin + cc;
    off = (int)((ur >= 0 ? ur % PPC : 0) * UT);
    if (u >= nun) c = c_end;                     // past the end
  };
  auto live_chunk = [&](int64_t c) { return c >= c_begin && c < c_end; };
  auto clamp_chunk = [&](int64_t c) -> int64_t { return c < c_begin ? c_begin : (c >= c_end ? c_end - 1 : c); };

  // state element (n, p) of value v of tile pt: n = 32 w + 8 (v / 4) + 4 hi + v % 4, p = 32 pt + l32
  f32x16 acc[2];
  const float* s_init = ADJ ? p.dh_last : (seg == 0 ? p.h0 : nullptr);
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[pt][v] = 0.f;
    if (s_init) {
      const float* src = s_init + (b * H + h) * PN + (int64_t)(32 * pt + l32) * N + 32 * w + 4 * hi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v4 = *reinterpret_cast<const float4*>(src + 8 * k);
        acc[pt][4 * k + 0] = v4.x; acc[pt][4 * k + 1] = v4.y; acc[pt][4 * k + 2] = v4.z; acc[pt][4 * k + 3] = v4.w;
      }
    }
  }
  // The initial state's loads (taken only with a state given) complete here, once: left in flight
  // into the loop, the compiler cannot tell at the loop head whether they are and waits for every
  // outstanding load there on each iteration.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- the x (dy, with z) of a step: item = (token pair jp, channel group pg of 8), so the eight
  // lanes of a row load its 128 bytes in one instruction. Column pair jp of the step belongs to
  // unit q = 2 jp / UT. Tokens past L (and units past the segment) read a valid stand-in and are
  // weighted 0.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  constexpr bool kGate = ADJ;
  struct StepX {
    u32x4 x[XPER][2];                          // [item][token]: 8 channels
    u32x4 z[kGate ? XPER : 1][kGate ? 2 : 1];  // the gate of the same elements
    f32x2 sp[XPER][2];                         // (S, phi) of the two tokens
    float se[XPER];                            // S at the end of their chunk
  };
  const bf16_t* xg = static_cast<const bf16_t*>(ADJ ? p.dy : p.x);
  const bf16_t* zg = ADJ ? static_cast<const bf16_t*>(p.z) : nullptr;
  auto load_x = [&](int64_t k, StepX& in) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < XPER; ++e) {
      const int it = std::min(tid + e * NT, kItems - 1), jp = it / (kP / 8), pg = it % (kP / 8);
      const int q = (2 * jp) / UT, j = (2 * jp) % UT;
      int64_t c;
      int off;
      unit_at(k, q, c, off);
      c = clamp_chunk(c);
      const float2* sp = p.ws_sphi + ((b * nch + c) * H + h) * QS;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t t = std::min<int64_t>(c * QS + off + j + u, L - 1);
        const int64_t o = ((b * L + t) * H + h) * kP + 8 * pg;
        in.x[e][u] = *reinterpret_cast<const u32x4*>(xg + o);
        if constexpr (kGate) {
          if (zg) in.z[e][u] = *reinterpret_cast<const u32x4*>(zg + o);
        }
        in.sp[e][u] = reinterpret_cast<const f32x2*>(sp)[off + j + u];
      }
      in.se[e] = sp[QS - 1].x;
    }
  };
  // x^T of the step weighted per token into buffer xsb (two tokens of one channel per 32-bit
  // word, word column XORed by xt_swizzle_words)
  auto stage = [&](int64_t k, const StepX& in, __bf16* xsb) __attribute__((always_inline)) {
    uint32_t* X32 = reinterpret_cast<uint32_t*>(xsb);
#pragma unroll
    for (int e = 0; e < XPER; ++e) {
      const int it = tid + e * NT, jp = it / (kP / 8), pg = it % (kP / 8);
      if (kItems < NT && it >= kItems) continue;
      const int q = (2 * jp) / UT, j = (2 * jp) % UT;
      int64_t c;
      int off;
      unit_at(k, q, c, off);
      float wt[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool live = live_chunk(c) && c * QS + off + j + u < L;
        const float wv = ADJ ? exp2_fast(a2 * in.sp[e][u].x) : exp2_fast(a2 * (in.se[e] - in.sp[e][u].x)) * in.sp[e][u].y;
        wt[u] = live ? wv : 0.f;
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        // channels 2qq (low halves) and 2qq+1 (high halves) of the two tokens
        float v[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          v[u][0] = bf16_lo(in.x[e][u][qq]);
          v[u][1] = bf16_hi(in.x[e][u][qq]);
          if constexpr (kGate) {
            if (zg) {
              v[u][0] *= silu(bf16_lo(in.z[e][u][qq]));
              v[u][1] *= silu(bf16_hi(in.z[e][u][qq]));
            }
          }
        }
        const int ra = pg * 8 + 2 * qq, rb = ra + 1;
        X32[ra * (XS / 2) + (jp ^ xt_swizzle_words<Q>(ra))] = pack_bf16x2(v[0][0] * wt[0], v[1][0] * wt[1]);
        X32[rb * (XS / 2) + (jp ^ xt_swizzle_words<Q>(rb))] = pack_bf16x2(v[0][1] * wt[0], v[1][1] * wt[1]);
      }
    }
  };
  // B operand of 16-token step s of the staged step: x^T rows p = 32 pt + l32, tokens
  // 16 s + 8 hi .. + 7
  auto frag_x = [&](const __bf16* xsb, int s, int pt) __attribute__((always_inline)) {
    const int row = 32 * pt + l32;
    const int col = 16 * s + 8 * hi;   // in bf16 elements; the XOR swizzle moves whole words
    return *reinterpret_cast<const bf16x8*>(&xsb[row * XS + (col ^ (2 * xt_swizzle_words<Q>(row)))]);
  };
  // A operands of step k: the 1 KB fragments of B^T (C^T) rows 32 w .. + 31 for each unit and
  // 16-token step (units past the segment read a valid stand-in, never used)
  auto load_ring = [&](int64_t k, bf16x8 (&r)[KQ]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      int64_t c;
      int off;
      unit_at(k, q, c, off);
      c = clamp_chunk(c);
#pragma unroll
      for (int s = 0; s < KU; ++s)
        r[q * KU + s] = load_frag(Bt_all + c * (int64_t)(N * QS) + ((int64_t)w * (QS / 16) + off / 16 + s) * 512 + lane * 8);
    }
  };
  bf16_t* hc_all = static_cast<bf16_t*>(ADJ ? p.ws_gout : p.ws_hin);
  auto store_carried = [&](int64_t c) __attribute__((always_inline)) {
    bf16_t* hc = hc_all + ((b * nch + c) * H + h) * PN;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<uint2*>(hc + (int64_t)(32 * pt + l32) * N + 32 * w + 8 * k + 4 * hi) =
            make_uint2(pack_bf16x2(acc[pt][4 * k], acc[pt][4 * k + 1]), pack_bf16x2(acc[pt][4 * k + 2], acc[pt][4 * k + 3]));
  };
  // segments: the sum of the step sizes of the segment's chunks before the current one
  float dsum = 0.f;

  // The step sizes summed over the chunks of step k's units (uniform loads), loaded one step
  // ahead of use.
  auto load_stot = [&](int64_t k, float (&st)[NU]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      int64_t c;
      int off;
      unit_at(k, q, c, off);
      st[q] = p.ws_sphi[((b * nch + clamp_chunk(c)) * H + h) * QS + QS - 1].x;
    }
  };
  // Loads in flight: the x of the next XA steps (XA register sets, by step parity), the B^T
  // fragments of the next step and (XA = 2) its step-size totals (two sets, used by step parity). The loop is
  // unrolled by two so every set is named statically, and within a step the loads are issued in
  // the order they are needed (totals, fragments, then x XA steps ahead): the memory counter
  // completes in order, so each wait then covers only what the step uses. Two steps of x ahead
  // at 128-token steps (the second set fits the registers of two waves per SIMD); one at
  // 256-token steps.
  static_assert(PPC <= 2, "a step covers whole chunks or one half of a chunk");
  constexpr int XA = Q <= 128 ? 2 : 1;
  bf16x8 ringA[KQ], ringB[KQ];
  float stA[NU], stB[NU];
  StepX inA, inB;   // (with XA = 1 only inA is used)
  if (nst > 0) {
    if constexpr (XA == 2) load_stot(0, stA);
    load_ring(0, ringA);
    load_x(0, inA);
    stage(0, inA, Xs[0]);
    if constexpr (XA == 2) {
      load_x(nst > 1 ? 1 : 0, inB);
      load_x(nst > 2 ? 2 : nst - 1, inA);
    } else {
      load_x(nst > 1 ? 1 : 0, inA);
    }
  }
  __syncthreads();
  // step k: START whether its first unit starts a chunk (with two steps of x ahead known at
  // compile time: always with whole chunks per step, on even steps with half chunks, since a
  // segment's first step starts its first chunk). TAIL: a step whose units may run past the
  // segment's end.
  auto step = [&](int64_t k, auto start_tag, auto tail_tag, const bf16x8 (&cur)[KQ], bf16x8 (&nxt)[KQ],
                  const float (&stp)[NU], float (&stn)[NU], StepX& xin) __attribute__((always_inline)) {
    // START: 1 / 0 known at compile time, -1 tested here
    constexpr int START = decltype(start_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;
    const __bf16* xsb = Xs[k & 1];
    // the totals of this step: prefetched with two steps of x in flight; else loaded here (the
    // registers of the 256-token steps are spent on x)
    float stc[NU];
    if constexpr (XA == 2) {
#pragma unroll
      for (int q = 0; q < NU; ++q) stc[q] = stp[q];
    } else {
      load_stot(k, stc);
    }
    // a chunk's first unit in the walk: store the carried state, then decay it over the chunk
    auto chunk_start = [&](int q, int64_t c) __attribute__((always_inline)) {
      store_carried(c);
      if (!ADJ && nseg > 1 && w == 0 && lane == 0) p.ws_dpre[(b * nch + c) * H + h] = dsum;
      dsum += stc[q];
      const float dec = exp2_fast(a2 * stc[q]);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[pt][v] *= dec;
    };
    // The first unit's stores go out before the step's loads, so that the waits of the next step
    // find them older than the loads it needs.
    int64_t c0;
    int off0;
    unit_at(k, 0, c0, off0);
    if constexpr (START == 1) {
      chunk_start(0, c0);
    } else if constexpr (START == -1) {
      if (live_chunk(c0) && off0 == (ADJ ? QS - UT : 0)) chunk_start(0, c0);   // uniform
    }
    // the next step's x^T into the other buffer (free since the last barrier); then the totals and
    // fragments of step k + 1 and the x of step k + 1 + XA (past the end: a repeated step, every
    // load stays unconditional)
    stage(k + 1, xin, Xs[(k + 1) & 1]);
    if constexpr (XA == 2) {
      load_stot(k + 1 < nst ? k + 1 : nst - 1, stn);
      load_ring(k + 1 < nst ? k + 1 : nst - 1, nxt);
      load_x(k + 3 < nst ? k + 3 : nst - 1, xin);
    } else {
      load_x(k + 2 < nst ? k + 2 : nst - 1, xin);
      load_ring(k + 1 < nst ? k + 1 : nst - 1, nxt);
    }
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      int64_t c;
      int off;
      unit_at(k, q, c, off);
      if constexpr (TAIL) {
        if (!live_chunk(c)) break;   // uniform: the remaining units are past the segment
      }
      if (q > 0 && off == (ADJ ? QS - UT : 0)) chunk_start(q, c);
      // x fragments read one step ahead of their products
      bf16x8 xf[2][2];
      xf[0][0] = frag_x(xsb, q * KU, 0);
      xf[0][1] = frag_x(xsb, q * KU, 1);
#pragma unroll
      for (int s = 0; s < KU; ++s) {
        if (s + 1 < KU) {
          xf[(s + 1) & 1][0] = frag_x(xsb, q * KU + s + 1, 0);
          xf[(s + 1) & 1][1] = frag_x(xsb, q * KU + s + 1, 1);
        }
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) acc[pt] = mfma32(cur[q * KU + s], xf[s & 1][pt], acc[pt]);
      }
    }
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using S1 = std::integral_constant<int, 1>;
  using SR = std::integral_constant<int, -1>;
  int64_t k = 0;
  if constexpr (XA == 2) {
    // even steps start a chunk (half chunks per step) or every step does (whole chunks); x of
    // step k + 1 is in the set of k + 1's parity (inB for even k, inA for odd k)
    using OddStart = std::integral_constant<int, PPC == 1 ? 1 : 0>;
    for (; k + 3 < nst; k += 2) {
      step(k, S1{}, F_{}, ringA, ringB, stA, stB, inB);
      step(k + 1, OddStart{}, F_{}, ringB, ringA, stB, stA, inA);
    }
    if (k < nst) step(k, S1{}, T_{}, ringA, ringB, stA, stB, inB);
    if (k + 1 < nst) step(k + 1, OddStart{}, T_{}, ringB, ringA, stB, stA, inA);
    if (k + 2 < nst) step(k + 2, S1{}, T_{}, ringA, ringB, stA, stB, inB);
  } else {
    // (the 256-token steps keep the run-time tests: their registers are full)
    for (; k + 1 < nst; k += 2) {
      step(k, SR{}, T_{}, ringA, ringB, stA, stB, inA);
      step(k + 1, SR{}, T_{}, ringB, ringA, stB, stA, inA);
    }
    if (k < nst) step(k, SR{}, T_{}, ringA, ringB, stA, stB, inA);
  }

  // the end state: the final one (one segment), else the segment's own (for the carry kernel)
  float* fin = ADJ ? p.dh0 : p.h_last;
  float* s_out = nseg > 1 ? p.ws_seg_h + ((b * nseg + seg) * H + h) * PN : (fin ? fin + (b * H + h) * PN : nullptr);
  if (s_out) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      float* dst = s_out + (int64_t)(32 * pt + l32) * N + 32 * w + 4 * hi;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2)
        *reinterpret_cast<float4*>(dst + 8 * k2) =
            make_float4(acc[pt][4 * k2], acc[pt][4 * k2 + 1], acc[pt][4 * k2 + 2], acc[pt][4 * k2 + 3]);
    }
  }
  if (nseg > 1 && tid == 0) p.ws_seg_s[(b * nseg + seg) * H + h] = dsum;
}

// grid (ceil(P N / 4 / 256), H, B): composes the segments of the chunk-state pass. The state
// entering segment s >= 1 is h_in[s] = exp(a S[s-1]) h_in[s-1] + e[s-1] with h_in[1] = e[0]:
// segment 0 ran from h0, so its end state e[0] already holds h0's part, while every later e[s]
// is the segment's own (from zero); S are the segments' sums of step sizes. h_in[s] for s >= 1
// goes to ws_seg_in (bf16, for the output kernel) and the state after the last segment to h_last.
__global__ __launch_bounds__(256) void ssd_seg_carry_kernel(SsdParams p, int nseg) {
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int64_t PN = p.P * p.N;
  const int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4 consecutive states
  if (e4 * 4 >= PN) return;
  const float a2 = p.A[h] * kLog2e;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);   // (h0 is inside e[0])
  for (int s = 0; s < nseg; ++s) {
    if (s > 0) {
      bf16_t* dst = static_cast<bf16_t*>(p.ws_seg_in) + ((b * nseg + s) * p.H + h) * PN + e4 * 4;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
    const float d = exp2_fast(a2 * p.ws_seg_s[(b * nseg + s) * p.H + h]);
    const float4 e = reinterpret_cast<const float4*>(p.ws_seg_h + ((b * nseg + s) * p.H + h) * PN)[e4];
    v = make_float4(fmaf(d, v.x, e.x), fmaf(d, v.y, e.y), fmaf(d, v.z, e.z), fmaf(d, v.w, e.w));
  }
  if (p.h_last) reinterpret_cast<float4*>(p.h_last + (b * p.H + h) * PN)[e4] = v;
}

}  // namespace
}  // namespace ssm
