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
#include "ssd_device.h"

namespace ssm {
namespace {

// ---------------------------------------------------------------------------- outputs
// Decay of a mask entry (i, j), j <= i: exp(a (S_i - S_j)) phi_j. It factors through the last
// token e of j's 16-token tile:
//   exp(a (S_i - S_e)) * [exp(a (S_e - S_j)) phi_j].
// The bracket depends on j only and is folded into x^T when it is staged, its exponent floored at
// 2^-64 (kSsdStageExpFloor). Off the diagonal (S_i >= S_e) the first factor is one exp per lane and
// tile, <= 1. On the diagonal tile (S_i <= S_e) it is not used: exp(a (S_i - S_e)) overflows once
// |a| times the step sizes of up to 15 tokens exceeds about 88, while the staged bracket underflows.
// There every entry divides the staged factor out of the direct difference instead,
//   2^(a2 (S_i - S_j) - max(a2 (S_e - S_j), -64)),
// whose exponent is at most 64 (it is a2 (S_i - S_e) <= 64 when the floor is not hit, and
// a2 (S_i - S_j) + 64 <= 64 when it is, since S_i >= S_j). So every mask entry is G_ij times a
// bounded factor, with the causal cut j <= i on the diagonal tile.
// One workgroup covers one chunk of one sequence and a run of consecutive heads of one group. The
// chunk's C rows and its G tiles depend only on the group: each wave loads the C fragments of its
// row block into registers once, and the G tiles on and below the diagonal (packed by the prep
// kernel) are copied into LDS once, for every head of the run. Per head only x, the carried-in
// state and the (S, phi) table are read. Those of the next head are loaded into registers while
// the current head is computed; per head a wave computes the carried-state term of its rows,
// waits at a barrier, stages the next head (x^T into the second of two buffers, the carried state,
// whose single buffer all waves have finished reading), then computes the within-chunk term.
template <int Q>
struct SsdOutCfg {
  static constexpr int NIB = Q / 16;                   // 16-row blocks of the chunk
  static constexpr int NW = NIB >= 16 ? 16 : 8;        // waves: one row block each
  static_assert(NIB <= NW, "one row block per wave");
};

template <int Q, int N>
__global__ __launch_bounds__(64 * SsdOutCfg<Q>::NW) void ssd_out_kernel(SsdParams p, int64_t hpw, int64_t wpg) {
  constexpr int NIB = SsdOutCfg<Q>::NIB, NW = SsdOutCfg<Q>::NW;
  constexpr int NT = 64 * NW;
  constexpr int NTILES = NIB * (NIB + 1) / 2; // G tiles on and below the diagonal
  constexpr int KS = N / 32;                  // K steps over the state dimension
  constexpr int XS = Q + 8, HSTR = N + 8;     // LDS row strides (bf16) of x^T and of the state
  constexpr int kItems = (Q / 2) * (kP / 8);  // (token pair, 8-channel group) items of x
  constexpr int XPER = (kItems + NT - 1) / NT;
  static_assert(kItems % NT == 0 || kItems < NT, "the x items divide over the threads");
  constexpr int kHP = kP * N / 8;             // 16-byte pieces of the carried state
  constexpr int HPER = (kHP + NT - 1) / NT;
  static_assert(kHP % NT == 0 || kHP < NT, "the state's pieces divide over the threads");
  __shared__ __attribute__((aligned(16))) __bf16 Gs[NTILES * 256];
  __shared__ __attribute__((aligned(16))) __bf16 Xt[2][kP * XS];
  // the carried-in state h_{c-1} (P x N bf16); rows padded by 8 elements so a wave's 16-byte
  // fragment reads (16 rows apart by one row) hit 64 banks
  __shared__ __attribute__((aligned(16))) __bf16 Hs[kP * HSTR];
  __shared__ float sS[2][Q];

  const int64_t c = blockIdx.y, b = blockIdx.z;
  const int64_t nch = gridDim.y;
  const int64_t hpg = p.H / p.G;                              // heads per group
  const int64_t grp = blockIdx.x / wpg;
  const int64_t h_begin = grp * hpg + (blockIdx.x % wpg) * hpw;
  const int64_t h_end = std::min<int64_t>((grp + 1) * hpg, h_begin + hpw);
  if (h_begin >= h_end) return;   // uniform
  const int nh = (int)(h_end - h_begin);
  const int tid = threadIdx.x;
  // the wave index is the same for all lanes of a wave: readfirstlane lets the compiler keep it
  // (and the row block derived from it) in scalar registers, so branches on it are not divergent
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, r16 = lane & 15;
  // This wave's row block. With 16 blocks over 16 waves, the four waves w = s, s + 4, s + 8,
  // s + 12 take the blocks s, 7 - s, 8 + s, 15 - s (34 tiles of the triangle each), so that the
  // waves sharing a SIMD (waves are dealt to the four SIMDs in turn) carry equal work.
  int ib = w;
  if constexpr (NIB == 16 && NW == 16) {
    const int sm = w & 3, slot = w >> 2;
    ib = slot == 0 ? sm : slot == 1 ? 7 - sm : slot == 2 ? 8 + sm : 15 - sm;
  }
  const bool active = ib < NIB;   // uniform
  // the L-segment of the state pass this chunk belongs to (segment s holds chunks
  // [s nch / S, (s + 1) nch / S))
  int cseg = 0;
  while (cseg + 1 < p.nseg && (int64_t)(cseg + 1) * nch / p.nseg <= c) ++cseg;
  const int64_t L = p.L, H = p.H, rs = p.G * N;   // token row stride of B and C
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  const bf16_t* zg = static_cast<const bf16_t*>(p.z);
  bf16_t* yg = static_cast<bf16_t*>(p.y);

  // ---- per-head inputs, loaded one head ahead into registers. Every load is unconditional:
  // tokens past L read the last token, whose phi is 0 when padded (its staged x is then 0), and
  // threads past the x items repeat the last item (their LDS writes are skipped).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  struct HeadIn {
    u32x4 x0[XPER], x1[XPER];   // tokens 2 jp and 2 jp + 1, 8 channels each
    f32x2 s0[XPER], s1[XPER];   // their (S, phi)
    float se[XPER];             // S at the end of their 16-token tile
    u32x4 hv[HPER];             // pieces of the carried-in state
    u32x4 sv[HPER];             // pieces of the state entering the chunk's segment (segments >= 1)
    float dpre;                 // step sizes of the segment's chunks before this one
  };
  // Addressing: per head a wave-uniform base (the chunk's first row of the head, its (S, phi)
  // table, its carried state) plus per-lane 32-bit byte offsets that are the same for every head
  // (tokens past L clamped to the last token). They stay below 2^31: a chunk of x spans
  // Q H P 2 bytes with Q <= 256, P = 64 and H <= 65535 (checked on the host).
  uint32_t xo0[XPER], xo1[XPER], so0[XPER];
#pragma unroll
  for (int k = 0; k < XPER; ++k) {
    const int gi = std::min(tid + k * NT, kItems - 1);
    const int jp = gi / (kP / 8), pg = gi % (kP / 8);
    const int64_t t0 = std::min<int64_t>(c * Q + 2 * jp, L - 1) - c * Q;
    const int64_t t1 = std::min<int64_t>(c * Q + 2 * jp + 1, L - 1) - c * Q;
    xo0[k] = (uint32_t)((t0 * H * kP + pg * 8) * 2);
    xo1[k] = (uint32_t)((t1 * H * kP + pg * 8) * 2);
    so0[k] = (uint32_t)(2 * jp * 8);
  }
  const bf16_t* xchunk = xg + (b * L + c * Q) * H * kP;   // the chunk's first row, head 0
  auto load_head = [&](int64_t hh, HeadIn& in) __attribute__((always_inline)) {
    const float2* sp = p.ws_sphi + ((b * nch + c) * H + hh) * Q;
    const bf16_t* xh = xchunk + hh * kP;
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
      in.x0[k] = ld_at<u32x4>(xh, xo0[k]);
      in.x1[k] = ld_at<u32x4>(xh, xo1[k]);
      in.s0[k] = ld_at<f32x2>(sp, so0[k]);
      in.s1[k] = ld_at<f32x2>(sp, so0[k] + 8u);
      in.se[k] = ld_at<float>(sp, so0[k] | 120u);   // token (2 jp) | 15
    }
    const bf16_t* hin = static_cast<const bf16_t*>(p.ws_hin) + ((b * nch + c) * H + hh) * (int64_t)(kP * N);
#pragma unroll
    for (int k = 0; k < HPER; ++k) in.hv[k] = ld_at<u32x4>(hin, (uint32_t)(std::min(tid + k * NT, kHP - 1) * 16));
    if (cseg > 0) {   // uniform
      const bf16_t* sin = static_cast<const bf16_t*>(p.ws_seg_in) + ((b * p.nseg + cseg) * H + hh) * (int64_t)(kP * N);
#pragma unroll
      for (int k = 0; k < HPER; ++k) in.sv[k] = ld_at<u32x4>(sin, (uint32_t)(std::min(tid + k * NT, kHP - 1) * 16));
      in.dpre = p.ws_dpre[(b * nch + c) * H + hh];
    }
  };
  // x^T of the head scaled by cp_j = 2^max(a2 (S_e - S_j), -64) phi_j (two tokens of one channel
  // per 32-bit word, word column XORed by xt_swizzle_words) into buffer buf, S (written by the
  // threads of the first channel group of each token pair) and the carried state
  auto stage = [&](const HeadIn& in, int buf, float a2) __attribute__((always_inline)) {
    uint32_t* X32 = reinterpret_cast<uint32_t*>(Xt[buf]);
#pragma unroll
    for (int k = 0; k < XPER; ++k) {
      const int gi = tid + k * NT;
      if (kItems < NT && gi >= kItems) continue;
      const int jp = gi / (kP / 8), pg = gi % (kP / 8);
      const float cp0 = exp2_fast(fmaxf(a2 * (in.se[k] - in.s0[k].x), kSsdStageExpFloor)) * in.s0[k].y;
      const float cp1 = exp2_fast(fmaxf(a2 * (in.se[k] - in.s1[k].x), kSsdStageExpFloor)) * in.s1[k].y;
      if (pg == 0) {
        sS[buf][2 * jp] = in.s0[k].x;
        sS[buf][2 * jp + 1] = in.s1[k].x;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // channels 2q (low halves) and 2q+1 (high halves) of the two tokens
        const int ra = pg * 8 + 2 * q, rb = ra + 1;
        X32[ra * (XS / 2) + (jp ^ xt_swizzle_words<Q>(ra))] = pack_bf16x2(bf16_lo(in.x0[k][q]) * cp0, bf16_lo(in.x1[k][q]) * cp1);
        X32[rb * (XS / 2) + (jp ^ xt_swizzle_words<Q>(rb))] = pack_bf16x2(bf16_hi(in.x0[k][q]) * cp0, bf16_hi(in.x1[k][q]) * cp1);
      }
    }
    // (a chunk of a later L-segment: the state pass started the segment from zero, so the
    // segment's entering state, decayed to the chunk, is added)
    const float fdec = cseg > 0 ? exp2_fast(a2 * in.dpre) : 0.f;
#pragma unroll
    for (int k = 0; k < HPER; ++k) {
      const int e = tid + k * NT, row = e / (N / 8), c8 = (e % (N / 8)) * 8;
      if (kHP < NT && e >= kHP) continue;
      u32x4 hv = in.hv[k];
      if (cseg > 0) {   // uniform
#pragma unroll
        for (int q = 0; q < 4; ++q)
          hv[q] = pack_bf16x2(fmaf(fdec, bf16_lo(in.sv[k][q]), bf16_lo(hv[q])), fmaf(fdec, bf16_hi(in.sv[k][q]), bf16_hi(hv[q])));
      }
      *reinterpret_cast<u32x4*>(&Hs[row * HSTR + c8]) = hv;
    }
  };

  // ---- the group's operands: this wave's C fragments (registers) and the packed G tiles (LDS)
  HeadIn in;
  load_head(h_begin, in);
  bf16x8 cf[KS];   // C rows of the block (B operand of the carried term: column i, k = n)
  {
    const bf16_t* Cg = static_cast<const bf16_t*>(p.Cm) + b * L * rs + grp * N;
    // rows past L take the last token's C: their outputs are never stored
    const int64_t ti = std::min<int64_t>(c * Q + (active ? ib : 0) * 16 + r16, L - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cf[ks] = load_frag(Cg + ti * rs + ks * 32 + 8 * g);
    const u32x4* Gg = reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(p.ws_G) +
                                                     ((b * p.G + grp) * nch + c) * (int64_t)(Q * Q));
    constexpr int kG16 = NTILES * 256 / 8;   // 16-byte pieces
    for (int e = tid; e < kG16; e += NT) reinterpret_cast<u32x4*>(Gs)[e] = Gg[e];
  }
  stage(in, 0, p.A[h_begin] * kLog2e);
  load_head(h_begin + (nh > 1 ? 1 : 0), in);
  __syncthreads();

  // ---- the run of heads. Every product is computed transposed (channels x tokens), so a lane
  // ends up holding four consecutive channels of one token: acc[pt][r] = y[il][pt 16 + 4 g + r].
  const int il = (active ? ib : 0) * 16 + r16;   // this lane's token row of M (B operand)
  // this lane's row of the block's G tiles: G[il][16 jt + 4 g .. + 3] at grow + 256 jt
  const __bf16* grow = &Gs[((active ? ib : 0) * ((active ? ib : 0) + 1) / 2) * 256 + r16 * 16 + 4 * g];
  for (int k = 0; k < nh; ++k) {
    const int64_t hh = h_begin + k;
    const int buf = k & 1;
    const float a2 = p.A[hh] * kLog2e;
    const float* S = sS[buf];
    const float Si = S[il];
    f32x4 acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // carried state: exp(a S_i) (C_i . h_in[p, :]), the row factor applied to the product
    if (active) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          acc[pt] = mfma16(*reinterpret_cast<const bf16x8*>(&Hs[(pt * 16 + r16) * HSTR + ks * 32 + 8 * g]), cf[ks],
                           acc[pt]);
    }
    __syncthreads();   // every wave is done with the carried state of head k
    if (k + 1 < nh) stage(in, buf ^ 1, p.A[hh + 1] * kLog2e);
    // (issued on the last heads too, repeating the last head: with every load of the loop
    // unconditional the compiler's count of outstanding memory operations stays exact)
    load_head(h_begin + std::min(k + 2, nh - 1), in);
    if (active) {
      const float eSi = exp2_fast(a2 * Si);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[pt][r] *= eSi;
      const __bf16* X = Xt[buf];
      // within the chunk: masked G_ij decay phi_j times x_j, two 16-token j tiles per product
      auto pair_product = [&](int jp, const float (&m)[8]) __attribute__((always_inline)) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m[4], m[5]),
                               pack_bf16x2(m[6], m[7])));
        const int jb = jp * 32;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const int sw = 2 * xt_swizzle_words<Q>(pt * 16);   // in bf16 elements, uniform over the wave
          const uint2 lo = *reinterpret_cast<const uint2*>(&X[(pt * 16 + r16) * XS + ((jb + 4 * g) ^ sw)]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&X[(pt * 16 + r16) * XS + ((jb + 16 + 4 * g) ^ sw)]);
          const uint4 pk = make_uint4(lo.x, lo.y, hi.x, hi.y);
          acc[pt] = mfma16(__builtin_bit_cast(bf16x8, pk), av, acc[pt]);
        }
      };
      // an off-diagonal tile jt < ib: G_ij exp(a (S_i - S_e)), one exp per lane and tile
      auto off_tile = [&](int jt, float* m) __attribute__((always_inline)) {
        const uint2 gw = *reinterpret_cast<const uint2*>(grow + jt * 256);
        const float r = exp2_fast(a2 * (Si - S[jt * 16 + 15]));
        m[0] = bf16_lo(gw.x) * r;
        m[1] = bf16_hi(gw.x) * r;
        m[2] = bf16_lo(gw.y) * r;
        m[3] = bf16_hi(gw.y) * r;
      };
      // pairs of two off-diagonal tiles
#pragma unroll 1
      for (int jp = 0; jp < ib / 2; ++jp) {
        float m[8];
        off_tile(2 * jp, m);
        off_tile(2 * jp + 1, m + 4);
        pair_product(jp, m);
      }
      // the pair holding the diagonal tile ib, whose other tile is off-diagonal (ib odd) or above
      // the diagonal (ib even, zero); on the diagonal each entry is
      // 2^(a2 (S_i - S_j) - max(a2 (S_e - S_j), -64)), cut at j <= i
      {
        float m[8];
        const int jd = ib, hd = ib & 1;   // diagonal tile and its half of the pair
        if (hd) off_tile(ib - 1, m);
        const uint2 gw = *reinterpret_cast<const uint2*>(grow + jd * 256);
        const float gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
        const float Se = S[jd * 16 + 15];
        const int j0 = jd * 16 + 4 * g;
        float md[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float Sj = S[j0 + q];
          const float r = exp2_fast(a2 * (Si - Sj) - fmaxf(a2 * (Se - Sj), kSsdStageExpFloor));
          md[q] = (j0 + q <= il) ? gv[q] * r : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (hd) m[4 + q] = md[q];
          else {
            m[q] = md[q];
            m[4 + q] = 0.f;
          }
        }
        pair_product(ib / 2, m);
      }

      // epilogue: D term, gate, store (8-byte loads of x and z, 8-byte store)
      if (c * Q + il < L) {
        const float dsk = p.Dskip && !p.dskip_per_channel ? p.Dskip[hh] : 0.f;
        // byte offset of the lane's output row from the head's first row of the chunk
        const uint32_t orow = (uint32_t)((il * H * kP + 4 * g) * 2);
        const bf16_t* xh = xchunk + hh * kP;
        bf16_t* yh = yg + (b * L + c * Q) * H * kP + hh * kP;
        const bf16_t* zh = zg ? zg + (b * L + c * Q) * H * kP + hh * kP : nullptr;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const uint32_t o = orow + pt * 32;
          float v[4] = {acc[pt][0], acc[pt][1], acc[pt][2], acc[pt][3]};
          if (p.Dskip) {
            const uint2 xr = ld_at<uint2>(xh, o);
            float d[4] = {dsk, dsk, dsk, dsk};
            if (p.dskip_per_channel) {   // channels pt 16 + 4 g .. + 3 of head hh
              const float4 dv = *reinterpret_cast<const float4*>(p.Dskip + hh * kP + pt * 16 + 4 * g);
              d[0] = dv.x; d[1] = dv.y; d[2] = dv.z; d[3] = dv.w;
            }
            v[0] = fmaf(d[0], bf16_lo(xr.x), v[0]);
            v[1] = fmaf(d[1], bf16_hi(xr.x), v[1]);
            v[2] = fmaf(d[2], bf16_lo(xr.y), v[2]);
            v[3] = fmaf(d[3], bf16_hi(xr.y), v[3]);
          }
          if (zh) {
            const uint2 zr = ld_at<uint2>(zh, o);
            v[0] *= silu(bf16_lo(zr.x));
            v[1] *= silu(bf16_hi(zr.x));
            v[2] *= silu(bf16_lo(zr.y));
            v[3] *= silu(bf16_hi(zr.y));
          }
          st_at(yh, o, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
        }
      }
    }
    __syncthreads();   // head k + 1 staged; every wave is done with x^T of head k
  }
}

template <int Q, int N>
hipError_t launch_qn(const SsdParams& p, hipStream_t stream) {
  const int64_t nch = (p.L + Q - 1) / Q;
  hipLaunchKernelGGL((ssd_cumsum_kernel<Q>), dim3((unsigned)((p.H + kCumHeads - 1) / kCumHeads), (unsigned)nch, (unsigned)p.B),
                     dim3(256), 0, stream, p);
  hipLaunchKernelGGL((ssd_prep_kernel<Q, N>), dim3(prep_parts<Q>(), (unsigned)nch, (unsigned)(p.B * p.G)), dim3(256), 0, stream,
                     p);
  // the state pass: 128-token steps (lighter on registers, so two workgroups share a CU), cut
  // into L-segments when the heads alone leave CUs idle; the carry kernel composes the segments
  constexpr int QST = Q < 128 ? Q : 128;
  hipLaunchKernelGGL((ssd_chunk_state_kernel<QST, Q, N>), dim3((unsigned)p.H, (unsigned)p.B, (unsigned)p.nseg),
                     dim3(64 * (N / 32)), 0, stream, p);
  if (p.nseg > 1)
    hipLaunchKernelGGL(ssd_seg_carry_kernel, dim3((unsigned)((kP * N / 4 + 255) / 256), (unsigned)p.H, (unsigned)p.B),
                       dim3(256), 0, stream, p, p.nseg);
  // output workgroups: runs of hpw heads inside one group, wpg runs per group, aiming at one
  // workgroup per CU (256) before splitting a group's heads further
  const int64_t hpg = p.H / p.G;
  int64_t wpg = std::min<int64_t>(hpg, std::max<int64_t>(1, (256 + p.B * nch * p.G - 1) / (p.B * nch * p.G)));
  const int64_t hpw = (hpg + wpg - 1) / wpg;
  wpg = (hpg + hpw - 1) / hpw;
  hipLaunchKernelGGL((ssd_out_kernel<Q, N>), dim3((unsigned)(p.G * wpg), (unsigned)nch, (unsigned)p.B),
                     dim3(64 * SsdOutCfg<Q>::NW), 0, stream, p, hpw, wpg);
  return hipGetLastError();
}

}  // namespace

// Workspace: carried states (bf16), G per chunk and group (bf16), transposed B per chunk and
// group (bf16), (S, phi) per chunk, head and token (float2), each 256-byte aligned.
static size_t ssd_align(size_t n) { return (n + 255) & ~(size_t)255; }

// L-segments of the state pass: enough (batch, head, segment) workgroups for about two per CU
// of MI355X's 256, at most 8 and at most one per chunk.
int64_t ssd_state_segments(int64_t B, int64_t H, int64_t nch) {
  const int64_t chains = std::max<int64_t>(1, B * H);
  return std::max<int64_t>(1, std::min<int64_t>({(512 + chains / 2) / chains, 8, nch}));
}

size_t ssd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q, bool io_f32) {
  const int64_t nch = (L + Q - 1) / Q;
  const int64_t nseg = ssd_state_segments(B, H, nch);
  size_t seg = 0;
  if (nseg > 1)
    seg = ssd_align((size_t)(B * nseg * H * P * N) * 4) + ssd_align((size_t)(B * nseg * H) * 4) +
          ssd_align((size_t)(B * nseg * H * P * N) * 2) + ssd_align((size_t)(B * nch * H) * 4);
  // float32 I/O: bf16 copies of x, z, B, C and y
  const size_t cvt = io_f32 ? 3 * ssd_align((size_t)(B * L * H * P) * 2) + 2 * ssd_align((size_t)(B * L * G * N) * 2) : 0;
  return ssd_align((size_t)(B * nch * H * P * N) * 2) + ssd_align((size_t)(B * G * nch * Q * Q) * 2) +
         ssd_align((size_t)(B * G * nch * N * Q) * 2) + ssd_align((size_t)(B * nch * H * Q) * 8) + seg + cvt;
}

void ssd_workspace_carve(SsdParams& p, void* ws) {
  const int64_t nch = (p.L + p.Q - 1) / p.Q;
  char* base = static_cast<char*>(ws);
  p.ws_hin = base;
  base += ssd_align((size_t)(p.B * nch * p.H * p.P * p.N) * 2);
  p.ws_G = base;
  base += ssd_align((size_t)(p.B * p.G * nch * p.Q * p.Q) * 2);
  p.ws_Btf = base;
  base += ssd_align((size_t)(p.B * p.G * nch * p.N * p.Q) * 2);
  p.ws_sphi = reinterpret_cast<float2*>(base);
  base += ssd_align((size_t)(p.B * nch * p.H * p.Q) * 8);
  p.nseg = (int)ssd_state_segments(p.B, p.H, nch);
  if (p.nseg > 1) {
    p.ws_seg_h = reinterpret_cast<float*>(base);
    base += ssd_align((size_t)(p.B * p.nseg * p.H * p.P * p.N) * 4);
    p.ws_seg_s = reinterpret_cast<float*>(base);
    base += ssd_align((size_t)(p.B * p.nseg * p.H) * 4);
    p.ws_seg_in = base;
    base += ssd_align((size_t)(p.B * p.nseg * p.H * p.P * p.N) * 2);
    p.ws_dpre = reinterpret_cast<float*>(base);
    base += ssd_align((size_t)(p.B * nch * p.H) * 4);
  }
  if (p.io_f32) {
    const size_t tok = ssd_align((size_t)(p.B * p.L * p.H * p.P) * 2), bc = ssd_align((size_t)(p.B * p.L * p.G * p.N) * 2);
    p.cvt_x = base;
    p.cvt_z = base + tok;
    p.cvt_y = base + 2 * tok;
    p.cvt_B = base + 3 * tok;
    p.cvt_C = base + 3 * tok + bc;
  }
}

namespace {
// float32 I/O: n4 groups of four elements rounded to bf16 (nearest even), and widened back
__global__ __launch_bounds__(256) void ssd_f32_to_bf16_kernel(const float* __restrict__ src, bf16_t* __restrict__ dst,
                                                             int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    reinterpret_cast<uint2*>(dst)[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}
__global__ __launch_bounds__(256) void ssd_bf16_to_f32_kernel(const bf16_t* __restrict__ src, float* __restrict__ dst,
                                                             int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const uint2 v = reinterpret_cast<const uint2*>(src)[i];
    reinterpret_cast<float4*>(dst)[i] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
  }
}
dim3 cvt_grid(int64_t n4) { return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 4096))); }

hipError_t launch_ssd_bf16(const SsdParams& p, hipStream_t stream) {
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
}  // namespace

hipError_t launch_ssd(const SsdParams& p, hipStream_t stream) {
  if (!p.io_f32) return launch_ssd_bf16(p, stream);
  // float32 I/O (the element counts are multiples of 4: P = 64, N in {64, 128})
  const int64_t ntok4 = p.B * p.L * p.H * p.P / 4, nbc4 = p.B * p.L * p.G * p.N / 4;
  auto to_bf16 = [&](const void* src, void* dst, int64_t n4) {
    hipLaunchKernelGGL(ssd_f32_to_bf16_kernel, cvt_grid(n4), dim3(256), 0, stream, static_cast<const float*>(src),
                       static_cast<bf16_t*>(dst), n4);
  };
  to_bf16(p.x, p.cvt_x, ntok4);
  if (p.z) to_bf16(p.z, p.cvt_z, ntok4);
  to_bf16(p.Bm, p.cvt_B, nbc4);
  to_bf16(p.Cm, p.cvt_C, nbc4);
  SsdParams q = p;
  q.io_f32 = 0;
  q.delta_f32 = 1;
  q.x = p.cvt_x;
  q.z = p.z ? p.cvt_z : nullptr;
  q.Bm = p.cvt_B;
  q.Cm = p.cvt_C;
  q.y = p.cvt_y;
  const hipError_t e = launch_ssd_bf16(q, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ssd_bf16_to_f32_kernel, cvt_grid(ntok4), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(p.cvt_y), static_cast<float*>(p.y), ntok4);
  return hipGetLastError();
}

}  // namespace ssm
