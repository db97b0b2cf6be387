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
constexpr int kOutWaves = 8;   // waves per output workgroup

template <int Q, int N>
__global__ __launch_bounds__(64 * kOutWaves) void ssd_out_kernel(SsdParams p) {
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
  {
    // the carried state's loads are issued first, to be in flight during the x staging
    constexpr int kNT = 64 * kOutWaves, kHPer = kP * N / 8 / kNT;
    static_assert((kP * N / 8) % kNT == 0, "the state's 16-byte pieces divide over the threads");
    const bf16_t* hin = static_cast<const bf16_t*>(p.ws_hin) + ((b * nch + c) * p.H + h) * (int64_t)(kP * N);
    uint4 hv[kHPer];
#pragma unroll
    for (int k = 0; k < kHPer; ++k) {
      const int e = tid + k * kNT, row = e / (N / 8), c8 = (e % (N / 8)) * 8;
      hv[k] = *reinterpret_cast<const uint4*>(hin + row * N + c8);
    }
    stage_x_transposed_scaled<Q, kNT>(p, b, c, h, Xt, sp, a2);
#pragma unroll
    for (int k = 0; k < kHPer; ++k) {
      const int e = tid + k * kNT, row = e / (N / 8), c8 = (e % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(&Hs[row * (N + 8) + c8]) = hv[k];
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
  constexpr int kBlocksPerWave = NIB >= 2 * kOutWaves ? NIB / kOutWaves : 1;
  auto block_of = [&](int kb) {
    if (NIB < 2 * kOutWaves) return w;
    const int pair = w + kOutWaves * (kb >> 1);
    return (kb & 1) ? (NIB - 1 - pair) : pair;
  };
  // carried-state fragments (the A operand of the carried term), the same for every row block;
  // every product here is computed transposed (channels x tokens) so a lane ends up holding four
  // consecutive channels of one token
  // (read from LDS at each use: kept in registers they would cost 16 KN / 8 VGPRs per lane)
  auto hfrag = [&](int ks, int pt) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(&Hs[(pt * 16 + r16) * (N + 8) + ks * 32 + 8 * g]);
  };
  auto load_c = [&](int ib, bf16x8 out[KS]) {
    const int64_t ti = c * Q + ib * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      out[ks] = ti < p.L ? load_frag(Cg + ti * rs + ks * 32 + 8 * g) : zero_frag();
  };
  bf16x8 cnext[KS];
  if (NIB >= kOutWaves || w < NIB) load_c(block_of(0), cnext);
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
        for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma16(hfrag(ks, pt), av, acc[pt]);
      }
    }

    // within the chunk: masked G_ij decay phi_j times x_j, two 16-token j tiles per product;
    // the G tiles of the next pair are requested while the current pair is processed
    auto load_g = [&](int jt) {
      return jt <= ib ? *reinterpret_cast<const uint2*>(Grow + jt * 16 + 4 * g) : make_uint2(0, 0);
    };
    // fully unrolled (at most NIB / 2 pairs, leaving at the diagonal): the G tiles are requested
    // kGPairs pairs ahead into registers named by tile, so several tiles' loads are in flight
    // while the current pair is processed
    constexpr int kGPairs = 4;
    uint2 gt[NIB + 2];
#pragma unroll
    for (int t = 0; t < 2 * kGPairs && t < NIB; ++t) gt[t] = load_g(t);
#pragma unroll
    for (int jp = 0; jp < (NIB + 1) / 2; ++jp) {
      if (2 * jp > ib) break;   // uniform (ib is a scalar)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * (jp + kGPairs) + u;
        if (t < NIB) gt[t] = load_g(t);
      }
      const uint2 gcur[2] = {gt[2 * jp], 2 * jp + 1 < NIB ? gt[2 * jp + 1] : make_uint2(0, 0)};
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
          const float Se = sS[jt * 16 + 15];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float Sj = sS[j0 + q];
            const float r = exp2_fast(a2 * (Si - Sj) - fmaxf(a2 * (Se - Sj), kSsdStageExpFloor));
            m[half * 4 + q] = (j0 + q <= il) ? gv[q] * r : 0.f;
          }
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
        out.x = pack_bf16x2(v[0], v[1]);
        out.y = pack_bf16x2(v[2], v[3]);
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
  hipLaunchKernelGGL((ssd_out_kernel<Q, N>), dim3((unsigned)p.H, (unsigned)nch, (unsigned)p.B), dim3(64 * kOutWaves), 0,
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
