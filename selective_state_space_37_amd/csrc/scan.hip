// Selective scan (S6) forward on gfx950.
//
// What is computed (pages "Beyond attention: exploring Mamba and state space models",
// state-space basics and selective-SSM sections; "Mamba and state space models", section
// "scan on the chip"): per token and channel, Delta = softplus(delta + bias), then for each of
// the N states Abar = exp(Delta A), h = Abar h + expm1(Delta A)/A * B_t x_t, the readout
// y = C_t . h + D x, and the optional gate y * z * sigmoid(z). The N-wide state stays in
// registers for the whole sequence and is never written to HBM; only y (and the final state)
// leave the chip.
//
// Work split (one workgroup = CH channels of one sequence, one L-segment):
//   * the N states of a channel are cut into KS slices of NS states; thread tid owns slice
//     tid / CH of channel tid % CH, so the readout of a channel is split over KS lanes.
//     At N = 16 the split is CH = 32, NS = 2, KS = 8: 256 threads, and the layer workload
//     (8 x 5120 channels) becomes 1280 workgroups -- exactly five per CU and five waves per SIMD
//     on MI355X's 256 CUs, so no SIMD carries an extra wave at the end.
//   * T-token tiles of (Delta, x) pairs (Delta activated once per element by the loader), z in
//     its storage type, and (B_n, C_n) pairs are staged through LDS with wide coalesced loads,
//     double buffered: the global loads of tile i+1 are in flight while tile i runs, and the loop
//     waits for memory once per tile (at the commit of the next tile; the y stores of a tile are
//     issued after that commit). Per token a lane then needs one 8-byte and one 16-byte LDS read.
//   * each lane writes its partial readout to LDS; after a barrier the threads split the tile's
//     (token, channel) outputs, add the KS partials in a fixed order (deterministic), add D x,
//     gate, round and store y with coalesced row stores.
//   * padded tokens (ragged L tail) are committed with Delta = 0, x = 0 and B = C = 0, which
//     makes the step the identity.
// Long, narrow inputs (few channel tiles) are cut into L-segments that run side by side. Every
// segment after the first starts from the zero state (the first from h0); besides its outputs
// it leaves its local end state h_loc and its sum of Delta. The state entering a segment then
// follows from the affine segment maps h -> exp(A sum Delta_s) h + h_loc[s] (an associative scan
// over segments), and the part of each output that the entering state contributes,
// C_t . exp(A S_t) h_in (S_t = sum of Delta from the segment start through t), is added
// afterwards for the tokens where that decay is still visible (scan_seg.hip). Segments exchange
// nothing but the state, as the pages' chunked view says.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace ssm {

namespace {

template <int CH, int NS, int KS, int T, int N, int GW>
struct ScanCfg {
  static_assert(NS * KS == N, "slices must cover the state");
  static_assert(T % KS == 0, "post-processing splits a tile's tokens over the slices");
  static constexpr int kThreads = CH * KS;
  static constexpr int kGroups = T * (CH / GW);                     // GW-channel groups per tensor
  static constexpr int kGroupsPerThr = (kGroups + kThreads - 1) / kThreads;
  static constexpr int kBC = T * N;                                  // B (and C) elements per tile
  static constexpr int kBCPerThr = (kBC + kThreads - 1) / kThreads;
};

// Raw storage bits of GW consecutive elements of io_t (kept unconverted while a load is in
// flight), with a buffer load and the conversion to float.
template <typename io_t, int GW> struct RawGroup;
template <> struct RawGroup<bf16_t, 2> {
  using type = uint32_t;
  __device__ __forceinline__ static type zero() { return 0u; }
  __device__ __forceinline__ static void load(Rsrc r, uint32_t off, type& v) {
    v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ static void unpack(type v, float* out) { out[0] = bf16_lo(v); out[1] = bf16_hi(v); }
};
template <> struct RawGroup<float, 2> {
  using type = uint2;
  __device__ __forceinline__ static type zero() { return make_uint2(0, 0); }
  __device__ __forceinline__ static void load(Rsrc r, uint32_t off, type& v) { buf_load(r, off, v); }
  __device__ __forceinline__ static void unpack(type v, float* out) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  }
};
template <typename io_t> struct RawGroup<io_t, 4> {
  using type = typename IoTraits<io_t>::raw4;
  __device__ __forceinline__ static type zero() { return IoTraits<io_t>::zero4(); }
  __device__ __forceinline__ static void load(Rsrc r, uint32_t off, type& v) { buf_load(r, off, v); }
  __device__ __forceinline__ static void unpack(type v, float* out) { IoTraits<io_t>::unpack4(v, out); }
};

// 16-byte chunking of a tile's B (and C) block in storage type io_t.
template <typename io_t, int T, int N, int kThreads>
struct BCChunks {
  static constexpr int kPerChunk = 16 / (int)sizeof(io_t);          // elements per 16 bytes
  static constexpr int kChunks = T * N / kPerChunk;
  static_assert((T * N) % kPerChunk == 0, "a tile's B block is whole 16-byte chunks");
  static_assert(kChunks <= kThreads, "one chunk per loading thread");
};

// OCC = waves per SIMD the launch plan needs resident (five at N = 16: <= 96 VGPRs per lane, as
// registers are allocated in blocks of 8 out of 512).
// CONV: the SSM input is the causal depthwise convolution (width <= 4) of x, formed by the loader
// (prefill in front of the decode step's convolution register).
// SEG (with FULL): one segment of a multi-segment plan: segments after the first start from the
// zero state; the local end state, the segment's sum of Delta and whether any Delta was negative
// go to the workspace (the final state is the carry pass's).
template <typename io_t, int CH, int NS, int KS, int T, int N, bool FULL, int OCC, bool CONV = false,
          bool SEG = false>
__global__ __launch_bounds__(CH * KS)
void scan_kernel(ScanParams p) {
  static_assert(FULL || !SEG, "the segment variant is a full pass");
  // Loader groups: GW consecutive channels of one token row per thread and tensor. Two spread
  // the loading and its conversion over every thread of the workgroup (all waves reach the tile
  // barrier with the same work); the convolution variant keeps groups of four, whose three halo
  // rows it also loads.
  constexpr int GW = CONV ? 4 : 2;
  using Cfg = ScanCfg<CH, NS, KS, T, N, GW>;
  using Io = IoTraits<io_t>;
  using raw4 = typename Io::raw4;
  using RG = RawGroup<io_t, GW>;
  using rawg = typename RG::type;
  static_assert(Cfg::kThreads % (CH / GW) == 0, "a thread always loads the same channel group");

  __shared__ __attribute__((aligned(16))) float2 s_dx[2][T][CH];          // (Delta, x)
  __shared__ __attribute__((aligned(16))) rawg s_z[FULL ? 2 : 1][FULL ? T : 1][CH / GW];
  __shared__ __attribute__((aligned(16))) float s_bc[2][T][N][2];          // (B_n, C_n)
  // partial readouts per slice; at CH = 32 a wave holds two slices, whose rows are offset by 32
  // banks so their writes do not collide
  // (only when the padding still lets OCC workgroups share a CU's 160 KB of LDS)
  constexpr int kLdsUnpadded = 2 * T * CH * 8 + (FULL ? 2 * T * (CH / GW) * (int)sizeof(rawg) : 16) +
                               2 * T * N * 8 + (FULL ? KS * T * CH * 4 : 4) +
                               (CONV ? CH * 16 + CH * 4 + 3 * CH * 4 + CH * 4 : 0);
  constexpr bool kPadY = FULL && CH < 64 && kLdsUnpadded + KS * 32 * 4 <= 163840 / OCC;
  constexpr int kYStride = FULL ? T * CH + (kPadY ? 32 : 0) : 1;
  __shared__ float s_y[FULL ? KS : 1][kYStride];
  // convolution: per channel the weights by lag (lag 0 = the newest input; zero past the width
  // or past D) and the bias, and the raw inputs before the sequence (the incoming register),
  // newest first
  __shared__ __attribute__((aligned(16))) float4 s_cw[CONV ? CH : 1];
  __shared__ __attribute__((aligned(16))) float s_cb[CONV ? CH : 4];
  __shared__ float s_cin[CONV ? 3 : 1][CONV ? CH : 1];
  __shared__ __attribute__((aligned(16))) float s_db[CONV ? CH : 4];

  const int tid = threadIdx.x;
  const int64_t D = p.D, L = p.L;
  // Workgroups are dispatched to the 8 XCDs round-robin by linear id. A CH-channel tile reads
  // half of each 128-byte line at CH = 32, so tiles 2k and 2k+1 are given linear ids 8 apart
  // (same XCD, same L2) to fetch each line from HBM once.
  int64_t tile, b, seg;
  {
    const int64_t gx = gridDim.x, gxy = gx * gridDim.y;
    const int64_t lin = blockIdx.x + gx * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t total = gxy * gridDim.z;
    int64_t logical = lin;
    if (CH < 64 && (lin | 15) < total) {
      const int64_t r = lin & 15;
      logical = (lin & ~(int64_t)15) + 2 * (r & 7) + (r >> 3);
    }
    // uniform over the workgroup: keep them in scalar registers (the 64-bit divisions above
    // partly run on the vector unit)
    tile = __builtin_amdgcn_readfirstlane((uint32_t)(logical % gx));
    b = __builtin_amdgcn_readfirstlane((uint32_t)((logical / gx) % gridDim.y));
    seg = __builtin_amdgcn_readfirstlane((uint32_t)(logical / gxy));
  }
  const int64_t c0 = tile * CH;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < L) ? t_begin + p.seg_len : L;
  const int ntiles = (int)((t_end - t_begin + T - 1) / T);

  const io_t* __restrict__ xg = static_cast<const io_t*>(p.x);
  const io_t* __restrict__ dg = static_cast<const io_t*>(p.delta);
  const io_t* __restrict__ zg = static_cast<const io_t*>(p.z);
  const io_t* __restrict__ Bg = static_cast<const io_t*>(p.Bm);
  const io_t* __restrict__ Cg = static_cast<const io_t*>(p.Cm);
  const bool has_z = FULL && (zg != nullptr);

  // ---- loader: this thread always handles channel group tid % (CH / GW)
  const int cg = tid % (CH / GW);
  const int64_t cgl = c0 + GW * cg;
  const bool cg_ok = cgl < D;  // D % 4 == 0: a group is wholly in or out
  // (the convolution variant keeps the step-size bias in LDS instead: registers for its halo rows)
  float biasg[GW];
#pragma unroll
  for (int k = 0; k < GW; ++k) biasg[k] = 0.f;
  if (!CONV && p.delta_bias && cg_ok)
#pragma unroll
    for (int k = 0; k < GW; ++k) biasg[k] = p.delta_bias[cgl + k];

  // segment variant: this thread's sum of the activated Delta of its channel group, and whether
  // any was negative (rows past the segment end commit Delta = 0)
  float dacc[SEG ? GW : 1];
#pragma unroll
  for (int k = 0; k < (SEG ? GW : 1); ++k) dacc[k] = 0.f;
  bool dneg = false;
  // Raw load registers (zeroed once for the threads that load nothing; z stays zero without z)
  rawg rx[Cfg::kGroupsPerThr], rd[Cfg::kGroupsPerThr], rz[Cfg::kGroupsPerThr];
#pragma unroll
  for (int k = 0; k < Cfg::kGroupsPerThr; ++k) rx[k] = rd[k] = rz[k] = RG::zero();
  // convolution: the x rows r-1 .. r-3 of each loaded row (lags 1..3) in registers; weights, bias
  // and the register entries before the sequence in LDS
  raw4 rxh[CONV ? Cfg::kGroupsPerThr : 1][3];
#pragma unroll
  for (int k = 0; k < (CONV ? Cfg::kGroupsPerThr : 1); ++k) rxh[k][0] = rxh[k][1] = rxh[k][2] = Io::zero4();
  if constexpr (CONV) {
    const int W = p.conv_W;
    if (tid < CH) {
      const bool ok = c0 + tid < D;
      float wl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wl[j] = (ok && j < W) ? p.conv_w[(c0 + tid) * W + (W - 1 - j)] : 0.f;
      s_cw[tid] = make_float4(wl[0], wl[1], wl[2], wl[3]);
      s_cb[tid] = (ok && p.conv_b) ? p.conv_b[c0 + tid] : 0.f;
      s_db[tid] = (ok && p.delta_bias) ? p.delta_bias[c0 + tid] : 0.f;
      // read through a descriptor with a uniform base (no per-lane copy of a shared address)
      constexpr int kEs = (int)sizeof(io_t);
      const Rsrc hc = make_rsrc(static_cast<const char*>(p.conv_in) + (b * D + c0) * W * kEs,
                                p.conv_in ? (int)((D - c0) * W * kEs) : 0);
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float v = 0.f;
        if (m < W) v = Io::from_bits(buf_load_bits(hc, (uint32_t)((tid * W + (W - 1 - m)) * kEs), (io_t*)nullptr));
        s_cin[m][tid] = (c0 + tid < D) ? v : 0.f;
      }
    }
    __syncthreads();
  }
  // B and C of a tile are T * N consecutive elements. When a row of N elements is whole 16-byte
  // chunks they move as chunks (threads below kChunks, a chunk never straddles a row, so a row
  // past the segment end reads as whole zero chunks); otherwise element by element. Either way the
  // registers keep the raw storage bits until the tile is committed, so the loads of tile i+1
  // stay in flight while tile i runs.
  // Outside the convolution variant, with N even, B and C move as element pairs instead, spread
  // over the workgroup: slot s < T N / 2 is the pair 2s, 2s + 1 of B, the next T N / 2 slots those
  // of C (a pair never straddles a row, so a row past the segment end reads as a zero pair).
  using BCC = BCChunks<io_t, T, N, Cfg::kThreads>;
  constexpr bool kPairBC = !CONV && N % 2 == 0;
  constexpr int kBCPairs = T * N / 2;
  constexpr int kBCSlots = FULL ? 2 * kBCPairs : kBCPairs;
  constexpr int kBCSlotsPerThr = (kBCSlots + Cfg::kThreads - 1) / Cfg::kThreads;
  using RP = RawGroup<io_t, 2>;
  typename RP::type rbc[kPairBC ? kBCSlotsPerThr : 1];
#pragma unroll
  for (int k = 0; k < (kPairBC ? kBCSlotsPerThr : 1); ++k) rbc[k] = RP::zero();
  constexpr bool kChunkBC = !kPairBC && N * (int)sizeof(io_t) >= 16;
  uint4 rbv = make_uint4(0, 0, 0, 0), rcv = make_uint4(0, 0, 0, 0);
  uint32_t rB[Cfg::kBCPerThr], rC[Cfg::kBCPerThr];
#pragma unroll
  for (int k = 0; k < Cfg::kBCPerThr; ++k) rB[k] = rC[k] = 0u;
  // tiles [0, n_full) have all T rows inside the segment (uniform 32-bit test)
  const int n_full = (int)((t_end - t_begin) / T);
  // Addressing: a tile's block of x / delta / z / y (T rows of D, from channel c0) and of B / C
  // (T rows of N) is one buffer descriptor (scalar registers, rebuilt per tile); each lane adds a
  // 32-bit byte offset that is the same for every tile (T D size < 2^31 since D <= 2^24, checked
  // on the host). Channel groups past D read the next row or zeros and are never stored.
  const int64_t seg_row0 = b * L + t_begin;
  uint32_t ld_boff[Cfg::kGroupsPerThr];
#pragma unroll
  for (int k = 0; k < Cfg::kGroupsPerThr; ++k) {
    const int g = tid + k * Cfg::kThreads;
    ld_boff[k] = (uint32_t)(((g / (CH / GW)) * D + GW * cg) * (int64_t)sizeof(io_t));
  }
  // rows of the tile inside the segment (T on the full tiles)
  auto tile_rows = [&](int tile) __attribute__((always_inline)) {
    return tile < n_full ? T : (int)(t_end - t_begin - (int64_t)tile * T);
  };
  // descriptor of the tile's block of a [*, row_len] tensor from column col0, ending with the
  // tile's last row inside the segment
  auto tile_rsrc = [&](const void* base, int64_t row_len, int64_t col0, int tile, int rows)
      __attribute__((always_inline)) {
    const char* blk = static_cast<const char*>(base) +
                      ((seg_row0 + (int64_t)tile * T) * row_len + col0) * (int64_t)sizeof(io_t);
    return make_rsrc(blk, (int)((rows * row_len - col0) * (int64_t)sizeof(io_t)));
  };

  // (the lambdas below are forced inline: what they capture by reference must stay in registers)
  auto issue_loads = [&](int tile) __attribute__((always_inline)) {
    const int rows = tile_rows(tile);
    const Rsrc xr = tile_rsrc(xg, D, c0, tile, rows);
    const Rsrc dr = tile_rsrc(dg, D, c0, tile, rows);
    const Rsrc zr = has_z ? tile_rsrc(zg, D, c0, tile, rows) : xr;
#pragma unroll
    for (int k = 0; k < Cfg::kGroupsPerThr; ++k) {
      if (tid + k * Cfg::kThreads < Cfg::kGroups) {
        RG::load(xr, ld_boff[k], rx[k]);
        RG::load(dr, ld_boff[k], rd[k]);
        if (has_z) RG::load(zr, ld_boff[k], rz[k]);
      }
    }
    if constexpr (CONV) {
      // rows r-1 .. r-3 of x for the convolution. Segments start at multiples of 16 tokens, so a
      // tile either starts the sequence or has three rows of x before it.
      // At the sequence's first tile the descriptor starts at the tile and the offsets of rows
      // before it wrap past 2^31: out of range, they read zero (the register supplies them at
      // commit).
      constexpr uint32_t kEs = sizeof(io_t);
      const uint32_t row_b = (uint32_t)D * kEs;
      const bool first = t_begin + (int64_t)tile * T == 0;
      const int64_t hrow = seg_row0 + (int64_t)tile * T - (first ? 0 : 3);
      const Rsrc hr = make_rsrc(reinterpret_cast<const char*>(xg) + (hrow * D + c0) * (int64_t)kEs,
                                (int)(((rows + (first ? 0 : 3)) * D - c0) * (int64_t)kEs));
      const uint32_t hoff = first ? 3u * row_b : 0u;
#pragma unroll
      for (int k = 0; k < Cfg::kGroupsPerThr; ++k)
        if (tid + k * Cfg::kThreads < Cfg::kGroups)
#pragma unroll
          for (int j = 1; j <= 3; ++j)
            buf_load(hr, ld_boff[k] + (uint32_t)(3 - j) * row_b - hoff, rxh[k][j - 1]);
    }
    const Rsrc br = tile_rsrc(Bg, N, 0, tile, rows);
    const Rsrc cr = tile_rsrc(Cg, N, 0, tile, rows);
    if constexpr (kPairBC) {
#pragma unroll
      for (int k = 0; k < kBCSlotsPerThr; ++k) {
        const int sl = tid + k * Cfg::kThreads;
        if (sl < kBCPairs)
          RP::load(br, (uint32_t)(2 * sl * (int)sizeof(io_t)), rbc[k]);
        else if (sl < kBCSlots)
          RP::load(cr, (uint32_t)(2 * (sl - kBCPairs) * (int)sizeof(io_t)), rbc[k]);
      }
    } else if constexpr (kChunkBC) {
      if (tid < BCC::kChunks) {
        buf_load(br, (uint32_t)tid * 16u, rbv);
        if (FULL) buf_load(cr, (uint32_t)tid * 16u, rcv);
      }
    } else {
#pragma unroll
      for (int k = 0; k < Cfg::kBCPerThr; ++k) {
        const int e = tid + k * Cfg::kThreads;
        if (e < Cfg::kBC) {
          rB[k] = buf_load_bits(br, (uint32_t)e * (uint32_t)sizeof(io_t), (io_t*)nullptr);
          if (FULL) rC[k] = buf_load_bits(cr, (uint32_t)e * (uint32_t)sizeof(io_t), (io_t*)nullptr);
        }
      }
    }
  };

  // Rows past the segment end (ragged last tile) load as x = 0, B = C = 0 and Delta = 0, and Delta
  // is committed as 0 after the bias and softplus as well: the identity step. RAGGED is a
  // compile-time switch so that full tiles carry no row tests at all.
  // FIRST: the sequence's first tile (only ever the prologue's commit), whose rows before the
  // sequence take the register for the convolution.
  auto commit_impl = [&](auto ragged_tag, auto first_tag, int tile, int buf) __attribute__((always_inline)) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const int rows = tile_rows(tile);
#pragma unroll
    for (int k = 0; k < Cfg::kGroupsPerThr; ++k) {
      const int g = tid + k * Cfg::kThreads;
      if (g < Cfg::kGroups) {
        const int r = g / (CH / GW);
        float xv[GW];
        RG::unpack(rx[k], xv);
        // (the convolution first: its halo registers are free before the step-size arithmetic)
        if constexpr (CONV) {
          // SSM input = bias + sum over lags j of w_j x_{t-j}; rows before the sequence come from
          // the register
          float xs[3][4];
#pragma unroll
          for (int j = 0; j < 3; ++j) Io::unpack4(rxh[k][j], xs[j]);
          if constexpr (FIRST) {
#pragma unroll
            for (int j = 1; j <= 3; ++j)
              if (r < j)
#pragma unroll
                for (int q = 0; q < 4; ++q) xs[j - 1][q] = s_cin[j - r - 1][4 * cg + q];
          }
          const float4 b4 = *reinterpret_cast<const float4*>(&s_cb[4 * cg]);
          const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 w = s_cw[4 * cg + q];
            float u = fmaf(w.x, xv[q], bq[q]);
            u = fmaf(w.y, xs[0][q], u);
            u = fmaf(w.z, xs[1][q], u);
            xv[q] = fmaf(w.w, xs[2][q], u);
          }
        }
        float dv[GW];
        RG::unpack(rd[k], dv);
        float db[GW];
#pragma unroll
        for (int q = 0; q < GW; ++q) db[q] = biasg[q];
        if constexpr (CONV) {
#pragma unroll
          for (int q = 0; q < GW; ++q) db[q] = s_db[GW * cg + q];
        }
#pragma unroll
        for (int q = 0; q < GW; ++q) {
          float u = dv[q] + db[q];   // zero without a bias
          if (p.delta_softplus) u = softplus_f32(u);
          dv[q] = (!RAGGED || r < rows) ? u : 0.f;
          if constexpr (SEG) {
            dacc[q] += dv[q];
            dneg = dneg || dv[q] < 0.f;
          }
        }
        float4* dst = reinterpret_cast<float4*>(&s_dx[buf][r][GW * cg]);
#pragma unroll
        for (int q = 0; q < GW / 2; ++q) dst[q] = make_float4(dv[2 * q], xv[2 * q], dv[2 * q + 1], xv[2 * q + 1]);
        if (has_z) s_z[buf][r][cg] = rz[k];
      }
    }
  };
  // B and C: rows past the segment end were loaded as zeros, so both tile kinds commit alike
  auto commit_bc = [&](int buf) __attribute__((always_inline)) {
    if constexpr (kPairBC) {
#pragma unroll
      for (int k = 0; k < kBCSlotsPerThr; ++k) {
        const int sl = tid + k * Cfg::kThreads;
        if (sl < kBCSlots) {
          const int which = sl < kBCPairs ? 0 : 1;            // B or C
          const int e = 2 * (sl - which * kBCPairs);           // first element of the pair
          float v[2];
          RP::unpack(rbc[k], v);
          float* bc = &s_bc[buf][0][0][0] + 2 * e + which;      // (B_n, C_n) interleaved
          bc[0] = v[0];
          bc[2] = v[1];
        }
      }
    } else if constexpr (kChunkBC) {
      if (tid < BCC::kChunks) {
        // kPerChunk consecutive (B, C) elements -> interleaved (B_n, C_n) pairs
        float bv[BCC::kPerChunk], cv[BCC::kPerChunk];
        Io::unpack_chunk(rbv, bv);
        if (FULL) Io::unpack_chunk(rcv, cv);
        float4* bc = reinterpret_cast<float4*>(&s_bc[buf][0][0][0] + 2 * tid * BCC::kPerChunk);
#pragma unroll
        for (int q = 0; q < BCC::kPerChunk / 2; ++q)
          bc[q] = make_float4(bv[2 * q], FULL ? cv[2 * q] : 0.f, bv[2 * q + 1], FULL ? cv[2 * q + 1] : 0.f);
      }
    } else {
#pragma unroll
      for (int k = 0; k < Cfg::kBCPerThr; ++k) {
        const int e = tid + k * Cfg::kThreads;
        if (e < Cfg::kBC) {
          float* bc = &s_bc[buf][0][0][0] + 2 * e;
          bc[0] = Io::from_bits(rB[k]);
          if (FULL) bc[1] = Io::from_bits(rC[k]);
        }
      }
    }
  };
  auto commit_tile = [&](int tile, int buf) __attribute__((always_inline)) {
    if (tile < n_full) commit_impl(std::false_type{}, std::false_type{}, tile, buf);
    else commit_impl(std::true_type{}, std::false_type{}, tile, buf);
    commit_bc(buf);
  };
  auto commit_first_tile = [&]() __attribute__((always_inline)) {
    if (CONV && t_begin == 0) {
      if (0 < n_full) commit_impl(std::false_type{}, std::true_type{}, 0, 0);
      else commit_impl(std::true_type{}, std::true_type{}, 0, 0);
      commit_bc(0);
    } else {
      commit_tile(0, 0);
    }
  };

  // ---- per-lane recurrence constants: channel c, states n0 .. n0+NS-1
  const int slice = tid / CH;
  const int chl = tid % CH;
  const int64_t c = c0 + chl;
  const bool c_ok = c < D;
  const int n0 = slice * NS;
  float a2[NS], ia[NS], h[NS];
  float amin = INFINITY;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float a = c_ok ? p.A[c * N + n0 + j] : -1.0f;
    a2[j] = a * kLog2e;
    ia[j] = 1.0f / a;
    h[j] = 0.f;
    amin = fminf(amin, fabsf(a2[j]));
  }
  // |Delta| below this puts some state of the lane under the series bound |Delta a2| < kZohSeriesT
  // (with a margin against rounding; a lane with a zero a2 always qualifies)
  const float series_dmax = kZohSeriesT * 1.01f / amin;
  // the sequence's first segment starts from h0, later segments of a segmented plan from zero
  if (FULL && c_ok && p.h0 && (!SEG || seg == 0)) {
    const float* hin = p.h0 + (b * D + c) * N + n0;
#pragma unroll
    for (int j = 0; j < NS; ++j) h[j] = hin[j];
  }
  float dsum = 0.f;

  // ---- post-processing constants: this thread finishes channel tid % CH of tokens
  //      slice, slice + KS, ... of each tile (the same channel as its recurrence lane)
  const float dsk = (FULL && p.Dskip && c_ok) ? p.Dskip[c] : 0.f;
  io_t* __restrict__ yg = static_cast<io_t*>(p.y);
  uint32_t y_boff[FULL ? T / KS : 1];   // byte offset of this thread's outputs inside a tile block
#pragma unroll
  for (int k = 0; k < (FULL ? T / KS : 1); ++k)
    y_boff[k] = (uint32_t)(((slice + k * KS) * D + chl) * (int64_t)sizeof(io_t));

  if (ntiles > 0) {
    issue_loads(0);
    commit_first_tile();
  }
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) issue_loads(tile + 1);

    // ---- recurrence over the tile (identity on padded tokens), in sub-tiles of PH tokens:
    //      phase 1 forms Abar and the input term of every token of the sub-tile (independent
    //      work, so several exps are in flight); phase 2 is the serial part, h = Abar h + u,
    //      and the readout.
    // (the convolution variant holds three more raw rows: two-token sub-tiles keep it at the
    // same occupancy)
    constexpr int PH = T < 4 ? T : (CONV ? 2 : 4);
    static_assert(T % PH == 0, "sub-tiles must cover the tile");
#pragma unroll
    for (int t0 = 0; t0 < T; t0 += PH) {
      float abar_t[PH][NS], u_t[PH][NS];
      auto phase1 = [&](auto accurate_tag) __attribute__((always_inline)) {
        constexpr bool ACCURATE = decltype(accurate_tag)::value;
#pragma unroll
        for (int i = 0; i < PH; ++i) {
          const float2 dx = s_dx[buf][t0 + i][chl];
          const float* bc = &s_bc[buf][t0 + i][n0][0];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float tx = dx.x * a2[j];
            const float abar = exp2_fast(tx);
            abar_t[i][j] = abar;
            // expm1(Delta a)/a B x
            u_t[i][j] = zoh_input_scale<ACCURATE>(abar, tx, dx.x, ia[j]) * (bc[2 * j] * dx.y);
          }
          if (!FULL) dsum += dx.x;
        }
      };
      if constexpr (std::is_same<io_t, float>::value) {
        // float32 I/O: the series of the input scale only where some state of the wave has
        // |Delta a| < 1/16 in the sub-tile (a uniform branch; the per-state choice is still made
        // inside), else the plain form
        float dmin = fabsf(s_dx[buf][t0][chl].x);
#pragma unroll
        for (int i = 1; i < PH; ++i) dmin = fminf(dmin, fabsf(s_dx[buf][t0 + i][chl].x));
        if (__any(!(dmin >= series_dmax) ? 1 : 0))
          phase1(std::true_type{});
        else
          phase1(std::false_type{});
      } else {
        phase1(std::false_type{});
      }
#pragma unroll
      for (int i = 0; i < PH; ++i) {
        const float* bc = &s_bc[buf][t0 + i][n0][0];
        float yp = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          h[j] = fmaf(abar_t[i][j], h[j], u_t[i][j]);
          if (FULL) yp = (j == 0) ? bc[1] * h[0] : fmaf(bc[2 * j + 1], h[j], yp);
        }
        if (FULL) s_y[slice][(t0 + i) * CH + chl] = yp;
      }
    }

    // ---- combine the KS partial readouts, D term, gate. The stores are issued only after the
    //      next tile is committed: stores count in the same memory counter as loads, so a store
    //      issued before the commit would make the commit wait for it as well.
    float yout[FULL ? T / KS : 1];
    if (FULL) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < T / KS; ++k) {
        const int t = slice + k * KS;
        float yv = s_y[0][t * CH + chl];
#pragma unroll
        for (int q = 1; q < KS; ++q) yv += s_y[q][t * CH + chl];
        yv = fmaf(dsk, s_dx[buf][t][chl].y, yv);
        if (has_z) yv *= silu(Io::load(reinterpret_cast<const io_t*>(&s_z[buf][t][0]), chl));
        yout[k] = yv;
      }
    }
    // every wave waits for the next tile's loads here, on every path (also waves that load
    // nothing, and the last tile), so no other point of the loop waits for memory operations
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (tile + 1 < ntiles) commit_tile(tile + 1, buf ^ 1);
    if (FULL) {
      // rows past the segment end fall outside the descriptor and are dropped
      const Rsrc yr = tile_rsrc(yg, D, c0, tile, tile_rows(tile));
      if (c_ok)
#pragma unroll
        for (int k = 0; k < T / KS; ++k) buf_store(yr, y_boff[k], yout[k], (io_t*)nullptr);
    }
    __syncthreads();
  }

  if constexpr (SEG) {
    // the segment's sum of Delta per channel: the loader threads of a channel group hold partial
    // sums over their rows (the tile buffers are free after the loop's last barrier)
    // (flags beside them; the readers of a channel are the first CH threads, all in wave 0)
    static_assert(KS * kYStride >= Cfg::kThreads * (GW + 1), "the partial sums fit the readout buffer");
    static_assert(CH <= 64, "the channel readers form one wave");
    float* s_red = &s_y[0][0];
    float* s_neg = s_red + Cfg::kThreads * GW;
#pragma unroll
    for (int q = 0; q < GW; ++q) s_red[tid * GW + q] = dacc[q];
    s_neg[tid] = dneg ? 1.f : 0.f;
    __syncthreads();
    if (tid < CH) {
      const int g0 = tid / GW, q = tid % GW;
      float s = 0.f;
      bool neg = false;
      for (int j = g0; j < Cfg::kThreads; j += CH / GW) {
        s += s_red[j * GW + q];
        neg = neg || s_neg[j] != 0.f;
      }
      if (c0 + tid < D) p.ws_sum[(b * p.nseg + seg) * D + c0 + tid] = s;
      const bool any_neg = __any(neg ? 1 : 0);
      if (tid == 0) p.ws_neg[(b * p.nseg + seg) * (int64_t)gridDim.x + tile] = any_neg ? 1 : 0;
    }
    if (c_ok) {
      float* hl = p.ws_h + ((b * p.nseg + seg) * D + c) * N + n0;
#pragma unroll
      for (int j = 0; j < NS; ++j) hl[j] = h[j];
    }
    return;
  }
  if (!c_ok) return;
  if (FULL) {
    if (p.h_last) {
      float* hl = p.h_last + (b * D + c) * N + n0;
#pragma unroll
      for (int j = 0; j < NS; ++j) hl[j] = h[j];
    }
  } else {
    float* hl = p.ws_h + ((b * p.nseg + seg) * D + c) * N + n0;
#pragma unroll
    for (int j = 0; j < NS; ++j) hl[j] = h[j];
    if (slice == 0) p.ws_sum[(b * p.nseg + seg) * D + c] = dsum;
  }
}

// Carry pass over segments, one thread per (b, d, n) chain:
// h_in[0] = h0 (or 0); h_in[s+1] = exp(A sum Delta_s) h_in[s] + h_loc[s].
// ws_h[b, s] holds h_loc[s] on entry and h_in[s] on exit (s = 0 .. nseg-1).
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanParams p) {
  const int64_t D = p.D, N = p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.B * D * N) return;
  const int64_t n = i % N;
  const int64_t c = (i / N) % D;
  const int64_t b = i / (N * D);
  const float a2 = p.A[c * N + n] * kLog2e;
  float h = p.h0 ? p.h0[(b * D + c) * N + n] : 0.f;
  for (int64_t s = 0; s + 1 < p.nseg; ++s) {
    float* slot = p.ws_h + ((b * p.nseg + s) * D + c) * N + n;
    const float hloc = *slot;
    const float decay = exp2_fast(a2 * p.ws_sum[(b * p.nseg + s) * D + c]);
    *slot = h;
    h = fmaf(decay, h, hloc);
  }
  p.ws_h[((b * p.nseg + p.nseg - 1) * D + c) * N + n] = h;
}

// The convolution register after the prefill: the last W raw inputs, oldest first (earlier
// register entries shifted in when L < W). One thread per (b, d); it runs after the scan, so the
// register may be updated in place.
template <typename io_t>
__global__ __launch_bounds__(256) void conv_register_kernel(ScanParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.B * p.D) return;
  const int64_t b = i / p.D, d = i % p.D;
  const int W = p.conv_W;
  using Io = IoTraits<io_t>;
  io_t* out = static_cast<io_t*>(p.conv_out) + i * W;
  const io_t* in = static_cast<const io_t*>(p.conv_in);
  for (int k = 0; k < W; ++k) {
    const int64_t t = p.L - W + k;
    if (t >= 0) {
      out[k] = static_cast<const io_t*>(p.x)[(b * p.L + t) * p.D + d];
    } else {
      // entries move left by L places; in place this reads index k + L > k before it is written
      const float v = in ? Io::load(in, i * W + k + p.L) : 0.f;
      Io::store(out, k, v);
    }
  }
}

template <typename io_t, int CH, int NS, int KS, int N, int OCC, bool CONV>
hipError_t launch_typed(const ScanParams& p, hipStream_t stream) {
  constexpr int T = 16;
  const dim3 block(CH * KS);
  const unsigned gx = (unsigned)((p.D + CH - 1) / CH);
  const dim3 grid(gx, (unsigned)p.B, (unsigned)p.nseg);
  if (p.nseg > 1) {
    hipLaunchKernelGGL((scan_kernel<io_t, CH, NS, KS, T, N, true, OCC, CONV, true>), grid, block, 0, stream, p);
    const hipError_t e = launch_scan_segment_fix(p, CH, stream);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((scan_kernel<io_t, CH, NS, KS, T, N, true, OCC, CONV>), grid, block, 0, stream, p);
  }
  if (CONV && p.conv_out) {
    const int64_t n = p.B * p.D;
    hipLaunchKernelGGL(conv_register_kernel<io_t>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// The segment carries alone: the state-only pass over segments 0 .. nseg-2 and the carry pass,
// which leave ws_h[b, s] = the state entering segment s (s = 0 .. nseg-1).
template <typename io_t, int CH, int NS, int KS, int N, int OCC>
hipError_t launch_carries_typed(const ScanParams& p, hipStream_t stream) {
  constexpr int T = 16;
  const dim3 block(CH * KS);
  const unsigned gx = (unsigned)((p.D + CH - 1) / CH);
  const dim3 grid_a(gx, (unsigned)p.B, (unsigned)(p.nseg - 1));
  hipLaunchKernelGGL((scan_kernel<io_t, CH, NS, KS, T, N, false, OCC>), grid_a, block, 0, stream, p);
  const int64_t chains = p.B * p.D * p.N;
  hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((chains + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename io_t>
hipError_t launch_carries_io(const ScanParams& p, hipStream_t stream) {
  switch (p.N) {
    case 1: return launch_carries_typed<io_t, 64, 1, 1, 1, 1>(p, stream);
    case 2: return launch_carries_typed<io_t, 64, 2, 1, 2, 1>(p, stream);
    case 4: return launch_carries_typed<io_t, 64, 2, 2, 4, 1>(p, stream);
    case 8: return launch_carries_typed<io_t, 32, 2, 4, 8, 1>(p, stream);
    case 16: return launch_carries_typed<io_t, 32, 2, 8, 16, 5>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename io_t, bool CONV>
hipError_t launch_io(const ScanParams& p, hipStream_t stream) {
  switch (p.N) {
    case 1: return launch_typed<io_t, 64, 1, 1, 1, 1, CONV>(p, stream);
    case 2: return launch_typed<io_t, 64, 2, 1, 2, 1, CONV>(p, stream);
    case 4: return launch_typed<io_t, 64, 2, 2, 4, 1, CONV>(p, stream);
    case 8: return launch_typed<io_t, 32, 2, 4, 8, 1, CONV>(p, stream);
    case 16: return launch_typed<io_t, 32, 2, 8, 16, 5, CONV>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t scan_channels_per_tile(int64_t N) { return N >= 8 ? 32 : 64; }

size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int64_t nseg) {
  if (nseg <= 1) return 0;
  const int64_t tiles = (D + scan_channels_per_tile(N) - 1) / scan_channels_per_tile(N);
  return (size_t)(B * nseg * D * N) * sizeof(float) + (size_t)(B * nseg * D) * sizeof(float) +
         (size_t)(B * nseg * tiles) * sizeof(int) + 256;
}

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
  if (p.conv_w)
    return p.io_bf16 ? launch_io<bf16_t, true>(p, stream) : launch_io<float, true>(p, stream);
  return p.io_bf16 ? launch_io<bf16_t, false>(p, stream) : launch_io<float, false>(p, stream);
}

hipError_t launch_scan_carries(const ScanParams& p, hipStream_t stream) {
  if (p.nseg < 2) return hipErrorInvalidValue;
  return p.io_bf16 ? launch_carries_io<bf16_t>(p, stream) : launch_carries_io<float>(p, stream);
}

}  // namespace ssm
