// Selective scan (S6) backward on gfx950: every input's gradient by state recomputation.
//
// The forward map (pages "Beyond attention: exploring Mamba and state space models", state-space
// basics and selective-SSM sections): per token and channel Delta = softplus(delta + bias) (or
// delta + bias), for each state Abar = exp(Delta a), phi = expm1(Delta a) / a,
// h_t = Abar h_{t-1} + phi B_t x_t, y_t = C_t . h_t + D x_t, out = y z sigmoid(z). Its
// reverse-mode derivative runs time backwards with the adjoint g_t = dL/dh_t:
//   g_t = C_t gy_t + Abar_{t+1} g_{t+1}            (gy = dL/dy before the gate)
//   dx_t = D gy_t + sum_n g phi B          dDelta_t = sum_n Abar g (a h_{t-1} + B x)
//   dB_t = sum_d g phi x                   dC_t = sum_d gy h_t
//   dA = sum_t (Delta Abar g (h_{t-1} + B x / a) - g phi B x / a)
// The state is never stored per token (it is N times the size of the input); the page "Mamba and
// state space models" names recomputation, with the fused scan, as what keeps the state on chip,
// and the backward recomputes it tile by tile from checkpoints.
//
// Plan (one workgroup = CH channels of one sequence and one L-segment, lanes as in the forward:
// thread tid owns states n0 .. n0+NS-1 of channel tid % CH):
//   ckpt  : forward over the segment from its entering state, storing the state at the start of
//           every 8-token tile (workspace).
//   adj   : (segmented plans) backward over the segment from a zero adjoint: the local adjoint
//           before the segment and the segment's sum of Delta. A carry pass then combines the
//           segments from the last one: E_{s-1} = exp(a sum Delta_s) E_s + q_s, E_last = dh_last.
//   full  : tiles in reverse order; per tile the forward is recomputed from the checkpoint with
//           (h_t, Abar_t) kept in registers, then the tile is walked backwards. dx, dDelta and
//           the recomputed y (for dz) are partial over the lane's states and are added over the
//           KS lanes of a channel through LDS; dB and dC are partial over channels and are added
//           over the workgroup's CH channels through LDS, then over the channel tiles by a
//           reduction kernel (fixed order: the result does not depend on scheduling).
//   reduce: dB, dC over channel tiles; dA, D and bias gradients over batch rows and segments.
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kTB = 8;  // tokens per tile of the backward kernels

enum BwdMode { kModeCkpt = 0, kModeAdj = 1, kModeFull = 2 };

template <typename io_t, int CH, int NS, int KS, int N, int MODE>
__global__ __launch_bounds__(CH * KS) void scan_bwd_kernel(ScanBwdParams p) {
  constexpr int T = kTB;
  constexpr int kThreads = CH * KS;
  constexpr bool kCkpt = MODE == kModeCkpt, kAdj = MODE == kModeAdj, kFull = MODE == kModeFull;
  static_assert(NS * KS == N, "slices must cover the state");
  static_assert(T % KS == 0, "post-processing splits a tile's tokens over the slices");
  constexpr int kEl = (T * CH + kThreads - 1) / kThreads;  // (token, channel) elements per thread
  constexpr int kBC = T * N;                               // B (and C) elements per tile
  static_assert(kBC <= kThreads, "one B/C element per loading thread");

  // Staged tile operands. The full pass keeps one copy (a barrier separates the last read of
  // a tile from the commit of the next, whose global loads were in flight meanwhile): 40 KB
  // per workgroup; the other passes double-buffer.
  constexpr int kNB = kFull ? 1 : 2;
  // per token and channel: (Delta, x) for the recurrence, (gy, sigmoid(u)) for the adjoint
  __shared__ __attribute__((aligned(16))) float2 s_dx[kNB][T][CH];
  __shared__ __attribute__((aligned(16))) float2 s_g[kCkpt ? 1 : kNB][kCkpt ? 1 : T][CH];
  __shared__ float s_dzc[kFull ? kNB : 1][kFull ? T : 1][CH];      // dz = y * s_dzc
  // B_n and C_n of each token, apart: the recomputed forward reads B only
  __shared__ __attribute__((aligned(16))) float s_b[kNB][T][N];
  __shared__ __attribute__((aligned(16))) float s_c[kNB][T][N];
  // partials over the slices (half a tile): dx, dDelta, y; two slices share a wave at CH = 32,
  // so their rows are 32 banks apart
  constexpr int kPStride = (T / 2) * CH + 32;
  __shared__ float s_p[kFull ? 3 : 1][kFull ? KS : 1][kFull ? kPStride : 1];
  // partials over the channels (half a tile), one column per channel. The lane of slice s, token i,
  // state n0 + j writes dB / dC (bc = 0 / 1) to q = (i NS + j) 2 + bc of its slice, stored at row
  // ((q / 8) KS + s) 8 + q % 8: the two slices of a wave write rows 8 apart (32 banks apart with
  // the row stride CH + 4), and rows of stride CH + 4 read as float4 hit distinct banks.
  constexpr int kQCols = CH;
  constexpr int kQRows = (T / 2) * N * 2, kQStride = kQCols + 4;
  static_assert(((T / 2) * NS * 2) % 8 == 0, "row blocks of 8");
  __shared__ __attribute__((aligned(16))) float s_q[kFull ? kQRows : 1][kFull ? kQStride : 4];

  const int tid = threadIdx.x;
  const int64_t D = p.D, L = p.L;
  int64_t tile_c, b, seg;
  {
    // same XCD-aware order as the forward scan: channel tiles 2k and 2k+1 share an L2
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
    tile_c = __builtin_amdgcn_readfirstlane((uint32_t)(logical % gx));
    b = __builtin_amdgcn_readfirstlane((uint32_t)((logical / gx) % gridDim.y));
    seg = __builtin_amdgcn_readfirstlane((uint32_t)(logical / gxy));
  }
  const int64_t c0 = tile_c * CH;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < L) ? t_begin + p.seg_len : L;
  const int ntiles = (int)((t_end - t_begin + T - 1) / T);
  const int n_full = (int)((t_end - t_begin) / T);
  const int64_t seg_row0 = b * L + t_begin;
  const int64_t tile0 = t_begin / T;                 // global index of the segment's first tile
  const int64_t ntt = (L + T - 1) / T;               // tiles per sequence

  const io_t* __restrict__ xg = static_cast<const io_t*>(p.x);
  const io_t* __restrict__ dg = static_cast<const io_t*>(p.delta);
  const io_t* __restrict__ zg = static_cast<const io_t*>(p.z);
  const io_t* __restrict__ gyg = static_cast<const io_t*>(p.dy);
  const io_t* __restrict__ Bg = static_cast<const io_t*>(p.Bm);
  const io_t* __restrict__ Cg = static_cast<const io_t*>(p.Cm);
  const bool has_z = !kCkpt && zg != nullptr;

  // ---- loader: thread tid handles elements e = tid + k kThreads of a tile (row e / CH, channel
  //      e % CH, the same every tile), and B/C element tid
  uint32_t el_off[kEl];
  float el_bias[kEl];
  bool el_col_ok[kEl];
#pragma unroll
  for (int k = 0; k < kEl; ++k) {
    const int e = tid + k * kThreads;
    const int col = e % CH;
    el_off[k] = (uint32_t)(((e / CH) * D + col) * (int64_t)sizeof(io_t));
    el_col_ok[k] = c0 + col < D;
    el_bias[k] = (p.delta_bias && el_col_ok[k]) ? p.delta_bias[c0 + col] : 0.f;
  }
  uint32_t rd[kEl], rx[kEl], rz[kEl], rg[kEl];
  uint32_t rB = 0u, rC = 0u;
#pragma unroll
  for (int k = 0; k < kEl; ++k) rd[k] = rx[k] = rz[k] = rg[k] = 0u;

  auto tile_rows = [&](int tile) __attribute__((always_inline)) {
    return tile < n_full ? T : (int)(t_end - t_begin - (int64_t)tile * T);
  };
  auto tile_rsrc = [&](const void* base, int64_t row_len, int64_t col0, int tile, int rows)
      __attribute__((always_inline)) {
    const char* blk = static_cast<const char*>(base) +
                      ((seg_row0 + (int64_t)tile * T) * row_len + col0) * (int64_t)sizeof(io_t);
    return make_rsrc(blk, (int)((rows * row_len - col0) * (int64_t)sizeof(io_t)));
  };

  // ---- lane constants: channel c, states n0 .. n0+NS-1
  const int slice = tid / CH;
  const int chl = tid % CH;
  const int64_t c = c0 + chl;
  const bool c_ok = c < D;
  const int n0 = slice * NS;
  float av[NS], a2[NS], ia[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    av[j] = c_ok ? p.A[c * N + n0 + j] : -1.0f;
    a2[j] = av[j] * kLog2e;
    ia[j] = 1.0f / av[j];
  }
  // checkpoint of this lane: ws_ck[((b ntt + tile) KS + slice) D + c] holds NS floats
  const int64_t ck_lane = (int64_t)slice * D + c;
  auto ck_ptr = [&](int tile) __attribute__((always_inline)) {
    return p.ws_ck + (((b * ntt + tile0 + tile) * KS) * D + ck_lane) * NS;
  };
  float ckn[NS], hck[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) ckn[j] = hck[j] = 0.f;

  auto issue_loads = [&](int tile) __attribute__((always_inline)) {
    const int rows = tile_rows(tile);
    const Rsrc dr = tile_rsrc(dg, D, c0, tile, rows);
    const Rsrc xr = tile_rsrc(xg, D, c0, tile, rows);
    const Rsrc gr = kCkpt ? xr : tile_rsrc(gyg, D, c0, tile, rows);
    const Rsrc zr = has_z ? tile_rsrc(zg, D, c0, tile, rows) : xr;
#pragma unroll
    for (int k = 0; k < kEl; ++k) {
      if (tid + k * kThreads < T * CH) {
        rd[k] = buf_load_bits(dr, el_off[k], (io_t*)nullptr);
        if (!kAdj) rx[k] = buf_load_bits(xr, el_off[k], (io_t*)nullptr);
        if (!kCkpt) rg[k] = buf_load_bits(gr, el_off[k], (io_t*)nullptr);
        if (has_z) rz[k] = buf_load_bits(zr, el_off[k], (io_t*)nullptr);
      }
    }
    if (tid < kBC) {
      const uint32_t off = (uint32_t)tid * (uint32_t)sizeof(io_t);
      if (!kAdj) rB = buf_load_bits(tile_rsrc(Bg, N, 0, tile, rows), off, (io_t*)nullptr);
      if (!kCkpt) rC = buf_load_bits(tile_rsrc(Cg, N, 0, tile, rows), off, (io_t*)nullptr);
    }
    if constexpr (kFull) {
      if (c_ok) {
        const float* q = ck_ptr(tile);
#pragma unroll
        for (int j = 0; j < NS; ++j) ckn[j] = q[j];
      }
    }
  };

  // Rows past the segment end and channels past D are committed as Delta = 0, x = 0, gy = 0:
  // the identity step with no gradient.
  auto commit = [&](int tile, int buf) __attribute__((always_inline)) {
    const int rows = tile_rows(tile);
#pragma unroll
    for (int k = 0; k < kEl; ++k) {
      const int e = tid + k * kThreads;
      if (e < T * CH) {
        const int r = e / CH, col = e % CH;
        const bool ok = el_col_ok[k] && r < rows;
        const float u = IoTraits<io_t>::from_bits(rd[k]) + el_bias[k];
        const float dt = ok ? (p.delta_softplus ? softplus_f32(u) : u) : 0.f;
        float2 v, w;
        v.x = dt;
        v.y = ok && !kAdj ? IoTraits<io_t>::from_bits(rx[k]) : 0.f;
        w.x = 0.f;
        w.y = 1.f;
        if constexpr (!kCkpt) {
          const float dyv = ok ? IoTraits<io_t>::from_bits(rg[k]) : 0.f;
          float gy = dyv, dzc = 0.f;
          if (has_z) {
            const float zv = IoTraits<io_t>::from_bits(rz[k]);
            const float sg = sigmoid_fast(zv);
            gy = dyv * zv * sg;
            dzc = dyv * sg * fmaf(zv, 1.0f - sg, 1.0f);
          }
          w.x = gy;
          if (p.delta_softplus) w.y = sigmoid_fast(u);
          if constexpr (kFull) s_dzc[buf][r][col] = dzc;
          s_g[buf][r][col] = w;
        }
        s_dx[buf][r][col] = v;
      }
    }
    if (tid < kBC) {
      if (!kAdj) s_b[buf][tid / N][tid % N] = IoTraits<io_t>::from_bits(rB);
      if (!kCkpt) s_c[buf][tid / N][tid % N] = IoTraits<io_t>::from_bits(rC);
    }
    if constexpr (kFull) {
#pragma unroll
      for (int j = 0; j < NS; ++j) hck[j] = ckn[j];
    }
  };

  if constexpr (kCkpt) {
    // ---------------------------------------------------------------- forward with checkpoints
    float h[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) h[j] = 0.f;
    if (c_ok) {
      const float* hin = nullptr;
      if (p.nseg > 1) hin = p.ws_h + ((b * p.nseg + seg) * D + c) * N + n0;
      else if (p.h0) hin = p.h0 + (b * D + c) * N + n0;
      if (hin)
#pragma unroll
        for (int j = 0; j < NS; ++j) h[j] = hin[j];
    }
    if (ntiles > 0) {
      issue_loads(0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      commit(0, 0);
    }
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      if (tile + 1 < ntiles) issue_loads(tile + 1);
      float hst[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) hst[j] = h[j];
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const float2 v = s_dx[buf][i][chl];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float bn = s_b[buf][i][n0 + j];
          const float abar = exp2_fast(v.x * a2[j]);
          h[j] = fmaf(abar, h[j], fmaf(abar, ia[j], -ia[j]) * (bn * v.y));
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      if (tile + 1 < ntiles) commit(tile + 1, buf ^ 1);
      if (c_ok) {
        float* q = ck_ptr(tile);
#pragma unroll
        for (int j = 0; j < NS; ++j) q[j] = hst[j];
      }
      __syncthreads();
    }
    return;
  }

  // ------------------------------------------------------------------ backward (adj and full)
  if constexpr (!kCkpt) {
  float g[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) g[j] = 0.f;
  if (kFull && c_ok) {
    const float* gin = nullptr;
    if (p.nseg > 1) gin = p.ws_E + ((b * p.nseg + seg) * D + c) * N + n0;
    else if (p.dh_last) gin = p.dh_last + (b * D + c) * N + n0;
    if (gin)
#pragma unroll
      for (int j = 0; j < NS; ++j) g[j] = gin[j];
  }
  float dAr[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) dAr[j] = 0.f;
  float dsum = 0.f;                 // adj: sum of Delta over the segment
  float accD = 0.f, accb = 0.f;     // full: this thread's outputs' D and bias gradients
  const float dsk = (kFull && p.Dskip && c_ok) ? p.Dskip[c] : 0.f;
  io_t* __restrict__ dxg = static_cast<io_t*>(p.dx);
  io_t* __restrict__ ddg = static_cast<io_t*>(p.ddelta);
  io_t* __restrict__ dzg = static_cast<io_t*>(p.dz);

  if (ntiles > 0) {
    issue_loads(ntiles - 1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    commit(ntiles - 1, 0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int tile = ntiles - 1 - it;
    const int buf = kFull ? 0 : (it & 1);
    if (tile > 0) issue_loads(tile - 1);

    if constexpr (kAdj) {
#pragma unroll
      for (int i = T - 1; i >= 0; --i) {
        const float dt = s_dx[buf][i][chl].x;
        const float gy = s_g[buf][i][chl].x;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float abar = exp2_fast(dt * a2[j]);
          g[j] = abar * fmaf(s_c[buf][i][n0 + j], gy, g[j]);
        }
        dsum += dt;
      }
    }

    // ---- full: the tile backwards in two halves of TH tokens; after each half the partials
    //      over the slices (dx, dDelta, y) and over the channels (dB, dC) are added from LDS
    //      (half-sized buffers: three workgroups fit a CU). Outputs are kept in registers and
    //      stored after the next tile's commit.
    constexpr int TH = T / 2;
    constexpr int kOutH = (TH + KS - 1) / KS;
    constexpr int kQRowsH = TH * N * 2;
    constexpr int kQPerThrH = (kQRowsH + kThreads - 1) / kThreads;
    float o_dx[kFull ? 2 : 1][kOutH], o_dd[kFull ? 2 : 1][kOutH], o_dz[kFull ? 2 : 1][kOutH];
    float o_q[kFull ? 2 : 1][kQPerThrH];
    const int rows = tile_rows(tile);
    if constexpr (kFull) {
      // forward recompute of the tile from its checkpoint, keeping h_t and Abar_t
      float H[T][NS], AB[T][NS];
      {
        float h[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) h[j] = hck[j];
#pragma unroll
        for (int i = 0; i < T; ++i) {
          const float2 v = s_dx[buf][i][chl];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float bn = s_b[buf][i][n0 + j];
            const float abar = exp2_fast(v.x * a2[j]);
            h[j] = fmaf(abar, h[j], fmaf(abar, ia[j], -ia[j]) * (bn * v.y));
            H[i][j] = h[j];
            AB[i][j] = abar;
          }
        }
      }
#pragma unroll
      for (int hf = 1; hf >= 0; --hf) {
#pragma unroll
        for (int il = TH - 1; il >= 0; --il) {
          const int i = hf * TH + il;
          const float2 v = s_dx[buf][i][chl];
          const float gy = s_g[buf][i][chl].x;
          float dxp = 0.f, ddp = 0.f, yp = 0.f;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float2 bc = make_float2(s_b[buf][i][n0 + j], s_c[buf][i][n0 + j]);
            const float hprev = i > 0 ? H[i - 1][j] : hck[j];
            const float abar = AB[i][j];
            const float gn = fmaf(bc.y, gy, g[j]);              // dL/dh_t
            const int q = (il * NS + j) * 2;
            const int row = ((q >> 3) * KS + slice) * 8 + (q & 7);
            s_q[row + 1][chl] = gy * H[i][j];                   // dC partial
            const float gphi = gn * fmaf(abar, ia[j], -ia[j]);
            s_q[row][chl] = gphi * v.y;                         // dB partial
            dxp = fmaf(gphi, bc.x, dxp);
            const float bx = bc.x * v.y;
            const float w = fmaf(av[j], hprev, bx);
            const float ga = gn * abar;
            const float vv = ga * w;
            ddp += vv;
            dAr[j] = fmaf(v.x, vv, dAr[j]);
            dAr[j] = fmaf(-gphi, bx, dAr[j]);
            g[j] = ga;                                          // on to dL/dh_{t-1}
            yp = fmaf(bc.y, H[i][j], yp);
          }
          s_p[0][slice][il * CH + chl] = dxp;
          s_p[1][slice][il * CH + chl] = ddp;
          if (has_z) s_p[2][slice][il * CH + chl] = yp;
        }
        __syncthreads();
        // outputs of this thread: tokens hf TH + slice + k KS of channel chl
#pragma unroll
        for (int k = 0; k < kOutH; ++k) {
          const int il = slice + k * KS;
          o_dx[hf][k] = o_dd[hf][k] = o_dz[hf][k] = 0.f;
          if (il < TH) {
            const int i = hf * TH + il;
            float sx = s_p[0][0][il * CH + chl], sd = s_p[1][0][il * CH + chl];
            float sy = has_z ? s_p[2][0][il * CH + chl] : 0.f;
#pragma unroll
            for (int q = 1; q < KS; ++q) {
              sx += s_p[0][q][il * CH + chl];
              sd += s_p[1][q][il * CH + chl];
              if (has_z) sy += s_p[2][q][il * CH + chl];
            }
            const float xv = s_dx[buf][i][chl].y;
            const float2 w = s_g[buf][i][chl];
            o_dx[hf][k] = fmaf(dsk, w.x, sx);
            o_dd[hf][k] = sd * w.y;
            o_dz[hf][k] = has_z ? fmaf(dsk, xv, sy) * s_dzc[buf][i][chl] : 0.f;
            if (i < rows) {
              accD = fmaf(w.x, xv, accD);
              accb += o_dd[hf][k];
            }
          }
        }
#pragma unroll
        for (int m = 0; m < kQPerThrH; ++m) {
          const int r = tid + m * kThreads;
          float sum = 0.f;
          if (r < kQRowsH) {
            const float4* row = reinterpret_cast<const float4*>(&s_q[r][0]);
#pragma unroll
            for (int k = 0; k < kQCols / 4; ++k) {
              const float4 q4 = row[k];
              sum += (q4.x + q4.y) + (q4.z + q4.w);
            }
          }
          o_q[hf][m] = sum;
        }
        if (hf == 1) __syncthreads();   // the second half reuses the buffers
      }
    }
    // every wave waits for the next tile's loads here (stores are issued after the commit:
    // they count in the same memory counter)
    if constexpr (kFull) __syncthreads();   // single-buffered operands: all reads done
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (tile > 0) commit(tile - 1, kFull ? 0 : buf ^ 1);
    if constexpr (kFull) {
      const Rsrc xr = tile_rsrc(dxg, D, c0, tile, rows);
      const Rsrc dr = tile_rsrc(ddg, D, c0, tile, rows);
      const Rsrc zr = has_z ? tile_rsrc(dzg, D, c0, tile, rows) : xr;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int k = 0; k < kOutH; ++k) {
          const int il = slice + k * KS;
          if (c_ok && il < TH) {
            const uint32_t off = (uint32_t)(((hf * TH + il) * D + chl) * (int64_t)sizeof(io_t));
            buf_store(xr, off, o_dx[hf][k], (io_t*)nullptr);
            buf_store(dr, off, o_dd[hf][k], (io_t*)nullptr);
            if (has_z) buf_store(zr, off, o_dz[hf][k], (io_t*)nullptr);
          }
        }
        // (dB, dC) partials of this channel tile: ws_pq[((b L + t) nct + tile_c) 2N + (n 2 + bc)]
#pragma unroll
        for (int m = 0; m < kQPerThrH; ++m) {
          // row r of s_q back to (token, state n, bc)
          const int r = tid + m * kThreads;
          const int q = (r / (8 * KS)) * 8 + (r & 7);
          const int i = hf * TH + q / (2 * NS);
          const int n = ((r >> 3) % KS) * NS + (q >> 1) % NS;
          if (r < kQRowsH && i < rows) {
            const int64_t t = seg_row0 + (int64_t)tile * T + i;
            p.ws_pq[(t * p.nct + tile_c) * (2 * N) + 2 * n + (q & 1)] = o_q[hf][m];
          }
        }
      }
    }
    __syncthreads();
  }

  if constexpr (kAdj) {
    if (c_ok) {
      float* q = p.ws_q + ((b * p.nseg + seg) * D + c) * N + n0;
#pragma unroll
      for (int j = 0; j < NS; ++j) q[j] = g[j];
      if (slice == 0) p.ws_dsum[(b * p.nseg + seg) * D + c] = dsum;
    }
    return;
  }
  // ---- full: per-(b, seg) partials of the parameter gradients, and dh0
  if constexpr (kFull) {
  if (c_ok) {
    float* pa = p.ws_pA + ((b * p.nseg + seg) * D + c) * N + n0;
#pragma unroll
    for (int j = 0; j < NS; ++j) pa[j] = dAr[j] * ia[j];
    if (seg == 0 && p.dh0) {
      float* d0 = p.dh0 + (b * D + c) * N + n0;
#pragma unroll
      for (int j = 0; j < NS; ++j) d0[j] = g[j];
    }
  }
  // D and bias gradients: add the KS threads of each channel in a fixed order
  s_p[0][slice][chl] = accD;
  s_p[1][slice][chl] = accb;
  __syncthreads();
  if (slice == 0 && c_ok) {
    float sD = 0.f, sb = 0.f;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      sD += s_p[0][q][chl];
      sb += s_p[1][q][chl];
    }
    p.ws_pD[(b * p.nseg + seg) * D + c] = sD;
    p.ws_pb[(b * p.nseg + seg) * D + c] = sb;
  }
  }  // kFull
  }  // !kCkpt
}

// Adjoint carry over segments, one thread per (b, d, n) chain, from the last segment:
// E_{nseg-1} = dh_last (or 0), E_{s-1} = exp(a sum Delta_s) E_s + q_s.
__global__ __launch_bounds__(256) void scan_bwd_adj_carry_kernel(ScanBwdParams p) {
  const int64_t D = p.D, N = p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.B * D * N) return;
  const int64_t n = i % N;
  const int64_t c = (i / N) % D;
  const int64_t b = i / (N * D);
  const float a2 = p.A[c * N + n] * kLog2e;
  float e = p.dh_last ? p.dh_last[(b * D + c) * N + n] : 0.f;
  for (int64_t s = p.nseg - 1; s >= 0; --s) {
    const int64_t k = ((b * p.nseg + s) * D + c) * N + n;
    p.ws_E[k] = e;
    e = fmaf(exp2_fast(a2 * p.ws_dsum[(b * p.nseg + s) * D + c]), e, p.ws_q[k]);
  }
}

// dB, dC: sum of the channel-tile partials, one thread per (b, t, n, B/C).
__global__ __launch_bounds__(256) void scan_bwd_reduce_bc_kernel(ScanBwdParams p) {
  const int64_t N2 = 2 * p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.B * p.L * N2) return;
  const int64_t row = i / N2, r = i % N2;
  const float* src = p.ws_pq + row * p.nct * N2 + r;
  // four independent partial sums (k mod 4) keep four loads in flight; fixed order throughout
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int64_t k = 0;
  for (; k + 4 <= p.nct; k += 4) {
    s0 += src[k * N2];
    s1 += src[(k + 1) * N2];
    s2 += src[(k + 2) * N2];
    s3 += src[(k + 3) * N2];
  }
  for (; k < p.nct; ++k) s0 += src[k * N2];
  (r & 1 ? p.dCm : p.dBm)[row * p.N + (r >> 1)] = (s0 + s1) + (s2 + s3);
}

// dA, dD, dbias: sum over batch rows and segments in order, one thread per (d, n).
__global__ __launch_bounds__(256) void scan_bwd_reduce_param_kernel(ScanBwdParams p) {
  const int64_t D = p.D, N = p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= D * N) return;
  const int64_t c = i / N, n = i % N;
  const int64_t parts = p.B * p.nseg;
  float s = 0.f;
  for (int64_t k = 0; k < parts; ++k) s += p.ws_pA[(k * D + c) * N + n];
  p.dA[i] = s;
  if (n == 0) {
    float sD = 0.f, sb = 0.f;
    for (int64_t k = 0; k < parts; ++k) {
      sD += p.ws_pD[k * D + c];
      sb += p.ws_pb[k * D + c];
    }
    if (p.dDskip) p.dDskip[c] = sD;
    if (p.ddelta_bias) p.ddelta_bias[c] = sb;
  }
}

template <typename io_t, int CH, int NS, int KS, int N>
hipError_t launch_bwd_typed(const ScanBwdParams& p, hipStream_t stream) {
  const dim3 block(CH * KS);
  const unsigned gx = (unsigned)((p.D + CH - 1) / CH);
  const dim3 grid(gx, (unsigned)p.B, (unsigned)p.nseg);
  if (p.nseg > 1) {
    ScanParams f{};
    f.B = p.B; f.L = p.L; f.D = p.D; f.N = p.N;
    f.io_bf16 = p.io_bf16;
    f.x = p.x; f.delta = p.delta; f.z = nullptr; f.Bm = p.Bm; f.Cm = p.Cm;
    f.delta_bias = p.delta_bias; f.A = p.A; f.Dskip = nullptr; f.h0 = p.h0;
    f.y = nullptr; f.h_last = nullptr; f.delta_softplus = p.delta_softplus;
    f.seg_len = p.seg_len; f.nseg = p.nseg; f.ws_h = p.ws_h; f.ws_sum = p.ws_sum;
    hipError_t e = launch_scan_carries(f, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_bwd_kernel<io_t, CH, NS, KS, N, kModeCkpt>), grid, block, 0, stream, p);
  if (p.nseg > 1) {
    hipLaunchKernelGGL((scan_bwd_kernel<io_t, CH, NS, KS, N, kModeAdj>), grid, block, 0, stream, p);
    const int64_t chains = p.B * p.D * p.N;
    hipLaunchKernelGGL(scan_bwd_adj_carry_kernel, dim3((unsigned)((chains + 255) / 256)), dim3(256), 0,
                       stream, p);
  }
  hipLaunchKernelGGL((scan_bwd_kernel<io_t, CH, NS, KS, N, kModeFull>), grid, block, 0, stream, p);
  const int64_t nbc = p.B * p.L * 2 * p.N;
  hipLaunchKernelGGL(scan_bwd_reduce_bc_kernel, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(scan_bwd_reduce_param_kernel, dim3((unsigned)((p.D * p.N + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename io_t>
hipError_t launch_bwd_io(const ScanBwdParams& p, hipStream_t stream) {
  switch (p.N) {
    case 1: return launch_bwd_typed<io_t, 64, 1, 1, 1>(p, stream);
    case 2: return launch_bwd_typed<io_t, 64, 2, 1, 2>(p, stream);
    case 4: return launch_bwd_typed<io_t, 64, 2, 2, 4>(p, stream);
    case 8: return launch_bwd_typed<io_t, 32, 2, 4, 8>(p, stream);
    case 16: return launch_bwd_typed<io_t, 32, 2, 8, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t scan_bwd_channels_per_wg(int64_t N) { return N >= 8 ? 32 : 64; }

size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseg) {
  const int64_t ntt = (L + kTB - 1) / kTB;
  const int64_t nct = (D + scan_bwd_channels_per_wg(N) - 1) / scan_bwd_channels_per_wg(N);
  int64_t floats = B * ntt * N * D      // checkpoints
                   + B * L * nct * 2 * N  // dB, dC partials
                   + B * nseg * D * N     // dA partials
                   + 2 * B * nseg * D;    // D and bias partials
  if (nseg > 1) floats += 3 * B * nseg * D * N + 2 * B * nseg * D;  // h_in, q, E; two sums
  return (size_t)floats * sizeof(float) + 16 * 10;
}

void scan_bwd_workspace_carve(ScanBwdParams& p, void* ws) {
  const int64_t B = p.B, L = p.L, D = p.D, N = p.N, nseg = p.nseg;
  const int64_t ntt = (L + kTB - 1) / kTB;
  char* cur = static_cast<char*>(ws);
  auto take = [&](int64_t floats) {
    float* r = reinterpret_cast<float*>(cur);
    cur += ((size_t)floats * sizeof(float) + 15) & ~(size_t)15;
    return r;
  };
  p.ws_ck = take(B * ntt * N * D);
  p.ws_pq = take(B * L * p.nct * 2 * N);
  p.ws_pA = take(B * nseg * D * N);
  p.ws_pD = take(B * nseg * D);
  p.ws_pb = take(B * nseg * D);
  if (nseg > 1) {
    p.ws_h = take(B * nseg * D * N);
    p.ws_sum = take(B * nseg * D);
    p.ws_q = take(B * nseg * D * N);
    p.ws_dsum = take(B * nseg * D);
    p.ws_E = take(B * nseg * D * N);
  } else {
    p.ws_h = p.ws_sum = p.ws_q = p.ws_dsum = p.ws_E = nullptr;
  }
}

hipError_t launch_scan_bwd(const ScanBwdParams& p, hipStream_t stream) {
  return p.io_bf16 ? launch_bwd_io<bf16_t>(p, stream) : launch_bwd_io<float>(p, stream);
}

}  // namespace ssm
