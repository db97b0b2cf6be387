// Segment carries and output correction of the segmented selective-scan forward on gfx950.
//
// Pages "Mamba and state space models", section "scan on the chip", and "Beyond attention:
// exploring Mamba and state space models", selective-SSM section: per channel and state the
// recurrence h_t = exp(Delta_t A) h_{t-1} + u_t is linear in h. Over a segment s it is the affine
// map h -> m_s h + h_loc[s] with m_s = exp(A sum Delta over s), where h_loc[s] is the segment's
// end state from the zero state; the state entering segment s is the composition of the maps of
// segments 0 .. s-1 applied to zero (segment 0 already started from h0). The segment pass ran
// every segment from its start state with these entering states left out; with S_t the sum of
// Delta from the segment start through token t, they add
//   y_t += g_t * sum_n C_t[n] exp(A[n] S_t) h_in[n]        (g_t = z_t sigmoid(z_t), or 1)
// to the outputs. The added term decays along the segment, so it is formed only while
// exp(A S_t) is still visible at the output precision.
#include "device_common.h"
#include "kernels.h"

namespace ssm {
namespace {

// Carry scan over segments: one wave per chain (b, c, n); lane l takes segments l, l + 64, ...
// Within a block of 64 segments an inclusive scan of the maps (m, v) over the lanes (composition
// (m2, v2) after (m1, v1) = (m2 m1, m2 v1 + v2)); the state before the block is carried in H.
// ws_h[b, s] holds h_loc[s] on entry and the state entering segment s on exit.
__global__ __launch_bounds__(256) void segment_carry_kernel(ScanParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t chain = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t D = p.D, N = p.N, S = p.nseg;
  if (chain >= p.B * D * N) return;   // uniform over the wave
  const int64_t n = chain % N, c = (chain / N) % D, b = chain / (N * D);
  const float a2 = p.A[c * N + n] * kLog2e;
  float H = 0.f;   // state after the segments of the previous blocks
  for (int64_t s0 = 0; s0 < S; s0 += 64) {
    const int64_t s = s0 + lane;
    float m = 1.f, v = 0.f;   // identity map for lanes past the last segment
    if (s < S) {
      v = p.ws_h[((b * S + s) * D + c) * N + n];
      m = exp2_fast(a2 * p.ws_sum[(b * S + s) * D + c]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float mo = __shfl_up(m, off, 64), vo = __shfl_up(v, off, 64);
      if (lane >= off) {
        v = fmaf(m, vo, v);
        m *= mo;
      }
    }
    // entering segment s: the maps of the segments before it (earlier lanes) applied to H
    float me = __shfl_up(m, 1, 64), ve = __shfl_up(v, 1, 64);
    if (lane == 0) {
      me = 1.f;
      ve = 0.f;
    }
    if (s < S) p.ws_h[((b * S + s) * D + c) * N + n] = fmaf(me, H, ve);
    H = fmaf(__shfl(m, 63, 64), H, __shfl(v, 63, 64));
  }
  if (p.h_last && lane == 0) p.h_last[(b * D + c) * N + n] = H;
}

// Base-2 exponent below which exp(A S_t) h_in no longer shows in an output: 2^-32 for float32
// outputs (eight bits below their 24-bit significand), 2^-24 for bf16 (fifteen bits below 9).
template <typename io_t> struct CorrectionCut;
template <> struct CorrectionCut<float> { static constexpr float value = -32.0f; };
template <> struct CorrectionCut<bf16_t> { static constexpr float value = -24.0f; };

// Output correction: grid (channel groups of 64, segments 1 .. nseg-1, B), 256 threads. Lane =
// channel; wave w holds states [w NPW, (w + 1) NPW) (no states when w NPW >= N). Per 16-token
// tile the four waves activate the tile's Delta (four rows each) and stage its C; every lane of a
// wave that still has visible states then runs S_t along the tile and writes its states' part of
// C_t . exp(A S_t) h_in; after a barrier wave w finishes rows 4w .. 4w+3 (the parts of the
// active waves added in wave order, gated, added to y in place).
// A wave goes idle once exp(A S_t) < 2^cut for each of its states with h_in != 0 (S only grows
// while Delta >= 0) and the workgroup ends when all four are idle -- unless the segment pass saw
// a negative Delta in these channels, in which case the whole segment is corrected.
template <typename io_t, int N>
__global__ __launch_bounds__(256) void segment_fix_kernel(ScanParams p, int ch_tile) {
  constexpr int T = 16;
  constexpr int NPW = (N + 3) / 4;
  constexpr float kCut = CorrectionCut<io_t>::value;
  using Io = IoTraits<io_t>;
  __shared__ float s_d[T][64];
  __shared__ float s_c[T][N];
  __shared__ float s_p[4][T][64];
  __shared__ int s_act[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t D = p.D, L = p.L;
  const int64_t c0 = (int64_t)blockIdx.x * 64, seg = (int64_t)blockIdx.y + 1, b = blockIdx.z;
  const int64_t c = c0 + lane;
  const bool c_ok = c < D;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = t_begin + p.seg_len < L ? t_begin + p.seg_len : L;
  const io_t* __restrict__ dg = static_cast<const io_t*>(p.delta);
  const io_t* __restrict__ zg = static_cast<const io_t*>(p.z);
  const io_t* __restrict__ Cg = static_cast<const io_t*>(p.Cm);
  io_t* __restrict__ yg = static_cast<io_t*>(p.y);

  bool may_stop = true;   // no negative Delta in the segment pass's tiles of these channels
  {
    const int64_t ntd = (D + ch_tile - 1) / ch_tile;
    const int64_t k0 = c0 / ch_tile, k1 = (c0 + 63 < D ? c0 + 63 : D - 1) / ch_tile;
    for (int64_t k = k0; k <= k1; ++k) may_stop = may_stop && p.ws_neg[(b * p.nseg + seg) * ntd + k] == 0;
  }
  const bool wave_has_states = w * NPW < N;   // uniform
  float a2[NPW], hin[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int n = w * NPW + j;
    const bool ok = wave_has_states && c_ok;
    a2[j] = ok ? p.A[c * N + n] * kLog2e : 0.f;
    hin[j] = ok ? p.ws_h[((b * p.nseg + seg) * D + c) * N + n] : 0.f;
  }
  const float bias = (c_ok && p.delta_bias) ? p.delta_bias[c] : 0.f;
  // visible: some state of the lane still adds more than 2^cut of its entering value
  auto visible = [&](float S) {
    bool v = false;
#pragma unroll
    for (int j = 0; j < NPW; ++j) v = v || (hin[j] != 0.f && !(a2[j] * S <= kCut));
    return v;
  };
  bool wave_on = wave_has_states && __any(visible(0.f) ? 1 : 0);
  if (!may_stop) wave_on = wave_has_states;
  if (!__syncthreads_or(wave_on ? 1 : 0)) return;   // nothing to add (every h_in is zero)
  float S = 0.f;

  // The tile's raw inputs are loaded one tile ahead (registers), so a tile waits for memory only
  // at its start and the loads overlap the previous tile's work: this thread's four Delta rows,
  // z and y of the four rows it finishes (the same rows), and one element of the tile's C.
  struct TileIn {
    float d[4], z[4], y[4], cv;
  };
  auto load_tile = [&](int64_t t0, TileIn& in) __attribute__((always_inline)) {
    const int rows = t_end - t0 < T ? (int)(t_end - t0) : T;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * w + i;
      const bool ok = r < rows && c_ok;
      const int64_t idx = (b * L + t0 + r) * D + c;
      in.d[i] = ok ? Io::load(dg, idx) : 0.f;
      in.z[i] = ok && zg ? Io::load(zg, idx) : 0.f;
      in.y[i] = ok ? Io::load(yg, idx) : 0.f;
    }
    in.cv = 0.f;
    if (tid < T * N) {
      const int r = tid / N, n = tid % N;
      if (r < rows) in.cv = Io::load(Cg, (b * L + t0 + r) * N + n);
    }
  };
  static_assert(T * N <= 256, "one C element per thread");
  TileIn nxt;
  load_tile(t_begin, nxt);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
    const TileIn cur = nxt;
    if (t0 + T < t_end) load_tile(t0 + T, nxt);
    const int rows = t_end - t0 < T ? (int)(t_end - t0) : T;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * w + i;
      float d = 0.f;
      if (r < rows && c_ok) {
        d = cur.d[i] + bias;
        if (p.delta_softplus) d = softplus_f32(d);
      }
      s_d[r][lane] = d;
    }
    if (tid < T * N) s_c[tid / N][tid % N] = cur.cv;
    if (lane == 0) s_act[w] = wave_on ? 1 : 0;
    __syncthreads();
    if (wave_on) {
#pragma unroll 4
      for (int r = 0; r < T; ++r) {
        S += s_d[r][lane];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NPW; ++j) acc = fmaf(s_c[r][w * NPW + j] * exp2_fast(a2[j] * S), hin[j], acc);
        s_p[w][r][lane] = acc;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * w + i;
      if (r < rows && c_ok) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (s_act[q]) v += s_p[q][r][lane];
        if (zg) v *= silu(cur.z[i]);
        Io::store(yg, (b * L + t0 + r) * D + c, cur.y[i] + v);
      }
    }
    if (may_stop && wave_on) wave_on = __any(visible(S) ? 1 : 0);
    // (also the barrier between this tile's reads of s_d, s_c, s_p, s_act and the next tile's
    // writes)
    if (!__syncthreads_or(wave_on ? 1 : 0)) break;
  }
}

template <typename io_t>
hipError_t launch_fix_io(const ScanParams& p, int ch_tile, hipStream_t stream) {
  const dim3 grid((unsigned)((p.D + 63) / 64), (unsigned)(p.nseg - 1), (unsigned)p.B);
  switch (p.N) {
    case 1: hipLaunchKernelGGL((segment_fix_kernel<io_t, 1>), grid, dim3(256), 0, stream, p, ch_tile); break;
    case 2: hipLaunchKernelGGL((segment_fix_kernel<io_t, 2>), grid, dim3(256), 0, stream, p, ch_tile); break;
    case 4: hipLaunchKernelGGL((segment_fix_kernel<io_t, 4>), grid, dim3(256), 0, stream, p, ch_tile); break;
    case 8: hipLaunchKernelGGL((segment_fix_kernel<io_t, 8>), grid, dim3(256), 0, stream, p, ch_tile); break;
    case 16: hipLaunchKernelGGL((segment_fix_kernel<io_t, 16>), grid, dim3(256), 0, stream, p, ch_tile); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_segment_fix(const ScanParams& p, int ch_tile, hipStream_t stream) {
  if (p.nseg < 2) return hipErrorInvalidValue;
  const int64_t chains = p.B * p.D * p.N;
  hipLaunchKernelGGL(segment_carry_kernel, dim3((unsigned)((chains + 3) / 4)), dim3(256), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return p.io_bf16 ? launch_fix_io<bf16_t>(p, ch_tile, stream) : launch_fix_io<float>(p, ch_tile, stream);
}

}  // namespace ssm
