// Internal launch interface between the C ABI layer and the gfx950 kernels (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct ScanParams {
  int64_t B, L, D, N;
  int io_bf16;             // 1: bf16 storage, 0: float
  const void* x;
  const void* delta;
  const void* z;           // nullable
  const void* Bm;
  const void* Cm;
  const float* delta_bias; // nullable
  const float* A;
  const float* Dskip;      // nullable
  const float* h0;         // nullable
  void* y;
  float* h_last;           // nullable
  int delta_softplus;
  int64_t seg_len;         // tokens per segment
  int64_t nseg;            // number of segments (1: single pass)
  float* ws_h;             // [B, nseg, D, N]   (nseg > 1)
  float* ws_sum;           // [B, nseg, D]      (nseg > 1)
  int* ws_neg;             // [B, nseg, channel tiles]: a segment's tile saw Delta < 0 (nseg > 1)
  // causal convolution in front of the scan (prefill); conv_w == nullptr: none
  const float* conv_w;     // [D, conv_W], conv_w[d, W-1] on the newest input
  const float* conv_b;     // nullable [D]
  const void* conv_in;     // nullable [B, D, conv_W] io: raw inputs before the sequence
  void* conv_out;          // nullable [B, D, conv_W] io: the register after the sequence
  int conv_W;              // 1 .. 4
};

// Channels per workgroup of the forward scan kernels for state size N.
int64_t scan_channels_per_tile(int64_t N);

// Workspace bytes for a plan with nseg segments (0 when nseg == 1): ws_h, ws_sum, ws_neg.
size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int64_t nseg);

// After the segment pass of a plan with nseg >= 2 (ws_h = local end states, ws_sum, ws_neg):
// the carry scan over segments (ws_h then holds the state entering each segment, h_last the
// final state) and the output correction of segments 1 .. nseg-1. ch_tile = channels per
// workgroup of the segment pass (the granularity of ws_neg).
hipError_t launch_scan_segment_fix(const ScanParams& p, int ch_tile, hipStream_t stream);

// Enqueue the scan (one to three kernels) on the stream. Returns hipSuccess or the launch error.
hipError_t launch_scan(const ScanParams& p, hipStream_t stream);

// dst[0 .. n) = src (or zeros without src), by a kernel on the stream.
hipError_t launch_state_fill(float* dst, const float* src, int64_t n, hipStream_t stream);

// Enqueue only the segment carries of a plan with nseg >= 2 (state-only pass and carry pass):
// afterwards ws_h[b, s] holds the state entering segment s. The segment length is a multiple
// of 16 tokens.
hipError_t launch_scan_carries(const ScanParams& p, hipStream_t stream);

// Selective-scan backward (gradients by state recomputation).
struct ScanBwdParams {
  int64_t B, L, D, N;
  int io_bf16;
  int delta_softplus;
  const void* x;
  const void* delta;
  const void* z;           // nullable
  const void* Bm;
  const void* Cm;
  const void* dy;          // dL/d(output) [B, L, D] io
  const float* delta_bias; // nullable
  const float* A;
  const float* Dskip;      // nullable
  const float* h0;         // nullable
  const float* dh_last;    // nullable: dL/dh_last [B, D, N]
  void* dx;                // [B, L, D] io
  void* ddelta;            // [B, L, D] io
  void* dz;                // [B, L, D] io (when z)
  float* dA;               // [D, N]
  float* dBm;              // [B, L, N]
  float* dCm;              // [B, L, N]
  float* dDskip;           // nullable [D]
  float* ddelta_bias;      // nullable [D]
  float* dh0;              // nullable [B, D, N]
  int64_t seg_len;         // multiple of 16 (or >= L)
  int64_t nseg;
  int64_t nct;             // channel tiles (D / channels per workgroup, rounded up)
  // workspace parts
  float* ws_ck;            // [B, ceil(L/8), N / NS, D, NS] state at the start of every 8-token tile
  float* ws_pq;            // [B, L, nct, N, 2]  (dB, dC) partial sums per channel tile
  float* ws_pA;            // [B, nseg, D, N]
  float* ws_pD;            // [B, nseg, D]
  float* ws_pb;            // [B, nseg, D]
  float* ws_h;             // [B, nseg, D, N]  state entering each segment   (nseg > 1)
  float* ws_sum;           // [B, nseg, D]     forward pass: sum of Delta    (nseg > 1)
  float* ws_q;             // [B, nseg, D, N]  local adjoint before the segment (nseg > 1)
  float* ws_dsum;          // [B, nseg, D]     sum of Delta over each segment (nseg > 1)
  float* ws_E;             // [B, nseg, D, N]  adjoint entering each segment from later tokens
};

// Channels per workgroup of the backward kernels for state size N.
int64_t scan_bwd_channels_per_wg(int64_t N);
size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t nseg);
void scan_bwd_workspace_carve(ScanBwdParams& p, void* ws);
hipError_t launch_scan_bwd(const ScanBwdParams& p, hipStream_t stream);

struct StepParams {
  int64_t B, D, N, W;
  int io_bf16;
  const void* x;
  const void* delta;
  const void* z;           // nullable
  const void* Bm;
  const void* Cm;
  const float* delta_bias; // nullable
  const float* A;
  const float* Dskip;      // nullable
  void* conv_state;        // nullable
  const float* conv_w;
  const float* conv_b;     // nullable
  float* h;
  void* y;
  int delta_softplus;
};

hipError_t launch_state_update(const StepParams& p, hipStream_t stream);

struct SsdParams {
  int64_t B, L, H, P, N, Q;  // Q = chunk length
  int64_t G;               // groups of B and C: head h reads group h / (H / G)
  const void* x;           // bf16 [B, L, H, P]
  const void* delta;       // bf16 [B, L, H], float32 with delta_f32
  int delta_f32;
  // float32 per-token tensors (launch_ssd): x, z, B and C are first rounded to the bf16 copies
  // cvt_x, cvt_z, cvt_B, cvt_C in the workspace, the layer runs on them with delta read as
  // float32, and y is widened from cvt_y
  int io_f32;
  void *cvt_x, *cvt_z, *cvt_B, *cvt_C, *cvt_y;
  const void* z;           // nullable
  const void* Bm;          // bf16 [B, L, G, N]
  const void* Cm;
  const float* delta_bias; // nullable [H]
  const float* A;          // [H]
  const float* Dskip;      // nullable: [H] per head, or [H, P] per channel
  int dskip_per_channel;
  const float* h0;         // nullable [B, H, P, N]
  void* y;
  float* h_last;           // nullable
  int delta_softplus;
  void* ws_hin;            // bf16 [B, nchunks, H, P, N]: state entering each chunk
  void* ws_G;              // forward: bf16 tiles of C_i . B_j on and below the diagonal, per chunk
  void* ws_Bt;             // backward: bf16 [B, G, nchunks, N, Q]: B of each chunk, transposed
  void* ws_Btf;            // bf16 [B, G, nchunks, N Q]: B^T of each chunk in MFMA fragment order
  void* ws_Ctf;            // backward: the same for C
  float2* ws_sphi;         // [B, nchunks, H, Q]: (inclusive cumulative Delta, ZOH input scale)
  // forward with the state pass cut into L-segments (NULL otherwise)
  float* ws_seg_h;         // [B, segments, H, P, N]: each segment's own end state
  float* ws_seg_s;         // [B, segments, H]: each segment's sum of step sizes
  void* ws_seg_in;         // bf16 [B, segments, H, P, N]: the state entering each segment
  float* ws_dpre;          // [B, nchunks, H]: the step sizes of the segment's chunks before each chunk
  int nseg;                // segments of the state pass (1: none)
  // backward only (NULL in the forward)
  const void* dy;          // bf16 [B, L, H, P]: dL/dy
  const float* dh_last;    // nullable [B, H, P, N]
  float* dh0;              // nullable [B, H, P, N] (out)
  void* ws_gout;           // bf16 [B, nchunks, H, P, N]: dL/d(state leaving each chunk)
  void* ws_Ct;             // bf16 [B, G, nchunks, N, Q]: C of each chunk, transposed
                           // (in the backward ws_G holds G in float32, [Q][Q])
};

size_t ssd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
                           bool io_f32 = false);
// Point the workspace fields of p at their parts of ws (ssd_workspace_bytes() bytes).
void ssd_workspace_carve(SsdParams& p, void* ws);
hipError_t launch_ssd(const SsdParams& p, hipStream_t stream);

// Gradients of the SSD layer. The backward cuts the sequence into chunks of its own (kSsdBwdQ
// tokens), independent of the forward's chunk length.
constexpr int64_t kSsdBwdQ = 64;
struct SsdBwdParams {
  SsdParams f;             // forward inputs, dy, dh_last, dh0 and the shared workspace parts
  void* dx;                // bf16 [B, L, H, P] (out)
  void* ddelta;            // bf16 [B, L, H] (out)
  void* dz;                // bf16 [B, L, H, P] (out) when z is given
  float* dA;               // [H] (out)
  float* dBm;              // [B, L, G, N] (out)
  float* dCm;
  float* dDskip;           // nullable (out): [H] or [H, P] (dskip_per_channel)
  float* ddelta_bias;      // nullable [H] (out)
  int64_t hb;              // heads per workgroup in the main pass (divides H / G)
  float* ws_dBp;           // [B, H / hb, L, N]: dB summed over each workgroup's heads
  float* ws_dCp;
  float* ws_pA;            // [B, nchunks, H] partial dA
  float* ws_pb;            // [B, nchunks, H] partial ddelta_bias
  float* ws_pD;            // [B, nchunks, H, P] partial dD (per channel)
};

// Products of M <= 128 token rows with a weight matrix: Y[m][n] = sum_k X[m][k] W[n][k] (+ R).
struct GemmParams {
  int64_t M, K, Nout;      // M <= 128, K % 128 == 0, Nout % 4 == 0
  int64_t ldx, ldy;        // row strides (elements) of X and of Y / R
  int64_t S, kslice;       // K splits and their length (set by launch_gemm)
  const void* x;           // bf16 [M, ldx]
  const void* w;           // bf16 [Nout, K]
  void* y;                 // bf16 [M, ldy]
  const void* residual;    // nullable bf16 [M, ldy]; may equal y
  float* partial;          // float [S, M, Nout] when S > 1
  // Optional conv + SiLU epilogue (gemm_xwt_kernel with K not split) for the outputs n < conv_D:
  // the register conv_state[m][n][0 .. conv_W - 1] (bf16) is shifted, the output (rounded to
  // bf16) appended, and u[m][n] = SiLU(sum_k conv_w[n][k] reg[k] + conv_b[n]) stored (row stride
  // conv_D); the outputs n >= conv_D go to y as usual. conv_state NULL = off.
  void* conv_state;
  const float* conv_w;     // [conv_D, conv_W]
  const float* conv_b;     // [conv_D] or NULL
  void* u;                 // bf16 [M, conv_D]
  int64_t conv_D, conv_W;
  // Optional x-projection epilogue (gemm_xwt_kernel with the conv epilogue, up to 2 row tiles):
  // each workgroup of the conv range multiplies its u tile (its rows x 128 channels) by the
  // matching 128 columns of xp_w [xp_n, conv_D] and stores float32 partials
  // xp_partial[conv_D / 128][M][xp_n], one per 128-channel slice, for gemm_reduce_kernel.
  const void* xp_w;
  int64_t xp_n;
  float* xp_partial;
};
// How a product runs. kind 0: the activations stream through LDS in K chunks (gemm_xwt_kernel, MT
// row tiles per row block, S splits of K). kind 1: the activation slice is resident in LDS
// (gemm_res_kernel, all rows in MT tiles, configuration cfg of kResCfgs, S = K / its slice).
// kind 2: as kind 0, but each row block's whole K slice is loaded into LDS once and the weight
// stream runs with no barrier (MT <= 2, K slice a multiple of 512 that fits; gemm_xres_fits).
struct GemmChoice {
  int kind, mt, cfg;
  int64_t S;
};
GemmChoice gemm_plan(int64_t M, int64_t K, int64_t Nout);
bool gemm_xres_fits(int mt, int64_t kslice);
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t Nout);
hipError_t launch_gemm(GemmParams p, hipStream_t stream);
hipError_t launch_gemm_with(GemmParams p, const GemmChoice& c, hipStream_t stream);
hipError_t launch_layernorm(int64_t M, int64_t D, const void* x, const float* w, const float* b, float eps, void* y,
                            hipStream_t stream);

// One decode token through a Mamba block (see block.hip).
struct BlockParams {
  int64_t B, Dm, Di, N, W, R;
  float eps;
  void* hidden;                       // bf16 [B, Dm], in/out (the residual stream)
  const float* ln_w;                  // [Dm]
  const float* ln_b;                  // [Dm]
  const void* W_in;                   // bf16 [2 Di, Dm]: rows [0, Di) the SSM branch, [Di, 2 Di) the gate
  const float* conv_w;                // [Di, W]
  const float* conv_b;                // nullable [Di]
  const void* W_xp;                   // bf16 [R + 2 N, Di]: rows Delta (rank R), B, C
  const void* W_dt;                   // bf16 [Di, R]
  const float* b_dt;                  // [Di]
  const float* A;                     // [Di, N]
  const float* Dskip;                 // nullable [Di]
  const void* W_out;                  // bf16 [Dm, Di]
  void* conv_state;                   // bf16 [B, Di, W], in/out
  float* h;                           // [B, Di, N], in/out
};
size_t block_workspace_bytes(int64_t B, int64_t Dm, int64_t Di, int64_t N, int64_t R);
hipError_t launch_block_step(const BlockParams& p, void* ws, hipStream_t stream);

size_t ssd_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t hb);
void ssd_bwd_workspace_carve(SsdBwdParams& p, void* ws);
hipError_t launch_ssd_bwd(const SsdBwdParams& p, hipStream_t stream);

}  // namespace ssm
