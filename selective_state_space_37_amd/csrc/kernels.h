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
};

// Workspace bytes for a plan with nseg segments (0 when nseg == 1).
size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int64_t nseg);

// Enqueue the scan (one to three kernels) on the stream. Returns hipSuccess or the launch error.
hipError_t launch_scan(const ScanParams& p, hipStream_t stream);

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
  const void* x;           // bf16 [B, L, H, P]
  const void* delta;       // bf16 [B, L, H]
  const void* z;           // nullable
  const void* Bm;          // bf16 [B, L, N]
  const void* Cm;
  const float* delta_bias; // nullable [H]
  const float* A;          // [H]
  const float* Dskip;      // nullable [H]
  const float* h0;         // nullable [B, H, P, N]
  void* y;
  float* h_last;           // nullable
  int delta_softplus;
  void* ws_hin;            // bf16 [B, nchunks, H, P, N]: state entering each chunk
  void* ws_G;              // bf16 [B, nchunks, Q, Q]: C_i . B_j inside each chunk
  void* ws_Bt;             // bf16 [B, nchunks, N, Q]: B of each chunk, transposed
  float2* ws_sphi;         // [B, nchunks, H, Q]: (inclusive cumulative Delta, ZOH input scale)
};

size_t ssd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t Q);
// Point the workspace fields of p at their parts of ws (ssd_workspace_bytes() bytes).
void ssd_workspace_carve(SsdParams& p, void* ws);
hipError_t launch_ssd(const SsdParams& p, hipStream_t stream);

}  // namespace ssm
