/*
 * ssm.h -- C ABI of libssm: the selective state-space (S6) forward pass on MI355X (gfx950).
 *
 * Three operations, as the Mamba pages state them (and the gradients of the first):
 *
 *   ssm_scan_fwd      The selective scan. Page "Beyond attention: exploring Mamba and state
 *                     space models" (ai-lab.club), state-space basics section: zero-order-hold
 *                     discretisation Abar = exp(Delta A), Bbar = (Delta A)^-1 (exp(Delta A) - I)
 *                     Delta B, recurrence h_t = Abar h_{t-1} + Bbar x_t, readout
 *                     y_t = C h_t + D x_t; selective-SSM section: Delta_t = softplus(. + b),
 *                     B_t and C_t per token. Page "Mamba and state space models"
 *                     (world.lapla.si), section "scan on the chip": the expanded state is never
 *                     written out; only y (and, here, the final state) leave the chip.
 *   ssm_state_update  One generated token with constant work: same page, section "fixed-size
 *                     state" -- per channel the N-number SSM state plus a short convolution
 *                     that keeps the last few (4) inputs.
 *   ssd_chunk_fwd     Mamba-2 with A a scalar times the identity per head: same page, section
 *                     "Mamba-2: two algorithms" -- the layer is a lower-triangular matrix
 *                     (C_i . B_j times all decay between steps j and i); the sequence is cut
 *                     into chunks, each chunk is a masked matrix product, and only the state
 *                     passes between chunks.
 *   ssd_chunk_bwd     gradients of ssd_chunk_fwd_grouped, with the same chunked split: within a
 *                     chunk every contraction is a masked matrix product on the matrix cores;
 *                     between chunks only the state (forwards) and its adjoint (backwards) pass.
 *   ssm_block_step    one decode token through a whole Mamba block for the generation workload
 *                     ("Mamba and state space models", section "how much faster": tokens per
 *                     second at batch 128): LayerNorm and residual (the code overview on "Beyond
 *                     attention"), the gated projections (the news write-up's "architecture"
 *                     section), the short convolution of the decode state ("fixed-size state")
 *                     with SiLU, Delta / B / C from small projections, the selective state update.
 *                     ssm_linear and ssm_layernorm are its products and its norm, exposed for the
 *                     model around the blocks (final norm, LM head).
 *   ssd_chunk_fwd_grouped  the same layer with B and C given per group of heads and D per head
 *                     or per channel. The page likens the layer to masked attention (C as the
 *                     queries, B as the keys, the input as the values); groups let several heads
 *                     share one B and C, as heads can share keys and queries. The pages do not
 *                     spell groups out: head h uses group h / (H / G), G = 1 is ssd_chunk_fwd.
 *
 * Conventions shared by every entry point
 *   - Sizes are int64_t. Tensors are dense, row-major, contiguous; no strides.
 *   - Tensor pointers are DEVICE pointers (memory the caller allocated on the current HIP
 *     device). The library never allocates, frees or keeps them. Scratch space, when an
 *     operation needs it, is a caller-provided device workspace whose size the matching
 *     *_workspace_bytes query returns.
 *   - io_dtype selects the storage type of the per-token tensors (x, delta, z, B, C, y and the
 *     decode conv register): SSM_F32 (float) or SSM_BF16 (bfloat16 bits). Parameters (A,
 *     delta_bias, D, conv weights) and states (h0, h_last, h) are always float32.
 *     All arithmetic is float32; bf16 results are rounded to nearest-even.
 *   - stream is a hipStream_t (NULL = the null stream). Calls only enqueue work; a device
 *     fault surfaces at the caller's next synchronisation.
 *   - Every argument is validated on the host before anything is enqueued; no call
 *     synchronises the device. A failed call returns a non-zero ssm_status, enqueues nothing
 *     and leaves the text in ssm_last_error_detail() (per thread).
 *   - Per-token pointers (x, delta, z, y, B, C) and the conv register must be 16-byte aligned.
 *   - A must be strictly negative (the decaying diagonal the pages use; A = 0 is the
 *     Delta * B limit, which the kernels do not special-case: it gives NaN).
 */
#ifndef SSM_H_
#define SSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 1

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARGUMENT = 1,   /* NULL required pointer, bad size, misalignment, aliasing */
  SSM_ERR_UNSUPPORTED = 2,        /* valid but not implemented: N, P, chunk, dtype combination */
  SSM_ERR_WORKSPACE_TOO_SMALL = 3,
  SSM_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} ssm_status;

typedef enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

/* Static text for a status code ("SSM_OK", ...). Never NULL. */
const char* ssm_status_string(ssm_status status);

/* Detail of the last failed call on this thread ("" if none). Valid until the next call. */
const char* ssm_last_error_detail(void);

/*
 * ssm_scan_fwd -- selective scan over L tokens for B sequences of D channels, N states each.
 *
 *   x, delta, z, y : [B, L, D]  io_dtype     (channels innermost)
 *   Bm, Cm         : [B, L, N]  io_dtype     (one N-vector per token, shared by all channels)
 *   A              : [D, N]     float32      (< 0)
 *   delta_bias     : [D]        float32 or NULL (0)
 *   Dskip          : [D]        float32 or NULL (no D x term)
 *   h0             : [B, D, N]  float32 or NULL (zero initial state)
 *   h_last         : [B, D, N]  float32 or NULL (final state not returned); may equal h0
 *   z              : NULL, or the gate input: y <- y * z * sigmoid(z) after the D term
 *
 *   Per (b, t, d): Delta = delta + delta_bias[d], then softplus(Delta) if delta_softplus != 0;
 *   for each n: Abar = exp(Delta A[d,n]), h[n] = Abar h[n] + expm1(Delta A[d,n]) / A[d,n]
 *   * Bm[b,t,n] * x[b,t,d]; y = sum_n Cm[b,t,n] h[n] + Dskip[d] x[b,t,d]; gate.
 *
 *   Requirements: B, L >= 0 (B == 0 or L == 0 is a no-op, except that with L == 0 h_last
 *   receives h0 or zeros); D >= 1 and D % 4 == 0; N in {1, 2, 4, 8, 16} and D <= 2^24 (else
 *   SSM_ERR_UNSUPPORTED); y must not overlap any input. workspace may be NULL when
 *   ssm_scan_fwd_workspace_bytes() returns 0.
 *
 *   Long, narrow inputs are split along L into segments whose carries are combined by a
 *   separate pass; that plan needs the workspace. The result does not depend on the plan
 *   beyond float32 rounding.
 */
size_t ssm_scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype);

ssm_status ssm_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                        const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                        const float* A, const void* Bm, const void* Cm, const float* Dskip,
                        const void* z, const float* h0, void* y, float* h_last,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments without
 * workspace / workspace_bytes, same plan and kernels, same results. The only scratch the scan
 * needs (the segment carries of a long, narrow input) lives in a device array inside the library,
 * SSM_SCAN_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, held from the library's load until the process
 * ends. The automatic plan splits L only while the channel tiles alone fill fewer than 512
 * workgroups, into at most about 1024 workgroups' worth of segments, so its workspace
 * (ssm_scan_fwd_workspace_bytes()) never exceeds about 3.4 MB.
 *
 *   Errors: those of ssm_scan_fwd; SSM_ERR_WORKSPACE_TOO_SMALL if a plan ever needed more than
 *   SSM_SCAN_NOALLOC_SCRATCH_BYTES, checked on the host before anything is enqueued; SSM_ERR_HIP
 *   if the array's address cannot be obtained on the current device.
 *   It calls no hipMalloc, hipFree, hipMemsetAsync or hipMemcpyAsync (the empty-sequence state
 *   copy is a kernel). The first call on a device looks the array's address up, a host-side query
 *   that enqueues nothing; a caller that captures graphs can make one ordinary call first.
 *   Every call on a GPU uses that GPU's one array and leaves its contents behind (nothing in it
 *   needs to start at zero): calls that overlap on one GPU (other streams, other host threads)
 *   race on it, and the caller must serialise them.
 */
#define SSM_SCAN_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

ssm_status ssm_scan_fwd_noalloc(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                                const void* x, const void* delta, const float* delta_bias,
                                int delta_softplus, const float* A, const void* Bm, const void* Cm,
                                const float* Dskip, const void* z, const float* h0, void* y,
                                float* h_last, void* stream);

/*
 * ssm_scan_fwd_segmented -- ssm_scan_fwd with an explicit segment length along L
 * (segment_len >= 1; segment_len >= L means one segment). The workspace size for it is
 * ssm_scan_fwd_segmented_workspace_bytes(). Used to check that results do not depend on the
 * split (the pages: only state passes between chunks).
 */
size_t ssm_scan_fwd_segmented_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                              int64_t segment_len);

ssm_status ssm_scan_fwd_segmented(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                                  const void* x, const void* delta, const float* delta_bias,
                                  int delta_softplus, const float* A, const void* Bm, const void* Cm,
                                  const float* Dskip, const void* z, const float* h0, void* y,
                                  float* h_last, int64_t segment_len,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_fwd_conv -- prefill: the depthwise causal convolution that the decode state keeps
 * (page "Mamba and state space models", section "fixed-size state": a short convolution over the
 * last few inputs), fused in front of ssm_scan_fwd. The scan input of channel d at token t is
 * u = sum_k conv_w[d, k] * r_t[k] + conv_b[d], where r_t holds the conv_width raw inputs up to and
 * including x_t, oldest first; u replaces x in the recurrence and in the D term, exactly as in
 * ssm_state_update, so a prefill followed by decode steps is one consistent sequence.
 *
 *   forward arguments : as ssm_scan_fwd (x holds the raw, unconvolved inputs)
 *   conv_width        : 1 .. 4 (else SSM_ERR_UNSUPPORTED)
 *   conv_w            : [D, conv_width] float32, conv_w[d, conv_width-1] on the newest input
 *   conv_b            : [D] float32 or NULL
 *   conv_state        : [B, D, conv_width] io_dtype, 16-byte aligned, or NULL. On entry: the raw
 *                       inputs before x (oldest first; NULL = zeros). On return: the register
 *                       after the last token (the last conv_width raw inputs), ready for
 *                       ssm_state_update.
 *   segment_len       : 0 = automatic plan; else the segment length along L, rounded up to a
 *                       multiple of 16 (workspace from ssm_scan_fwd_conv_workspace_bytes()).
 *
 *   Requirements: those of ssm_scan_fwd; conv_state overlaps no other tensor.
 */
size_t ssm_scan_fwd_conv_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                         int64_t segment_len);

ssm_status ssm_scan_fwd_conv(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                             const void* x, const void* delta, const float* delta_bias,
                             int delta_softplus, const float* A, const void* Bm, const void* Cm,
                             const float* Dskip, const void* z, const float* h0, int64_t conv_width,
                             const float* conv_w, const float* conv_b, void* conv_state, void* y,
                             float* h_last, int64_t segment_len, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * ssm_scan_bwd -- gradients of ssm_scan_fwd (training): the derivative of the forward map for
 * a loss L, given dy = dL/dy and optionally dh_last = dL/dh_last. The forward is the
 * recurrence of the page "Beyond attention: exploring Mamba and state space models"
 * (state-space basics and selective-SSM sections); its state is recomputed from checkpoints
 * instead of being stored, the recomputation named on the page "Mamba and state space
 * models" (section "scan on the chip").
 *
 *   forward inputs : as ssm_scan_fwd (x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip,
 *                    z, h0), unchanged
 *   dy             : [B, L, D]  io_dtype     dL/dy (y after the gate)
 *   dh_last        : [B, D, N]  float32 or NULL (zero)
 *   dx, ddelta     : [B, L, D]  io_dtype     (out) dL/dx, dL/ddelta (ddelta is the gradient of
 *                                            the raw delta: through the softplus when it is on)
 *   dz             : [B, L, D]  io_dtype     (out) dL/dz; required when z is given, else ignored
 *   dA             : [D, N]     float32      (out)
 *   dBm, dCm       : [B, L, N]  float32      (out; sums over channels are kept in float32)
 *   dDskip         : [D]        float32 or NULL (out; the gradient at Dskip, at zero if Dskip
 *                                            is NULL)
 *   ddelta_bias    : [D]        float32 or NULL (out; likewise at delta_bias or zero)
 *   dh0            : [B, D, N]  float32 or NULL (out; dL/dh0, at h0 or at the zero state)
 *
 *   Sums over channels (dBm, dCm) and over batch rows and time (dA, dDskip, ddelta_bias) are
 *   formed in a fixed order, so repeated calls give identical bits.
 *   Requirements: those of ssm_scan_fwd; no output may overlap an input or another output;
 *   the workspace (ssm_scan_bwd_workspace_bytes(), about 4 N / (storage size) times the size
 *   of x plus partial sums) is required whenever B, L > 0. B == 0 or L == 0 writes zeros to
 *   dA, dDskip, ddelta_bias and (B > 0) dh0 = dh_last or zeros.
 */
size_t ssm_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype);

ssm_status ssm_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                        const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                        const float* A, const void* Bm, const void* Cm, const float* Dskip,
                        const void* z, const float* h0, const void* dy, const float* dh_last,
                        void* dx, void* ddelta, float* dA, float* dBm, float* dCm, float* dDskip,
                        float* ddelta_bias, void* dz, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_bwd_segmented -- ssm_scan_bwd with an explicit segment length along L (rounded up
 * to a multiple of 16; >= L means one segment). Used to check that the gradients do not depend
 * on the split.
 */
size_t ssm_scan_bwd_segmented_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                              int64_t segment_len);

ssm_status ssm_scan_bwd_segmented(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_dtype,
                                  const void* x, const void* delta, const float* delta_bias,
                                  int delta_softplus, const float* A, const void* Bm, const void* Cm,
                                  const float* Dskip, const void* z, const float* h0, const void* dy,
                                  const float* dh_last, void* dx, void* ddelta, float* dA, float* dBm,
                                  float* dCm, float* dDskip, float* ddelta_bias, void* dz, float* dh0,
                                  int64_t segment_len, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * ssm_state_update -- one decode token for B sequences of D channels (N states each).
 *
 *   x, delta, z, y : [B, D]      io_dtype
 *   Bm, Cm         : [B, N]      io_dtype
 *   A              : [D, N]      float32 (< 0)
 *   delta_bias     : [D] float32 or NULL;  Dskip : [D] float32 or NULL;  z : [B, D] or NULL
 *   h              : [B, D, N]   float32, read and overwritten with the new state
 *   conv_state     : [B, D, W]   io_dtype, oldest input first, read and overwritten; or NULL
 *   conv_w         : [D, W]      float32 (conv_w[d, W-1] multiplies the newest input)
 *   conv_b         : [D]         float32 or NULL
 *
 *   With conv_state: the register shifts by one, x enters as the newest entry, and the SSM
 *   input of the channel is u = sum_k conv_w[d,k] * register[k] + conv_b[d] (no activation);
 *   without it, u = x. Then the scan step on u (u is also the input of the D term), then gate.
 *
 *   Requirements: B >= 0 (0 is a no-op), D >= 1, N in {1, 2, 4, 8, 16}, 1 <= W <= 8 when
 *   conv_state is given (conv_width is ignored otherwise); y must not overlap any input;
 *   h, A and conv_w (besides the per-token tensors) are 16-byte aligned.
 */
ssm_status ssm_state_update(int64_t B, int64_t D, int64_t N, int64_t conv_width, ssm_dtype io_dtype,
                            const void* x, const void* delta, const float* delta_bias,
                            int delta_softplus, const float* A, const void* Bm, const void* Cm,
                            const float* Dskip, const void* z, void* conv_state,
                            const float* conv_w, const float* conv_b, float* h, void* y,
                            void* stream);

/*
 * ssd_chunk_fwd -- Mamba-2 layer: H heads of P channels, one scalar A per head, N states.
 *
 *   x, z, y        : [B, L, H, P]   io_dtype
 *   delta          : [B, L, H]      io_dtype (one step size per token and head)
 *   Bm, Cm         : [B, L, N]      io_dtype (shared by all heads)
 *   A              : [H] float32 (< 0);  delta_bias, Dskip : [H] float32 or NULL
 *   h0, h_last     : [B, H, P, N] float32 or NULL; h_last may equal h0
 *
 *   Result: per head the plain recurrence S <- exp(Delta a) S + expm1(Delta a)/a x B^T,
 *   y = S C (+ D x, gate), computed chunk by chunk: within a chunk the masked matrix
 *   (C_i . B_j) exp(a (cumsum Delta_i - cumsum Delta_j)) expm1(a Delta_j)/a on the matrix
 *   cores (bf16 operands, float32 accumulation); between chunks the float32 state.
 *
 *   io_dtype SSM_BF16, or SSM_F32: then x, z, Bm and Cm are first rounded to bf16 copies in the
 *   workspace (they are the matrix-core operands either way), delta is read as float32, and y
 *   is written as float32 (widened from a bf16 result); the accuracy is that of bf16 operands.
 *   The float32 workspace is larger by 3 B L H P + 2 B L N bf16 elements.
 *
 *   Requirements: P == 64; N in {64, 128}; chunk in {64, 128, 256};
 *   B, L >= 0 (0 is a no-op; with L == 0 h_last receives h0 or zeros); 1 <= H <= 65535,
 *   B <= 65535 and at most 65535 chunks (grid dimensions).
 */
size_t ssd_chunk_fwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N,
                                     int64_t chunk, ssm_dtype io_dtype);

ssm_status ssd_chunk_fwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t chunk,
                         ssm_dtype io_dtype, const void* x, const void* delta,
                         const float* delta_bias, int delta_softplus, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip, const void* z,
                         const float* h0, void* y, float* h_last, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * ssd_chunk_fwd_grouped -- ssd_chunk_fwd with G groups of B and C and an optional per-channel D.
 *
 *   Bm, Cm         : [B, L, G, N]   io_dtype; head h reads group h / (H / G) (heads
 *                                   [k H/G, (k+1) H/G) share group k)
 *   Dskip          : NULL, [H] float32 (dskip_per_channel == 0) or [H, P] float32
 *                    (dskip_per_channel != 0: y[.., h, p] += Dskip[h, p] x[.., h, p]; then
 *                    16-byte aligned)
 *   every other argument as in ssd_chunk_fwd.
 *
 *   Requirements: those of ssd_chunk_fwd; G >= 1 and G divides H; B * G <= 65535, H <= 65535
 *   and at most 65535 chunks. The workspace grows with G (C B^T and B per chunk are kept per
 *   group, and with SSM_F32 the bf16 copies of Bm and Cm); query it with
 *   ssd_chunk_fwd_grouped_workspace_bytes.
 */
size_t ssd_chunk_fwd_grouped_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N,
                                             int64_t G, int64_t chunk, ssm_dtype io_dtype);

ssm_status ssd_chunk_fwd_grouped(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                                 int64_t chunk, ssm_dtype io_dtype, const void* x,
                                 const void* delta, const float* delta_bias, int delta_softplus,
                                 const float* A, const void* Bm, const void* Cm,
                                 const float* Dskip, int dskip_per_channel, const void* z,
                                 const float* h0, void* y, float* h_last, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * ssm_linear -- y = x W^T (+ residual) for a batch of token rows, the block's projections.
 *   x        : [M, K] bf16       W : [Nout, K] bf16 (row n = output n)
 *   residual : [M, Nout] bf16 or NULL; may equal y (then y += x W^T)
 *   y        : [M, Nout] bf16 (out); float32 accumulation, rounded once
 *   Requirements: 0 <= M <= 128 (M == 0 is a no-op); K a positive multiple of 128; Nout a positive
 *   multiple of 4; x, W, y, residual 16-byte aligned; y overlaps neither x nor W. The workspace
 *   (ssm_linear_workspace_bytes(), 0 when the product needs no split of K) holds float32 partial
 *   sums. Sums over K are formed in a fixed order.
 */
size_t ssm_linear_workspace_bytes(int64_t M, int64_t K, int64_t Nout);

ssm_status ssm_linear(int64_t M, int64_t K, int64_t Nout, const void* x, const void* W,
                      const void* residual, void* y, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * ssm_layernorm -- per row, (x - mean) / sqrt(var + eps) * w + b (biased variance), float32
 * arithmetic. x, y: [M, D] bf16 (y may equal x; 16-byte aligned); w, b: [D] float32; eps > 0;
 * D a multiple of 8 up to 8192.
 */
ssm_status ssm_layernorm(int64_t M, int64_t D, const void* x, const float* w, const float* b,
                         float eps, void* y, void* stream);

/*
 * ssm_block_step -- one decode token through a Mamba block, for B sequences:
 *   xn = LayerNorm(hidden; ln_w, ln_b, eps)
 *   [xi | zi] = xn W_in^T                                         [B, 2 d_inner]
 *   u  = SiLU(conv(register with xi appended; conv_w, conv_b))        (register updated)
 *   [dl | Bt | Ct] = u W_xp^T,  dt = dl W_dt^T                        (rank-R Delta path)
 *   y  = the selective state update of ssm_state_update on u with delta dt, delta_bias b_dt,
 *        softplus, A, Bt, Ct, Dskip and gate zi (h updated in place)
 *   hidden += y W_out^T
 *
 *   hidden     : [B, d_model] bf16, in/out        conv_state : [B, d_inner, W] bf16, in/out
 *   h          : [B, d_inner, N] float32, in/out
 *   ln_w, ln_b : [d_model] float32      W_in : [2 d_inner, d_model] bf16 (SSM branch rows, then gate rows)
 *   conv_w     : [d_inner, W] float32   conv_b : [d_inner] float32 or NULL
 *   W_xp       : [R + 2 N, d_inner] bf16 (Delta rank rows, B rows, C rows)   W_dt : [d_inner, R] bf16
 *   b_dt       : [d_inner] float32      A : [d_inner, N] float32 (< 0)   Dskip : [d_inner] or NULL
 *   W_out      : [d_model, d_inner] bf16
 *   Intermediate activations (xn, zi, u, [dl | Bt | Ct], y) are bf16 in the workspace
 *   (ssm_block_step_workspace_bytes()); dt stays float32 from the product to the softplus.
 *   Requirements: 0 <= B <= 128 (0 is a no-op); d_model a multiple of 128 up to 8192; d_inner and
 *   R multiples of 128; N in {4, 8, 16}; 1 <= W <= 8; eps > 0; the in/out tensors overlap no
 *   weight, each other or the workspace; pointers of bf16 tensors, A, conv_state and h 16-byte
 *   aligned.
 */
size_t ssm_block_step_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t N,
                                      int64_t W, int64_t R);

ssm_status ssm_block_step(int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t W,
                          int64_t R, void* hidden, const float* ln_w, const float* ln_b, float eps,
                          const void* W_in, const float* conv_w, const float* conv_b,
                          const void* W_xp, const void* W_dt, const float* b_dt, const float* A,
                          const float* Dskip, const void* W_out, void* conv_state, float* h,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssd_chunk_bwd -- gradients of ssd_chunk_fwd_grouped (training): the derivative of the forward
 * map for a loss L, given dy = dL/dy and optionally dh_last = dL/dh_last. Same page and section
 * as ssd_chunk_fwd: inside each chunk the products are masked matrix products; between chunks
 * the state is carried forwards and its adjoint backwards. The state entering each chunk is
 * recomputed, not taken from the forward call.
 *
 *   forward inputs : as ssd_chunk_fwd_grouped (x, delta, delta_bias, delta_softplus, A, Bm, Cm
 *                    [B, L, G, N], Dskip with dskip_per_channel, z, h0), unchanged
 *   dy             : [B, L, H, P]  io_dtype     dL/dy (y after the gate)
 *   dh_last        : [B, H, P, N]  float32 or NULL (zero)
 *   dx, dz         : [B, L, H, P]  io_dtype     (out) dz required when z is given, else ignored
 *   ddelta         : [B, L, H]     io_dtype     (out) gradient of the raw delta (through the
 *                                               softplus when it is on)
 *   dA             : [H]           float32      (out)
 *   dBm, dCm       : [B, L, G, N]  float32      (out) summed over the heads of each group
 *   dDskip         : float32 or NULL (out) [H, P] when dskip_per_channel, else [H]; the
 *                    gradient at Dskip, at zero if Dskip is NULL
 *   ddelta_bias    : [H] float32 or NULL (out; at delta_bias or zero)
 *   dh0            : [B, H, P, N] float32 or NULL (out; at h0 or at the zero state)
 *
 *   The backward works in chunks of 64 tokens whatever chunk the forward used (the result does
 *   not depend on the chunk). Sums over heads (dBm, dCm), over batch rows and time (dA, dDskip,
 *   ddelta_bias) are formed in a fixed order, so repeated calls give identical bits.
 *   Requirements: io_dtype SSM_BF16; P == 64; N in {64, 128}; G >= 1 divides H; B * G <= 65535,
 *   H <= 65535, at most 65535 chunks of 64 tokens; no output may overlap an input or another
 *   output; the workspace (ssd_chunk_bwd_workspace_bytes(): two bf16 states per chunk and
 *   head, per-head float32 partial dB and dC, and small per-chunk terms) is required whenever
 *   B, L > 0. B == 0 or L == 0 writes zeros to dA, dDskip, ddelta_bias and (B > 0) dh0 =
 *   dh_last or zeros.
 */
size_t ssd_chunk_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N,
                                     int64_t G, ssm_dtype io_dtype);

ssm_status ssd_chunk_bwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                         ssm_dtype io_dtype, const void* x, const void* delta,
                         const float* delta_bias, int delta_softplus, const float* A,
                         const void* Bm, const void* Cm, const float* Dskip,
                         int dskip_per_channel, const void* z, const float* h0, const void* dy,
                         const float* dh_last, void* dx, void* ddelta, float* dA, float* dBm,
                         float* dCm, float* dDskip, float* ddelta_bias, void* dz, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H_ */
