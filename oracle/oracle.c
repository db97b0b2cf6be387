/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the selective state-space (S6) forward pass and
 * its gradients, its one-token decode step, and the Mamba-2 scalar-A (SSD) layer and its
 * gradients.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. It shares no code, header, table or constant with the GPU library;
 * the product path never calls it.
 *
 * Every input arrives as fp64 (the callers upcast the stored bf16 / fp32 values, which is
 * exact). Every loop runs in the order the definitions are written: sequential in time,
 * one channel (or head) at a time. OpenMP splits only the independent (batch, channel) or
 * (batch, head) pairs, so the result does not depend on the thread count.
 *
 * Sources (web pages on Mamba / selective state-space models):
 *   "Beyond attention: exploring Mamba and state space models" (ai-lab.club), section on
 *     state-space basics: the continuous system h' = A h + B x, y = C h + D x and its
 *     zero-order-hold discretisation  Abar = exp(dA),  Bbar = (dA)^-1 (exp(dA) - I) dB,
 *     h_t = Abar h_{t-1} + Bbar x_t,  y_t = C h_t + D x_t.
 *   Same page, section on the selective SSM: Delta_t = softplus(W x_t + b), B_t, C_t per token.
 *   "Mamba and state space models" (world.lapla.si), section "fixed-size state": the decode
 *     state is the SSM state plus a short convolution holding the last 4 inputs.
 *   Same page, section "Mamba-2: two algorithms": with A a scalar times identity, the layer is
 *     multiplication by a lower-triangular matrix whose (i, j) entry is C at step i times B at
 *     step j times all decay between the two steps.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - A is diagonal, given as A[d, n] (the pages' discretisation specialised to diagonal A:
 *     Bbar_n = expm1(Delta A_n) / A_n * B_n, with the limit Delta * B_n when A_n == 0).
 *   - B_t and C_t are N-wide per token and shared by all channels (and by all SSD heads, or
 *     by the heads of one group when the SSD layer has G groups: head h uses group h / (H / G)).
 *   - D multiplies the SSM input of the channel; NULL means no D term.
 *   - The optional gate is applied after the D term: y <- y * z * sigmoid(z). NULL z: no gate.
 *   - The initial state is zero unless h0 is given.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(u) = log(1 + e^u), evaluated without overflow for either sign. */
static double o_softplus(double u) {
  return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));
}

/* logistic sigmoid, evaluated without overflow for either sign. */
static double o_sigmoid(double v) {
  if (v >= 0.0) return 1.0 / (1.0 + exp(-v));
  double e = exp(v);
  return e / (1.0 + e);
}

/* Zero-order-hold input scale for one diagonal entry: (Delta a)^-1 (exp(Delta a) - 1) Delta
 * = expm1(Delta a) / a, whose limit at a == 0 is Delta. */
static double o_zoh_scale(double dt, double a) {
  return a == 0.0 ? dt : expm1(dt * a) / a;
}

static double o_step_size(double delta, const double* delta_bias, int64_t idx, int delta_softplus) {
  double u = delta + (delta_bias ? delta_bias[idx] : 0.0);
  return delta_softplus ? o_softplus(u) : u;
}

/*
 * oracle_scan: selective scan, one (b, d) channel at a time, sequential in t.
 *   x, delta, z, y : [Bsz, L, D]      delta_bias, Dskip : [D]      A : [D, N]
 *   Bm, Cm         : [Bsz, L, N]      h0, h_last        : [Bsz, D, N]
 * delta_bias, Dskip, z, h0, h_last may be NULL.
 */
void oracle_scan(int64_t Bsz, int64_t L, int64_t D, int64_t N,
                 const double* x, const double* delta, const double* delta_bias, int delta_softplus,
                 const double* A, const double* Bm, const double* Cm, const double* Dskip,
                 const double* z, const double* h0, double* y, double* h_last) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < Bsz; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double* h = (double*)malloc((size_t)N * sizeof(double));
      for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t io = (b * L + t) * D + d;
        const double* Bt = Bm + (b * L + t) * N;
        const double* Ct = Cm + (b * L + t) * N;
        const double dt = o_step_size(delta[io], delta_bias, d, delta_softplus);
        const double xt = x[io];
        double out = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[d * N + n];
          const double abar = exp(dt * a);
          const double bbar = o_zoh_scale(dt, a) * Bt[n];
          h[n] = abar * h[n] + bbar * xt;
          out += Ct[n] * h[n];
        }
        if (Dskip) out += Dskip[d] * xt;
        if (z) out *= z[io] * o_sigmoid(z[io]);
        y[io] = out;
      }
      if (h_last)
        for (int64_t n = 0; n < N; ++n) h_last[(b * D + d) * N + n] = h[n];
      free(h);
    }
  }
}

/*
 * oracle_scan_bwd: gradients of oracle_scan (its reverse-mode derivative, written out).
 *   inputs as oracle_scan, plus dy = dL/dy [Bsz, L, D] and dh_last = dL/dh_last [Bsz, D, N]
 *   (NULL: zero);
 *   outputs dx, ddelta, dz [Bsz, L, D]; dA [D, N]; dBm, dCm [Bsz, L, N]; dDskip, ddelta_bias [D];
 *   dh0 [Bsz, D, N]. dz is written only when z is given; dDskip, ddelta_bias, dh0 may be NULL
 *   (they are the gradients at the given values, also when Dskip, delta_bias or h0 is absent:
 *   then at zero).
 * Per (b, d) the forward recurrence is run again keeping every state h_t, then t walks
 * backwards with the adjoint g = dL/dh_t: it takes C_t times the gradient reaching the readout,
 * feeds the derivatives of h_t = Abar h_{t-1} + phi B_t x_t with respect to its inputs, and
 * passes Abar_t g on to h_{t-1}. Derivatives used (a = A[d, n], Abar = exp(Delta a),
 * phi = expm1(Delta a) / a):
 *   d Abar / d Delta = a Abar,  d phi / d Delta = Abar,
 *   d Abar / d a = Delta Abar,  d phi / d a = (Delta Abar - phi) / a  (Delta^2 / 2 at a = 0),
 *   d softplus(u) / du = sigmoid(u),  d (z sigmoid(z)) / dz = sigmoid(z) (1 + z (1 - sigmoid(z))).
 * OpenMP splits the batch rows only (dBm, dCm sum over channels inside one row); the parameter
 * gradients are summed per row and then over rows in order, so the result is independent of
 * the thread count.
 */
void oracle_scan_bwd(int64_t Bsz, int64_t L, int64_t D, int64_t N,
                     const double* x, const double* delta, const double* delta_bias, int delta_softplus,
                     const double* A, const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* h0, const double* dy, const double* dh_last,
                     double* dx, double* ddelta, double* dA, double* dBm, double* dCm,
                     double* dDskip, double* ddelta_bias, double* dz, double* dh0) {
  double* pA = (double*)calloc((size_t)(Bsz * D * N) + 1, sizeof(double));
  double* pD = (double*)calloc((size_t)(Bsz * D) + 1, sizeof(double));
  double* pb = (double*)calloc((size_t)(Bsz * D) + 1, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < Bsz; ++b) {
    double* hs = (double*)malloc((size_t)((L + 1) * N) * sizeof(double));  /* hs[t+1] = h_t */
    double* g = (double*)malloc((size_t)N * sizeof(double));
    for (int64_t i = 0; i < L * N; ++i) dBm[b * L * N + i] = dCm[b * L * N + i] = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t io = (b * L + t) * D + d;
        const double* Bt = Bm + (b * L + t) * N;
        const double dt = o_step_size(delta[io], delta_bias, d, delta_softplus);
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[d * N + n];
          hs[(t + 1) * N + n] = exp(dt * a) * hs[t * N + n] + o_zoh_scale(dt, a) * Bt[n] * x[io];
        }
      }
      for (int64_t n = 0; n < N; ++n) g[n] = dh_last ? dh_last[(b * D + d) * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t io = (b * L + t) * D + d;
        const double* Bt = Bm + (b * L + t) * N;
        const double* Ct = Cm + (b * L + t) * N;
        const double u = delta[io] + (delta_bias ? delta_bias[d] : 0.0);
        const double dt = delta_softplus ? o_softplus(u) : u;
        const double xt = x[io];
        /* gradient reaching y before the gate; the gate's own derivative needs y */
        double gy = dy[io];
        if (z) {
          double yt = 0.0;
          for (int64_t n = 0; n < N; ++n) yt += Ct[n] * hs[(t + 1) * N + n];
          if (Dskip) yt += Dskip[d] * xt;
          const double zt = z[io], sg = o_sigmoid(zt);
          dz[io] = dy[io] * yt * sg * (1.0 + zt * (1.0 - sg));
          gy = dy[io] * zt * sg;
        }
        double gx = Dskip ? Dskip[d] * gy : 0.0;
        double gdt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const double a = A[d * N + n];
          const double abar = exp(dt * a);
          const double phi = o_zoh_scale(dt, a);
          const double hprev = hs[t * N + n];
          const double gn = g[n] + Ct[n] * gy;          /* dL/dh_t */
          dCm[(b * L + t) * N + n] += gy * hs[(t + 1) * N + n];
          dBm[(b * L + t) * N + n] += gn * phi * xt;
          gx += gn * phi * Bt[n];
          gdt += gn * (a * abar * hprev + abar * Bt[n] * xt);
          const double dphi_da = a == 0.0 ? 0.5 * dt * dt : (dt * abar - phi) / a;
          pA[(b * D + d) * N + n] += gn * (dt * abar * hprev + dphi_da * Bt[n] * xt);
          g[n] = abar * gn;                             /* on to dL/dh_{t-1} */
        }
        const double gu = delta_softplus ? gdt * o_sigmoid(u) : gdt;
        dx[io] = gx;
        ddelta[io] = gu;
        pb[b * D + d] += gu;
        pD[b * D + d] += gy * xt;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = g[n];
    }
    free(g);
    free(hs);
  }
  for (int64_t d = 0; d < D; ++d) {
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t b = 0; b < Bsz; ++b) s += pA[(b * D + d) * N + n];
      dA[d * N + n] = s;
    }
    double sD = 0.0, sb = 0.0;
    for (int64_t b = 0; b < Bsz; ++b) {
      sD += pD[b * D + d];
      sb += pb[b * D + d];
    }
    if (dDskip) dDskip[d] = sD;
    if (ddelta_bias) ddelta_bias[d] = sb;
  }
  free(pb);
  free(pD);
  free(pA);
}

/*
 * oracle_conv1d: the depthwise causal convolution the decode state keeps (page "Mamba and state
 * space models", section "fixed-size state": a short convolution over the last inputs), run over
 * a whole sequence for the prefill.
 *   x, u        : [Bsz, L, D]    conv_w : [D, W] (conv_w[d, W-1] multiplies the newest input)
 *   conv_b      : [D] or NULL    conv_in, conv_out : [Bsz, D, W] (oldest input first) or NULL
 * u[b, t, d] = sum_k conv_w[d, k] * r_t[k] (+ conv_b[d]), where r_t holds the W raw inputs up to
 * and including x_t, oldest first; inputs before the sequence come from conv_in (zeros if NULL).
 * conv_out receives the register after the last token.
 */
void oracle_conv1d(int64_t Bsz, int64_t L, int64_t D, int64_t W, const double* x,
                   const double* conv_w, const double* conv_b, const double* conv_in,
                   double* u, double* conv_out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < Bsz; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      double* reg = (double*)malloc((size_t)W * sizeof(double));
      for (int64_t k = 0; k < W; ++k) reg[k] = conv_in ? conv_in[(b * D + d) * W + k] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        for (int64_t k = 0; k + 1 < W; ++k) reg[k] = reg[k + 1];
        reg[W - 1] = x[(b * L + t) * D + d];
        double acc = conv_b ? conv_b[d] : 0.0;
        for (int64_t k = 0; k < W; ++k) acc += conv_w[d * W + k] * reg[k];
        u[(b * L + t) * D + d] = acc;
      }
      if (conv_out)
        for (int64_t k = 0; k < W; ++k) conv_out[(b * D + d) * W + k] = reg[k];
      free(reg);
    }
  }
}

/*
 * oracle_step: one decode token per (b, d).
 *   x, delta, z, y : [Bsz, D]   Bm, Cm : [Bsz, N]   A : [D, N]   h : [Bsz, D, N] (in/out)
 *   conv_state     : [Bsz, D, W] (in/out; oldest input first, newest last) or NULL
 *   conv_w         : [D, W] (conv_w[d, W-1] multiplies the newest input)   conv_b : [D] or NULL
 * With conv_state == NULL the SSM input is x itself; otherwise the register is shifted by one,
 * x enters at the newest slot, and the SSM input is the depthwise causal convolution
 * u = sum_k conv_w[d, k] * register[k] (+ conv_b[d]). u replaces x in the D term too.
 */
void oracle_step(int64_t Bsz, int64_t D, int64_t N, int64_t W,
                 const double* x, const double* delta, const double* delta_bias, int delta_softplus,
                 const double* A, const double* Bm, const double* Cm, const double* Dskip,
                 const double* z, double* conv_state, const double* conv_w, const double* conv_b,
                 double* h, double* y) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < Bsz; ++b) {
    for (int64_t d = 0; d < D; ++d) {
      const int64_t io = b * D + d;
      double u = x[io];
      if (conv_state) {
        double* reg = conv_state + io * W;
        for (int64_t k = 0; k + 1 < W; ++k) reg[k] = reg[k + 1];
        reg[W - 1] = x[io];
        u = conv_b ? conv_b[d] : 0.0;
        for (int64_t k = 0; k < W; ++k) u += conv_w[d * W + k] * reg[k];
      }
      const double dt = o_step_size(delta[io], delta_bias, d, delta_softplus);
      double* hs = h + io * N;
      double out = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double a = A[d * N + n];
        hs[n] = exp(dt * a) * hs[n] + o_zoh_scale(dt, a) * Bm[b * N + n] * u;
        out += Cm[b * N + n] * hs[n];
      }
      if (Dskip) out += Dskip[d] * u;
      if (z) out *= z[io] * o_sigmoid(z[io]);
      y[io] = out;
    }
  }
}

/*
 * oracle_ssd: Mamba-2 layer with one scalar A per head, run as the plain recurrence
 * (the chunk size plays no part in the result).
 *   x, z, y : [Bsz, L, H, P]   delta : [Bsz, L, H]   delta_bias, A : [H]
 *   Bm, Cm  : [Bsz, L, G, N]: G groups of heads share one B and C (head hd uses group
 *             hd / (H / G); G = 1: shared by all heads)
 *   Dskip   : [H] (one D per head) or, with dskip_per_channel, [H, P]
 *   h0, h_last : [Bsz, H, P, N]
 * State per (b, h): S[p, n] <- exp(Delta a) S[p, n] + expm1(Delta a)/a * x[p] * B[n];
 * y[p] = sum_n C[n] S[p, n] (+ D x[p]), then the optional gate.
 */
void oracle_ssd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                const double* x, const double* delta, const double* delta_bias, int delta_softplus,
                const double* A, const double* Bm, const double* Cm, const double* Dskip,
                int dskip_per_channel, const double* z, const double* h0, double* y, double* h_last) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < Bsz; ++b) {
    for (int64_t hd = 0; hd < H; ++hd) {
      double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
      for (int64_t i = 0; i < P * N; ++i) S[i] = h0 ? h0[(b * H + hd) * P * N + i] : 0.0;
      const double a = A[hd];
      const int64_t grp = hd / (H / G);
      for (int64_t t = 0; t < L; ++t) {
        const double dt = o_step_size(delta[(b * L + t) * H + hd], delta_bias, hd, delta_softplus);
        const double abar = exp(dt * a);
        const double phi = o_zoh_scale(dt, a);
        const double* Bt = Bm + ((b * L + t) * G + grp) * N;
        const double* Ct = Cm + ((b * L + t) * G + grp) * N;
        const double* xt = x + ((b * L + t) * H + hd) * P;
        const double* zt = z ? z + ((b * L + t) * H + hd) * P : NULL;
        double* yt = y + ((b * L + t) * H + hd) * P;
        for (int64_t p = 0; p < P; ++p) {
          double out = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            S[p * N + n] = abar * S[p * N + n] + phi * xt[p] * Bt[n];
            out += Ct[n] * S[p * N + n];
          }
          if (Dskip) out += (dskip_per_channel ? Dskip[hd * P + p] : Dskip[hd]) * xt[p];
          if (zt) out *= zt[p] * o_sigmoid(zt[p]);
          yt[p] = out;
        }
      }
      if (h_last)
        for (int64_t i = 0; i < P * N; ++i) h_last[(b * H + hd) * P * N + i] = S[i];
      free(S);
    }
  }
}

/*
 * oracle_ssd_bwd: the gradients of oracle_ssd's map (B and C in G groups of heads, D per head or
 * per channel) for a loss with dL/dy = dy (the gated output) and dL/dh_last = dh_last (NULL: 0).
 * Reverse mode of the plain recurrence, as oracle_scan_bwd does for the selective scan, with the
 * state of a head a P x N matrix: per (b, head) the states are rebuilt from checkpoints kept every
 * 64 steps, then time is walked backwards with g = dL/dh_t:
 *   dL/dh_t   = g + ybar_t C_t^T            (ybar = dy before the gate's factor z sigma(z))
 *   dC_t     += h_t^T ybar_t                dB_t += phi (dL/dh_t)^T x_t
 *   dx_t      = phi (dL/dh_t) B_t + D ybar_t
 *   dDelta_t  = sum (dL/dh_t) o (a abar h_{t-1} + abar x_t B_t^T)
 *   dA       += sum (dL/dh_t) o (Delta abar h_{t-1} + dphi/da x_t B_t^T)
 *   g         = abar dL/dh_t
 * with abar = exp(Delta a), phi = expm1(Delta a) / a, dphi/da = (Delta abar - phi) / a
 * (Delta^2 / 2 at a = 0); ddelta is taken through the softplus when it is on. dB and dC are
 * summed over the heads of a group, dA, dD and ddelta_bias over batch rows (and tokens), each in
 * a fixed order.
 *   dx, dz : [Bsz, L, H, P]   ddelta : [Bsz, L, H]   dA, ddelta_bias : [H]
 *   dBm, dCm : [Bsz, L, G, N]   dDskip : as Dskip   dh0 : [Bsz, H, P, N]
 * Gradients of absent optional inputs (dz without z, dDskip without D, ...) may be NULL; those
 * given for absent inputs are the derivatives at zero.
 */
void oracle_ssd_bwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* x, const double* delta, const double* delta_bias, int delta_softplus,
                    const double* A, const double* Bm, const double* Cm, const double* Dskip,
                    int dskip_per_channel, const double* z, const double* h0, const double* dy,
                    const double* dh_last, double* dx, double* ddelta, double* dA, double* dBm,
                    double* dCm, double* dDskip, double* ddelta_bias, double* dz, double* dh0) {
  const int64_t K = 64;                        /* checkpoint spacing */
  const int64_t nck = (L + K - 1) / K;
  const int64_t PN = P * N;
  /* per (b, head) partial sums, reduced in a fixed order at the end */
  double* pB = (double*)calloc((size_t)(Bsz * H * L * N) + 1, sizeof(double));
  double* pC = (double*)calloc((size_t)(Bsz * H * L * N) + 1, sizeof(double));
  double* pA = (double*)calloc((size_t)(Bsz * H) + 1, sizeof(double));
  double* pb = (double*)calloc((size_t)(Bsz * H) + 1, sizeof(double));
  double* pD = (double*)calloc((size_t)(Bsz * H * P) + 1, sizeof(double));
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < Bsz; ++b) {
    for (int64_t hd = 0; hd < H; ++hd) {
      const double a = A[hd];
      const int64_t grp = hd / (H / G);
      double* ck = (double*)malloc((size_t)(nck * PN + 1) * sizeof(double));  /* state before token s K */
      double* hs = (double*)malloc((size_t)((K + 1) * PN) * sizeof(double));  /* hs[k] = state before token s K + k */
      double* g = (double*)malloc((size_t)PN * sizeof(double));
      double* ybar = (double*)malloc((size_t)P * sizeof(double));
      double* gx = (double*)malloc((size_t)P * sizeof(double));
      for (int64_t i = 0; i < PN; ++i) hs[i] = h0 ? h0[(b * H + hd) * PN + i] : 0.0;
      /* forward: keep the checkpoints */
      for (int64_t t = 0; t < L; ++t) {
        if (t % K == 0) memcpy(ck + (t / K) * PN, hs, (size_t)PN * sizeof(double));
        const double dt = o_step_size(delta[(b * L + t) * H + hd], delta_bias, hd, delta_softplus);
        const double abar = exp(dt * a), phi = o_zoh_scale(dt, a);
        const double* Bt = Bm + ((b * L + t) * G + grp) * N;
        const double* xt = x + ((b * L + t) * H + hd) * P;
        for (int64_t p = 0; p < P; ++p)
          for (int64_t n = 0; n < N; ++n) hs[p * N + n] = abar * hs[p * N + n] + phi * xt[p] * Bt[n];
      }
      for (int64_t i = 0; i < PN; ++i) g[i] = dh_last ? dh_last[(b * H + hd) * PN + i] : 0.0;
      /* backward, one checkpoint segment at a time */
      for (int64_t sgm = nck - 1; sgm >= 0; --sgm) {
        const int64_t t0 = sgm * K, t1 = t0 + K < L ? t0 + K : L;
        memcpy(hs, ck + sgm * PN, (size_t)PN * sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
          const double dt = o_step_size(delta[(b * L + t) * H + hd], delta_bias, hd, delta_softplus);
          const double abar = exp(dt * a), phi = o_zoh_scale(dt, a);
          const double* Bt = Bm + ((b * L + t) * G + grp) * N;
          const double* xt = x + ((b * L + t) * H + hd) * P;
          double* hn = hs + (t - t0 + 1) * PN;
          const double* hp = hs + (t - t0) * PN;
          for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) hn[p * N + n] = abar * hp[p * N + n] + phi * xt[p] * Bt[n];
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
          const int64_t it = (b * L + t) * H + hd;      /* token-head index */
          const double u = delta[it] + (delta_bias ? delta_bias[hd] : 0.0);
          const double dt = delta_softplus ? o_softplus(u) : u;
          const double abar = exp(dt * a), phi = o_zoh_scale(dt, a);
          const double dphi_da = a == 0.0 ? 0.5 * dt * dt : (dt * abar - phi) / a;
          const double* Bt = Bm + ((b * L + t) * G + grp) * N;
          const double* Ct = Cm + ((b * L + t) * G + grp) * N;
          const double* xt = x + it * P;
          const double* hcur = hs + (t - t0 + 1) * PN;
          const double* hprev = hs + (t - t0) * PN;
          double* pBt = pB + ((b * H + hd) * L + t) * N;
          double* pCt = pC + ((b * H + hd) * L + t) * N;
          for (int64_t p = 0; p < P; ++p) {
            const double Dp = Dskip ? (dskip_per_channel ? Dskip[hd * P + p] : Dskip[hd]) : 0.0;
            const double g_out = dy[it * P + p];
            ybar[p] = g_out;
            if (z) {
              double yp = Dp * xt[p];
              for (int64_t n = 0; n < N; ++n) yp += Ct[n] * hcur[p * N + n];
              const double zt = z[it * P + p], sg = o_sigmoid(zt);
              if (dz) dz[it * P + p] = g_out * yp * sg * (1.0 + zt * (1.0 - sg));
              ybar[p] = g_out * zt * sg;
            }
            gx[p] = Dp * ybar[p];
            pD[(b * H + hd) * P + p] += ybar[p] * xt[p];
          }
          double gdt = 0.0, ga = 0.0;
          for (int64_t p = 0; p < P; ++p) {
            for (int64_t n = 0; n < N; ++n) {
              const double gn = g[p * N + n] + Ct[n] * ybar[p];   /* dL/dh_t */
              pCt[n] += ybar[p] * hcur[p * N + n];
              pBt[n] += gn * phi * xt[p];
              gx[p] += gn * phi * Bt[n];
              gdt += gn * (a * abar * hprev[p * N + n] + abar * xt[p] * Bt[n]);
              ga += gn * (dt * abar * hprev[p * N + n] + dphi_da * xt[p] * Bt[n]);
              g[p * N + n] = abar * gn;                         /* on to dL/dh_{t-1} */
            }
          }
          for (int64_t p = 0; p < P; ++p) dx[it * P + p] = gx[p];
          const double gu = delta_softplus ? gdt * o_sigmoid(u) : gdt;
          ddelta[it] = gu;
          pb[b * H + hd] += gu;
          pA[b * H + hd] += ga;
        }
      }
      if (dh0)
        for (int64_t i = 0; i < PN; ++i) dh0[(b * H + hd) * PN + i] = g[i];
      free(gx);
      free(ybar);
      free(g);
      free(hs);
      free(ck);
    }
  }
  for (int64_t b = 0; b < Bsz; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t k = 0; k < G; ++k)
        for (int64_t n = 0; n < N; ++n) {
          double sb = 0.0, sc = 0.0;
          for (int64_t hd = k * (H / G); hd < (k + 1) * (H / G); ++hd) {
            sb += pB[((b * H + hd) * L + t) * N + n];
            sc += pC[((b * H + hd) * L + t) * N + n];
          }
          dBm[((b * L + t) * G + k) * N + n] = sb;
          dCm[((b * L + t) * G + k) * N + n] = sc;
        }
  for (int64_t hd = 0; hd < H; ++hd) {
    double sa = 0.0, sb = 0.0;
    for (int64_t b = 0; b < Bsz; ++b) {
      sa += pA[b * H + hd];
      sb += pb[b * H + hd];
    }
    dA[hd] = sa;
    if (ddelta_bias) ddelta_bias[hd] = sb;
    if (dDskip) {
      if (dskip_per_channel) {
        for (int64_t p = 0; p < P; ++p) {
          double s = 0.0;
          for (int64_t b = 0; b < Bsz; ++b) s += pD[(b * H + hd) * P + p];
          dDskip[hd * P + p] = s;
        }
      } else {
        double s = 0.0;
        for (int64_t b = 0; b < Bsz; ++b)
          for (int64_t p = 0; p < P; ++p) s += pD[(b * H + hd) * P + p];
        dDskip[hd] = s;
      }
    }
  }
  free(pD);
  free(pb);
  free(pA);
  free(pC);
  free(pB);
}

/* Thread count for the following OpenMP regions (n >= 1); used to time a single core. The
   results do not depend on it. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Number of threads an OpenMP region would use (reported beside CPU timings). */
int oracle_num_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
