/*
 * Driver of the fp64 oracle for the AddressSanitizer / UndefinedBehaviorSanitizer build: every
 * oracle routine on small seeded inputs, with the optional arguments on and off, ragged shapes
 * (L not a multiple of the chunk or checkpoint spacing) and one group of heads or several.
 * Outputs are checked to be finite. Exit status 0 on success; a sanitizer report aborts.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_scan(int64_t Bsz, int64_t L, int64_t D, int64_t N, const double* x, const double* delta,
                 const double* delta_bias, int delta_softplus, const double* A, const double* Bm,
                 const double* Cm, const double* Dskip, const double* z, const double* h0, double* y,
                 double* h_last);
void oracle_scan_bwd(int64_t Bsz, int64_t L, int64_t D, int64_t N, const double* x, const double* delta,
                     const double* delta_bias, int delta_softplus, const double* A, const double* Bm,
                     const double* Cm, const double* Dskip, const double* z, const double* h0,
                     const double* dy, const double* dh_last, double* dx, double* ddelta, double* dA,
                     double* dBm, double* dCm, double* dDskip, double* ddelta_bias, double* dz, double* dh0);
void oracle_conv1d(int64_t Bsz, int64_t L, int64_t D, int64_t W, const double* x, const double* conv_w,
                   const double* conv_b, const double* conv_in, double* u, double* conv_out);
void oracle_step(int64_t Bsz, int64_t D, int64_t N, int64_t W, const double* x, const double* delta,
                 const double* delta_bias, int delta_softplus, const double* A, const double* Bm,
                 const double* Cm, const double* Dskip, const double* z, double* conv_state,
                 const double* conv_w, const double* conv_b, double* h, double* y);
void oracle_ssd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double* x,
                const double* delta, const double* delta_bias, int delta_softplus, const double* A,
                const double* Bm, const double* Cm, const double* Dskip, int dskip_per_channel,
                const double* z, const double* h0, double* y, double* h_last);
void oracle_ssd_bwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double* x,
                    const double* delta, const double* delta_bias, int delta_softplus, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip, int dskip_per_channel,
                    const double* z, const double* h0, const double* dy, const double* dh_last, double* dx,
                    double* ddelta, double* dA, double* dBm, double* dCm, double* dDskip,
                    double* ddelta_bias, double* dz, double* dh0);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double unit(void) {   /* splitmix64 to [-1, 1) */
  uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}
static double* arr(int64_t n, double lo, double hi) {   /* uniform in [lo, hi); one spare element */
  double* a = (double*)malloc(sizeof(double) * (size_t)(n + 1));
  for (int64_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (unit() + 1.0);
  return a;
}
static int bad = 0;
static void finite(const char* what, const double* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) { fprintf(stderr, "%s[%lld] not finite\n", what, (long long)i); ++bad; return; }
}

static void scan_case(int64_t B, int64_t L, int64_t D, int64_t N, int opt) {
  const int64_t t = B * L * D, bc = B * L * N, st = B * D * N;
  double *x = arr(t, -1, 1), *dl = arr(t, -3, 1), *z = arr(t, -2, 2), *Bm = arr(bc, -1, 1), *Cm = arr(bc, -1, 1);
  double *A = arr(D * N, -4, -0.5), *bias = arr(D, -1, 0), *Dk = arr(D, -1, 1), *h0 = arr(st, -1, 1);
  double *dy = arr(t, -1, 1), *dhl = arr(st, -1, 1);
  double *y = arr(t, 0, 0), *hl = arr(st, 0, 0), *dx = arr(t, 0, 0), *dd = arr(t, 0, 0), *dz = arr(t, 0, 0);
  double *dA = arr(D * N, 0, 0), *dB = arr(bc, 0, 0), *dC = arr(bc, 0, 0), *dD = arr(D, 0, 0), *db = arr(D, 0, 0);
  double *dh0 = arr(st, 0, 0);
  const int on = opt & 1;
  oracle_scan(B, L, D, N, x, dl, on ? bias : NULL, on, A, Bm, Cm, on ? Dk : NULL, on ? z : NULL, on ? h0 : NULL,
              y, hl);
  finite("scan y", y, t);
  finite("scan h", hl, st);
  oracle_scan_bwd(B, L, D, N, x, dl, on ? bias : NULL, on, A, Bm, Cm, on ? Dk : NULL, on ? z : NULL,
                  on ? h0 : NULL, dy, on ? dhl : NULL, dx, dd, dA, dB, dC, on ? dD : NULL, on ? db : NULL,
                  on ? dz : NULL, dh0);
  finite("scan_bwd dx", dx, t);
  finite("scan_bwd dA", dA, D * N);
  finite("scan_bwd dh0", dh0, st);
  free(x); free(dl); free(z); free(Bm); free(Cm); free(A); free(bias); free(Dk); free(h0); free(dy); free(dhl);
  free(y); free(hl); free(dx); free(dd); free(dz); free(dA); free(dB); free(dC); free(dD); free(db); free(dh0);
}

static void conv_step_case(int64_t B, int64_t L, int64_t D, int64_t N, int64_t W, int opt) {
  double *x = arr(B * L * D, -1, 1), *cw = arr(D * W, -1, 1), *cb = arr(D, -1, 1), *cin = arr(B * D * W, -1, 1);
  double *u = arr(B * L * D, 0, 0), *cout = arr(B * D * W, 0, 0);
  oracle_conv1d(B, L, D, W, x, cw, opt ? cb : NULL, opt ? cin : NULL, u, cout);
  finite("conv u", u, B * L * D);
  double *xt = arr(B * D, -1, 1), *dt = arr(B * D, -2, 1), *A = arr(D * N, -4, -0.5), *Bm = arr(B * N, -1, 1);
  double *Cm = arr(B * N, -1, 1), *h = arr(B * D * N, -1, 1), *y = arr(B * D, 0, 0), *z = arr(B * D, -1, 1);
  oracle_step(B, D, N, opt ? W : 0, xt, dt, NULL, 1, A, Bm, Cm, NULL, opt ? z : NULL, opt ? cin : NULL,
              opt ? cw : NULL, opt ? cb : NULL, h, y);
  finite("step y", y, B * D);
  free(x); free(cw); free(cb); free(cin); free(u); free(cout); free(xt); free(dt); free(A); free(Bm); free(Cm);
  free(h); free(y); free(z);
}

static void ssd_case(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int opt) {
  const int64_t t = B * L * H * P, th = B * L * H, bc = B * L * G * N, st = B * H * P * N;
  double *x = arr(t, -1, 1), *dl = arr(th, -3, 1), *A = arr(H, -4, -0.5), *Bm = arr(bc, -1, 1), *Cm = arr(bc, -1, 1);
  double *bias = arr(H, -1, 0), *Dk = arr(H * P, -1, 1), *z = arr(t, -2, 2), *h0 = arr(st, -1, 1);
  double *dy = arr(t, -1, 1), *dhl = arr(st, -1, 1);
  double *y = arr(t, 0, 0), *hl = arr(st, 0, 0), *dx = arr(t, 0, 0), *dd = arr(th, 0, 0), *dA = arr(H, 0, 0);
  double *dB = arr(bc, 0, 0), *dC = arr(bc, 0, 0), *dD = arr(H * P, 0, 0), *db = arr(H, 0, 0), *dz = arr(t, 0, 0);
  double *dh0 = arr(st, 0, 0);
  const int on = opt & 1, pc = (opt >> 1) & 1;
  oracle_ssd(B, L, H, P, N, G, x, dl, on ? bias : NULL, on, A, Bm, Cm, on ? Dk : NULL, pc, on ? z : NULL,
             on ? h0 : NULL, y, hl);
  finite("ssd y", y, t);
  oracle_ssd_bwd(B, L, H, P, N, G, x, dl, on ? bias : NULL, on, A, Bm, Cm, on ? Dk : NULL, pc, on ? z : NULL,
                 on ? h0 : NULL, dy, on ? dhl : NULL, dx, dd, dA, dB, dC, on ? dD : NULL, on ? db : NULL,
                 on ? dz : NULL, dh0);
  finite("ssd_bwd dx", dx, t);
  finite("ssd_bwd dB", dB, bc);
  free(x); free(dl); free(A); free(Bm); free(Cm); free(bias); free(Dk); free(z); free(h0); free(dy); free(dhl);
  free(y); free(hl); free(dx); free(dd); free(dA); free(dB); free(dC); free(dD); free(db); free(dz); free(dh0);
}

int main(void) {
  for (int opt = 0; opt < 2; ++opt) {
    scan_case(2, 37, 12, 16, opt);
    scan_case(1, 5, 4, 1, opt);
    scan_case(1, 0, 4, 2, opt);
    conv_step_case(2, 7, 8, 4, 4, opt);
    conv_step_case(1, 2, 4, 16, 3, opt);
  }
  for (int opt = 0; opt < 4; ++opt) {
    ssd_case(1, 70, 4, 8, 6, 1, opt);    /* L past one 64-token checkpoint */
    ssd_case(2, 17, 4, 4, 3, 2, opt);    /* two groups of two heads */
    ssd_case(1, 1, 2, 2, 2, 2, opt);
  }
  if (bad) return 1;
  printf("oracle driver ok\n");
  return 0;
}
