/*
 * fp64 oracle of the Mamba-2 layer core -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load or call this library. It shares no code, header, table or
 * helper with the HIP library and is built with gcc, never hipcc.
 *
 * What it computes (the Mamba-2 mixer of the Nemotron-Nano-2 report: hyper.ai
 * summary, section "方法", and neurohive article, section "Архитектура": 8 groups,
 * state dimension 128, head dimension 64, conv window 4; fp32 SSM cache per the
 * neurohive section "Развертывание"), written out in double precision on the
 * exact decoded input values:
 *
 *   conv:   v[t,c] = bias[c] + sum_{k<W} w[c,k] * u[t-(W-1)+k, c]
 *           (history u[-W+1..-1] from conv_state, slot 0 the oldest, zeros if
 *            absent); out = SiLU(v) = v / (1 + e^-v).
 *   dt:     dt[t,h] = softplus(dt_raw[t,h] + dt_bias[h]);  a = exp(dt * A[h]).
 *   scan:   h_t = a_t * h_{t-1} + dt_t * B[t,g] x[t,h]^T      (an N x P matrix)
 *           y_t = h_t^T C[t,g] + D[h] * x[t,h];  out = y * SiLU(z[t,h]).
 *   group of head h: g = floor(h / (H / G)) (contiguous heads share B and C).
 *
 * Readings where the pages are silent: conv taps are a cross-correlation with
 * w[c][W-1] on the current token; SiLU follows the conv bias on every channel;
 * dt * B x^T is taken literally (no zero-order-hold factor); the scan's output
 * carries no RMSNorm.
 *
 * Group RMSNorm of the gated output (the block's RMSNorm, hyper.ai summary,
 * section "方法", applied after the SiLU(z) gate): each row of width channels
 * is cut into G contiguous groups; within a group,
 *   out[k] = g[k] / sqrt(mean_group(g^2) + eps) * weight[k].
 *
 * Three forms are provided so that they pin one another:
 *   O1 oracle_ssd_scan     -- the plain recurrence above, token by token;
 *   O2 oracle_ssd_chunked  -- the same map evaluated chunk by chunk (state
 *                             passed between chunks, quadratic form inside);
 *   decode                 -- conv + scan with L = 1 and states updated in place.
 * The brute-force unrolled form (O3) lives in brute.py.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }
static double silu(double v) { return v / (1.0 + exp(-v)); }

int oracle_threads(int requested) {
#ifdef _OPENMP
  return requested > 0 ? requested : omp_get_max_threads();
#else
  (void)requested;
  return 1;
#endif
}

/* u, out: [B][L][Cc]; w: [Cc][W]; bias: [Cc] or NULL; state_in/out: [B][W-1][Cc] or NULL. */
void oracle_conv1d(long B, long L, long Cc, long W, const double* u, const double* w,
                   const double* bias, const double* state_in, double* out, double* state_out,
                   int nthreads) {
  int nt = oracle_threads(nthreads);
  long hist = W - 1;
#pragma omp parallel for num_threads(nt) schedule(static)
  for (long bc = 0; bc < B * Cc; ++bc) {
    long b = bc / Cc, c = bc % Cc;
    /* extended sequence e[i], i = 0 .. hist+L-1: e[i] = u[i-hist] */
    for (long t = 0; t < L; ++t) {
      double v = bias ? bias[c] : 0.0;
      for (long k = 0; k < W; ++k) {
        long i = t + k; /* index into e */
        double e;
        if (i < hist)
          e = state_in ? state_in[(b * hist + i) * Cc + c] : 0.0;
        else
          e = u[(b * L + (i - hist)) * Cc + c];
        v += w[c * W + k] * e;
      }
      out[(b * L + t) * Cc + c] = silu(v);
    }
  }
  if (state_out) {
    /* final history = e[L .. L+hist-1]; computed into a temporary so that
       state_out may alias state_in */
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(B * hist * Cc));
    for (long b = 0; b < B; ++b)
      for (long j = 0; j < hist; ++j)
        for (long c = 0; c < Cc; ++c) {
          long i = L + j;
          double e;
          if (i < hist)
            e = state_in ? state_in[(b * hist + i) * Cc + c] : 0.0;
          else
            e = u[(b * L + (i - hist)) * Cc + c];
          tmp[(b * hist + j) * Cc + c] = e;
        }
    memcpy(state_out, tmp, sizeof(double) * (size_t)(B * hist * Cc));
    free(tmp);
  }
}

/* O1. x, z, y: [B][L][H*P]; Bm, Cm: [B][L][G*N]; dt_raw: [B][L][H]; h0, h_final: [B][H][N][P].
   heads: list of n_sel head indices to compute (NULL: all H); other heads are not written. */
void oracle_ssd_scan(long B, long L, long H, long P, long G, long N, const double* x,
                     const double* Bm, const double* Cm, const double* dt_raw,
                     const double* dt_bias, const double* A, const double* D, const double* z,
                     const double* h0, double* y, double* h_final, const int* heads, long n_sel,
                     int nthreads) {
  int nt = oracle_threads(nthreads);
  long nh = heads ? n_sel : H;
  long hpg = H / G;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
  for (long bi = 0; bi < B * nh; ++bi) {
    long b = bi / nh;
    long h = heads ? heads[bi % nh] : bi % nh;
    long g = h / hpg;
    double* S = (double*)malloc(sizeof(double) * (size_t)(N * P));
    for (long i = 0; i < N * P; ++i) S[i] = h0 ? h0[(b * H + h) * N * P + i] : 0.0;
    for (long t = 0; t < L; ++t) {
      long row = b * L + t;
      double dt = softplus(dt_raw[row * H + h] + dt_bias[h]);
      double a = exp(dt * A[h]);
      const double* xr = x + row * H * P + h * P;
      const double* Br = Bm + row * G * N + g * N;
      const double* Cr = Cm + row * G * N + g * N;
      for (long n = 0; n < N; ++n) {
        double coef = dt * Br[n];
        for (long p = 0; p < P; ++p) S[n * P + p] = a * S[n * P + p] + coef * xr[p];
      }
      for (long p = 0; p < P; ++p) {
        double acc = 0.0;
        for (long n = 0; n < N; ++n) acc += S[n * P + p] * Cr[n];
        double v = acc + (D ? D[h] * xr[p] : 0.0);
        if (z) v *= silu(z[row * H * P + h * P + p]);
        y[row * H * P + h * P + p] = v;
      }
    }
    if (h_final)
      for (long i = 0; i < N * P; ++i) h_final[(b * H + h) * N * P + i] = S[i];
    free(S);
  }
}

/* O2. Same arguments as O1 plus the chunk length Q (any Q >= 1; the last chunk may be short).
   Inside chunk [c0, c1): l_i = sum_{r=c0..c0+i} dt_r A (inclusive), and
     y_t = exp(l_t) C_t . S_prev                                 (state carried in)
         + sum_{c0<=s<=t} (C_t . B_s) exp(l_t - l_s) dt_s x_s    (within the chunk)
         + D x_t, then gated;
     S_next = exp(l_end) S_prev + sum_s exp(l_end - l_s) dt_s B_s x_s^T.
   Both follow from unrolling the recurrence: prod_{r=s+1..t} a_r = exp(l_t - l_s). */
void oracle_ssd_chunked(long B, long L, long H, long P, long G, long N, long Q, const double* x,
                        const double* Bm, const double* Cm, const double* dt_raw,
                        const double* dt_bias, const double* A, const double* D,
                        const double* z, const double* h0, double* y, double* h_final,
                        const int* heads, long n_sel, int nthreads) {
  int nt = oracle_threads(nthreads);
  long nh = heads ? n_sel : H;
  long hpg = H / G;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
  for (long bi = 0; bi < B * nh; ++bi) {
    long b = bi / nh;
    long h = heads ? heads[bi % nh] : bi % nh;
    long g = h / hpg;
    double* S = (double*)malloc(sizeof(double) * (size_t)(N * P));
    double* dt = (double*)malloc(sizeof(double) * (size_t)Q);
    double* l = (double*)malloc(sizeof(double) * (size_t)Q);
    double* acc = (double*)malloc(sizeof(double) * (size_t)P);
    for (long i = 0; i < N * P; ++i) S[i] = h0 ? h0[(b * H + h) * N * P + i] : 0.0;
    for (long c0 = 0; c0 < L; c0 += Q) {
      long n = (L - c0 < Q) ? (L - c0) : Q;
      double run = 0.0;
      for (long i = 0; i < n; ++i) {
        long row = b * L + c0 + i;
        dt[i] = softplus(dt_raw[row * H + h] + dt_bias[h]);
        run += dt[i] * A[h];
        l[i] = run;
      }
      for (long i = 0; i < n; ++i) {
        long rt = b * L + c0 + i;
        const double* Ct = Cm + rt * G * N + g * N;
        double el = exp(l[i]);
        for (long p = 0; p < P; ++p) {
          double s = 0.0;
          for (long k = 0; k < N; ++k) s += Ct[k] * S[k * P + p];
          acc[p] = el * s;
        }
        for (long j = 0; j <= i; ++j) {
          long rs = b * L + c0 + j;
          const double* Bs = Bm + rs * G * N + g * N;
          double cb = 0.0;
          for (long k = 0; k < N; ++k) cb += Ct[k] * Bs[k];
          double coef = cb * exp(l[i] - l[j]) * dt[j];
          const double* xs = x + rs * H * P + h * P;
          for (long p = 0; p < P; ++p) acc[p] += coef * xs[p];
        }
        const double* xt = x + rt * H * P + h * P;
        for (long p = 0; p < P; ++p) {
          double v = acc[p] + (D ? D[h] * xt[p] : 0.0);
          if (z) v *= silu(z[rt * H * P + h * P + p]);
          y[rt * H * P + h * P + p] = v;
        }
      }
      double lend = l[n - 1], dend = exp(lend);
      for (long i = 0; i < N * P; ++i) S[i] *= dend;
      for (long j = 0; j < n; ++j) {
        long rs = b * L + c0 + j;
        const double* Bs = Bm + rs * G * N + g * N;
        const double* xs = x + rs * H * P + h * P;
        double wgt = exp(lend - l[j]) * dt[j];
        for (long k = 0; k < N; ++k) {
          double cbk = wgt * Bs[k];
          for (long p = 0; p < P; ++p) S[k * P + p] += cbk * xs[p];
        }
      }
    }
    if (h_final)
      for (long i = 0; i < N * P; ++i) h_final[(b * H + h) * N * P + i] = S[i];
    free(acc);
    free(l);
    free(dt);
    free(S);
  }
}

/* Decode: one new token per sequence, states updated in place. It is the conv and the
   scan above with L = 1: u_t [B][Cc] raw xBC of the token, conv_state [B][W-1][Cc],
   dt_raw_t [B][H], z_t [B][H*P] or NULL, ssm_state [B][H][N][P], y_t [B][H*P]. */
void oracle_state_update(long B, long H, long P, long G, long N, long W, const double* u_t,
                         const double* w, const double* bias, double* conv_state,
                         const double* dt_raw_t, const double* dt_bias, const double* A,
                         const double* D, const double* z_t, double* ssm_state, double* y_t,
                         int nthreads) {
  long di = H * P, gn = G * N, Cc = di + 2 * gn;
  double* xbc = (double*)malloc(sizeof(double) * (size_t)(B * Cc));
  oracle_conv1d(B, 1, Cc, W, u_t, w, bias, conv_state, xbc, conv_state, nthreads);
  double* xs = (double*)malloc(sizeof(double) * (size_t)(B * di));
  double* bs = (double*)malloc(sizeof(double) * (size_t)(B * gn));
  double* cs = (double*)malloc(sizeof(double) * (size_t)(B * gn));
  for (long b = 0; b < B; ++b) {
    memcpy(xs + b * di, xbc + b * Cc, sizeof(double) * (size_t)di);
    memcpy(bs + b * gn, xbc + b * Cc + di, sizeof(double) * (size_t)gn);
    memcpy(cs + b * gn, xbc + b * Cc + di + gn, sizeof(double) * (size_t)gn);
  }
  oracle_ssd_scan(B, 1, H, P, G, N, xs, bs, cs, dt_raw_t, dt_bias, A, D, z_t, ssm_state, y_t,
                  ssm_state, NULL, 0, nthreads);
  free(cs);
  free(bs);
  free(xs);
  free(xbc);
}

/* Group RMSNorm of rows of the gated output g (rows x width, width divisible by G):
 * out[r][k] = g[r][k] / sqrt(mean over k' in k's group of g[r][k']^2 + eps) * weight[k]
 * (weight NULL means ones). */
void oracle_group_rmsnorm(long rows, long width, long G, const double* g, const double* weight,
                          double eps, double* out) {
  const long gs = width / G;
  for (long r = 0; r < rows; ++r) {
    for (long q = 0; q < G; ++q) {
      const double* gr = g + r * width + q * gs;
      double ss = 0.0;
      for (long k = 0; k < gs; ++k) ss += gr[k] * gr[k];
      const double inv = 1.0 / sqrt(ss / (double)gs + eps);
      for (long k = 0; k < gs; ++k)
        out[r * width + q * gs + k] = gr[k] * inv * (weight ? weight[q * gs + k] : 1.0);
    }
  }
}
