/*
 * gdn_oracle.c -- f64 CPU oracle for the Gated DeltaNet mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU path.
 *
 * Everything here is the plain definition, computed token by token in double
 * precision, in the order the pages state it.  Parallelism (OpenMP) runs only
 * over independent (batch, head) sequences or channels; every recurrence stays
 * sequential.  Inputs arrive as f64 arrays holding exactly the (rounded) values
 * the GPU receives; nothing here emulates GPU rounding.
 *
 * Source passages (cited by page title and section):
 *   [card]  "Qwen3.8 27B" model card (nest.franknoh.dev), "Gated DeltaNet"
 *           bullet: projection -> width-4 depthwise causal conv + silu over
 *           q/k/v; L2-normalised q and k; per value head a [128,128] state
 *           decayed by exp(-exp(A_log)*softplus(a+dt_bias)) and written at
 *           rate sigmoid(b) by the gated delta rule; head outputs
 *           RMS-normalised and gated by silu(z).  "Norms" bullet: scale by
 *           1+w, in f32.  State paragraph: conv history and recurrent state
 *           kept per row in f32.
 *   [viz]   "Qwen/Qwen3.8-27B" architecture viewer (llm-arch-viz), module
 *           tree: conv1d 10240x1x4 (41.0K parameters, hence no bias),
 *           Qwen3_5RMSNormGated of width 128; header "RMSNorm eps 1e-06".
 *   [viz]   module tree, linear layers of the mixer: in_proj_qkv 5120->10240,
 *           in_proj_z 5120->6144, in_proj_a and in_proj_b 5120->48,
 *           out_proj 6144->5120 (a Linear maps x to x W^T, W stored
 *           [out][in]).
 *   [cuda]  "qwen38" code-generation page (docs.logicaffeine.com), extra
 *           kernels: the two 48-wide gate projections keep f32 weights.
 *   Update rule as written out in the project statement:
 *           S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *           o_t = S_t q_t.
 *
 * Parity status of each function (what pins it; see tests/test_oracle_*.py):
 *   gdn_oracle_gates           pinned: closed forms at 0 and +-inf, numpy/scipy
 *                              library routines for softplus and the logistic.
 *   gdn_oracle_conv_silu       pinned: identity tap, impulse response (tap
 *                              order), numpy.convolve, split-run invariance.
 *   gdn_oracle_l2norm_heads    pinned: unit norm, constant-vector closed form,
 *                              numpy.linalg.norm.
 *   gdn_oracle_recurrence      pinned: exact-rational brute force of the
 *                              matrix-product form, beta=0 / unit-key closed
 *                              forms, orthonormal-key masked matmul, scalar EMA,
 *                              split invariance, head-sharing map, chunked WY
 *                              form.
 *   gdn_oracle_gated_rmsnorm   pinned: constant-vector closed form, z=0,
 *                              w=-1, scale invariance, logistic library.
 *   gdn_oracle_linear          pinned: numpy matmul, identity and permutation
 *                              weights, exact small-integer brute force,
 *                              linearity.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_num_threads(void);
void gdn_oracle_set_num_threads(int n);

#ifdef _OPENMP
#include <omp.h>
int gdn_oracle_num_threads(void) { return omp_get_max_threads(); }
void gdn_oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int gdn_oracle_num_threads(void) { return 1; }
void gdn_oracle_set_num_threads(int n) { (void)n; }
#endif

/* silu(x) = x * logistic(x) = x / (1 + e^-x). */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written in the overflow-free form
 * max(x, 0) + log1p(e^-|x|).  No threshold cut-off. */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* logistic(x) = 1 / (1 + e^-x); gives exactly 0 at -inf and 1 at +inf. */
static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Gates [card, Gated DeltaNet bullet]:
 *   g     = -exp(A_log[h]) * softplus(a + dt_bias[h])   (log of the decay)
 *   alpha = exp(g)
 *   beta  = logistic(b)
 * a, b, alpha, beta, g are [N, H] row-major; A_log, dt_bias are [H].
 * g may be NULL.
 */
void gdn_oracle_gates(const double* a, const double* b, const double* A_log,
                      const double* dt_bias, double* alpha, double* beta,
                      double* g, int64_t N, int32_t H) {
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t i = n * H + h;
      const double gl = -exp(A_log[h]) * softplus(a[i] + dt_bias[h]);
      if (g) g[i] = gl;
      alpha[i] = exp(gl);
      beta[i] = logistic(b[i]);
    }
  }
}

/*
 * Depthwise causal conv of width W followed by silu [card; viz conv1d
 * 10240x1x4 without bias].  Cross-correlation over the padded sequence
 * xhat = [hist (W-1 rows); x (T rows)]:
 *   y[b,t,c] = silu( sum_{i<W} w[c,i] * xhat[b, t+i, c] )
 * so w[c, W-1] multiplies the current token and w[c, 0] the oldest.
 * hist_out[b, j, c] = xhat[b, T+j, c] for j < W-1 (the last W-1 inputs).
 *   x, y     : [B, T, C]
 *   w        : [C, W]
 *   hist_in  : [B, W-1, C] or NULL (zero history, as for a fresh row)
 *   hist_out : [B, W-1, C] or NULL
 */
void gdn_oracle_conv_silu(const double* x, const double* w,
                          const double* hist_in, double* y, double* hist_out,
                          int32_t B, int32_t T, int32_t C, int32_t W) {
  const int32_t P = W - 1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t bb = 0; bb < B; ++bb) {
    for (int32_t c = 0; c < C; ++c) {
      double* xh = (double*)malloc(sizeof(double) * (size_t)(P + T));
      for (int32_t j = 0; j < P; ++j)
        xh[j] = hist_in ? hist_in[((int64_t)bb * P + j) * C + c] : 0.0;
      for (int32_t t = 0; t < T; ++t) xh[P + t] = x[((int64_t)bb * T + t) * C + c];
      for (int32_t t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int32_t i = 0; i < W; ++i) acc += w[(int64_t)c * W + i] * xh[t + i];
        y[((int64_t)bb * T + t) * C + c] = silu(acc);
      }
      if (hist_out)
        for (int32_t j = 0; j < P; ++j) hist_out[((int64_t)bb * P + j) * C + c] = xh[T + j];
      free(xh);
    }
  }
}

/*
 * L2 normalisation of q and k heads [card: "queries and keys are
 * L2-normalized"].  For each of the N token rows of width C, the first
 * l2_channels channels are split into groups of head_dim and each group is
 * divided by sqrt(sum of squares + eps).  In place.
 */
void gdn_oracle_l2norm_heads(double* y, int64_t N, int32_t C,
                             int32_t l2_channels, int32_t head_dim, double eps) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t g0 = 0; g0 + head_dim <= l2_channels; g0 += head_dim) {
      double* r = y + n * C + g0;
      double ss = 0.0;
      for (int32_t i = 0; i < head_dim; ++i) ss += r[i] * r[i];
      const double inv = 1.0 / sqrt(ss + eps);
      for (int32_t i = 0; i < head_dim; ++i) r[i] *= inv;
    }
  }
}

/*
 * The gated delta rule, token by token.  Per (batch b, value head h), with
 * q/k head kh = h / (Hv / Hk) (consecutive value heads share a q/k head):
 *   S <- alpha_t S (I - beta_t k k^T) + beta_t v k^T
 * evaluated as  u = S k;  S <- alpha_t S + beta_t (v - alpha_t u) k^T,
 * which is the same expression with the product expanded, and then
 *   o_t = S (q_scale * q)   using the updated S.
 * S is [dv, dk] (row i is value channel i, column j key channel j).
 *   q, k   : [B, T, Hk, dk]       v, o : [B, T, Hv, dv]
 *   alpha, beta : [B, T, Hv]
 *   S0, S_out   : [B, Hv, dv, dk]; S0 NULL = zero state; S_out may be NULL.
 */
void gdn_oracle_recurrence(const double* q, const double* k, const double* v,
                           const double* alpha, const double* beta,
                           const double* S0, double* S_out, double* o,
                           int32_t B, int32_t T, int32_t Hk, int32_t Hv,
                           int32_t dk, int32_t dv, double q_scale) {
  const int32_t group = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int32_t bb = 0; bb < B; ++bb) {
    for (int32_t h = 0; h < Hv; ++h) {
      const int32_t kh = h / group;
      double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
      double* u = (double*)malloc(sizeof(double) * (size_t)dv);
      const int64_t sbase = ((int64_t)bb * Hv + h) * dv * dk;
      for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = S0 ? S0[sbase + e] : 0.0;
      for (int32_t t = 0; t < T; ++t) {
        const int64_t bt = (int64_t)bb * T + t;
        const double* kt = k + (bt * Hk + kh) * dk;
        const double* qt = q + (bt * Hk + kh) * dk;
        const double* vt = v + (bt * Hv + h) * dv;
        const double al = alpha[bt * Hv + h];
        const double be = beta[bt * Hv + h];
        for (int32_t i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * kt[j];
          u[i] = acc;
        }
        for (int32_t i = 0; i < dv; ++i) {
          const double d = be * (vt[i] - al * u[i]);
          for (int32_t j = 0; j < dk; ++j)
            S[(int64_t)i * dk + j] = al * S[(int64_t)i * dk + j] + d * kt[j];
        }
        double* ot = o + (bt * Hv + h) * dv;
        for (int32_t i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (q_scale * qt[j]);
          ot[i] = acc;
        }
      }
      if (S_out)
        for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S_out[sbase + e] = S[e];
      free(u);
      free(S);
    }
  }
}

/*
 * Gated RMSNorm per (token, head) [card: outputs RMS-normalised and gated by
 * silu(z); "Norms": scale 1+w; viz: RMSNormGated of width 128, eps 1e-06]:
 *   y = x / sqrt(mean(x^2) + eps) * (1 + w) * silu(z)
 * x, z, y : [N, H, D]; w : [D], shared by all heads.
 */
void gdn_oracle_gated_rmsnorm(const double* x, const double* z, const double* w,
                              double* y, int64_t N, int32_t H, int32_t D, double eps) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t base = (n * H + h) * D;
      double ss = 0.0;
      for (int32_t d = 0; d < D; ++d) ss += x[base + d] * x[base + d];
      const double r = 1.0 / sqrt(ss / D + eps);
      for (int32_t d = 0; d < D; ++d)
        y[base + d] = x[base + d] * r * (1.0 + w[d]) * silu(z[base + d]);
    }
  }
}

/*
 * Linear map of every mixer projection [viz: in_proj_qkv, in_proj_z,
 * in_proj_a, in_proj_b, out_proj; cuda: gate projections with f32 weights]:
 *   y[m][n] = sum_k x[m][k] W[n][k]
 * x : [M, K]; W : [N, K] (the Linear layout, output-major); y : [M, N].
 * The sum runs over k in order, in double precision.
 */
void gdn_oracle_linear(const double* x, const double* W, double* y, int64_t M, int32_t N,
                       int32_t K) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int32_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k) acc += x[m * K + k] * W[(int64_t)n * K + k];
      y[m * N + n] = acc;
    }
  }
}
