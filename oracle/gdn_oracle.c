/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet (GDN) sublayer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant with the HIP library; the two meet only through the seeded input
 * generators, which hold none of the method's arithmetic.
 *
 * Every routine is the obvious definition, written for a reader to check by
 * eye: fp64 throughout, direct loops, no blocking, fusion or reordering.  The
 * only parallelism is OpenMP over independent (sequence, channel) or
 * (sequence, value-head) pairs, which does not change any result.
 *
 * Sources (web pages; cited by title and section):
 *  [GOLDEN]  pegainfer PR #1152, "Reference golden for the Gated DeltaNet
 *            sublayer of Qwen3.8-Flash-Next": Summary (geometry 16 K / 48 V
 *            heads of 128, conv kernel 4, repeat_interleave ratio 3, sigmoid
 *            gated norm), Consumer (conv1d prefill -> chunk-wise gated delta
 *            rule with prepare = head-expand, L2-norm, split v; then
 *            cumsum -> A -> solve -> recompute -> state -> output; then the
 *            shared gated RMSNorm with the sigmoid activation), Negative
 *            controls (SiLU gate, skipped conv and dropped state carry are the
 *            named faults), code review (gated norm is rsqrt(variance + eps)).
 *  [LEDGER]  "Qwen3.8 kernel architecture and TDD ledger", Current dense-27B
 *            kernel map: scalar GDN recurrence with fused output gate checked
 *            against a CPU oracle; batched/prefill recurrence checked against
 *            one- and multi-chunk sequential oracles.
 *  [GLM]     "GLM-5.3-Flash kernel TDD ledger", Slice ledger rows I2 (FP32
 *            [value,key] state, decay sign, beta, q output scale 1/sqrt(Dk)),
 *            I2a (Q/K unit-L2 x/sqrt(sum(x^2)+eps)), I3 (a conv step equals
 *            the full width-4 causal conv), I4 (chunked equals sequential).
 *  [SSM]     spark_model layers/qwen3_ssm/layer_struct.rs, Qwen3SsmLayer
 *            fields: sequential [Q|K|V|Z] projection layout; per-key-channel
 *            decay appears in the KDA rows of [GLM].
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - conv activation: none or SiLU, selected by the caller (act = 0 / 1);
 *  - conv tap order: w[c][3] multiplies the current token, w[c][0] the
 *    oldest; conv state rows are oldest first;
 *  - recurrence order per token: decay, predict from the decayed state,
 *    write, then read the output from the updated state;
 *  - v-head h reads k-head floor(h * Hk / Hv) (repeat_interleave);
 *  - state layout [value][key] (dv rows, dk columns), row-major.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double conv_act(double y, int32_t act) { return act ? y * sigmoid(y) : y; }

/* Value of channel c at position s of sequence n, where s counts from the
 * sequence start and may be -3..-1 (then it comes from the carried conv state,
 * rows oldest first, or is zero when no state is given). */
static double conv_input(const double* x, int32_t C, int64_t t0, int32_t n,
                         const double* state_in, int64_t s, int32_t c) {
  if (s >= 0) return x[(t0 + s) * C + c];
  if (!state_in) return 0.0;
  return state_in[((int64_t)n * 3 + (3 + s)) * C + c];
}

/*
 * Depthwise causal conv1d of width 4 over N packed sequences [GOLDEN Consumer;
 * GLM row I3].
 *   x        [T][C]       inputs (the projected mixed_qkv rows)
 *   cu       [N+1]        sequence offsets, cu[0] = 0, cu[N] = T
 *   w        [C][4]       taps, w[c][3] on the current token
 *   state_in [N][3][C]    last three inputs before each sequence, or NULL
 *   y        [T][C]       output, after the optional SiLU
 *   state_out[N][3][C]    last three inputs of each sequence, or NULL; may
 *                         alias state_in
 */
void gdn_oracle_conv1d(const double* x, int32_t C, const int32_t* cu, int32_t N,
                       const double* w, const double* state_in, int32_t act,
                       double* y, double* state_out) {
  for (int32_t n = 0; n < N; ++n) {
    const int64_t t0 = cu[n];
    const int64_t len = (int64_t)cu[n + 1] - cu[n];
#pragma omp parallel for schedule(static)
    for (int32_t c = 0; c < C; ++c) {
      for (int64_t t = 0; t < len; ++t) {
        double acc = 0.0;
        for (int i = 0; i < 4; ++i)
          acc += w[c * 4 + i] * conv_input(x, C, t0, n, state_in, t - 3 + i, c);
        y[(t0 + t) * C + c] = conv_act(acc, act);
      }
      if (state_out) {
        double keep[3];
        for (int r = 0; r < 3; ++r) keep[r] = conv_input(x, C, t0, n, state_in, len - 3 + r, c);
        for (int r = 0; r < 3; ++r) state_out[((int64_t)n * 3 + r) * C + c] = keep[r];
      }
    }
  }
}

/*
 * One decode token per sequence [GLM row I3: the step form of the same conv].
 * The window is (state rows 0,1,2, x); the state becomes (rows 1,2, x).
 *   x [B][C], w [C][4], state [B][3][C] (in place), y [B][C].
 */
void gdn_oracle_conv1d_step(const double* x, int32_t B, int32_t C, const double* w,
                            double* state, int32_t act, double* y) {
  for (int32_t b = 0; b < B; ++b) {
    double* st = state + (int64_t)b * 3 * C;
    for (int32_t c = 0; c < C; ++c) {
      const double window[4] = {st[0 * C + c], st[1 * C + c], st[2 * C + c], x[(int64_t)b * C + c]};
      double acc = 0.0;
      for (int i = 0; i < 4; ++i) acc += w[c * 4 + i] * window[i];
      y[(int64_t)b * C + c] = conv_act(acc, act);
      st[0 * C + c] = window[1];
      st[1 * C + c] = window[2];
      st[2 * C + c] = window[3];
    }
  }
}

/* out = x / sqrt(sum(x^2) + eps) [GLM row I2a]; with l2norm == 0 a copy. */
static void l2_normalize(const double* x, int32_t d, int32_t l2norm, double eps, double* out) {
  double ss = 0.0;
  for (int32_t i = 0; i < d; ++i) ss += x[i] * x[i];
  const double inv = l2norm ? 1.0 / sqrt(ss + eps) : 1.0;
  for (int32_t i = 0; i < d; ++i) out[i] = x[i] * inv;
}

/*
 * Gated delta rule, token by token [LEDGER kernel map; GLM row I2; GOLDEN
 * Consumer].  Per sequence n and value head h, with S the fp64 [dv][dk] state
 * started from state_in (or zero), each token t does
 *     decay    S[i][j] *= exp(g)            (per key channel: exp(g[j]))
 *     predict  p[i] = sum_j S[i][j] * khat[j]
 *     delta    u[i] = beta * (v[i] - p[i])
 *     write    S[i][j] += u[i] * khat[j]
 *     read     o[i] = sum_j S[i][j] * qtil[j]
 * where khat = L2(k), qtil = L2(q) * q_scale, and value head h reads key head
 * h / (Hv / Hk).
 *
 *   q, k      row t at q + t*qk_stride; head kh at offset kh*dk
 *   v         row t at v + t*v_stride; head h at offset h*dv
 *   g         [T][Hv] (scalar decay) or [T][Hv][dk] (per key channel)
 *   beta      [T][Hv]
 *   cu        [N+1] sequence offsets
 *   state_in  [N][Hv][dv][dk] or NULL (zero)
 *   o         [T][Hv][dv]
 *   state_out [N][Hv][dv][dk] or NULL; may alias state_in
 */
void gdn_oracle_delta_rule(int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                           int32_t per_channel, int32_t l2norm, double l2_eps, double q_scale,
                           const double* q, const double* k, int64_t qk_stride,
                           const double* v, int64_t v_stride,
                           const double* g, const double* beta,
                           const int32_t* cu, int32_t N, const double* state_in,
                           double* o, double* state_out) {
  const int32_t ratio = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < Hv; ++h) {
      const int32_t kh = h / ratio;
      double* S = (double*)calloc((size_t)dv * dk, sizeof(double));
      double* kn = (double*)malloc(sizeof(double) * dk);
      double* qn = (double*)malloc(sizeof(double) * dk);
      double* a = (double*)malloc(sizeof(double) * dk);
      double* u = (double*)malloc(sizeof(double) * dv);
      const int64_t sidx = ((int64_t)n * Hv + h) * dv * dk;
      if (state_in) memcpy(S, state_in + sidx, sizeof(double) * dv * dk);
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        l2_normalize(k + t * qk_stride + (int64_t)kh * dk, dk, l2norm, l2_eps, kn);
        l2_normalize(q + t * qk_stride + (int64_t)kh * dk, dk, l2norm, l2_eps, qn);
        for (int32_t j = 0; j < dk; ++j) qn[j] *= q_scale;
        for (int32_t j = 0; j < dk; ++j)
          a[j] = per_channel ? exp(g[(t * Hv + h) * dk + j]) : exp(g[t * Hv + h]);
        const double b = beta[t * Hv + h];
        const double* vt = v + t * v_stride + (int64_t)h * dv;
        for (int32_t i = 0; i < dv; ++i)
          for (int32_t j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= a[j];
        for (int32_t i = 0; i < dv; ++i) {
          double p = 0.0;
          for (int32_t j = 0; j < dk; ++j) p += S[(int64_t)i * dk + j] * kn[j];
          u[i] = b * (vt[i] - p);
        }
        for (int32_t i = 0; i < dv; ++i)
          for (int32_t j = 0; j < dk; ++j) S[(int64_t)i * dk + j] += u[i] * kn[j];
        double* ot = o + (t * Hv + h) * dv;
        for (int32_t i = 0; i < dv; ++i) {
          double acc = 0.0;
          for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qn[j];
          ot[i] = acc;
        }
      }
      if (state_out) memcpy(state_out + sidx, S, sizeof(double) * dv * dk);
      free(S); free(kn); free(qn); free(a); free(u);
    }
  }
}

/*
 * The same recurrence computed chunk by chunk in the WY form, fp64, following
 * the stage order the golden PR names: cumsum -> A -> solve -> recompute ->
 * state -> output [GOLDEN Consumer / Shipped-line diff].  It exists only to
 * pin that this algebra reaches the token-by-token result (chunked equals
 * sequential [GLM row I4; LEDGER kernel map]); it is not the parity reference.
 *
 * Per chunk of L <= chunk tokens, with S0 the state entering the chunk and
 * gam[r][c] the within-chunk cumulative sum of the log decay:
 *   A[r][j]  = beta_r * sum_c khat_r[c] khat_j[c] exp(gam_r[c] - gam_j[c]), j < r
 *   T        = (I + A)^-1                     (forward substitution)
 *   W        = T diag(beta) [khat_j * exp(gam_j)]_j
 *   U        = T diag(beta) V
 *   Vnew     = U - W S0^T
 *   o_r      = S0 (qtil_r * exp(gam_r)) + sum_{j<=r} Vnew_j ((khat_j * exp(gam_r - gam_j)) . qtil_r)
 *   S_L      = S0 diag(exp(gam_L)) + sum_j Vnew_j (khat_j * exp(gam_L - gam_j))^T
 * Exponents are formed as differences, never as a product of exp(+) and exp(-).
 * Arguments are those of gdn_oracle_delta_rule plus the chunk length.
 */
void gdn_oracle_delta_rule_chunked(int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                                   int32_t per_channel, int32_t l2norm, double l2_eps, double q_scale,
                                   const double* q, const double* k, int64_t qk_stride,
                                   const double* v, int64_t v_stride,
                                   const double* g, const double* beta,
                                   const int32_t* cu, int32_t N, const double* state_in,
                                   int32_t chunk, double* o, double* state_out) {
  const int32_t ratio = Hv / Hk;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t n = 0; n < N; ++n) {
    for (int32_t h = 0; h < Hv; ++h) {
      const int32_t kh = h / ratio;
      const int64_t sidx = ((int64_t)n * Hv + h) * dv * dk;
      double* S = (double*)calloc((size_t)dv * dk, sizeof(double));
      double* S1 = (double*)malloc(sizeof(double) * dv * dk);
      double* K = (double*)malloc(sizeof(double) * chunk * dk);
      double* Q = (double*)malloc(sizeof(double) * chunk * dk);
      double* V = (double*)malloc(sizeof(double) * chunk * dv);
      double* gam = (double*)malloc(sizeof(double) * chunk * dk);
      double* bet = (double*)malloc(sizeof(double) * chunk);
      double* A = (double*)malloc(sizeof(double) * chunk * chunk);
      double* Tm = (double*)malloc(sizeof(double) * chunk * chunk);
      double* Wm = (double*)malloc(sizeof(double) * chunk * dk);
      double* Um = (double*)malloc(sizeof(double) * chunk * dv);
      double* Vn = (double*)malloc(sizeof(double) * chunk * dv);
      if (state_in) memcpy(S, state_in + sidx, sizeof(double) * dv * dk);
      for (int64_t c0 = cu[n]; c0 < cu[n + 1]; c0 += chunk) {
        const int32_t L = (int32_t)((cu[n + 1] - c0) < chunk ? (cu[n + 1] - c0) : chunk);
        /* prepare: normalise, scale q, gather the chunk */
        for (int32_t r = 0; r < L; ++r) {
          const int64_t t = c0 + r;
          l2_normalize(k + t * qk_stride + (int64_t)kh * dk, dk, l2norm, l2_eps, K + (int64_t)r * dk);
          l2_normalize(q + t * qk_stride + (int64_t)kh * dk, dk, l2norm, l2_eps, Q + (int64_t)r * dk);
          for (int32_t c = 0; c < dk; ++c) Q[(int64_t)r * dk + c] *= q_scale;
          for (int32_t i = 0; i < dv; ++i) V[(int64_t)r * dv + i] = v[t * v_stride + (int64_t)h * dv + i];
          bet[r] = beta[t * Hv + h];
        }
        /* cumsum */
        for (int32_t c = 0; c < dk; ++c) {
          double run = 0.0;
          for (int32_t r = 0; r < L; ++r) {
            const int64_t t = c0 + r;
            run += per_channel ? g[(t * Hv + h) * dk + c] : g[t * Hv + h];
            gam[(int64_t)r * dk + c] = run;
          }
        }
        /* A */
        for (int32_t r = 0; r < L; ++r)
          for (int32_t j = 0; j < L; ++j) {
            double acc = 0.0;
            if (j < r)
              for (int32_t c = 0; c < dk; ++c)
                acc += K[(int64_t)r * dk + c] * K[(int64_t)j * dk + c] *
                       exp(gam[(int64_t)r * dk + c] - gam[(int64_t)j * dk + c]);
            A[r * chunk + j] = bet[r] * acc;
          }
        /* solve: (I + A) T = I, row r from rows < r */
        for (int32_t r = 0; r < L; ++r)
          for (int32_t col = 0; col < L; ++col) {
            double acc = (r == col) ? 1.0 : 0.0;
            for (int32_t j = 0; j < r; ++j) acc -= A[r * chunk + j] * Tm[j * chunk + col];
            Tm[r * chunk + col] = acc;
          }
        /* recompute W and U */
        for (int32_t r = 0; r < L; ++r) {
          for (int32_t c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < L; ++j)
              acc += Tm[r * chunk + j] * bet[j] * K[(int64_t)j * dk + c] * exp(gam[(int64_t)j * dk + c]);
            Wm[(int64_t)r * dk + c] = acc;
          }
          for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < L; ++j) acc += Tm[r * chunk + j] * bet[j] * V[(int64_t)j * dv + i];
            Um[(int64_t)r * dv + i] = acc;
          }
        }
        /* state (values entering the chunk's writes) */
        for (int32_t r = 0; r < L; ++r)
          for (int32_t i = 0; i < dv; ++i) {
            double acc = Um[(int64_t)r * dv + i];
            for (int32_t c = 0; c < dk; ++c) acc -= Wm[(int64_t)r * dk + c] * S[(int64_t)i * dk + c];
            Vn[(int64_t)r * dv + i] = acc;
          }
        /* output */
        for (int32_t r = 0; r < L; ++r) {
          double* ot = o + ((c0 + r) * Hv + h) * dv;
          for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t c = 0; c < dk; ++c)
              acc += S[(int64_t)i * dk + c] * Q[(int64_t)r * dk + c] * exp(gam[(int64_t)r * dk + c]);
            for (int32_t j = 0; j <= r; ++j) {
              double kq = 0.0;
              for (int32_t c = 0; c < dk; ++c)
                kq += K[(int64_t)j * dk + c] * exp(gam[(int64_t)r * dk + c] - gam[(int64_t)j * dk + c]) *
                      Q[(int64_t)r * dk + c];
              acc += Vn[(int64_t)j * dv + i] * kq;
            }
            ot[i] = acc;
          }
        }
        /* carry the state to the next chunk */
        for (int32_t i = 0; i < dv; ++i)
          for (int32_t c = 0; c < dk; ++c) {
            const double gl = gam[(int64_t)(L - 1) * dk + c];
            double acc = S[(int64_t)i * dk + c] * exp(gl);
            for (int32_t j = 0; j < L; ++j)
              acc += Vn[(int64_t)j * dv + i] * K[(int64_t)j * dk + c] * exp(gl - gam[(int64_t)j * dk + c]);
            S1[(int64_t)i * dk + c] = acc;
          }
        memcpy(S, S1, sizeof(double) * dv * dk);
      }
      if (state_out) memcpy(state_out + sidx, S, sizeof(double) * dv * dk);
      free(S); free(S1); free(K); free(Q); free(V); free(gam); free(bet);
      free(A); free(Tm); free(Wm); free(Um); free(Vn);
    }
  }
}

/*
 * Gate derivation from the a / b projections.  The pages name the step (the
 * TDD ledger's GDN alpha/beta transform kernels; the golden PR's prepare stage
 * "derives the raw g/beta" from in_proj_a / in_proj_b outputs with the layer's
 * A_log and dt_bias vectors, which its fixture does not store) but do not
 * print the formula.  Reading: A_log is the log of a positive per-head decay
 * rate and dt_bias a per-head bias of the a projection, so per token t and
 * value head h
 *     g[t][h]    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *     beta[t][h] = sigmoid(b[t][h])
 * with softplus(x) = log(1 + exp(x)) (evaluated as x + log1p(exp(-x)) for
 * x > 0, the same function without overflow).  a, b, g, beta are [rows][Hv].
 */
static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

void gdn_oracle_gates(const double* a, const double* b, const double* A_log, const double* dt_bias,
                      int64_t rows, int32_t Hv, double* g, double* beta) {
  for (int64_t t = 0; t < rows; ++t) {
    for (int32_t h = 0; h < Hv; ++h) {
      g[t * Hv + h] = -exp(A_log[h]) * softplus(a[t * Hv + h] + dt_bias[h]);
      beta[t * Hv + h] = sigmoid(b[t * Hv + h]);
    }
  }
}

/*
 * Gated RMSNorm with the sigmoid gate [GOLDEN Summary, Negative controls and
 * code review: rsqrt(variance + eps), sigmoid not SiLU].  Over each of the
 * `vectors` rows of length d:
 *     out[i] = o[i] / sqrt(mean(o^2) + eps) * w[i] * sigmoid(z[i])
 * w [d] is shared by every head.
 */
void gdn_oracle_gated_rmsnorm(const double* o, const double* z, const double* w, int64_t vectors,
                              int32_t d, double eps, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < vectors; ++r) {
    const double* orow = o + r * d;
    const double* zrow = z + r * d;
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += orow[i] * orow[i];
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int32_t i = 0; i < d; ++i) out[r * d + i] = orow[i] * inv * w[i] * sigmoid(zrow[i]);
  }
}

/*
 * One fused decode step for B sequences of one token each [LEDGER kernel map:
 * scalar recurrence with fused output gate; SSM fields gdn_f32_conv_norm_k
 * and the strided norm twins]: conv step over all Cc = 2*Hk*dk + Hv*dv
 * channels (q | k | v), the recurrence with that single token, then the
 * sigmoid gated norm.  conv_state [B][3][Cc] and state [B][Hv][dv][dk] are
 * updated in place; out is [B][Hv][dv].
 */
void gdn_oracle_decode_step(int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                            int32_t per_channel, int32_t act, double l2_eps, double q_scale,
                            double rms_eps, int32_t B,
                            const double* x, const double* conv_w, double* conv_state,
                            const double* g, const double* beta, const double* z,
                            const double* norm_w, double* state, double* out) {
  const int32_t Cc = 2 * Hk * dk + Hv * dv;
  double* y = (double*)malloc(sizeof(double) * B * Cc);
  double* o = (double*)malloc(sizeof(double) * B * Hv * dv);
  int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
  for (int32_t b = 0; b <= B; ++b) cu[b] = b;
  gdn_oracle_conv1d_step(x, B, Cc, conv_w, conv_state, act, y);
  gdn_oracle_delta_rule(Hk, Hv, dk, dv, per_channel, 1, l2_eps, q_scale,
                        y, y + Hk * dk, Cc, y + 2 * Hk * dk, Cc, g, beta, cu, B, state, o, state);
  gdn_oracle_gated_rmsnorm(o, z, norm_w, (int64_t)B * Hv, dv, rms_eps, out);
  free(y); free(o); free(cu);
}
