/*
 * m2_oracle.c -- plain fp64 CPU oracle of the Mamba-2 mixer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the HIP path is
 * compared against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library, and it does not include or call it.
 *
 * What it computes (the steps of the Zamba2 mixer as the article "Transformers 中
 * Zamba2 混合架构模型解析" lays them out in §三 "Mamba2 Mixer": causal depthwise
 * conv1d of width mamba_d_conv followed by SiLU, then the selective state-space
 * scan for a whole prompt, or the single-token recurrent update when a cached
 * state exists):
 *
 *   conv    out[t,c] = SiLU(bias[c] + sum_k w[c,k] * x[t-(W-1)+k, c])
 *           (cross-correlation, left history of W-1 tokens, last tap on the current token)
 *   dt      dt = softplus(dt_raw + dt_bias[h]), optionally clamped to [dt_min, dt_max]
 *   scan    S_t = exp(dt_t * A_h) * S_{t-1} + dt_t * x_t (outer) B_t     (S is P x N)
 *           y_t = S_t . C_t + D_h * x_t
 *   step    the same for one token, with the conv window taken from a ring of the
 *           last W tokens (the cache of conv state + recurrent state, §三)
 *   scan backward  the gradients of L = sum_t dy_t . y_t + <dS, S_final> with respect to every
 *           input of the scan (the training path of the stateful mixer, §三), by the adjoint
 *           recurrence in reverse time from the stored forward states:
 *             Gt = adjoint of S_t:  Gt = a_{t+1} G_{t+1} + dy_t (outer) C_t,  G_{L-1} includes dS
 *             dx_t = D dy_t + dt_t Gt B_t      dB_t = dt_t Gt^T x_t      dC_t = S_t^T dy_t
 *             d(dt_t) = <Gt, x_t B_t^T> + A a_t <Gt, S_{t-1}>,   a_t = exp(dt_t A)
 *             dA = sum_t dt_t a_t <Gt, S_{t-1}>   dD = sum_t dy_t . x_t   dstate_in = a_0 G_0
 *           then through the clamp and softplus to dt_raw and dt_bias
 *   norm    the gated group RMSNorm after the scan (§三, the gated normalisation: group RMSNorm times
 *           SiLU of the gate z, over intermediate_size in groups; eps from §五 rms_norm_eps):
 *             gate first (norm_before_gate = 0):  g = y * SiLU(z),
 *                                                 out = g / sqrt(mean_group(g^2) + eps) * w
 *             norm first (norm_before_gate = 1):  out = y / sqrt(mean_group(y^2) + eps) * w * SiLU(z)
 *
 * Everything is evaluated in double precision, sequentially in t, straight
 * from the definitions: no chunking, no blocking, no reordering.  OpenMP only
 * spreads independent (batch, channel) or (batch, head) units over threads.
 *
 * Layouts (row-major, innermost last):
 *   x        [B, L, H, P]        B_in, C_in  [B, L, G, N]     dt_raw [B, L, H]
 *   state    [B, H, P, N]        y           [B, L, H, P]
 *   conv x   [B, L, Cd]          w           [Cd, W]          bias   [Cd]
 *   ring     [B, W, Cd]  slot-major.  A ring "at phase s" holds the W most recent
 *            tokens; the token j places before the next one to be consumed
 *            (j = 1..W) sits in slot (s - j) mod W.  Consuming a token at phase s
 *            overwrites slot s mod W, the one token no longer in the window.
 * Head h reads group g(h) = h / (H / G).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* softplus(v) = log(1 + e^v).  For v > 30 the same quantity is written as
 * v + log1p(e^-v) so that e^v does not overflow; the two are equal. */
static double softplus(double v) { return v > 30.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

static int64_t pmod(int64_t a, int64_t m) { int64_t r = a % m; return r < 0 ? r + m : r; }

static double step_size(double raw, double bias, double dt_min, double dt_max) {
    double dt = softplus(raw + bias);
    if (dt < dt_min) dt = dt_min;
    if (dt > dt_max) dt = dt_max;
    return dt;
}

/* Causal depthwise conv1d + SiLU over a prompt (article §三: groups = conv_dim,
 * kernel width mamba_d_conv, SiLU on the output; §五: use_conv_bias).
 * ring_in (nullable) supplies the W-1 tokens before t = 0 at phase ring_in_step;
 * ring_out (nullable) receives the last W tokens at phase 0.
 * lens (nullable): sequence b holds only its first lens[b] tokens (the rest is padding): outputs
 * past them are not written and ring_out holds the W tokens before lens[b]. */
void oracle_conv1d(int64_t Bn, int64_t L, int64_t Cd, int64_t W,
                   const double* x, const double* w, const double* bias,
                   const double* ring_in, int64_t ring_in_step,
                   double* ring_out, double* out, const int64_t* lens)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t c = 0; c < Cd; ++c) {
            const double* xb = x + b * L * Cd;
            const int64_t Lb = lens ? lens[b] : L;
            for (int64_t t = 0; t < Lb; ++t) {
                double v = bias ? bias[c] : 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    int64_t tau = t - (W - 1) + k;  /* token index feeding tap k */
                    double xv;
                    if (tau >= 0) xv = xb[tau * Cd + c];
                    else if (ring_in) xv = ring_in[(b * W + pmod(ring_in_step + tau, W)) * Cd + c];
                    else xv = 0.0;
                    v += w[c * W + k] * xv;
                }
                out[(b * L + t) * Cd + c] = silu(v);
            }
            if (ring_out) {
                for (int64_t j = 0; j < W; ++j) {
                    int64_t tau = Lb - W + j;  /* slot j at phase 0 */
                    double xv;
                    if (tau >= 0) xv = xb[tau * Cd + c];
                    else if (ring_in) xv = ring_in[(b * W + pmod(ring_in_step + tau, W)) * Cd + c];
                    else xv = 0.0;
                    ring_out[(b * W + j) * Cd + c] = xv;
                }
            }
        }
    }
}

/* Selective state-space recurrence over a prompt, one token at a time
 * (the chunked scan of article §三 computes exactly this sum; here it is
 * evaluated sequentially).  state_in / D nullable (zero).
 * lens (nullable): sequence b consumes only its first lens[b] tokens; y past them is not written
 * and state_out is the state after token lens[b] - 1. */
void oracle_ssd_scan(int64_t Bn, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                     const double* x, const double* Bm, const double* Cm,
                     const double* dt_raw, const double* dt_bias, const double* A, const double* D,
                     double dt_min, double dt_max,
                     const double* state_in, double* y, double* state_out, const int64_t* lens)
{
    const int64_t hpg = H / G;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / hpg;
            double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
            for (int64_t i = 0; i < P * N; ++i)
                S[i] = state_in ? state_in[((b * H + h) * P) * N + i] : 0.0;
            const double Dh = D ? D[h] : 0.0;
            const int64_t Lb = lens ? lens[b] : L;
            for (int64_t t = 0; t < Lb; ++t) {
                const int64_t bt = b * L + t;
                const double dt = step_size(dt_raw[bt * H + h], dt_bias[h], dt_min, dt_max);
                const double decay = exp(dt * A[h]);
                const double* xt = x + (bt * H + h) * P;
                const double* Bt = Bm + (bt * G + g) * N;
                const double* Ct = Cm + (bt * G + g) * N;
                double* yt = y + (bt * H + h) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        double s = decay * S[p * N + n] + dt * xt[p] * Bt[n];
                        S[p * N + n] = s;
                        acc += s * Ct[n];
                    }
                    yt[p] = acc + Dh * xt[p];
                }
            }
            if (state_out)
                for (int64_t i = 0; i < P * N; ++i) state_out[((b * H + h) * P) * N + i] = S[i];
            free(S);
        }
    }
}

/* One decode token for every sequence (article §三: with a cached state and a
 * sequence of length 1 the mixer takes the recurrent single-step update; the
 * cache holds each layer's conv state and recurrent state).
 * ring [B, W, Cd] and state [B, H, P, N] are updated in place; y is [B, H, P].
 * The channels of the conv output are x (H*P) | B (G*N) | C (G*N). */
void oracle_ssd_step(int64_t Bn, int64_t H, int64_t P, int64_t N, int64_t G, int64_t W,
                     const double* xbc_tok, const double* dt_tok,
                     const double* w, const double* bias,
                     const double* dt_bias, const double* A, const double* D,
                     double dt_min, double dt_max,
                     double* ring, int64_t step, double* state, double* y)
{
    const int64_t Di = H * P, Cd = Di + 2 * G * N, hpg = H / G;
    double* act = (double*)malloc((size_t)(Bn * Cd) * sizeof(double));
    /* conv of the window (W-1 ring tokens + the new one) */
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t c = 0; c < Cd; ++c) {
            double v = bias ? bias[c] : 0.0;
            for (int64_t k = 0; k < W; ++k) {
                int64_t rel = k - (W - 1);   /* token position relative to the new one */
                double xv = rel == 0 ? xbc_tok[b * Cd + c]
                                     : ring[(b * W + pmod(step + rel, W)) * Cd + c];
                v += w[c * W + k] * xv;
            }
            act[b * Cd + c] = silu(v);
        }
        /* the new token replaces the one that just left the window */
        for (int64_t c = 0; c < Cd; ++c) ring[(b * W + pmod(step, W)) * Cd + c] = xbc_tok[b * Cd + c];
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / hpg;
            const double* xt = act + b * Cd + h * P;
            const double* Bt = act + b * Cd + Di + g * N;
            const double* Ct = act + b * Cd + Di + G * N + g * N;
            const double dt = step_size(dt_tok[b * H + h], dt_bias[h], dt_min, dt_max);
            const double decay = exp(dt * A[h]);
            const double Dh = D ? D[h] : 0.0;
            double* S = state + ((b * H + h) * P) * N;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    double s = decay * S[p * N + n] + dt * xt[p] * Bt[n];
                    S[p * N + n] = s;
                    acc += s * Ct[n];
                }
                y[(b * H + h) * P + p] = acc + Dh * xt[p];
            }
        }
    }
    free(act);
}

/* Softplus as the oracle evaluates it, exported so its pin can call it directly. */
double oracle_softplus(double v) { return softplus(v); }

/* Gated group RMSNorm over rows of D channels, in groups of GS consecutive channels.
 * y, z, out [T, D]; w [D]. */
void oracle_gated_rmsnorm(int64_t T, int64_t D, int64_t GS, const double* y, const double* z, const double* w,
                          double eps, int64_t norm_before_gate, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t g0 = 0; g0 < D; g0 += GS) {
            const double* yr = y + t * D + g0;
            const double* zr = z + t * D + g0;
            double ss = 0.0;
            for (int64_t c = 0; c < GS; ++c) {
                const double v = norm_before_gate ? yr[c] : yr[c] * silu(zr[c]);
                ss += v * v;
            }
            const double r = 1.0 / sqrt(ss / (double)GS + eps);
            for (int64_t c = 0; c < GS; ++c) {
                const double v = norm_before_gate ? yr[c] * r * w[g0 + c] * silu(zr[c])
                                                  : yr[c] * silu(zr[c]) * r * w[g0 + c];
                out[t * D + g0 + c] = v;
            }
        }
    }
}

/* Gradients of L = sum_t dy_t . y_t + <dstate_out, S_final> for the scan of oracle_ssd_scan.
 * dstate_out / state_in / D nullable (zero).  Outputs: dx [B,L,H,P], dB and dC [B,L,G,N]
 * (summed over the heads of the group), ddt_raw [B,L,H], ddt_bias / dA / dD [H] (summed over
 * the batch), dstate_in [B,H,P,N].  The forward states of a (sequence, head) are kept, then
 * the adjoint runs from its last token down to 0.  The clamped softplus passes the gradient
 * where dt_min <= softplus(v) <= dt_max, else 0.  lens (nullable): sequence b consumes only
 * its first lens[b] tokens, as in oracle_ssd_scan (S_final is the state after the last of
 * them); per-token outputs past them are not written. */
void oracle_ssd_scan_bwd(int64_t Bn, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                         const double* x, const double* Bm, const double* Cm,
                         const double* dt_raw, const double* dt_bias, const double* A, const double* D,
                         double dt_min, double dt_max, const double* state_in,
                         const double* dy, const double* dstate_out,
                         double* dx, double* dB, double* dC, double* ddt_raw,
                         double* ddt_bias, double* dA, double* dD, double* dstate_in, const int64_t* lens)
{
    const int64_t hpg = H / G, PN = P * N;
    /* per (sequence, head) partial sums, added up after the parallel loop */
    double* pdB = (double*)calloc((size_t)(Bn * H * L * N), sizeof(double));
    double* pdC = (double*)calloc((size_t)(Bn * H * L * N), sizeof(double));
    double* pdA = (double*)calloc((size_t)(Bn * H), sizeof(double));
    double* pdD = (double*)calloc((size_t)(Bn * H), sizeof(double));
    double* pdb = (double*)calloc((size_t)(Bn * H), sizeof(double));
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < Bn; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / hpg, bh = b * H + h;
            const double Dh = D ? D[h] : 0.0;
            const int64_t Lb = lens ? lens[b] : L;
            /* forward: S[t + 1] is the state after token t, S[0] the initial state */
            double* S = (double*)malloc((size_t)((L + 1) * PN) * sizeof(double));
            double* dts = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
            for (int64_t i = 0; i < PN; ++i) S[i] = state_in ? state_in[bh * PN + i] : 0.0;
            for (int64_t t = 0; t < Lb; ++t) {
                const int64_t bt = b * L + t;
                const double dt = step_size(dt_raw[bt * H + h], dt_bias[h], dt_min, dt_max);
                const double a = exp(dt * A[h]);
                const double* xt = x + (bt * H + h) * P;
                const double* Bt = Bm + (bt * G + g) * N;
                dts[t] = dt;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        S[(t + 1) * PN + p * N + n] = a * S[t * PN + p * N + n] + dt * xt[p] * Bt[n];
            }
            /* reverse: Gm is the adjoint of the state after token t */
            double* Gm = (double*)malloc((size_t)PN * sizeof(double));
            for (int64_t i = 0; i < PN; ++i) Gm[i] = dstate_out ? dstate_out[bh * PN + i] : 0.0;
            for (int64_t t = Lb - 1; t >= 0; --t) {
                const int64_t bt = b * L + t;
                const double dt = dts[t];
                const double a = exp(dt * A[h]);
                const double* xt = x + (bt * H + h) * P;
                const double* Bt = Bm + (bt * G + g) * N;
                const double* Ct = Cm + (bt * G + g) * N;
                const double* dyt = dy + (bt * H + h) * P;
                const double* St = S + (t + 1) * PN;
                const double* Sp = S + t * PN;
                /* y_t = S_t C_t + D x_t: the state after t receives dy_t (outer) C_t */
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) Gm[p * N + n] += dyt[p] * Ct[n];
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += St[p * N + n] * dyt[p];
                    pdC[(bh * L + t) * N + n] = acc;
                }
                double xdy = 0.0;
                for (int64_t p = 0; p < P; ++p) xdy += dyt[p] * xt[p];
                pdD[bh] += xdy;
                /* S_t = a S_{t-1} + dt x_t B_t^T */
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += Gm[p * N + n] * Bt[n];
                    dx[(bt * H + h) * P + p] = Dh * dyt[p] + dt * acc;
                }
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += Gm[p * N + n] * xt[p];
                    pdB[(bh * L + t) * N + n] = dt * acc;
                }
                double gxb = 0.0, gs = 0.0;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) {
                        gxb += Gm[p * N + n] * xt[p] * Bt[n];
                        gs += Gm[p * N + n] * Sp[p * N + n];
                    }
                const double ddt = gxb + A[h] * a * gs;
                pdA[bh] += dt * a * gs;
                /* dt = clamp(softplus(v)), v = dt_raw + dt_bias; softplus'(v) = 1 / (1 + e^-v) */
                const double v = dt_raw[bt * H + h] + dt_bias[h];
                const double sp = softplus(v);
                const double g_raw = (sp < dt_min || sp > dt_max) ? 0.0 : ddt / (1.0 + exp(-v));
                ddt_raw[bt * H + h] = g_raw;
                pdb[bh] += g_raw;
                for (int64_t i = 0; i < PN; ++i) Gm[i] *= a;
            }
            for (int64_t i = 0; i < PN; ++i) dstate_in[bh * PN + i] = Gm[i];
            free(Gm);
            free(dts);
            free(S);
        }
    }
    for (int64_t b = 0; b < Bn; ++b)
        for (int64_t t = 0; t < (lens ? lens[b] : L); ++t)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t n = 0; n < N; ++n) {
                    double sb = 0.0, sc = 0.0;
                    for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                        sb += pdB[((b * H + h) * L + t) * N + n];
                        sc += pdC[((b * H + h) * L + t) * N + n];
                    }
                    dB[((b * L + t) * G + g) * N + n] = sb;
                    dC[((b * L + t) * G + g) * N + n] = sc;
                }
    for (int64_t h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0, sbias = 0.0;
        for (int64_t b = 0; b < Bn; ++b) {
            sa += pdA[b * H + h];
            sd += pdD[b * H + h];
            sbias += pdb[b * H + h];
        }
        dA[h] = sa;
        dD[h] = sd;
        ddt_bias[h] = sbias;
    }
    free(pdB);
    free(pdC);
    free(pdA);
    free(pdD);
    free(pdb);
}
