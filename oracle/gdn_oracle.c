/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, fp64 CPU reference for one pipeline chunk of the gated
 * delta-rule recurrence (Gated DeltaNet), forward and backward, token by
 * token.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg load this library.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Source of the method:
 *   "Pith review of StateFlow: Sequence Pipeline Parallelism for
 *   Long-Context Modeling with Linear Recurrence" (pith.science).
 *     - "What carries the argument": a chunk C_i starts from its boundary
 *       state S_i^in and emits S_i^out; the forward chain is
 *       S_{i+1}^in = S_i^out (Eq. 5) and the backward chain is
 *       Sbar_i^out = Sbar_{i+1}^in (Eq. 7).
 *     - "Referee Report", major comment 1: the recurrence is the gated
 *       delta rule of the page's Eq. (1) (Gated DeltaNet), and chunking is
 *       claimed to be exact.
 *   The page names Eq. (1) but does not print it.  The recurrence used here
 *   is the standard Gated DeltaNet update, with a d_v x d_k state S:
 *       S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = S_t q_t
 *   with scalar gates alpha_t (decay) and beta_t (write strength) per token
 *   and head, no query scaling and no normalisation inside the operation.
 *
 * Layouts (all C-contiguous, fp64):
 *   q, k   [B, T, H, Dk]     v, o, dO   [B, T, H, Dv]
 *   alpha, beta, dalpha, dbeta          [B, T, H]
 *   S_in, S_out, dS_out, dS_in          [B, H, Dv, Dk]
 * A NULL S_in or dS_out means zeros.  Each (b, h) is an independent
 * sequence; OpenMP runs them in parallel.
 */
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TOK(b, t, h, T, H) (((size_t)(b) * (T) + (t)) * (H) + (h))

/* Forward of one (b,h) sequence.  S (Dv x Dk) holds the entry state on input
 * and the exit state on output.  Row-vector products are written out as
 * loops on purpose, so that each line reads as one term of the update. */
static void fwd_one(int b, int h, int T, int H, int Dk, int Dv,
                    const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta,
                    double *S, double *o, double *u /* scratch, Dv */)
{
    for (int t = 0; t < T; ++t) {
        size_t tok = IDX_TOK(b, t, h, T, H);
        const double *kt = k + tok * Dk;
        const double *qt = q + tok * Dk;
        const double *vt = v + tok * Dv;
        double a = alpha[tok], be = beta[tok];
        /* S_{t-1}(I - beta k k^T) = S_{t-1} - beta (S_{t-1} k) k^T, so the
         * update is S_t = a S_{t-1} + beta (v - a S_{t-1} k) k^T. */
        for (int i = 0; i < Dv; ++i) {
            double sk = 0.0;
            for (int j = 0; j < Dk; ++j) sk += S[(size_t)i * Dk + j] * kt[j];
            u[i] = vt[i] - a * sk;
        }
        for (int i = 0; i < Dv; ++i)
            for (int j = 0; j < Dk; ++j)
                S[(size_t)i * Dk + j] = a * S[(size_t)i * Dk + j] + be * u[i] * kt[j];
        if (o) {
            double *ot = o + tok * Dv;
            for (int i = 0; i < Dv; ++i) {
                double acc = 0.0;
                for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * qt[j];
                ot[i] = acc;
            }
        }
    }
}

static int threads_for(int nseq, int nthreads)
{
    int nt = nthreads;
#ifdef _OPENMP
    if (nt <= 0) nt = omp_get_max_threads();
#else
    nt = 1;
#endif
    if (nt > nseq) nt = nseq;
    if (nt < 1) nt = 1;
    return nt;
}

/* Returns the number of threads used, or a negative value on a bad argument
 * or allocation failure. */
int oracle_gdn_fwd(int B, int T, int H, int Dk, int Dv,
                   const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *S_in,
                   double *o, double *S_out, int nthreads)
{
    if (B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    int nseq = B * H;
    int nt = threads_for(nseq, nthreads);
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int bh = 0; bh < nseq; ++bh) {
        int b = bh / H, h = bh % H;
        size_t ss = (size_t)Dv * Dk;
        double *S = (double *)malloc(ss * sizeof(double));
        double *u = (double *)malloc((size_t)Dv * sizeof(double));
        if (!S || !u) {
            free(S); free(u);
            #pragma omp atomic write
            err = 1;
            continue;
        }
        if (S_in) memcpy(S, S_in + (size_t)bh * ss, ss * sizeof(double));
        else memset(S, 0, ss * sizeof(double));
        fwd_one(b, h, T, H, Dk, Dv, q, k, v, alpha, beta, S, o, u);
        if (S_out) memcpy(S_out + (size_t)bh * ss, S, ss * sizeof(double));
        free(S); free(u);
    }
    return err ? -2 : nt;
}

/*
 * Backward of the loss L = sum_t <dO_t, o_t> + <dS_out, S_T> by reverse
 * accumulation through the token loop.  With P = S_{t-1}, y = P k_t,
 * u = v_t - alpha_t y and G = dL/dS_t (the gradient of everything after
 * token t plus o_t's own term), the step S_t = alpha P + beta u k^T gives
 *     Gk       = G k_t
 *     dv_t     = beta Gk
 *     dbeta_t  = u . Gk
 *     dalpha_t = <G, P> - beta (Gk . y)
 *     dk_t     = beta (G^T u - alpha P^T Gk)
 *     dL/dP    = alpha (G - beta Gk k_t^T)
 * and o_t = S_t q_t gives dq_t = S_t^T dO_t and G += dO_t q_t^T.
 * States are needed in reverse order: the forward pass stores S every CK
 * tokens and each stretch of CK tokens is recomputed from its checkpoint.
 */
#define CK 64

int oracle_gdn_bwd(int B, int T, int H, int Dk, int Dv,
                   const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *S_in,
                   const double *dO, const double *dS_out,
                   double *dq, double *dk, double *dv,
                   double *dalpha, double *dbeta, double *dS_in, int nthreads)
{
    if (B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    int nseq = B * H;
    int nt = threads_for(nseq, nthreads);
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int bh = 0; bh < nseq; ++bh) {
        int b = bh / H, h = bh % H;
        size_t ss = (size_t)Dv * Dk;
        int nck = (T + CK - 1) / CK;
        /* ckpt[c] = state entering token c*CK; seg[i] = state after token
         * c*CK + i within the stretch being processed. */
        double *ckpt = (double *)malloc((size_t)(nck > 0 ? nck : 1) * ss * sizeof(double));
        double *seg = (double *)malloc((size_t)CK * ss * sizeof(double));
        double *G = (double *)malloc(ss * sizeof(double));
        double *u = (double *)malloc((size_t)Dv * sizeof(double));
        double *y = (double *)malloc((size_t)Dv * sizeof(double));
        double *Gk = (double *)malloc((size_t)Dv * sizeof(double));
        double *S = (double *)malloc(ss * sizeof(double));
        if (!ckpt || !seg || !G || !u || !y || !Gk || !S) {
            free(ckpt); free(seg); free(G); free(u); free(y); free(Gk); free(S);
            #pragma omp atomic write
            err = 1;
            continue;
        }
        /* Forward pass, keeping one checkpoint per stretch. */
        if (S_in) memcpy(S, S_in + (size_t)bh * ss, ss * sizeof(double));
        else memset(S, 0, ss * sizeof(double));
        for (int c = 0; c < nck; ++c) {
            memcpy(ckpt + (size_t)c * ss, S, ss * sizeof(double));
            int t0 = c * CK, t1 = t0 + CK < T ? t0 + CK : T;
            for (int t = t0; t < t1; ++t) {
                size_t tok = IDX_TOK(b, t, h, T, H);
                const double *kt = k + tok * Dk;
                const double *vt = v + tok * Dv;
                double a = alpha[tok], be = beta[tok];
                for (int i = 0; i < Dv; ++i) {
                    double sk = 0.0;
                    for (int j = 0; j < Dk; ++j) sk += S[(size_t)i * Dk + j] * kt[j];
                    u[i] = vt[i] - a * sk;
                }
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j)
                        S[(size_t)i * Dk + j] = a * S[(size_t)i * Dk + j] + be * u[i] * kt[j];
            }
        }
        /* Reverse pass. */
        if (dS_out) memcpy(G, dS_out + (size_t)bh * ss, ss * sizeof(double));
        else memset(G, 0, ss * sizeof(double));
        for (int c = nck - 1; c >= 0; --c) {
            int t0 = c * CK, t1 = t0 + CK < T ? t0 + CK : T;
            /* Recompute S_t for t in [t0, t1): seg[t - t0] = S_t. */
            memcpy(S, ckpt + (size_t)c * ss, ss * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                size_t tok = IDX_TOK(b, t, h, T, H);
                const double *kt = k + tok * Dk;
                const double *vt = v + tok * Dv;
                double a = alpha[tok], be = beta[tok];
                for (int i = 0; i < Dv; ++i) {
                    double sk = 0.0;
                    for (int j = 0; j < Dk; ++j) sk += S[(size_t)i * Dk + j] * kt[j];
                    u[i] = vt[i] - a * sk;
                }
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j)
                        S[(size_t)i * Dk + j] = a * S[(size_t)i * Dk + j] + be * u[i] * kt[j];
                memcpy(seg + (size_t)(t - t0) * ss, S, ss * sizeof(double));
            }
            for (int t = t1 - 1; t >= t0; --t) {
                size_t tok = IDX_TOK(b, t, h, T, H);
                const double *kt = k + tok * Dk;
                const double *qt = q + tok * Dk;
                const double *vt = v + tok * Dv;
                const double *dot = dO + tok * Dv;
                double a = alpha[tok], be = beta[tok];
                const double *St = seg + (size_t)(t - t0) * ss;
                const double *P = (t > t0) ? seg + (size_t)(t - t0 - 1) * ss
                                           : ckpt + (size_t)c * ss;
                /* Output term: G += dO_t q_t^T, dq_t = S_t^T dO_t. */
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j)
                        G[(size_t)i * Dk + j] += dot[i] * qt[j];
                double *dqt = dq + tok * Dk;
                for (int j = 0; j < Dk; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < Dv; ++i) acc += St[(size_t)i * Dk + j] * dot[i];
                    dqt[j] = acc;
                }
                /* Rebuild y = P k and u = v - a y for this token. */
                for (int i = 0; i < Dv; ++i) {
                    double sk = 0.0;
                    for (int j = 0; j < Dk; ++j) sk += P[(size_t)i * Dk + j] * kt[j];
                    y[i] = sk;
                    u[i] = vt[i] - a * sk;
                }
                for (int i = 0; i < Dv; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < Dk; ++j) acc += G[(size_t)i * Dk + j] * kt[j];
                    Gk[i] = acc;
                }
                double *dvt = dv + tok * Dv;
                double db = 0.0, gy = 0.0, gp = 0.0;
                for (int i = 0; i < Dv; ++i) {
                    dvt[i] = be * Gk[i];
                    db += u[i] * Gk[i];
                    gy += Gk[i] * y[i];
                }
                for (size_t e = 0; e < ss; ++e) gp += G[e] * P[e];
                dbeta[tok] = db;
                dalpha[tok] = gp - be * gy;
                double *dkt = dk + tok * Dk;
                for (int j = 0; j < Dk; ++j) {
                    double gu = 0.0, pg = 0.0;
                    for (int i = 0; i < Dv; ++i) {
                        gu += G[(size_t)i * Dk + j] * u[i];
                        pg += P[(size_t)i * Dk + j] * Gk[i];
                    }
                    dkt[j] = be * (gu - a * pg);
                }
                /* Gradient with respect to S_{t-1}. */
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j)
                        G[(size_t)i * Dk + j] = a * (G[(size_t)i * Dk + j] - be * Gk[i] * kt[j]);
            }
        }
        if (dS_in) memcpy(dS_in + (size_t)bh * ss, G, ss * sizeof(double));
        free(ckpt); free(seg); free(G); free(u); free(y); free(Gk); free(S);
    }
    return err ? -2 : nt;
}

/* ------------------------------------------------------------------------
 * Short causal depthwise convolution with a boundary state (TEST
 * INFRASTRUCTURE, like the rest of this file).
 *
 * Source: Pith review of StateFlow, "What carries the argument" (each chunk
 * also carries auxiliary local-convolution states across its boundary) and
 * "Referee Report", major comment 1 (the short-convolution boundary states
 * must be reconstructed for the chunked backward to be exact).  The pages do
 * not print the convolution; the plainest reading, used here, is the usual
 * causal depthwise 1-D convolution of width W over the token axis, per
 * channel, applied to a chunk's inputs with the previous chunk's last W-1
 * inputs in front of them:
 *     xe = [conv_in (W-1 rows) ; x (T rows)]          per (b, channel c)
 *     z_t[c] = sum_{j=0}^{W-1} w[c][j] * xe[t + W-1 - j][c]
 *     y_t[c] = z_t[c]            (act = 0)
 *     y_t[c] = z_t / (1 + e^-z)  (act = 1, SiLU)
 *     conv_out = the last W-1 rows of xe (the next chunk's conv_in).
 * Tap j multiplies the input j tokens back.  conv_in NULL means zeros (the
 * start of a sequence).
 * Layouts (fp64, C-contiguous): x, y, dy, dx [B, T, C]; w, dw [C, W];
 * conv_in, conv_out, dconv_in, dconv_out [B, W-1, C].
 * ---------------------------------------------------------------------- */
static double xe_at(const double *x, const double *cin, int b, int u, int T, int C, int W,
                    int c)
{
    if (u < W - 1)
        return cin ? cin[((size_t)b * (W - 1) + u) * C + c] : 0.0;
    return x[((size_t)b * T + (u - (W - 1))) * C + c];
}

void oracle_shortconv_fwd(int B, int T, int C, int W, int act, const double *x, const double *w,
                          const double *conv_in, double *y, double *conv_out)
{
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) {
                double z = 0.0;
                for (int j = 0; j < W; ++j)
                    z += w[(size_t)c * W + j] * xe_at(x, conv_in, b, t + W - 1 - j, T, C, W, c);
                y[((size_t)b * T + t) * C + c] = act ? z / (1.0 + exp(-z)) : z;
            }
    if (conv_out)
        for (int b = 0; b < B; ++b)
            for (int m = 0; m < W - 1; ++m)
                for (int c = 0; c < C; ++c)
                    conv_out[((size_t)b * (W - 1) + m) * C + c] =
                        xe_at(x, conv_in, b, T + m, T, C, W, c);
}

/* Backward of the loss L = <dy, y> + <dconv_out, conv_out>.  Writes dx, dw
 * (summed over b and t) and dconv_in (NULL dconv_out means zeros). */
void oracle_shortconv_bwd(int B, int T, int C, int W, int act, const double *x, const double *w,
                          const double *conv_in, const double *dy, const double *dconv_out,
                          double *dx, double *dw, double *dconv_in)
{
    const int U = T + W - 1;                   /* rows of xe */
    double *dxe = (double *)calloc((size_t)U * C, sizeof(double));
    memset(dw, 0, sizeof(double) * (size_t)C * W);
    for (int b = 0; b < B; ++b) {
        memset(dxe, 0, sizeof(double) * (size_t)U * C);
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) {
                double z = 0.0;
                for (int j = 0; j < W; ++j)
                    z += w[(size_t)c * W + j] * xe_at(x, conv_in, b, t + W - 1 - j, T, C, W, c);
                double g = dy[((size_t)b * T + t) * C + c];
                if (act) {
                    const double s = 1.0 / (1.0 + exp(-z));
                    g *= s * (1.0 + z * (1.0 - s));    /* d/dz of z * sigmoid(z) */
                }
                for (int j = 0; j < W; ++j) {
                    const int u = t + W - 1 - j;
                    dxe[(size_t)u * C + c] += w[(size_t)c * W + j] * g;
                    dw[(size_t)c * W + j] += g * xe_at(x, conv_in, b, u, T, C, W, c);
                }
            }
        if (dconv_out)                            /* conv_out = xe rows T .. T+W-2 */
            for (int m = 0; m < W - 1; ++m)
                for (int c = 0; c < C; ++c)
                    dxe[(size_t)(T + m) * C + c] += dconv_out[((size_t)b * (W - 1) + m) * C + c];
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c)
                dx[((size_t)b * T + t) * C + c] = dxe[(size_t)(t + W - 1) * C + c];
        if (dconv_in)
            for (int m = 0; m < W - 1; ++m)
                for (int c = 0; c < C; ++c)
                    dconv_in[((size_t)b * (W - 1) + m) * C + c] = dxe[(size_t)m * C + c];
    }
    free(dxe);
}
