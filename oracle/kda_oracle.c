/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * loads this file; it is compiled into its own shared object (liboracle_kda.so)
 * and used only by the tests, by the smoke check and by the benchmark's
 * cpu_baseline leg.  It shares no code, header, table or helper with the HIP
 * path.
 *
 * What it computes (Kimi Linear summary page, "De la atencion lineal a Gated
 * DeltaNet" and "Control fino de memoria en Kimi Delta Attention"): per head a
 * matrix-valued fast-weight state S (dk x dv; row = key channel, column = value
 * channel) updated token by token with the gated delta rule whose forget gate
 * is a per-key-channel diagonal,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t          (output read AFTER the update),
 *
 * with alpha_t = exp(g_t) (g is the natural log of the gate, passed in).
 * The step is evaluated in its delta-rule form -- decay first, then one online
 * gradient step on the reconstruction loss 1/2 ||S^T k - v||^2 with step size
 * beta -- which expands to exactly the product above:
 *
 *     S <- Diag(exp(g_t)) S
 *     u  = S^T k_t                     (what the state recalls for k_t)
 *     S <- S + beta_t k_t (v_t - u)^T  (write the correction)
 *     o_t = scale * S^T q_t
 *
 * No chunking, no reordering: the exact result, one token at a time, in fp64
 * on the exact input values (fp32 arrays; bf16 inputs are upcast exactly by
 * the caller).  Independent (sequence, head) chains run in parallel with
 * OpenMP, each chain strictly in token order.
 *
 * Layouts (all contiguous, row-major):
 *   q, k  [B, T, H, dk]   v [B, T, H, dv]   g [B, T, H, dk]   beta [B, T, H]
 *   o     [B, T, H, dv]   (fp64)
 *   S0, S_final  [N, H, dk, dv] (fp64); S0 may be NULL (= zero state)
 *   cu_seqlens   int32 [N + 1] or NULL.  Non-NULL requires B == 1: sequence n
 *                occupies tokens [cu[n], cu[n+1]) and starts from S0[n].
 *                NULL means N == B and sequence n is batch row n.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on state S (dk x dv, fp64), on fp64 token
 * vectors q, k (dk), v (dv) and the log gate lg (dk).
 * drop_erase != 0 removes the k k^T (erase) term, leaving the plain additive
 * write S <- Diag(alpha) S + beta k v^T; it exists only so the tests can
 * reduce the oracle to textbook linear attention and is never used for
 * parity against the GPU path. */
static void kda_token(int dk, int dv, double scale, const double *q,
                      const double *k, const float *v, const double *lg,
                      double beta, double *S, double *u, double *o,
                      int drop_erase)
{
    for (int i = 0; i < dk; ++i) {
        const double a = exp(lg[i]);
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] *= a;
    }
    for (int j = 0; j < dv; ++j) u[j] = 0.0;
    if (!drop_erase) {
        for (int i = 0; i < dk; ++i) {
            const double ki = k[i];
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) u[j] += row[j] * ki;
        }
    }
    for (int j = 0; j < dv; ++j) u[j] = beta * ((double)v[j] - u[j]);
    for (int i = 0; i < dk; ++i) {
        const double ki = k[i];
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] += ki * u[j];
    }
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = q[i];
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) o[j] += row[j] * qi;
        }
        for (int j = 0; j < dv; ++j) o[j] *= scale;
    }
}

/* Optional preparation of one token's inputs, as a model layer does before
 * the operator (summary page, "Configuracion del modelo Kimi Linear": L2
 * normalisation of queries and keys; a per-channel decay gate computed with a
 * GDN/Mamba-style decay function).  The page names the decay function only
 * by family; the form taken is the Mamba/GDN one, per key channel:
 *     log alpha_c = -exp(A_log[h]) * softplus(g_c + dt_bias[h, c]).
 * flags bit 0: q, k <- x / sqrt(sum x^2 + eps)      (L2 normalisation)
 * flags bit 1: beta <- 1 / (1 + exp(-beta))         (beta given as a logit)
 * A_log != NULL: g holds the gate pre-activation (dt_bias may be NULL = 0).
 * Without any of these the values are passed through unchanged. */
typedef struct {
    int flags;
    double eps;
    const float *A_log;     /* [H] */
    const float *dt_bias;   /* [H, dk] */
} prep_t;

static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

static void prepare_token(const prep_t *p, int h, int dk, const float *q,
                          const float *k, const float *g, float beta,
                          double *qd, double *kd, double *lg, double *bd)
{
    for (int i = 0; i < dk; ++i) {
        qd[i] = (double)q[i];
        kd[i] = (double)k[i];
        lg[i] = (double)g[i];
    }
    *bd = (double)beta;
    if (!p) return;
    if (p->flags & 1) {
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) {
            sq += qd[i] * qd[i];
            sk += kd[i] * kd[i];
        }
        /* a zero vector (with eps = 0) stays zero */
        const double nq = sq + p->eps > 0.0 ? 1.0 / sqrt(sq + p->eps) : 0.0;
        const double nk = sk + p->eps > 0.0 ? 1.0 / sqrt(sk + p->eps) : 0.0;
        for (int i = 0; i < dk; ++i) {
            qd[i] *= nq;
            kd[i] *= nk;
        }
    }
    if (p->flags & 2) *bd = 1.0 / (1.0 + exp(-*bd));
    if (p->A_log) {
        const double rate = exp((double)p->A_log[h]);
        for (int i = 0; i < dk; ++i) {
            const double bias = p->dt_bias ? (double)p->dt_bias[(size_t)h * dk + i] : 0.0;
            lg[i] = -rate * softplus(lg[i] + bias);
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Optional output epilogue of a Kimi Linear layer (summary page,
 * "Configuracion del modelo Kimi Linear": per-head RMSNorm and a
 * data-dependent output gate before the output projection).  The gate's
 * activation is not named on the page; the sigmoid is taken.  On one output
 * row o (dv) of one head:
 *     y_j = o_j / sqrt(mean_j o_j^2 + eps) * w_j * sigmoid(z_j)
 * w: [dv] or NULL (= 1); z: the row's gate logits [dv] or NULL (no gate). */
typedef struct {
    double eps;
    const float *w;       /* [dv] */
    const float *z;       /* [.., H, dv] like o */
} epi_t;

static void epilogue_row(const epi_t *e, int dv, const float *z, double *o)
{
    double ms = 0.0;
    for (int j = 0; j < dv; ++j) ms += o[j] * o[j];
    ms /= dv;
    const double r = ms + e->eps > 0.0 ? 1.0 / sqrt(ms + e->eps) : 0.0;
    for (int j = 0; j < dv; ++j) {
        double y = o[j] * r;
        if (e->w) y *= (double)e->w[j];
        if (z) y *= 1.0 / (1.0 + exp(-(double)z[j]));
        o[j] = y;
    }
}

/* Full forward over B rows (or N packed sequences), with optional input
 * preparation (see prepare_token; prep == NULL passes inputs through).
 * Returns 0 on success, nonzero on a malformed argument. */
static int kda_fwd_impl(int B, int T, int H, int dk, int dv, double scale,
                        const float *q, const float *k, const float *v,
                        const float *g, const float *beta, const double *S0,
                        const int32_t *cu_seqlens, int N, int drop_erase,
                        const prep_t *prep, const epi_t *epi, double *o,
                        double *S_final)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens) {
        if (B != 1 || N <= 0) return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return 3;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return 4;
    } else {
        N = B;
    }
    const size_t tok_k = (size_t)H * dk, tok_v = (size_t)H * dv;
    const long chains = (long)N * H;
    int err = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *tv = (double *)malloc(sizeof(double) * (size_t)dk * 3);
        if (!S || !u || !tv) {
#pragma omp atomic write
            err = 5;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long c = 0; c < chains; ++c) {
                const int n = (int)(c / H), h = (int)(c % H);
                long t0, t1, base;
                if (cu_seqlens) { t0 = cu_seqlens[n]; t1 = cu_seqlens[n + 1]; base = 0; }
                else { t0 = 0; t1 = T; base = (long)n * T; }
                const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;
                if (S0) memcpy(S, S0 + sidx, sizeof(double) * (size_t)dk * dv);
                else memset(S, 0, sizeof(double) * (size_t)dk * dv);
                for (long t = t0; t < t1; ++t) {
                    const size_t tok = (size_t)(base + t);
                    double bd;
                    prepare_token(prep, h, dk, q + tok * tok_k + (size_t)h * dk,
                                  k + tok * tok_k + (size_t)h * dk,
                                  g + tok * tok_k + (size_t)h * dk, beta[tok * H + h],
                                  tv, tv + dk, tv + 2 * dk, &bd);
                    double *orow = o ? o + tok * tok_v + (size_t)h * dv : NULL;
                    kda_token(dk, dv, scale, tv, tv + dk, v + tok * tok_v + (size_t)h * dv,
                              tv + 2 * dk, bd, S, u, orow, drop_erase);
                    if (epi && orow)
                        epilogue_row(epi, dv, epi->z ? epi->z + tok * tok_v + (size_t)h * dv : NULL,
                                     orow);
                }
                if (S_final) memcpy(S_final + sidx, S, sizeof(double) * (size_t)dk * dv);
            }
        }
        free(S);
        free(u);
        free(tv);
    }
    return err;
}

int oracle_kda_fwd(int B, int T, int H, int dk, int dv, double scale,
                   const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const double *S0,
                   const int32_t *cu_seqlens, int N, int drop_erase,
                   double *o, double *S_final)
{
    return kda_fwd_impl(B, T, H, dk, dv, scale, q, k, v, g, beta, S0, cu_seqlens, N,
                        drop_erase, NULL, NULL, o, S_final);
}

/* The forward with input preparation (flags, eps, A_log [H] or NULL,
 * dt_bias [H, dk] or NULL; see prepare_token) and output epilogue (epi_on,
 * epi_eps, w [dv] or NULL, z [B, T, H, dv] or NULL; see epilogue_row). */
int oracle_kda_fwd_ex(int B, int T, int H, int dk, int dv, double scale,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta, const double *S0,
                      const int32_t *cu_seqlens, int N, int flags, double eps,
                      const float *A_log, const float *dt_bias, int epi_on,
                      double epi_eps, const float *w, const float *z,
                      double *o, double *S_final)
{
    prep_t p = {flags, eps, A_log, dt_bias};
    epi_t e = {epi_eps, w, z};
    return kda_fwd_impl(B, T, H, dk, dv, scale, q, k, v, g, beta, S0, cu_seqlens, N, 0,
                        &p, epi_on ? &e : NULL, o, S_final);
}

/* One decode step: the same token update applied once to each sequence's
 * cached state.  state is [num_slots, H, dk, dv] fp64, updated in place;
 * sequence n uses slot slot_idx[n] (or n when slot_idx is NULL).  Sequences
 * whose slot is out of range are skipped and their output row is left as is.
 * q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H]; o [N, H, dv] (fp64). */
static int kda_decode_impl(int N, int H, int dk, int dv, double scale,
                           const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *state,
                           int num_slots, const int32_t *slot_idx,
                           const prep_t *prep, const epi_t *epi, double *o)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || num_slots < 0) return 1;
    if (!slot_idx && N > num_slots) return 2;
    const long chains = (long)N * H;
    int err = 0;
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *tv = (double *)malloc(sizeof(double) * (size_t)dk * 3);
        if (!u || !tv) {
#pragma omp atomic write
            err = 5;
        } else {
#pragma omp for schedule(static)
            for (long c = 0; c < chains; ++c) {
                const int n = (int)(c / H), h = (int)(c % H);
                const int slot = slot_idx ? slot_idx[n] : n;
                if (slot < 0 || slot >= num_slots) continue;
                double *S = state + ((size_t)slot * H + h) * (size_t)dk * dv;
                const size_t r = (size_t)n * H + h;
                double bd;
                prepare_token(prep, h, dk, q + r * dk, k + r * dk, g + r * dk, beta[r], tv,
                              tv + dk, tv + 2 * dk, &bd);
                kda_token(dk, dv, scale, tv, tv + dk, v + r * dv, tv + 2 * dk, bd, S, u,
                          o + r * dv, 0);
                if (epi) epilogue_row(epi, dv, epi->z ? epi->z + r * dv : NULL, o + r * dv);
            }
        }
        free(u);
        free(tv);
    }
    return err;
}

int oracle_kda_decode_step(int N, int H, int dk, int dv, double scale,
                           const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *state,
                           int num_slots, const int32_t *slot_idx, double *o)
{
    return kda_decode_impl(N, H, dk, dv, scale, q, k, v, g, beta, state, num_slots,
                           slot_idx, NULL, NULL, o);
}

int oracle_kda_decode_step_ex(int N, int H, int dk, int dv, double scale,
                              const float *q, const float *k, const float *v,
                              const float *g, const float *beta, double *state,
                              int num_slots, const int32_t *slot_idx, int flags,
                              double eps, const float *A_log, const float *dt_bias,
                              int epi_on, double epi_eps, const float *w,
                              const float *z, double *o)
{
    prep_t p = {flags, eps, A_log, dt_bias};
    epi_t e = {epi_eps, w, z};
    return kda_decode_impl(N, H, dk, dv, scale, q, k, v, g, beta, state, num_slots,
                           slot_idx, &p, epi_on ? &e : NULL, o);
}

/* ------------------------------------------------------------------------
 * Gradients of the forward (reverse mode through the same token recurrence,
 * in fp64).  For the loss L = sum(o * d_o) + sum(S_final * d_S_final), with
 * each token step written as
 *     a  = exp(g_t);  S1 = Diag(a) S_{t-1};  u = S1^T k;  e = beta (v - u);
 *     S_t = S1 + k e^T;  o_t = scale S_t^T q,
 * the adjoints, taken in reverse token order, are
 *     dS_t += scale q do^T;        dq = scale S_t do
 *     dk   = dS_t e;               de = dS_t^T k
 *     dbeta = de . (v - u);        dv = beta de;       du = -beta de
 *     dS1  = dS_t + k du^T;        dk += S1 du
 *     dS_{t-1} = Diag(a) dS1;      dg = a * rowsum(dS1 * S_{t-1})
 * The states of one chain are kept for the whole sequence (test sizes only).
 * Outputs dq, dk, dg [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H], and dS0
 * [N,H,dk,dv] when non-NULL; d_S_final may be NULL (zero).
 * ------------------------------------------------------------------------ */
int oracle_kda_bwd(int B, int T, int H, int dk, int dv, double scale,
                   const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const double *S0,
                   const int32_t *cu_seqlens, int N, const double *d_o,
                   const double *d_S_final, double *dq, double *dkk,
                   double *dvv, double *dg, double *dbeta, double *dS0)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens) {
        if (B != 1 || N <= 0) return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return 3;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return 4;
    } else {
        N = B;
    }
    const size_t tok_k = (size_t)H * dk, tok_v = (size_t)H * dv, SZ = (size_t)dk * dv;
    const long chains = (long)N * H;
    int err = 0;
#pragma omp parallel
    {
        const long maxlen = cu_seqlens ? T : T;
        double *hist = (double *)malloc(sizeof(double) * SZ * (size_t)(maxlen + 1));
        double *dS = (double *)malloc(sizeof(double) * SZ);
        double *S1 = (double *)malloc(sizeof(double) * SZ);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        double *de = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!hist || !dS || !S1 || !u || !e || !de || !du) {
#pragma omp atomic write
            err = 5;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long c = 0; c < chains; ++c) {
                const int n = (int)(c / H), h = (int)(c % H);
                long t0, t1, base;
                if (cu_seqlens) { t0 = cu_seqlens[n]; t1 = cu_seqlens[n + 1]; base = 0; }
                else { t0 = 0; t1 = T; base = (long)n * T; }
                const size_t sidx = ((size_t)n * H + h) * SZ;
                /* forward: hist[j] = state after j tokens of this chain */
                if (S0) memcpy(hist, S0 + sidx, sizeof(double) * SZ);
                else memset(hist, 0, sizeof(double) * SZ);
                for (long t = t0; t < t1; ++t) {
                    const size_t tok = (size_t)(base + t);
                    const float *kt = k + tok * tok_k + (size_t)h * dk;
                    const float *vt = v + tok * tok_v + (size_t)h * dv;
                    const float *gt = g + tok * tok_k + (size_t)h * dk;
                    const double bt = (double)beta[tok * H + h];
                    const double *Sp = hist + (size_t)(t - t0) * SZ;
                    double *Sn = hist + (size_t)(t - t0 + 1) * SZ;
                    for (int i = 0; i < dk; ++i) {
                        const double a = exp((double)gt[i]);
                        for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] = a * Sp[(size_t)i * dv + j];
                    }
                    for (int j = 0; j < dv; ++j) u[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) u[j] += Sn[(size_t)i * dv + j] * (double)kt[i];
                    for (int j = 0; j < dv; ++j) e[j] = bt * ((double)vt[j] - u[j]);
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) Sn[(size_t)i * dv + j] += (double)kt[i] * e[j];
                }
                /* reverse */
                if (d_S_final) memcpy(dS, d_S_final + sidx, sizeof(double) * SZ);
                else memset(dS, 0, sizeof(double) * SZ);
                for (long t = t1 - 1; t >= t0; --t) {
                    const size_t tok = (size_t)(base + t);
                    const float *qt = q + tok * tok_k + (size_t)h * dk;
                    const float *kt = k + tok * tok_k + (size_t)h * dk;
                    const float *vt = v + tok * tok_v + (size_t)h * dv;
                    const float *gt = g + tok * tok_k + (size_t)h * dk;
                    const double bt = (double)beta[tok * H + h];
                    const double *Sp = hist + (size_t)(t - t0) * SZ;
                    const double *St = hist + (size_t)(t - t0 + 1) * SZ;
                    const double *dot = d_o + tok * tok_v + (size_t)h * dv;
                    double *dqt = dq + tok * tok_k + (size_t)h * dk;
                    double *dkt = dkk + tok * tok_k + (size_t)h * dk;
                    double *dvt = dvv + tok * tok_v + (size_t)h * dv;
                    double *dgt = dg + tok * tok_k + (size_t)h * dk;
                    /* recompute S1, u, e of this token */
                    for (int i = 0; i < dk; ++i) {
                        const double a = exp((double)gt[i]);
                        for (int j = 0; j < dv; ++j) S1[(size_t)i * dv + j] = a * Sp[(size_t)i * dv + j];
                    }
                    for (int j = 0; j < dv; ++j) u[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) u[j] += S1[(size_t)i * dv + j] * (double)kt[i];
                    for (int j = 0; j < dv; ++j) e[j] = bt * ((double)vt[j] - u[j]);
                    /* output */
                    for (int i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            dS[(size_t)i * dv + j] += scale * (double)qt[i] * dot[j];
                            acc += St[(size_t)i * dv + j] * dot[j];
                        }
                        dqt[i] = scale * acc;
                    }
                    /* write */
                    for (int j = 0; j < dv; ++j) de[j] = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            acc += dS[(size_t)i * dv + j] * e[j];
                            de[j] += dS[(size_t)i * dv + j] * (double)kt[i];
                        }
                        dkt[i] = acc;
                    }
                    double db = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        db += de[j] * ((double)vt[j] - u[j]);
                        dvt[j] = bt * de[j];
                        du[j] = -bt * de[j];
                    }
                    dbeta[tok * H + h] = db;
                    /* recall u = S1^T k */
                    for (int i = 0; i < dk; ++i) {
                        double acc = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            dS[(size_t)i * dv + j] += (double)kt[i] * du[j];
                            acc += S1[(size_t)i * dv + j] * du[j];
                        }
                        dkt[i] += acc;
                    }
                    /* decay */
                    for (int i = 0; i < dk; ++i) {
                        const double a = exp((double)gt[i]);
                        double acc = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            acc += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
                            dS[(size_t)i * dv + j] *= a;
                        }
                        dgt[i] = a * acc;
                    }
                }
                if (dS0) memcpy(dS0 + sidx, dS, sizeof(double) * SZ);
            }
        }
        free(hist); free(dS); free(S1); free(u); free(e); free(de); free(du);
    }
    return err;
}

/* ------------------------------------------------------------------------
 * General diagonal-plus-low-rank (DPLR) transition, the family KDA belongs to
 * (summary page, "Menor cantidad de operaciones que DPLR general": both allow
 * fine-grained decay, and KDA ties both low-rank vectors of the transition to
 * the key).  The page gives no formula; the form used here is
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
 *     o_t = scale * S_t^T q_t,                  alpha_t = exp(g_t),
 *
 * so that KDA is the case a_t = beta_t k_t, b_t = alpha_t * k_t with the
 * write key beta_t k_t.  Token by token:
 *     u = S^T b_t                 (read through b, before the step)
 *     S <- Diag(alpha_t) S - a_t u^T + k_t v_t^T
 *     o_t = scale * S^T q_t
 * Layouts as for the KDA forward, with a, b [B, T, H, dk] (float32).
 * ------------------------------------------------------------------------ */
int oracle_dplr_fwd(int B, int T, int H, int dk, int dv, double scale,
                    const float *q, const float *k, const float *v,
                    const float *a, const float *b, const float *g,
                    const double *S0, const int32_t *cu_seqlens, int N,
                    double *o, double *S_final)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens) {
        if (B != 1 || N <= 0) return 2;
        if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return 3;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return 4;
    } else {
        N = B;
    }
    const size_t tok_k = (size_t)H * dk, tok_v = (size_t)H * dv, SZ = (size_t)dk * dv;
    const long chains = (long)N * H;
    int err = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * SZ);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !u) {
#pragma omp atomic write
            err = 5;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long c = 0; c < chains; ++c) {
                const int n = (int)(c / H), h = (int)(c % H);
                long t0, t1, base;
                if (cu_seqlens) { t0 = cu_seqlens[n]; t1 = cu_seqlens[n + 1]; base = 0; }
                else { t0 = 0; t1 = T; base = (long)n * T; }
                const size_t sidx = ((size_t)n * H + h) * SZ;
                if (S0) memcpy(S, S0 + sidx, sizeof(double) * SZ);
                else memset(S, 0, sizeof(double) * SZ);
                for (long t = t0; t < t1; ++t) {
                    const size_t tk = (size_t)(base + t) * tok_k + (size_t)h * dk;
                    const size_t tv = (size_t)(base + t) * tok_v + (size_t)h * dv;
                    /* u = S^T b (old state) */
                    for (int j = 0; j < dv; ++j) u[j] = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        const double bi = (double)b[tk + i];
                        const double *row = S + (size_t)i * dv;
                        for (int j = 0; j < dv; ++j) u[j] += bi * row[j];
                    }
                    /* S <- Diag(alpha) S - a u^T + k v^T */
                    for (int i = 0; i < dk; ++i) {
                        const double al = exp((double)g[tk + i]);
                        const double ai = (double)a[tk + i], ki = (double)k[tk + i];
                        double *row = S + (size_t)i * dv;
                        for (int j = 0; j < dv; ++j)
                            row[j] = al * row[j] - ai * u[j] + ki * (double)v[tv + j];
                    }
                    if (o) {
                        double *orow = o + tv;
                        for (int j = 0; j < dv; ++j) orow[j] = 0.0;
                        for (int i = 0; i < dk; ++i) {
                            const double qi = (double)q[tk + i];
                            const double *row = S + (size_t)i * dv;
                            for (int j = 0; j < dv; ++j) orow[j] += qi * row[j];
                        }
                        for (int j = 0; j < dv; ++j) orow[j] *= scale;
                    }
                }
                if (S_final) memcpy(S_final + sidx, S, sizeof(double) * SZ);
            }
        }
        free(S);
        free(u);
    }
    return err;
}
