/*
 * KDA (Kimi Delta Attention) mixer: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library under hybrid_linear_attention_rule_amd/csrc/.
 *
 * Plain, slow and written to be checked by eye: every quantity is a double,
 * every loop is the definition, and nothing is blocked, fused or reordered
 * beyond what the recurrence itself states.
 *
 * What is computed, and where it comes from:
 *
 *   "Extend NVIDIA/TensorRT-LLM#19991 with isolated NVFP4 Kimi K3 targets"
 *   (fork pull request), Description: the KDA mixer fuses a short
 *   convolution, an FP32 recurrence and a gated output normalisation; the
 *   recurrent state is stored as FP32 or BF16 while the recurrence itself
 *   stays FP32, and verify keeps FP32 per-token draft records under either
 *   storage dtype.
 *
 *   "Kimi K3 on modeling_v2: stateful catalog entries, ..." section 5: the
 *   speculative path keeps per-token KDA verify states (kda_token_states).
 *   Section 6: KDA hands its output back before o_proj on every path, so the
 *   mixer ends at the gated norm.
 *
 *   The pages print no formula.  The recurrence is the gated delta rule in
 *   its usual statement, per sequence and head, for each token t:
 *
 *     1. history   x_{t-3}, x_{t-2}, x_{t-1} of the raw q, k, v channels
 *                  (zero before the sequence's first token);
 *     2. conv      c = sum_{j=0..W-1} w[., j] * x_{t-(W-1)+j}, depthwise,
 *                  tap W-1 on the current token, no bias, no activation;
 *     3. normalise qh = s * c_q / sqrt(|c_q|^2 + eps_l2),
 *                  kh = c_k / sqrt(|c_k|^2 + eps_l2),  vt = c_v;
 *     4. decay     S <- Diag(alpha_t) S            (rows = key channels);
 *     5. write     u = S^T kh;  S <- S + beta_t kh (vt - u)^T,
 *                  so S_t = (I - beta kh kh^T) Diag(alpha) S_{t-1}
 *                           + beta kh vt^T;
 *     6. read-out  o = S^T qh, after the write;
 *     7. gated norm y = w_n * o / sqrt(mean(o^2) + eps_n) * gate(g_t),
 *                  gate = sigmoid (default) or silu;
 *     8. store     FP32 storage keeps S; BF16 storage replaces S by its
 *                  nearest bfloat16 value (ties to even), and the next token
 *                  starts from that value.
 *
 *   Verify runs steps 1-7 over n draft tokens with no rounding between them
 *   and records S after each token; commit(m) makes record m the stored state
 *   (rounded once for BF16 storage) and the last W-1 raw tokens of
 *   (old history || drafts 1..m) the new history; m = 0 changes nothing.
 *   Prefill is steps 1-7 over the whole sequence, stored once at the end.
 *
 *   Gate inputs.  The decay and write strengths may arrive as logits instead
 *   (cfg->gates = 1): the mixer fuses the f_b projection that produces them
 *   (first page, Description), and the plain reading of the per-channel
 *   decay is alpha = exp(-softplus(a)) in (0, 1), of the per-head write
 *   strength beta = sigmoid(b) in (0, 1); both are formed before step 4 of
 *   each token.
 *
 *   kda_ref_run_chunked restates steps 4-6 in the chunkwise WY/UT form (the
 *   derivation is written out above that function).  It exists so that tests
 *   can check that the chunk algebra reaches the sequential result.
 *
 * Layouts (all dense, row-major, doubles):
 *   S      [dk][dv], S[i*dv + j]: row i is key channel i, column j value ch.
 *   hist   [W-1][2dk+dv], oldest first; channels ordered q | k | v.
 *   wconv  [2dk+dv][W] for the head; the same q | k | v channel order.
 *   q, k, alpha [T][dk]; v, g [T][dv]; beta [T]; y [T][dv] (alpha and beta
 *   hold the logits a and b when cfg->gates = 1).
 *   records [T][dk][dv] (nullable).
 *
 * Return value: 0 on success, -1 on a bad argument, -2 when out of memory.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int dk;          /* key channels per head */
    int dv;          /* value channels per head */
    int width;       /* conv taps, including the current token */
    int gate;        /* 0: sigmoid, 1: silu */
    double q_scale;  /* s in step 3 */
    double l2_eps;   /* eps_l2 in step 3 */
    double norm_eps; /* eps_n in step 7 */
    int gates;       /* 0: alpha and beta given; 1: their logits a and b */
} kda_ref_cfg;

/* Nearest bfloat16 value of x, ties to even (IEEE-754 binary16 "brain"
 * format: 8 significant bits, float32's exponent range).  frexp gives
 * x = f * 2^e with 0.5 <= |f| < 1, so f * 2^8 holds the 8 significant bits
 * and nearbyint rounds the rest to nearest, ties to even (default mode). */
double kda_ref_bf16(double x)
{
    int e;
    double f;
    if (x == 0.0 || !isfinite(x))
        return x;
    f = frexp(x, &e);
    return ldexp(nearbyint(ldexp(f, 8)), e - 8);
}

void kda_ref_round_bf16(double *x, long n)
{
    long i;
    for (i = 0; i < n; ++i)
        x[i] = kda_ref_bf16(x[i]);
}

static double gate_fn(int gate, double x)
{
    double sig = 1.0 / (1.0 + exp(-x));
    return gate == 1 ? x * sig : sig;
}

static int cfg_ok(const kda_ref_cfg *cfg)
{
    return cfg && cfg->dk > 0 && cfg->dv > 0 && cfg->width >= 1 &&
           (cfg->gate == 0 || cfg->gate == 1) &&
           (cfg->gates == 0 || cfg->gates == 1);
}

/* softplus(x) = log(1 + e^x), split at 0 so that e^x never overflows. */
static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* The T tokens' alpha [T][dk] and beta [T] from the inputs: copies when they
 * are given, else alpha = exp(-softplus(a)) and beta = 1 / (1 + e^-b) of the
 * logits.  Returns 0, or -2 when out of memory (*al, *be then NULL). */
static int gate_values(const kda_ref_cfg *cfg, int T, const double *alpha,
                       const double *beta, double **al, double **be)
{
    long n = (long)T * cfg->dk, i;
    *al = malloc(sizeof(double) * (n > 0 ? n : 1));
    *be = malloc(sizeof(double) * (T > 0 ? T : 1));
    if (!*al || !*be) {
        free(*al); free(*be);
        *al = *be = NULL;
        return -2;
    }
    for (i = 0; i < n; ++i)
        (*al)[i] = cfg->gates ? exp(-softplus(alpha[i])) : alpha[i];
    for (i = 0; i < T; ++i)
        (*be)[i] = cfg->gates ? 1.0 / (1.0 + exp(-beta[i])) : beta[i];
    return 0;
}

/* Steps 1-3 for one token: the causal conv over (hist || x_t) and the
 * normalisations.  xq, xk, xv are the raw current-token channels. */
static void conv_and_normalise(const kda_ref_cfg *cfg, const double *hist,
                               const double *xq, const double *xk,
                               const double *xv, const double *wconv,
                               double *qh, double *kh, double *vt)
{
    const int dk = cfg->dk, dv = cfg->dv, W = cfg->width;
    const int nch = 2 * dk + dv;
    int ch, j;
    double sq = 0.0, sk = 0.0, rq, rk;

    for (ch = 0; ch < nch; ++ch) {
        double cur, acc = 0.0;
        if (ch < dk)
            cur = xq[ch];
        else if (ch < 2 * dk)
            cur = xk[ch - dk];
        else
            cur = xv[ch - 2 * dk];
        /* tap j multiplies x_{t-(W-1)+j}: taps 0..W-2 read the history,
         * tap W-1 the current token */
        for (j = 0; j < W - 1; ++j)
            acc += wconv[ch * W + j] * hist[j * nch + ch];
        acc += wconv[ch * W + (W - 1)] * cur;
        if (ch < dk)
            qh[ch] = acc;
        else if (ch < 2 * dk)
            kh[ch - dk] = acc;
        else
            vt[ch - 2 * dk] = acc;
    }
    for (j = 0; j < dk; ++j) {
        sq += qh[j] * qh[j];
        sk += kh[j] * kh[j];
    }
    rq = cfg->q_scale / sqrt(sq + cfg->l2_eps);
    rk = 1.0 / sqrt(sk + cfg->l2_eps);
    for (j = 0; j < dk; ++j) {
        qh[j] *= rq;
        kh[j] *= rk;
    }
    (void)dv;
}

/* Step 7 on one token's read-out o[dv]. */
static void gated_norm(const kda_ref_cfg *cfg, const double *o,
                       const double *g, const double *norm_w, double *y)
{
    const int dv = cfg->dv;
    int j;
    double ms = 0.0, r;
    for (j = 0; j < dv; ++j)
        ms += o[j] * o[j];
    ms /= (double)dv;
    r = 1.0 / sqrt(ms + cfg->norm_eps);
    for (j = 0; j < dv; ++j)
        y[j] = (norm_w ? norm_w[j] : 1.0) * o[j] * r * gate_fn(cfg->gate, g[j]);
}

/* Shift the history one token: drop the oldest, append x_t (q | k | v). */
static void push_history(const kda_ref_cfg *cfg, double *hist,
                         const double *xq, const double *xk, const double *xv)
{
    const int dk = cfg->dk, dv = cfg->dv, W = cfg->width;
    const int nch = 2 * dk + dv;
    int j;
    if (W < 2)
        return;
    for (j = 0; j < W - 2; ++j)
        memcpy(hist + j * nch, hist + (j + 1) * nch, sizeof(double) * nch);
    memcpy(hist + (W - 2) * nch, xq, sizeof(double) * dk);
    memcpy(hist + (W - 2) * nch + dk, xk, sizeof(double) * dk);
    memcpy(hist + (W - 2) * nch + 2 * dk, xv, sizeof(double) * dv);
}

/* Steps 1-8 over T tokens of one (sequence, head), token by token. */
int kda_ref_run(const kda_ref_cfg *cfg, int T, double *S, double *hist,
                const double *q, const double *k, const double *v,
                const double *alpha, const double *beta, const double *g,
                const double *wconv, const double *norm_w,
                int round_each_token, double *y, double *records)
{
    int dk, dv, t, i, j;
    double *qh, *kh, *vt, *u, *o, *al = NULL, *be = NULL;

    if (!cfg_ok(cfg) || T < 0 || !S || !hist || (T > 0 && (!q || !k || !v ||
        !alpha || !beta || !g || !wconv || !y)))
        return -1;
    dk = cfg->dk;
    dv = cfg->dv;
    if (T > 0 && gate_values(cfg, T, alpha, beta, &al, &be) != 0)
        return -2;
    qh = malloc(sizeof(double) * dk);
    kh = malloc(sizeof(double) * dk);
    vt = malloc(sizeof(double) * dv);
    u = malloc(sizeof(double) * dv);
    o = malloc(sizeof(double) * dv);
    if (!qh || !kh || !vt || !u || !o) {
        free(qh); free(kh); free(vt); free(u); free(o); free(al); free(be);
        return -2;
    }

    for (t = 0; t < T; ++t) {
        const double *xq = q + (long)t * dk, *xk = k + (long)t * dk;
        const double *xv = v + (long)t * dv, *a = al + (long)t * dk;
        const double b = be[t];

        conv_and_normalise(cfg, hist, xq, xk, xv, wconv, qh, kh, vt);

        /* 4. decay the rows of S */
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[i * dv + j] *= a[i];

        /* 5. delta-rule write: u = S^T kh, S += beta kh (vt - u)^T */
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i)
                acc += S[i * dv + j] * kh[i];
            u[j] = acc;
        }
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[i * dv + j] += b * kh[i] * (vt[j] - u[j]);

        /* 6. read-out after the write */
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (i = 0; i < dk; ++i)
                acc += S[i * dv + j] * qh[i];
            o[j] = acc;
        }

        /* 7. gated RMSNorm */
        gated_norm(cfg, o, g + (long)t * dv, norm_w, y + (long)t * dv);

        /* 8. store */
        if (round_each_token)
            kda_ref_round_bf16(S, (long)dk * dv);
        if (records)
            memcpy(records + (long)t * dk * dv, S, sizeof(double) * dk * dv);

        push_history(cfg, hist, xq, xk, xv);
    }
    free(qh); free(kh); free(vt); free(u); free(o); free(al); free(be);
    return 0;
}

/* Commit the accepted prefix of a verify over n draft tokens: m in [0, n].
 * records [n][dk][dv] are the verify's per-token states; draft_q/k/v are the
 * raw draft tokens [n][dk|dv].  store_bf16 rounds the committed state once. */
int kda_ref_commit(const kda_ref_cfg *cfg, int n, int m, int store_bf16,
                   double *S, double *hist, const double *records,
                   const double *draft_q, const double *draft_k,
                   const double *draft_v)
{
    int dk, dv, t;
    if (!cfg_ok(cfg) || n < 0 || m < 0 || m > n || !S || !hist)
        return -1;
    if (m == 0)
        return 0;
    if (!records || !draft_q || !draft_k || !draft_v)
        return -1;
    dk = cfg->dk;
    dv = cfg->dv;
    memcpy(S, records + (long)(m - 1) * dk * dv, sizeof(double) * dk * dv);
    if (store_bf16)
        kda_ref_round_bf16(S, (long)dk * dv);
    for (t = 0; t < m; ++t)
        push_history(cfg, hist, draft_q + (long)t * dk, draft_k + (long)t * dk,
                     draft_v + (long)t * dv);
    return 0;
}

/*
 * Chunkwise (WY/UT) form of steps 4-6, no rounding (prefill semantics).
 *
 * Within a chunk of L <= C tokens starting from state S0, write
 * G_t = sum_{s<=t} log alpha_s (per key channel, cumulative inside the
 * chunk) and D_t = Diag(exp(G_t)).  The write vector of token t,
 *     w_t = beta_t (vt_t - (Diag(alpha_t) S_{t-1})^T kh_t),
 * gives S_t = Diag(alpha_t) S_{t-1} + kh_t w_t^T, hence
 *     S_t = D_t S0 + sum_{i<=t} D_t D_i^{-1} kh_i w_i^T.
 * Substituting S_{t-1} into w_t:
 *     w_t + sum_{i<t} A_ti w_i = beta_t (vt_t - S0^T D_t kh_t),
 *     A_ti = beta_t kh_t^T D_t D_i^{-1} kh_i   (i < t),
 * i.e. (I + A) Wr = diag(beta) (V - K_D S0) with K_D rows (e^{G_t} * kh_t).
 * With Tm = (I + A)^{-1}:  Wr = Ut - Wm S0,  Ut = Tm diag(beta) V,
 * Wm = Tm diag(beta) K_D.  The read-outs and the chunk's final state are
 *     o_t = S0^T (e^{G_t} * qh_t) + sum_{i<=t} P_ti w_i,
 *     P_ti = qh_t^T D_t D_i^{-1} kh_i,
 *     S_L = D_L S0 + sum_i (e^{G_L - G_i} * kh_i) w_i^T.
 * Everything here is formed explicitly, in that order, from doubles.
 */
int kda_ref_run_chunked(const kda_ref_cfg *cfg, int T, int C, double *S,
                        double *hist, const double *q, const double *k,
                        const double *v, const double *alpha_in,
                        const double *beta_in, const double *g,
                        const double *wconv, const double *norm_w, double *y)
{
    int dk, dv, c0, t, i, j, c, L;
    double *QH, *KH, *VT, *G, *A, *Tm, *Wm, *Ut, *Wr, *O, *S0;
    double *alpha = NULL, *beta = NULL;
    int ok = 1;

    if (!cfg_ok(cfg) || T < 0 || C < 1 || !S || !hist || (T > 0 && (!q ||
        !k || !v || !alpha_in || !beta_in || !g || !wconv || !y)))
        return -1;
    dk = cfg->dk;
    dv = cfg->dv;
    QH = malloc(sizeof(double) * C * dk);
    KH = malloc(sizeof(double) * C * dk);
    VT = malloc(sizeof(double) * C * dv);
    G = malloc(sizeof(double) * C * dk);
    A = malloc(sizeof(double) * C * C);
    Tm = malloc(sizeof(double) * C * C);
    Wm = malloc(sizeof(double) * C * dk);
    Ut = malloc(sizeof(double) * C * dv);
    Wr = malloc(sizeof(double) * C * dv);
    O = malloc(sizeof(double) * C * dv);
    S0 = malloc(sizeof(double) * dk * dv);
    if (!QH || !KH || !VT || !G || !A || !Tm || !Wm || !Ut || !Wr || !O || !S0)
        ok = 0;
    if (ok && T > 0 && gate_values(cfg, T, alpha_in, beta_in, &alpha, &beta) != 0)
        ok = 0;

    for (c0 = 0; ok && c0 < T; c0 += C) {
        L = T - c0 < C ? T - c0 : C;
        /* steps 1-3 per token, and the cumulative log decay */
        for (t = 0; t < L; ++t) {
            const long tt = c0 + t;
            conv_and_normalise(cfg, hist, q + tt * dk, k + tt * dk, v + tt * dv,
                               wconv, QH + t * dk, KH + t * dk, VT + t * dv);
            push_history(cfg, hist, q + tt * dk, k + tt * dk, v + tt * dv);
            for (i = 0; i < dk; ++i)
                G[t * dk + i] = log(alpha[tt * dk + i]) +
                                (t > 0 ? G[(t - 1) * dk + i] : 0.0);
        }
        /* A_ti for i < t, zero elsewhere */
        for (t = 0; t < L; ++t)
            for (i = 0; i < L; ++i) {
                double acc = 0.0;
                if (i < t)
                    for (c = 0; c < dk; ++c)
                        acc += KH[t * dk + c] * KH[i * dk + c] *
                               exp(G[t * dk + c] - G[i * dk + c]);
                A[t * C + i] = beta[c0 + t] * acc;
            }
        /* Tm = (I + A)^{-1}, unit lower triangular, by forward substitution
         * on the columns of the identity */
        for (t = 0; t < L; ++t)
            for (i = 0; i < L; ++i) {
                double acc = (t == i) ? 1.0 : 0.0;
                for (c = 0; c < t; ++c)
                    acc -= A[t * C + c] * Tm[c * C + i];
                Tm[t * C + i] = acc;
            }
        /* Wm = Tm diag(beta) K_D, Ut = Tm diag(beta) V */
        for (t = 0; t < L; ++t) {
            for (c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (i = 0; i < L; ++i)
                    acc += Tm[t * C + i] * beta[c0 + i] *
                           exp(G[i * dk + c]) * KH[i * dk + c];
                Wm[t * dk + c] = acc;
            }
            for (j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (i = 0; i < L; ++i)
                    acc += Tm[t * C + i] * beta[c0 + i] * VT[i * dv + j];
                Ut[t * dv + j] = acc;
            }
        }
        /* write vectors Wr = Ut - Wm S0 */
        memcpy(S0, S, sizeof(double) * dk * dv);
        for (t = 0; t < L; ++t)
            for (j = 0; j < dv; ++j) {
                double acc = Ut[t * dv + j];
                for (c = 0; c < dk; ++c)
                    acc -= Wm[t * dk + c] * S0[c * dv + j];
                Wr[t * dv + j] = acc;
            }
        /* read-outs o_t = S0^T (e^{G_t} qh_t) + sum_{i<=t} P_ti w_i */
        for (t = 0; t < L; ++t)
            for (j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (c = 0; c < dk; ++c)
                    acc += exp(G[t * dk + c]) * QH[t * dk + c] * S0[c * dv + j];
                for (i = 0; i <= t; ++i) {
                    double p = 0.0;
                    for (c = 0; c < dk; ++c)
                        p += QH[t * dk + c] * KH[i * dk + c] *
                             exp(G[t * dk + c] - G[i * dk + c]);
                    acc += p * Wr[i * dv + j];
                }
                O[t * dv + j] = acc;
            }
        /* final state of the chunk */
        for (c = 0; c < dk; ++c)
            for (j = 0; j < dv; ++j) {
                const double gl = G[(L - 1) * dk + c];
                double acc = exp(gl) * S0[c * dv + j];
                for (i = 0; i < L; ++i)
                    acc += exp(gl - G[i * dk + c]) * KH[i * dk + c] *
                           Wr[i * dv + j];
                S[c * dv + j] = acc;
            }
        for (t = 0; t < L; ++t)
            gated_norm(cfg, O + t * dv, g + (long)(c0 + t) * dv, norm_w,
                       y + (long)(c0 + t) * dv);
    }
    free(QH); free(KH); free(VT); free(G); free(A); free(Tm); free(Wm);
    free(Ut); free(Wr); free(O); free(S0); free(alpha); free(beta);
    return ok ? 0 : -2;
}
