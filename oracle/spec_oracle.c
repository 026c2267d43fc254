/* spec_oracle.c - plain fp64 CPU oracle of the speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline leg of the benchmark, never by the product path.  Slow on purpose:
 * one sequence at a time, one row at a time, sums in ascending index order,
 * libm exp/log in double precision.  Shares nothing with the HIP library.
 *
 * Sources (cited by page and section):
 *   [QH]  quochung.cyou, "A.I" category page, tutorial on speculative decoding:
 *         sections "Chọn token: greedy vs sampling", "Một vòng speculative
 *         decoding", "Draft model kém hơn target...", "Modified rejection
 *         sampling" (subsections "Giải pháp", "Khi reject thì lấy token từ
 *         đâu?", "Toàn bộ thuật toán cho một token", "Áp dụng thuật toán").
 *   [NL]  nalar.dev, "Speculative decoding: memverifikasi token draft secara
 *         paralel": sections "Sampling eksak memerlukan aturan koreksi" and
 *         "Penolakan memotong prefix yang diterima".
 *   [MC]  ml-canon-ru card 57 "Speculative Decoding": section "Приёмка и
 *         почему распределение НЕ портится" and the Python sketch of one round.
 *
 * Readings where the pages leave a step open (each restated where used):
 *   R1  p = softmax(l/T), q = softmax(d/T), one T > 0 for both.
 *   R2  accept iff u < alpha (strict, u in [0,1)), the sketch's form in [MC].
 *   R3  uniforms[b, j] (j < K) drives test j; uniforms[b, K] drives the one
 *       final draw (correction or bonus).
 *   R4  "sample from a distribution" = inverse CDF in ascending token index:
 *       smallest i with C_i > u*S; rounding overrun -> last i with r_i > 0.
 *   R5  residual mass exactly 0 after a reject (rounding only) -> draw from p_n,
 *       flagged.
 *   R6  bonus token drawn from p_K when all K drafts pass ([QH] "Áp dụng").
 *   R8  argmax ties go to the lowest index, on raw logits.
 *   R9  greedy sequences ignore T, uniforms and draft logits.
 *   R10 accepted_len = n in [0, K]; n + 1 tokens are emitted; padding -1.
 *   R11 q(x) = 0: alpha = 1 if p(x) > 0, else 0.
 *   R12 a row that the method examines and that holds NaN or +Inf, or is all
 *       -Inf, a token outside [0, V) or a uniform outside [0, 1) that the
 *       method uses, makes the sequence invalid: accepted_len = -1, row -1.
 *       -Inf logits are legal (masked tokens).  Rows past the first rejection
 *       are never examined ([QH] "Một vòng": candidates after the rejected
 *       one are dropped unchecked).
 */
#include "spec_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- exact widening of stored logits ----------------------------------- */

static double load_logit(const void* base, int dtype, size_t i)
{
    if (dtype == 0) return (double)((const float*)base)[i];
    if (dtype == 2) return ((const double*)base)[i];
    /* bf16: the 16 stored bits are the top half of an fp32 word */
    uint32_t w = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) { return dtype == 0 ? 4 : (dtype == 1 ? 2 : 8); }

static const void* row_ptr(const void* base, int dtype, size_t row, int32_t V)
{
    return (const char*)base + row * (size_t)V * elem_size(dtype);
}

/* ---- softmax at temperature T ([QH] "Forward pass": a probability table
 * over the vocabulary summing to 100%; R1 for the temperature) ------------ */

int oracle_row_softmax(const void* row, int dtype, int32_t V, double T, double* p, double* lse)
{
    double m = -INFINITY;
    for (int32_t i = 0; i < V; ++i) {
        double v = load_logit(row, dtype, (size_t)i);
        if (isnan(v) || v == INFINITY) return 0;          /* R12 */
        if (v > m) m = v;
    }
    if (m == -INFINITY) return 0;                         /* all -Inf: R12 */
    double Z = 0.0;
    for (int32_t i = 0; i < V; ++i) {
        double v = load_logit(row, dtype, (size_t)i);
        double e = (v == -INFINITY) ? 0.0 : exp((v - m) / T);
        p[i] = e;
        Z += e;                                           /* ascending i */
    }
    for (int32_t i = 0; i < V; ++i) p[i] /= Z;
    if (lse) *lse = m / T + log(Z);
    return 1;
}

/* ---- greedy choice ([QH] "Chọn token": greedy picks the most likely token;
 * R8 for ties) ------------------------------------------------------------ */

int oracle_row_argmax(const void* row, int dtype, int32_t V, int32_t* idx)
{
    double best = -INFINITY;
    int32_t bi = -1;
    for (int32_t i = 0; i < V; ++i) {
        double v = load_logit(row, dtype, (size_t)i);
        if (isnan(v) || v == INFINITY) return 0;          /* R12 */
        if (v > best) { best = v; bi = i; }               /* strict: first maximum wins */
    }
    if (bi < 0) return 0;                                 /* all -Inf */
    *idx = bi;
    return 1;
}

/* ---- inverse-CDF draw (R4; [QH] "Chọn token": the 100-sided die) -------- */

int32_t oracle_draw(const double* r, int32_t V, double u, double* S_out, double* margin)
{
    double S = 0.0;
    for (int32_t i = 0; i < V; ++i) S += r[i];            /* ascending i */
    *S_out = S;
    if (!(S > 0.0)) { *margin = 0.0; return -1; }
    double t = u * S;
    double C = 0.0;
    for (int32_t i = 0; i < V; ++i) {
        double Cprev = C;
        C += r[i];
        if (C > t) {
            double a = t - Cprev, b = C - t;
            *margin = a < b ? a : b;
            return i;
        }
    }
    /* rounding overrun: the last token with positive weight */
    for (int32_t i = V - 1; i >= 0; --i)
        if (r[i] > 0.0) { *margin = 0.0; return i; }
    *margin = 0.0;
    return -1;
}

/* ---- one sequence -------------------------------------------------------- */

typedef struct {
    const void* target; const void* draft; int dtype; int ddtype;
    const int32_t* tokens; const float* uniforms; double T; const uint8_t* greedy;
    int32_t B, K, V;
    int32_t* acc; int32_t* out;
    const oracle_diag* dg;
    int32_t b0, b1;
} job_t;

static void set_d(double* a, size_t i, double v) { if (a) a[i] = v; }

static void mark_invalid(const job_t* J, int32_t b)
{
    int32_t K = J->K;
    J->acc[b] = -1;
    for (int32_t j = 0; j <= K; ++j) J->out[(size_t)b * (K + 1) + j] = -1;
    const oracle_diag* d = J->dg;
    if (!d) return;
    for (int32_t j = 0; j < K; ++j) {
        set_d(d->p_tok, (size_t)b * K + j, NAN);
        set_d(d->q_tok, (size_t)b * K + j, NAN);
        set_d(d->lse_q, (size_t)b * K + j, NAN);
        set_d(d->test_margin, (size_t)b * K + j, NAN);
    }
    for (int32_t j = 0; j <= K; ++j) set_d(d->lse_p, (size_t)b * (K + 1) + j, NAN);
    set_d(d->res_mass, (size_t)b, NAN);
    set_d(d->draw_margin, (size_t)b, NAN);
    if (d->flags) d->flags[b] = 0;
}

static int u_ok(float u) { return u >= 0.0f && u < 1.0f; }   /* NaN fails both */

/* Greedy sequence ([QH] "Draft model kém hơn target...": keep the draft token
 * while it equals the target's choice, otherwise emit the target's token and
 * stop; all K pass -> one more token from the target, [QH] "Áp dụng").       */
static void verify_greedy(const job_t* J, int32_t b)
{
    int32_t K = J->K, V = J->V;
    int32_t* out = J->out + (size_t)b * (K + 1);
    int32_t n = K, y = -1;
    for (int32_t j = 0; j <= K; ++j) {
        int32_t g;
        if (!oracle_row_argmax(row_ptr(J->target, J->dtype, (size_t)b * (K + 1) + j, V),
                               J->dtype, V, &g)) { mark_invalid(J, b); return; }
        if (j == K) { n = K; y = g; break; }
        int32_t x = J->tokens[(size_t)b * K + j];
        if (x < 0 || x >= V) { mark_invalid(J, b); return; }
        if (x != g) { n = j; y = g; break; }
    }
    for (int32_t j = 0; j < n; ++j) out[j] = J->tokens[(size_t)b * K + j];
    out[n] = y;
    for (int32_t j = n + 1; j <= K; ++j) out[j] = -1;
    J->acc[b] = n;
    if (J->dg) set_d(J->dg->res_mass, (size_t)b, 0.0);
}

/* Sampling sequence: modified rejection sampling, left to right.
 *   alpha_j = min(1, p_j(x_j) / q_j(x_j))        [QH] "Giải pháp"; [NL]; [MC]
 *   accept iff u_j < alpha_j                      R2 ([MC] sketch)
 *   first reject at n: y ~ norm(max(0, p_n - q_n)) [QH] "Khi reject..."; [NL]; [MC]
 *   all accepted: bonus y ~ p_K                   [QH] "Áp dụng thuật toán"
 *   positions after n are never examined          [QH] "Một vòng"; [NL] "Penolakan..." */
static void verify_sampling(const job_t* J, int32_t b, double* p, double* q, double* r)
{
    int32_t K = J->K, V = J->V;
    const oracle_diag* dg = J->dg;
    int32_t* out = J->out + (size_t)b * (K + 1);
    const float* u = J->uniforms + (size_t)b * (K + 1);
    int flags = 0;
    int32_t n = K;

    for (int32_t j = 0; j < K; ++j) {
        double lp, lq;
        if (!oracle_row_softmax(row_ptr(J->target, J->dtype, (size_t)b * (K + 1) + j, V),
                                J->dtype, V, J->T, p, &lp)) { mark_invalid(J, b); return; }
        if (!oracle_row_softmax(row_ptr(J->draft, J->ddtype, (size_t)b * K + j, V),
                                J->ddtype, V, J->T, q, &lq)) { mark_invalid(J, b); return; }
        int32_t x = J->tokens[(size_t)b * K + j];
        if (x < 0 || x >= V || !u_ok(u[j])) { mark_invalid(J, b); return; }
        double px = p[x], qx = q[x];
        double alpha;
        if (qx > 0.0) alpha = (px / qx < 1.0) ? px / qx : 1.0;
        else alpha = (px > 0.0) ? 1.0 : 0.0;              /* R11 */
        double uj = (double)u[j];
        double mg = fabs(uj - alpha);
        if (dg) {
            set_d(dg->p_tok, (size_t)b * K + j, px);
            set_d(dg->q_tok, (size_t)b * K + j, qx);
            set_d(dg->lse_p, (size_t)b * (K + 1) + j, lp);
            set_d(dg->lse_q, (size_t)b * K + j, lq);
            set_d(dg->test_margin, (size_t)b * K + j, mg);
        }
        if (mg < ORACLE_NEAR) flags |= ORACLE_FLAG_TEST_NEAR;
        if (!(uj < alpha)) { n = j; break; }              /* first rejection ends the round */
    }

    if (!u_ok(u[K])) { mark_invalid(J, b); return; }
    double uK = (double)u[K];
    int32_t y;
    double S, mg;
    if (n < K) {
        /* p and q still hold row n: residual max(0, p - q) */
        for (int32_t i = 0; i < V; ++i) r[i] = (p[i] - q[i] > 0.0) ? p[i] - q[i] : 0.0;
        y = oracle_draw(r, V, uK, &S, &mg);
        if (y < 0) {                                      /* R5 */
            flags |= ORACLE_FLAG_FALLBACK;
            double S0;
            y = oracle_draw(p, V, uK, &S0, &mg);
            S = 0.0;
        }
    } else {
        double lp;
        if (!oracle_row_softmax(row_ptr(J->target, J->dtype, (size_t)b * (K + 1) + K, V),
                                J->dtype, V, J->T, p, &lp)) { mark_invalid(J, b); return; }
        if (dg) set_d(dg->lse_p, (size_t)b * (K + 1) + K, lp);
        y = oracle_draw(p, V, uK, &S, &mg);
    }
    if (mg < ORACLE_NEAR) flags |= ORACLE_FLAG_DRAW_NEAR;

    for (int32_t j = 0; j < n; ++j) out[j] = J->tokens[(size_t)b * K + j];
    out[n] = y;
    for (int32_t j = n + 1; j <= K; ++j) out[j] = -1;
    J->acc[b] = n;
    if (dg) {
        set_d(dg->res_mass, (size_t)b, S);
        set_d(dg->draw_margin, (size_t)b, mg);
        if (dg->flags) dg->flags[b] = flags;
    }
}

static void clear_diag(const job_t* J, int32_t b)
{
    const oracle_diag* d = J->dg;
    int32_t K = J->K;
    if (!d) return;
    for (int32_t j = 0; j < K; ++j) {
        set_d(d->p_tok, (size_t)b * K + j, NAN);
        set_d(d->q_tok, (size_t)b * K + j, NAN);
        set_d(d->lse_q, (size_t)b * K + j, NAN);
        set_d(d->test_margin, (size_t)b * K + j, NAN);
    }
    for (int32_t j = 0; j <= K; ++j) set_d(d->lse_p, (size_t)b * (K + 1) + j, NAN);
    set_d(d->res_mass, (size_t)b, NAN);
    set_d(d->draw_margin, (size_t)b, NAN);
    if (d->flags) d->flags[b] = 0;
}

static void* run_job(void* arg)
{
    const job_t* J = (const job_t*)arg;
    size_t V = (size_t)J->V;
    double* buf = (double*)malloc(3 * V * sizeof(double));
    if (!buf) return (void*)1;
    for (int32_t b = J->b0; b < J->b1; ++b) {
        clear_diag(J, b);
        if (J->greedy && J->greedy[b]) verify_greedy(J, b);
        else verify_sampling(J, b, buf, buf + V, buf + 2 * V);
    }
    free(buf);
    return NULL;
}

int oracle_verify(const void* target, int dtype, const void* draft, int ddtype,
                  const int32_t* tokens, const float* uniforms, double T,
                  const uint8_t* greedy, int32_t B, int32_t K, int32_t V,
                  int32_t* accepted_len, int32_t* out_tokens,
                  const oracle_diag* diag, int nthreads)
{
    if (B < 0 || K < 0 || V < 1 || dtype < 0 || dtype > 2 || ddtype < 0 || ddtype > 2) return -1;
    if (B == 0) return 0;
    if (!target || !uniforms || !accepted_len || !out_tokens) return -1;
    if (K > 0 && !tokens) return -1;
    if (K > 0 && !draft) {
        if (!greedy) return -1;
        for (int32_t b = 0; b < B; ++b) if (!greedy[b]) return -1;
    }
    if (!(T > 0.0) || !isfinite(T)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = B;

    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        job_t J = { target, draft, dtype, ddtype, tokens, uniforms, T, greedy, B, K, V,
                    accepted_len, out_tokens, diag,
                    (int32_t)((int64_t)B * t / nthreads), (int32_t)((int64_t)B * (t + 1) / nthreads) };
        jobs[t] = J;
    }
    if (nthreads == 1) {
        if (run_job(&jobs[0])) rc = -1;
    } else {
        int started = 0;
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) { rc = -1; break; }
            ++started;
        }
        for (int t = 0; t < started; ++t) {
            void* ret = NULL;
            pthread_join(th[t], &ret);
            if (ret) rc = -1;
        }
    }
    free(jobs);
    free(th);
    return rc;
}
