/*
 * wyo_oracle.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see wyo_oracle.h).
 *
 * Every routine is the definition written out with plain loops: no blocking, fusion or
 * reordering beyond what the cited passage states.  Sums run in ascending index order.
 * Threads only split the list of independent units; they never change the arithmetic.
 *
 * Pages cited: [Inv] "TileLang 实战：单位下三角矩阵求逆"; [QLA] the FlashQLA announcement.
 */
#include "wyo_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- input decoding ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32; widening to double is exact. */
static double decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* base, int32_t dtype, int64_t idx)
{
    if (dtype == WYO_BF16) return decode_bf16(((const uint16_t*)base)[idx]);
    return (double)((const float*)base)[idx];
}

/* ---- work map: chunks restart at each sequence start ([QLA] usage: cu_seqlens) ----------- */

static int problem_ok(const wyo_problem* p, const int32_t* cu)
{
    if (!p) return 0;
    if (p->batch < 0 || p->seqlen < 0 || p->num_qk_heads <= 0 || p->num_v_heads <= 0) return 0;
    if (p->num_v_heads % p->num_qk_heads != 0) return 0;
    if (p->head_dim_k <= 0 || p->head_dim_v <= 0 || p->chunk_size <= 0) return 0;
    if (p->kv_dtype != WYO_BF16 && p->kv_dtype != WYO_F32) return 0;
    if (cu) {
        if (p->batch != 1 || p->num_seqs < 0) return 0;
        if (cu[0] != 0 || cu[p->num_seqs] != p->seqlen) return 0;
        for (int32_t s = 0; s < p->num_seqs; ++s)
            if (cu[s + 1] < cu[s]) return 0;
    }
    return 1;
}

int64_t wyo_list_chunks(const wyo_problem* p, const int32_t* cu, int64_t* chunk_start,
                        int32_t* chunk_len, int64_t cap)
{
    if (!problem_ok(p, cu)) return -1;
    const int64_t C = p->chunk_size;
    int64_t count = 0;
    const int64_t nseq = cu ? p->num_seqs : p->batch;
    for (int64_t s = 0; s < nseq; ++s) {
        const int64_t s0 = cu ? cu[s] : s * (int64_t)p->seqlen;
        const int64_t s1 = cu ? cu[s + 1] : (s + 1) * (int64_t)p->seqlen;
        for (int64_t t0 = s0; t0 < s1; t0 += C) {
            if (chunk_start) {
                if (count >= cap) return -1;
                chunk_start[count] = t0;
                chunk_len[count] = (int32_t)((s1 - t0) < C ? (s1 - t0) : C);
            }
            ++count;
        }
    }
    return count;
}

int64_t wyo_count_chunks(const wyo_problem* p, const int32_t* cu)
{
    return wyo_list_chunks(p, cu, NULL, NULL, 0);
}

/* ---- [Inv] section 2.1: X = L^{-1} row by row ------------------------------------------- */
/* X[k,:] = e_k^T - sum_{j<k} L[k,j] X[j,:].  X[j,:] is zero right of column j, so the update
 * of row k from row j touches columns 0..j only.  The product with X[j,j] = 1 (column i = j)
 * is free; the counted ("necessary") products are those with i < j < k. */
int64_t wyo_row_forward_inverse(int32_t n, const double* L, int32_t ldl, double* X, int32_t ldx)
{
    int64_t fma = 0;
    for (int32_t k = 0; k < n; ++k) {
        double* xk = X + (int64_t)k * ldx;
        for (int32_t i = 0; i < n; ++i) xk[i] = (i == k) ? 1.0 : 0.0;
        for (int32_t j = 0; j < k; ++j) {
            const double lkj = L[(int64_t)k * ldl + j];
            const double* xj = X + (int64_t)j * ldx;
            for (int32_t i = 0; i <= j; ++i) {
                xk[i] -= lkj * xj[i];
                if (i < j) ++fma;
            }
        }
    }
    return fma;
}

/* ---- [Inv] section 2.2: the 2x2 block identity, applied recursively ----------------------
 * L = [[L00, 0], [L10, L11]]  =>  L^{-1} = [[L00^{-1}, 0], [-L11^{-1} L10 L00^{-1}, L11^{-1}]].
 * The two diagonal inverses are independent; the coupling is two dense products. */
int64_t wyo_block_recursive_inverse(int32_t n, int32_t base, const double* L, int32_t ldl,
                                    double* X, int32_t ldx, int32_t* depth)
{
    if (n <= base || n < 2) {
        if (depth) *depth = n > 0 ? n - 1 : 0;
        return wyo_row_forward_inverse(n, L, ldl, X, ldx);
    }
    const int32_t h = n / 2, m = n - h;
    int32_t d0 = 0, d1 = 0;
    int64_t fma = wyo_block_recursive_inverse(h, base, L, ldl, X, ldx, &d0);
    fma += wyo_block_recursive_inverse(m, base, L + (int64_t)h * ldl + h, ldl,
                                       X + (int64_t)h * ldx + h, ldx, &d1);
    for (int32_t i = 0; i < h; ++i)
        for (int32_t j = h; j < n; ++j) X[(int64_t)i * ldx + j] = 0.0;

    /* tmp = L10 X00  (m x h) */
    double* tmp = (double*)malloc(sizeof(double) * (size_t)m * (size_t)h);
    for (int32_t i = 0; i < m; ++i)
        for (int32_t j = 0; j < h; ++j) {
            double s = 0.0;
            for (int32_t q = 0; q < h; ++q) {
                s += L[(int64_t)(h + i) * ldl + q] * X[(int64_t)q * ldx + j];
                ++fma;
            }
            tmp[(int64_t)i * h + j] = s;
        }
    /* X10 = -(X11 tmp)  (m x h) */
    for (int32_t i = 0; i < m; ++i)
        for (int32_t j = 0; j < h; ++j) {
            double s = 0.0;
            for (int32_t q = 0; q < m; ++q) {
                s += X[(int64_t)(h + i) * ldx + (h + q)] * tmp[(int64_t)q * h + j];
                ++fma;
            }
            X[(int64_t)(h + i) * ldx + j] = -s;
        }
    free(tmp);
    if (depth) *depth = (d0 > d1 ? d0 : d1) + 2;
    return fma;
}

/* ---- one unit: ([Inv] section 1 equations, section 3.2 for the diagonal rule) ------------ */

typedef struct {
    double* K;  /* n x dk */
    double* V;  /* n x dv */
    double* b;  /* n */
    double* G;  /* n: chunk-local inclusive prefix sums of the log gates (0 without gates) */
    double* E;  /* n: exp(G), the decay from the chunk start through token j */
    double* A;  /* n x n */
    double* X;  /* n x n */
} unit_scratch;

static int scratch_alloc(unit_scratch* s, const wyo_problem* p)
{
    const size_t C = (size_t)p->chunk_size;
    s->K = (double*)malloc(sizeof(double) * C * (size_t)p->head_dim_k);
    s->V = (double*)malloc(sizeof(double) * C * (size_t)p->head_dim_v);
    s->b = (double*)malloc(sizeof(double) * C);
    s->G = (double*)malloc(sizeof(double) * C);
    s->E = (double*)malloc(sizeof(double) * C);
    s->A = (double*)malloc(sizeof(double) * C * C);
    s->X = (double*)malloc(sizeof(double) * C * C);
    return s->K && s->V && s->b && s->G && s->E && s->A && s->X;
}

static void scratch_free(unit_scratch* s)
{
    free(s->K); free(s->V); free(s->b); free(s->G); free(s->E); free(s->A); free(s->X);
}

/* Computes T (n x n, into s->X), and W, U (n x dk, n x dv) for the chunk [tok0, tok0 + n) of
 * value head hv.  Returns the forward-substitution count.
 *
 * Gates (g != NULL; [Inv] section 5, item 12: with gating the coefficient is
 * diag(beta)(Gamma o K K^T)): g holds log alpha_t per token and value head.  G_i is the sum of
 * g over the chunk's tokens 0..i, Gamma[i][j] = exp(G_i - G_j) is the decay from token j to
 * token i, and W takes the decay from the chunk start, W = T diag(beta exp(G)) K, while
 * U = T diag(beta) V keeps its form.  (Those two W / U forms are what the gated delta rule
 * S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T needs; the FlashQLA page
 * names the recurrence and its alpha_i in (0, 1), but its formula did not survive.)
 * Without gates G = 0, every exp() below is exactly 1 and the result is the ungated one. */
/* Decodes K, V (when v != NULL), beta and the gates of the chunk into s and forms
 * A = I + strictLower(diag(beta) (Gamma o K K^T)) in s->A (n x n). */
static void unit_form_a(const wyo_problem* p, const void* k, const void* v, const float* beta,
                        const float* gate, int64_t tok0, int32_t n, int32_t hv, unit_scratch* s)
{
    const int32_t dk = p->head_dim_k, dv = p->head_dim_v;
    const int32_t Hq = p->num_qk_heads, Hv = p->num_v_heads;
    const int32_t hk = hv / (Hv / Hq);

    for (int32_t i = 0; i < n; ++i) {
        const int64_t tok = tok0 + i;
        for (int32_t d = 0; d < dk; ++d)
            s->K[(int64_t)i * dk + d] = load_elem(k, p->kv_dtype, (tok * Hq + hk) * dk + d);
        if (v)
            for (int32_t e = 0; e < dv; ++e)
                s->V[(int64_t)i * dv + e] = load_elem(v, p->kv_dtype, (tok * Hv + hv) * dv + e);
        s->b[i] = (double)beta[tok * Hv + hv];
        const double gi = gate ? (double)gate[tok * Hv + hv] : 0.0;
        s->G[i] = (i == 0 ? 0.0 : s->G[i - 1]) + gi;
        s->E[i] = exp(s->G[i]);
    }

    /* A = I + strictLower(diag(beta) (Gamma o K K^T)): beta scales row i; the diagonal is 1. */
    for (int32_t i = 0; i < n; ++i)
        for (int32_t j = 0; j < n; ++j) {
            double a;
            if (j < i) {
                double g = 0.0;
                for (int32_t d = 0; d < dk; ++d)
                    g += s->K[(int64_t)i * dk + d] * s->K[(int64_t)j * dk + d];
                const double decay = exp(s->G[i] - s->G[j]);
                a = s->b[i] * decay * g;
            } else {
                a = (i == j) ? 1.0 : 0.0;
            }
            s->A[(int64_t)i * n + j] = a;
        }
}

static int64_t unit_solve(const wyo_problem* p, const void* k, const void* v, const float* beta,
                          const float* gate, int64_t tok0, int32_t n, int32_t hv,
                          unit_scratch* s, double* W, double* U)
{
    const int32_t dk = p->head_dim_k, dv = p->head_dim_v;
    unit_form_a(p, k, v, beta, gate, tok0, n, hv, s);

    /* T = A^{-1} */
    const int64_t fma = wyo_row_forward_inverse(n, s->A, n, s->X, n);

    /* W = T diag(beta exp(G)) K, U = T diag(beta) V  (full products over j = 0..n-1) */
    if (W) {
        for (int32_t i = 0; i < n; ++i) {
            for (int32_t d = 0; d < dk; ++d) {
                double acc = 0.0;
                for (int32_t j = 0; j < n; ++j)
                    acc += (s->X[(int64_t)i * n + j] * s->b[j] * s->E[j]) * s->K[(int64_t)j * dk + d];
                W[(int64_t)i * dk + d] = acc;
            }
            for (int32_t e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int32_t j = 0; j < n; ++j)
                    acc += (s->X[(int64_t)i * n + j] * s->b[j]) * s->V[(int64_t)j * dv + e];
                U[(int64_t)i * dv + e] = acc;
            }
        }
    }
    return fma;
}

/* The single right-hand side ([Inv] section 5, item 10: when T would be used only once, the
 * forward substitution is applied straight to the right-hand side and T is never formed):
 * X = A^{-1} diag(beta) R for the chunk's rows of R (the rhs, value-head layout, in s->V),
 * row by row, X[i,:] = beta_i R[i,:] - sum_{j<i} A[i,j] X[j,:] (ascending j), into Xout (n x dv).
 * With R = V this is U = T diag(beta) V. */
static void unit_rhs_solve(const wyo_problem* p, const void* k, const void* rhs, const float* beta,
                           const float* gate, int64_t tok0, int32_t n, int32_t hv,
                           unit_scratch* s, double* Xout)
{
    const int32_t dv = p->head_dim_v;
    unit_form_a(p, k, rhs, beta, gate, tok0, n, hv, s);
    for (int32_t i = 0; i < n; ++i)
        for (int32_t e = 0; e < dv; ++e) {
            double x = s->b[i] * s->V[(int64_t)i * dv + e];
            for (int32_t j = 0; j < i; ++j)
                x -= s->A[(int64_t)i * n + j] * Xout[(int64_t)j * dv + e];
            Xout[(int64_t)i * dv + e] = x;
        }
}

/* ---- threading over independent units ------------------------------------------------- */

typedef struct {
    const wyo_problem* p;
    const void* k;
    const void* v;
    const float* beta;
    const float* gate;     /* NULL: no gates */
    const int64_t* start;
    const int32_t* len;
    const int32_t* heads;  /* NULL: unit u = (chunk u / Hv, head u % Hv) */
    int64_t num_units;
    int compact;           /* 1: compact [M,C,*] outputs; 0: scatter into [B,T,Hv,*] */
    int rhs_solve;         /* 1: v is a right-hand side R; only X = A^{-1} diag(beta) R, into U */
    double* T;
    double* W;
    double* U;
    int32_t tid, nthreads;
    int64_t fma;
    int ok;
} job;

static void* job_run(void* arg)
{
    job* jb = (job*)arg;
    const wyo_problem* p = jb->p;
    const int32_t C = p->chunk_size, dk = p->head_dim_k, dv = p->head_dim_v;
    const int32_t Hv = p->num_v_heads;
    unit_scratch s;
    double* W = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dk);
    double* U = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dv);
    jb->ok = scratch_alloc(&s, p) && W && U;
    jb->fma = 0;
    if (jb->ok) {
        for (int64_t u = jb->tid; u < jb->num_units; u += jb->nthreads) {
            const int64_t c = jb->heads ? u : u / Hv;
            const int32_t hv = jb->heads ? jb->heads[u] : (int32_t)(u % Hv);
            const int64_t tok0 = jb->start[c];
            const int32_t n = jb->len[c];
            if (jb->rhs_solve) {
                unit_rhs_solve(p, jb->k, jb->v, jb->beta, jb->gate, tok0, n, hv, &s, U);
                for (int32_t i = 0; i < n; ++i)
                    memcpy(jb->U + ((tok0 + i) * Hv + hv) * dv, U + (int64_t)i * dv,
                           sizeof(double) * (size_t)dv);
                continue;
            }
            const int want_wu = jb->W != NULL;
            jb->fma += unit_solve(p, jb->k, want_wu ? jb->v : NULL, jb->beta, jb->gate, tok0, n,
                                  hv, &s, want_wu ? W : NULL, want_wu ? U : NULL);
            for (int32_t i = 0; i < n; ++i) {
                double* trow;
                double* wrow = NULL;
                double* urow = NULL;
                if (jb->compact) {
                    trow = jb->T + (u * C + i) * (int64_t)C;
                    if (want_wu) {
                        wrow = jb->W + (u * C + i) * (int64_t)dk;
                        urow = jb->U + (u * C + i) * (int64_t)dv;
                    }
                } else {
                    const int64_t row = (tok0 + i) * Hv + hv;
                    trow = jb->T + row * C;
                    if (want_wu) {
                        wrow = jb->W + row * dk;
                        urow = jb->U + row * dv;
                    }
                }
                for (int32_t j = 0; j < C; ++j) trow[j] = (j < n) ? s.X[(int64_t)i * n + j] : 0.0;
                if (want_wu) {
                    memcpy(wrow, W + (int64_t)i * dk, sizeof(double) * (size_t)dk);
                    memcpy(urow, U + (int64_t)i * dv, sizeof(double) * (size_t)dv);
                }
            }
        }
    }
    scratch_free(&s);
    free(W);
    free(U);
    return NULL;
}

static int run_jobs(job* proto, int32_t nthreads)
{
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    job* jobs = (job*)calloc((size_t)nthreads, sizeof(job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 0; }
    for (int32_t t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
    }
    int32_t started = 0;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, job_run, &jobs[t]) != 0) break;
        started = t;
    }
    /* threads that failed to start: run their share here */
    for (int32_t t = started + 1; t < nthreads; ++t) job_run(&jobs[t]);
    job_run(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    int ok = 1;
    proto->fma = 0;
    for (int32_t t = 0; t < nthreads; ++t) {
        ok = ok && jobs[t].ok;
        proto->fma += jobs[t].fma;
    }
    free(jobs);
    free(th);
    return ok;
}

int32_t wyo_wy_prepare(const wyo_problem* p, const void* k, const void* v, const float* g,
                       const float* beta, const int32_t* cu, double* T_out, double* W_out,
                       double* U_out, int32_t nthreads, int64_t* fma_out)
{
    if (!problem_ok(p, cu) || !k || !beta || !T_out) return 1;
    if ((W_out == NULL) != (U_out == NULL) || (W_out && !v)) return 1;
    const int64_t nchunks = wyo_count_chunks(p, cu);
    if (nchunks < 0) return 1;
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nchunks + 1));
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nchunks + 1));
    if (!start || !len) { free(start); free(len); return 2; }
    wyo_list_chunks(p, cu, start, len, nchunks);
    job proto;
    memset(&proto, 0, sizeof proto);
    proto.p = p; proto.k = k; proto.v = v; proto.beta = beta; proto.gate = g;
    proto.start = start; proto.len = len; proto.heads = NULL;
    proto.num_units = nchunks * p->num_v_heads;
    proto.compact = 0;
    proto.T = T_out; proto.W = W_out; proto.U = U_out;
    const int ok = run_jobs(&proto, nthreads);
    if (fma_out) *fma_out = proto.fma;
    free(start);
    free(len);
    return ok ? 0 : 2;
}

int32_t wyo_solve_rhs(const wyo_problem* p, const void* k, const void* rhs, const float* g,
                      const float* beta, const int32_t* cu, double* X_out, int32_t nthreads)
{
    if (!problem_ok(p, cu) || !k || !rhs || !beta || !X_out) return 1;
    const int64_t nchunks = wyo_count_chunks(p, cu);
    if (nchunks < 0) return 1;
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nchunks + 1));
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nchunks + 1));
    if (!start || !len) { free(start); free(len); return 2; }
    wyo_list_chunks(p, cu, start, len, nchunks);
    job proto;
    memset(&proto, 0, sizeof proto);
    proto.p = p; proto.k = k; proto.v = rhs; proto.beta = beta; proto.gate = g;
    proto.start = start; proto.len = len; proto.heads = NULL;
    proto.num_units = nchunks * p->num_v_heads;
    proto.compact = 0;
    proto.rhs_solve = 1;
    proto.U = X_out;
    const int ok = run_jobs(&proto, nthreads);
    free(start);
    free(len);
    return ok ? 0 : 2;
}

int32_t wyo_units(const wyo_problem* p, const void* k, const void* v, const float* g,
                  const float* beta, int64_t num_units, const int64_t* chunk_start, const int32_t* chunk_len,
                  const int32_t* v_head, double* T_out, double* W_out, double* U_out,
                  int32_t nthreads)
{
    if (!problem_ok(p, NULL) || !k || !beta || !T_out || num_units < 0) return 1;
    if (!chunk_start || !chunk_len || !v_head) return 1;
    if ((W_out == NULL) != (U_out == NULL) || (W_out && !v)) return 1;
    const int64_t total_tokens = (int64_t)p->batch * p->seqlen;
    for (int64_t u = 0; u < num_units; ++u)
        if (chunk_len[u] < 1 || chunk_len[u] > p->chunk_size || v_head[u] < 0 ||
            v_head[u] >= p->num_v_heads || chunk_start[u] < 0 ||
            chunk_start[u] + chunk_len[u] > total_tokens)
            return 1;
    const int64_t C = p->chunk_size;
    memset(T_out, 0, sizeof(double) * (size_t)(num_units * C * C));
    if (W_out) {
        memset(W_out, 0, sizeof(double) * (size_t)(num_units * C * p->head_dim_k));
        memset(U_out, 0, sizeof(double) * (size_t)(num_units * C * p->head_dim_v));
    }
    job proto;
    memset(&proto, 0, sizeof proto);
    proto.p = p; proto.k = k; proto.v = v; proto.beta = beta; proto.gate = g;
    proto.start = chunk_start; proto.len = chunk_len; proto.heads = v_head;
    proto.num_units = num_units;
    proto.compact = 1;
    proto.T = T_out; proto.W = W_out; proto.U = U_out;
    return run_jobs(&proto, nthreads) ? 0 : 2;
}

/* ---- the gated delta rule, token by token (see wyo_oracle.h) ----------------------------- */

typedef struct {
    const wyo_problem* p;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* h0;
    double scale;
    const int32_t* cu;
    double* o;
    double* hT;
    const uint8_t* mask;
    int32_t tid, nthreads;
    int ok;
} gdn_job;

static void* gdn_run(void* arg)
{
    gdn_job* jb = (gdn_job*)arg;
    const wyo_problem* p = jb->p;
    const int32_t dk = p->head_dim_k, dv = p->head_dim_v;
    const int32_t Hq = p->num_qk_heads, Hv = p->num_v_heads;
    const int64_t nseq = jb->cu ? p->num_seqs : p->batch;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
    jb->ok = S && kt && qt && e;
    if (jb->ok) {
        for (int64_t pair = jb->tid; pair < nseq * Hv; pair += jb->nthreads) {
            if (jb->mask && !jb->mask[pair]) continue;
            const int64_t seq = pair / Hv;
            const int32_t hv = (int32_t)(pair % Hv), hk = hv / (Hv / Hq);
            const int64_t s0 = jb->cu ? jb->cu[seq] : seq * (int64_t)p->seqlen;
            const int64_t s1 = jb->cu ? jb->cu[seq + 1] : (seq + 1) * (int64_t)p->seqlen;
            const float* h0 = jb->h0 ? jb->h0 + pair * (int64_t)dk * dv : NULL;
            for (int64_t i = 0; i < (int64_t)dk * dv; ++i) S[i] = h0 ? (double)h0[i] : 0.0;
            for (int64_t t = s0; t < s1; ++t) {
                const double alpha = jb->g ? exp((double)jb->g[t * Hv + hv]) : 1.0;
                const double b = (double)jb->beta[t * Hv + hv];
                for (int32_t d = 0; d < dk; ++d) {
                    kt[d] = load_elem(jb->k, p->kv_dtype, (t * Hq + hk) * dk + d);
                    qt[d] = load_elem(jb->q, p->kv_dtype, (t * Hq + hk) * dk + d);
                }
                /* S <- alpha S; e = beta (v_t - S^T k_t); S <- S + k_t e^T */
                for (int64_t i = 0; i < (int64_t)dk * dv; ++i) S[i] *= alpha;
                for (int32_t c = 0; c < dv; ++c) {
                    double r = 0.0;
                    for (int32_t d = 0; d < dk; ++d) r += kt[d] * S[(int64_t)d * dv + c];
                    e[c] = b * (load_elem(jb->v, p->kv_dtype, (t * Hv + hv) * dv + c) - r);
                }
                for (int32_t d = 0; d < dk; ++d)
                    for (int32_t c = 0; c < dv; ++c) S[(int64_t)d * dv + c] += kt[d] * e[c];
                /* o_t = scale S^T q_t */
                for (int32_t c = 0; c < dv; ++c) {
                    double r = 0.0;
                    for (int32_t d = 0; d < dk; ++d) r += qt[d] * S[(int64_t)d * dv + c];
                    jb->o[(t * Hv + hv) * (int64_t)dv + c] = jb->scale * r;
                }
            }
            if (jb->hT)
                memcpy(jb->hT + pair * (int64_t)dk * dv, S, sizeof(double) * (size_t)dk * (size_t)dv);
        }
    }
    free(S); free(kt); free(qt); free(e);
    return NULL;
}

int32_t wyo_gdn_forward(const wyo_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, double scale,
                        const int32_t* cu, double* o_out, double* hT_out,
                        const uint8_t* pair_mask, int32_t nthreads)
{
    if (!problem_ok(p, cu) || !q || !k || !v || !beta || !o_out) return 1;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    gdn_job* jobs = (gdn_job*)calloc((size_t)nthreads, sizeof(gdn_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 2; }
    for (int32_t t = 0; t < nthreads; ++t) {
        gdn_job* jb = &jobs[t];
        jb->p = p; jb->q = q; jb->k = k; jb->v = v; jb->g = g; jb->beta = beta; jb->h0 = h0;
        jb->scale = scale; jb->cu = cu; jb->o = o_out; jb->hT = hT_out; jb->mask = pair_mask;
        jb->tid = t; jb->nthreads = nthreads;
    }
    int32_t started = 0;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, gdn_run, &jobs[t]) != 0) break;
        started = t;
    }
    for (int32_t t = started + 1; t < nthreads; ++t) gdn_run(&jobs[t]);
    gdn_run(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    int ok = 1;
    for (int32_t t = 0; t < nthreads; ++t) ok = ok && jobs[t].ok;
    free(jobs);
    free(th);
    return ok ? 0 : 2;
}

/* ---- backward of the preparation step (see wyo_oracle.h) ------------------------------------
 * Forward, per chunk and value head (D = diag(beta), E = diag(exp(G)), Gamma[i][j] =
 * exp(G_i - G_j)):  L = strictLower(D (Gamma o K K^T)),  A = I + L,  T = A^{-1},
 * W = T D E K,  U = T D V.  Reverse, for the upstream dT, dW, dU:
 *   dT_tot = dT + dW (D E K)^T + dU (D V)^T
 *   d(D E K) = T^T dW  ->  dK += D E (T^T dW),  dbeta_i += sum_d (T^T dW)[i][d] e^{G_i} K[i][d],
 *                          dG_i += sum_d (T^T dW)[i][d] beta_i e^{G_i} K[i][d]
 *   d(D V)   = T^T dU  ->  dV = D (T^T dU),      dbeta_i += sum_d (T^T dU)[i][d] V[i][d]
 *   dA = -T^T dT_tot T^T  (the derivative of the inverse); M = strictLower(dA)
 *   L_ij = beta_i Gamma_ij (k_i . k_j), i > j:
 *       dbeta_i += M_ij Gamma_ij (k_i . k_j);  dK_i += M_ij beta_i Gamma_ij k_j,
 *       dK_j += M_ij beta_i Gamma_ij k_i;      dG_i += Z_ij, dG_j -= Z_ij with
 *       Z_ij = M_ij beta_i Gamma_ij (k_i . k_j)
 *   G_i = g_0 + ... + g_i  ->  dg_t = sum_{i >= t} dG_i.
 */
typedef struct {
    const wyo_problem* p;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* dT;
    const void* dW;
    const void* dU;
    const int64_t* start;
    const int32_t* len;
    int64_t nchunks;
    double* dk;
    double* dv;
    double* db;
    double* dg;
    int32_t tid, nthreads;
    int ok;
} bwd_job;

static void* bwd_run(void* arg)
{
    bwd_job* jb = (bwd_job*)arg;
    const wyo_problem* p = jb->p;
    const int32_t C = p->chunk_size, dk = p->head_dim_k, dv = p->head_dim_v;
    const int32_t Hq = p->num_qk_heads, Hv = p->num_v_heads, r = Hv / Hq;
    unit_scratch s;
    const size_t CC = (size_t)C * (size_t)C;
    double* dTt = (double*)malloc(sizeof(double) * CC);   /* dT_tot */
    double* Y = (double*)malloc(sizeof(double) * CC);     /* dT_tot T^T */
    double* M = (double*)malloc(sizeof(double) * CC);     /* strictLower(dA) */
    double* TdW = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dk);
    double* TdU = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dv);
    double* dWc = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dk);
    double* dUc = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dv);
    double* dK = (double*)malloc(sizeof(double) * (size_t)C * (size_t)dk);
    double* dG = (double*)malloc(sizeof(double) * (size_t)C);
    jb->ok = scratch_alloc(&s, p) && dTt && Y && M && TdW && TdU && dWc && dUc && dK && dG;
    if (jb->ok) {
        for (int64_t job = jb->tid; job < jb->nchunks * Hq; job += jb->nthreads) {
            const int64_t c = job / Hq;
            const int32_t hk = (int32_t)(job % Hq);
            const int64_t tok0 = jb->start[c];
            const int32_t n = jb->len[c];
            for (int64_t i = 0; i < (int64_t)n * dk; ++i) dK[i] = 0.0;
            for (int32_t hv = hk * r; hv < (hk + 1) * r; ++hv) {
                /* forward: K, V, beta, G, E and T = A^{-1} (into s.X) */
                unit_solve(p, jb->k, jb->v, jb->beta, jb->g, tok0, n, hv, &s, NULL, NULL);
                const double* K = s.K;
                const double* V = s.V;
                const double* b = s.b;
                const double* E = s.E;
                const double* T = s.X;
                for (int32_t i = 0; i < n; ++i) {
                    const int64_t row = (tok0 + i) * Hv + hv;
                    for (int32_t d = 0; d < dk; ++d)
                        dWc[(int64_t)i * dk + d] = load_elem(jb->dW, p->kv_dtype, row * dk + d);
                    for (int32_t d = 0; d < dv; ++d)
                        dUc[(int64_t)i * dv + d] = load_elem(jb->dU, p->kv_dtype, row * dv + d);
                }
                /* dT_tot[i][j] = dT[i][j] + sum_d dW[i][d] beta_j e^{G_j} K[j][d]
                 *                         + sum_d dU[i][d] beta_j V[j][d] */
                for (int32_t i = 0; i < n; ++i)
                    for (int32_t j = 0; j < n; ++j) {
                        double a = jb->dT ? (double)jb->dT[((tok0 + i) * Hv + hv) * (int64_t)C + j] : 0.0;
                        double w = 0.0, u = 0.0;
                        for (int32_t d = 0; d < dk; ++d) w += dWc[(int64_t)i * dk + d] * K[(int64_t)j * dk + d];
                        for (int32_t d = 0; d < dv; ++d) u += dUc[(int64_t)i * dv + d] * V[(int64_t)j * dv + d];
                        dTt[(int64_t)i * n + j] = a + w * b[j] * E[j] + u * b[j];
                    }
                /* T^T dW and T^T dU */
                for (int32_t i = 0; i < n; ++i) {
                    for (int32_t d = 0; d < dk; ++d) {
                        double acc = 0.0;
                        for (int32_t m = 0; m < n; ++m) acc += T[(int64_t)m * n + i] * dWc[(int64_t)m * dk + d];
                        TdW[(int64_t)i * dk + d] = acc;
                    }
                    for (int32_t d = 0; d < dv; ++d) {
                        double acc = 0.0;
                        for (int32_t m = 0; m < n; ++m) acc += T[(int64_t)m * n + i] * dUc[(int64_t)m * dv + d];
                        TdU[(int64_t)i * dv + d] = acc;
                    }
                }
                double* dbrow = jb->db;
                for (int32_t i = 0; i < n; ++i) {
                    const int64_t row = (tok0 + i) * Hv + hv;
                    double dbi = 0.0, dgi = 0.0;
                    for (int32_t d = 0; d < dk; ++d) {
                        const double t = TdW[(int64_t)i * dk + d];
                        dK[(int64_t)i * dk + d] += b[i] * E[i] * t;
                        dbi += t * E[i] * K[(int64_t)i * dk + d];
                        dgi += t * b[i] * E[i] * K[(int64_t)i * dk + d];
                    }
                    for (int32_t d = 0; d < dv; ++d) {
                        const double t = TdU[(int64_t)i * dv + d];
                        jb->dv[row * dv + d] = b[i] * t;
                        dbi += t * V[(int64_t)i * dv + d];
                    }
                    dbrow[row] = dbi;
                    dG[i] = dgi;
                }
                /* dA = -T^T dT_tot T^T:  Y = dT_tot T^T, M = strictLower(-T^T Y) */
                for (int32_t i = 0; i < n; ++i)
                    for (int32_t j = 0; j < n; ++j) {
                        double acc = 0.0;
                        for (int32_t m = 0; m < n; ++m) acc += dTt[(int64_t)i * n + m] * T[(int64_t)j * n + m];
                        Y[(int64_t)i * n + j] = acc;
                    }
                for (int32_t i = 0; i < n; ++i)
                    for (int32_t j = 0; j < n; ++j) {
                        double acc = 0.0;
                        if (j < i)
                            for (int32_t m = 0; m < n; ++m) acc += T[(int64_t)m * n + i] * Y[(int64_t)m * n + j];
                        M[(int64_t)i * n + j] = -acc;
                    }
                /* through L_ij = beta_i Gamma_ij (k_i . k_j), i > j */
                for (int32_t i = 0; i < n; ++i)
                    for (int32_t j = 0; j < i; ++j) {
                        const double mij = M[(int64_t)i * n + j];
                        const double gam = exp(s.G[i] - s.G[j]);
                        double kk = 0.0;
                        for (int32_t d = 0; d < dk; ++d) kk += K[(int64_t)i * dk + d] * K[(int64_t)j * dk + d];
                        const int64_t row = (tok0 + i) * Hv + hv;
                        dbrow[row] += mij * gam * kk;
                        const double rr = mij * b[i] * gam;
                        for (int32_t d = 0; d < dk; ++d) {
                            dK[(int64_t)i * dk + d] += rr * K[(int64_t)j * dk + d];
                            dK[(int64_t)j * dk + d] += rr * K[(int64_t)i * dk + d];
                        }
                        const double z = rr * kk;
                        dG[i] += z;
                        dG[j] -= z;
                    }
                /* dg_t = sum_{i >= t} dG_i */
                if (jb->dg) {
                    double run = 0.0;
                    for (int32_t t = n - 1; t >= 0; --t) {
                        run += dG[t];
                        jb->dg[(tok0 + t) * Hv + hv] = run;
                    }
                }
            }
            for (int32_t i = 0; i < n; ++i)
                memcpy(jb->dk + ((tok0 + i) * Hq + hk) * (int64_t)dk, dK + (int64_t)i * dk,
                       sizeof(double) * (size_t)dk);
        }
    }
    scratch_free(&s);
    free(dTt); free(Y); free(M); free(TdW); free(TdU); free(dWc); free(dUc); free(dK); free(dG);
    return NULL;
}

int32_t wyo_wy_backward(const wyo_problem* p, const void* k, const void* v, const float* g,
                        const float* beta, const int32_t* cu, const float* dT, const void* dW,
                        const void* dU, double* dk_out, double* dv_out, double* dbeta_out,
                        double* dg_out, int32_t nthreads)
{
    if (!problem_ok(p, cu) || !k || !v || !beta || !dW || !dU) return 1;
    if (!dk_out || !dv_out || !dbeta_out || (g && !dg_out)) return 1;
    const int64_t nchunks = wyo_count_chunks(p, cu);
    if (nchunks < 0) return 1;
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nchunks + 1));
    int32_t* len = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nchunks + 1));
    if (!start || !len) { free(start); free(len); return 2; }
    wyo_list_chunks(p, cu, start, len, nchunks);
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); free(start); free(len); return 2; }
    for (int32_t t = 0; t < nthreads; ++t) {
        bwd_job* jb = &jobs[t];
        jb->p = p; jb->k = k; jb->v = v; jb->g = g; jb->beta = beta; jb->dT = dT; jb->dW = dW;
        jb->dU = dU; jb->start = start; jb->len = len; jb->nchunks = nchunks; jb->dk = dk_out;
        jb->dv = dv_out; jb->db = dbeta_out; jb->dg = g ? dg_out : NULL;
        jb->tid = t; jb->nthreads = nthreads;
    }
    int32_t started = 0;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, bwd_run, &jobs[t]) != 0) break;
        started = t;
    }
    for (int32_t t = started + 1; t < nthreads; ++t) bwd_run(&jobs[t]);
    bwd_run(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    int ok = 1;
    for (int32_t t = 0; t < nthreads; ++t) ok = ok && jobs[t].ok;
    free(jobs); free(th); free(start); free(len);
    return ok ? 0 : 2;
}
