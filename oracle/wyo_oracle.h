/*
 * wyo_oracle.h -- plain fp64 CPU oracle for the per-chunk WY/UT preparation of chunkwise
 * (Gated) DeltaNet.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline load this library.  It shares no code, header, table or helper with the HIP path
 * under chunkwise_gated_deltanet_amd/ and never includes a HIP header.
 *
 * Pages cited (by title and section):
 *   [Inv]  "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
 *          lower-triangular matrix), sections 1, 2.1-2.4, 3.2, 4.
 *   [QLA]  The FlashQLA announcement, section "使用方式" (usage): tensor shapes of k, v, beta
 *          and the optional cu_seqlens.
 *
 * What it computes, for every chunk of C tokens of every sequence and every value head
 * ([Inv] section 1, first equation and the W / U equations):
 *     A = I + strictLower(diag(beta) K K^T)
 *     T = A^{-1}                      (row-wise forward substitution, [Inv] section 2.1)
 *     W = T diag(beta) K,  U = T diag(beta) V
 * With per-token log gates g ([Inv] section 5, item 12 for the gated coefficient; [QLA] usage
 * for g [B,T,Hv]): G_i = g_0 + ... + g_i over the chunk's tokens, Gamma[i][j] = exp(G_i - G_j),
 *     A = I + strictLower(diag(beta) (Gamma o K K^T))
 *     W = T diag(beta exp(G)) K,  U = T diag(beta) V
 * (the W / U forms of the gated delta rule; without gates G = 0 and this is the line above).
 * All arithmetic is IEEE double; inputs are decoded exactly from the caller's bf16 / fp32 data.
 *
 * Conventions (readings of the pages where they leave a choice open):
 *   - Token-major layouts as in [QLA] usage: k [B,T,Hq,dk], v [B,T,Hv,dv], beta [B,T,Hv],
 *     g [B,T,Hv] (float32 log alpha_t, or NULL for no gates).
 *   - Value head h reads key head h / (Hv/Hq) (contiguous groups).
 *   - With cu_seqlens (B must be 1) chunks restart at every sequence start; the last chunk of
 *     a sequence may hold n < C tokens and is solved as an n x n system.
 *   - T is returned as [B,T,Hv,C]: row t holds row (t - chunk start) of its chunk's T, with
 *     chunk-relative columns; columns >= n of a short chunk are 0.
 *   - W [B,T,Hv,dk], U [B,T,Hv,dv].
 * All pointers are host pointers owned by the caller.
 */
#ifndef WYO_ORACLE_H
#define WYO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { WYO_BF16 = 0, WYO_F32 = 1 };

typedef struct {
    int32_t batch;        /* B (1 when cu_seqlens is given) */
    int32_t seqlen;       /* T per batch row, or total packed tokens with cu_seqlens */
    int32_t num_qk_heads; /* Hq */
    int32_t num_v_heads;  /* Hv, a multiple of Hq */
    int32_t head_dim_k;   /* dk */
    int32_t head_dim_v;   /* dv */
    int32_t chunk_size;   /* C */
    int32_t num_seqs;     /* N, used only with cu_seqlens */
    int32_t kv_dtype;     /* WYO_BF16 (k, v given as raw bf16 bit patterns) or WYO_F32 */
} wyo_problem;

/* Number of chunks (over all sequences); -1 on invalid arguments. */
int64_t wyo_count_chunks(const wyo_problem* p, const int32_t* cu_seqlens);

/* Writes the first-token index (flattened b*T + t) and the length of every chunk, in
 * sequence order; returns the count, or -1 if it exceeds cap or the arguments are invalid. */
int64_t wyo_list_chunks(const wyo_problem* p, const int32_t* cu_seqlens, int64_t* chunk_start,
                        int32_t* chunk_len, int64_t cap);

/* Row-wise forward substitution ([Inv] section 2.1): X = L^{-1} for the n x n unit lower
 * triangular L (only the strict lower part of L is read; its diagonal is taken as 1).
 * Returns the number of necessary multiply-adds: products L[k,j] * X[j,i] with i < j < k. */
int64_t wyo_row_forward_inverse(int32_t n, const double* L, int32_t ldl, double* X,
                                int32_t ldx);

/* Independent second algorithm, used only to pin the 2x2 block identity ([Inv] section 2.2):
 * X = L^{-1} by halving recursion down to blocks of at most `base` rows, each solved by
 * wyo_row_forward_inverse, coupled by X10 = -X11 L10 X00 (two dense products).
 * Returns the multiply-add count (dense products counted in full); *depth receives the
 * dependency depth in steps: n-1 for a leaf, +2 per recursion level. */
int64_t wyo_block_recursive_inverse(int32_t n, int32_t base, const double* L, int32_t ldl,
                                    double* X, int32_t ldx, int32_t* depth);

/* Whole-tensor oracle.  T_out [B,T,Hv,C], W_out [B,T,Hv,dk], U_out [B,T,Hv,dv] (fp64).
 * v / W_out / U_out may be NULL together (T only); g may be NULL (no gates).  nthreads <= 0
 * means 1.  *fma_out (may be NULL) receives the summed forward-substitution count.
 * Returns 0 on success, nonzero on invalid arguments. */
int32_t wyo_wy_prepare(const wyo_problem* p, const void* k, const void* v, const float* g,
                       const float* beta, const int32_t* cu_seqlens, double* T_out,
                       double* W_out, double* U_out, int32_t nthreads, int64_t* fma_out);

/* A single right-hand side, T never formed ([Inv] section 5, item 10: when T would be used only
 * once, apply the forward substitution straight to the right-hand side instead of materialising
 * it).  For every chunk and value head h: X = A^{-1} diag(beta) R, where R holds the chunk's rows
 * of rhs for value head h and A is wyo_wy_prepare's (gates included), by row-wise forward
 * substitution on the right-hand side: X[i,:] = beta_i R[i,:] - sum_{j<i} A[i,j] X[j,:].  With
 * rhs = v, X is U.  rhs [B,T,Hv,dv] (kv_dtype), X_out [B,T,Hv,dv] (fp64).  Returns 0 on success. */
int32_t wyo_solve_rhs(const wyo_problem* p, const void* k, const void* rhs, const float* g,
                      const float* beta, const int32_t* cu_seqlens, double* X_out,
                      int32_t nthreads);

/* Selected units only: unit u is the chunk starting at flattened token chunk_start[u] with
 * chunk_len[u] tokens, for value head v_head[u].  Outputs are compact and zero-padded:
 * T_out [M,C,C], W_out [M,C,dk], U_out [M,C,dv] (W_out / U_out may be NULL with v).
 * Returns 0 on success. */
int32_t wyo_units(const wyo_problem* p, const void* k, const void* v, const float* g,
                  const float* beta, int64_t num_units, const int64_t* chunk_start,
                  const int32_t* chunk_len,
                  const int32_t* v_head, double* T_out, double* W_out, double* U_out,
                  int32_t nthreads);

/* The gated delta rule itself, token by token -- the recurrence whose chunk form the WY / UT
 * preparation serves ([Inv] section 1: the chunk's C Householder transforms; [QLA] gate section:
 * the GDN recurrence with alpha_i in (0, 1), whose formula did not survive extraction; [QLA]
 * usage: o, final_state = chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state, ...)
 * with initial_state [B, Hv, K, V]).  Per sequence and value head h (key / query head
 * h / (Hv/Hq)), with S the dk x dv state:
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   alpha_t = exp(g_t)
 *     o_t = scale * S_t^T q_t                      (read after token t's own write)
 * S_{-1} = h0[seq][h] (zeros when h0 is NULL).  q, k [B,T,Hq,dk]; v [B,T,Hv,dv]; g, beta
 * [B,T,Hv]; h0, hT_out [N,Hv,dk,dv] with N = num_seqs (cu_seqlens) or B; o_out [B,T,Hv,dv].
 * Outputs fp64.  pair_mask [N*Hv] (may be NULL = all): only pairs (seq, head) with a nonzero
 * byte are computed; the rest of o_out / hT_out is left untouched.  Returns 0 on success. */
int32_t wyo_gdn_forward(const wyo_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* h0, double scale,
                        const int32_t* cu_seqlens, double* o_out, double* hT_out,
                        const uint8_t* pair_mask, int32_t nthreads);

/* Backward of the preparation step: the gradient of
 *     L = <dT, T> + <dW, W> + <dU, U>
 * (sums over every chunk and value head) with respect to k, v, beta and g, for upstream
 * gradients dT [B,T,Hv,C] (float32, may be NULL = 0; only its entries left of the diagonal of
 * each chunk matter), dW [B,T,Hv,dk] and dU [B,T,Hv,dv] (kv_dtype).  T, W, U are the
 * functions of k, v, beta, g that wyo_wy_prepare computes; the oracle takes the derivative of
 * its steps in reverse order (chain rule, fp64 plain loops; see wyo_oracle.c).  Outputs (fp64):
 * dk [B,T,Hq,dk] (summed over the value heads that read each key head), dv [B,T,Hv,dv],
 * dbeta [B,T,Hv], dg [B,T,Hv] (written only when g is given; may then be NULL).
 * Returns 0 on success. */
int32_t wyo_wy_backward(const wyo_problem* p, const void* k, const void* v, const float* g,
                        const float* beta, const int32_t* cu_seqlens, const float* dT,
                        const void* dW, const void* dU, double* dk_out, double* dv_out,
                        double* dbeta_out, double* dg_out, int32_t nthreads);

#ifdef __cplusplus
}
#endif

#endif /* WYO_ORACLE_H */
