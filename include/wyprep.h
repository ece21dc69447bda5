/*
 * wyprep.h -- C ABI of the MI355X (gfx950) per-chunk WY/UT preparation of chunkwise
 * (Gated) DeltaNet.
 *
 * Pages cited (by title and section):
 *   [Inv]  "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
 *          lower-triangular matrix).
 *   [QLA]  The FlashQLA announcement (FlashQLA: a TileLang GDN chunked-prefill operator
 *          library), section "使用方式" (usage).
 *
 * For every chunk of C tokens of every sequence and every value head h the library computes
 * ([Inv] section 1, the coefficient-matrix equation and the W / U equations):
 *     A = I + strictLower(diag(beta) K K^T)       (beta scales rows; diagonal 1, [Inv] 3.2)
 *     T = A^{-1}                                  (block recursion of [Inv] section 2.2:
 *                                                  independent 16x16 forward substitutions,
 *                                                  then the coupling -X11 L10 X00 per level)
 *     W = T diag(beta) K,   U = T diag(beta) V
 * K is the chunk's keys of key head h / (Hv/Hq), V its values of value head h.
 *
 * Gates (optional; g == NULL means alpha = 1 everywhere and gives exactly the lines above).
 * [Inv] section 5, item 12 states the gated coefficient diag(beta)(Gamma o K K^T); [QLA]
 * usage passes g [B,T,Hv] beside beta.  g_t = log alpha_t is the per-token log decay of the
 * value head (finite; alpha_t in (0, 1] is the decaying regime the tolerances are stated for).
 * With G_i = g_0 + ... + g_i summed over the chunk's own tokens (restarting at every chunk)
 * and Gamma[i][j] = exp(G_i - G_j), the decay from token j to token i:
 *     A = I + strictLower(diag(beta) (Gamma o K K^T)),   T = A^{-1}
 *     W = T diag(beta exp(G)) K,   U = T diag(beta) V
 * These W and U are the ones the gated delta rule S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T)
 * + beta_t v_t k_t^T needs to advance a chunk in one step (the recurrence the FlashQLA page
 * recalls, with alpha_i in (0, 1)).
 *
 * Layouts (row-major, contiguous, token-major as in [QLA] usage):
 *   k      [B, T, Hq, dk]    dtype kv_dtype
 *   v      [B, T, Hv, dv]    dtype kv_dtype
 *   beta   [B, T, Hv]        float32
 *   g      [B, T, Hv]        float32 log gates, or NULL
 *   T_out  [B, T, Hv, C]     float32; row t holds row (t - chunk start) of its chunk's T with
 *                            chunk-relative columns; every entry right of the diagonal
 *                            (including columns >= n of a short chunk) is written as 0.0 and
 *                            the diagonal as 1.0.
 *   W_out  [B, T, Hv, dk]    dtype kv_dtype
 *   U_out  [B, T, Hv, dv]    dtype kv_dtype
 *   cu_seqlens  int32 [N+1] (device) or NULL.  With it, B must be 1, T is the total packed
 *               token count, and chunks restart at every sequence start ([QLA] usage lists
 *               cu_seqlens as the variable-length option).  The last chunk of a sequence may
 *               hold n < C tokens; it is solved as an n x n system (the same result as padding
 *               k with zero rows and beta = 0).
 *
 * Ownership: every tensor pointer is a DEVICE pointer owned by the caller.  The library
 * never allocates, frees or synchronises device memory, keeps no per-call state and needs no
 * workspace.  k, v, T_out, W_out and U_out must be 16-byte aligned; beta, g and cu_seqlens
 * 4-byte aligned.
 *
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * call returns without waiting for it.
 *
 * Errors: problems detectable on the host return WYP_ERR_INVALID_ARGUMENT or
 * WYP_ERR_UNSUPPORTED before any HIP call and launch nothing; a failed launch returns
 * WYP_ERR_HIP.  wyp_last_error() then describes the failure (per calling thread).  No C++
 * exception crosses this boundary.  A problem with T == 0 tokens is a no-op returning WYP_OK.
 * The device contents of cu_seqlens are trusted, not checked (that would need a
 * synchronisation): cu[0] = 0, non-decreasing, cu[N] = T.
 *
 * Supported: dk = dv = 128; C in {32, 64, 128}; kv_dtype WYP_BF16 (bf16 MFMA, fp32
 * accumulation) or WYP_F32 (fp32 MFMA throughout); Hv a multiple of Hq.  Anything else
 * returns WYP_ERR_UNSUPPORTED.
 */
#ifndef WYPREP_H
#define WYPREP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WYP_ABI_VERSION 8  /* 2: log gates g; 3: wyp_chunk_fwd; 4: wyp_wy_backward; 5: wyp_chunk_fwd_cp;
                              6: wyp_chunk_fwd_cp_noalloc; 7: wyp_solve_rhs; 8: cu_seqlens in the
                              split forward and its workspace query */

/* Bytes of the static device scratch behind wyp_chunk_fwd_cp_noalloc (one array per GPU). */
#define WYP_CP_SCRATCH_BYTES (32 * 1024 * 1024)

typedef enum {
    WYP_OK = 0,
    WYP_ERR_INVALID_ARGUMENT = 1,
    WYP_ERR_UNSUPPORTED = 2,
    WYP_ERR_HIP = 3
} wyp_status;

typedef enum { WYP_BF16 = 0, WYP_F32 = 1 } wyp_dtype;

/* Problem sizes.  The struct is read, never kept. */
typedef struct {
    int32_t batch;        /* B (must be 1 when cu_seqlens is given)                     */
    int32_t seqlen;       /* T per batch row; total packed tokens with cu_seqlens        */
    int32_t num_qk_heads; /* Hq: key heads                                               */
    int32_t num_v_heads;  /* Hv: value heads, a multiple of Hq                          */
    int32_t head_dim_k;   /* dk (128)                                                   */
    int32_t head_dim_v;   /* dv (128)                                                   */
    int32_t chunk_size;   /* C: 32, 64 or 128                                           */
    int32_t num_seqs;     /* N: number of packed sequences (only with cu_seqlens)        */
    int32_t kv_dtype;     /* wyp_dtype of k, v, W_out, U_out                             */
} wyp_problem;

/* Version of this ABI (WYP_ABI_VERSION of the build). */
int32_t wyp_abi_version(void);

/* Static text for a status code. */
const char* wyp_status_string(int32_t status);

/* Detail of the calling thread's last non-OK return ("" if none).  Valid until the thread's
 * next call into the library. */
const char* wyp_last_error(void);

/* kkt_solve ([Inv] section 3: takes only K and beta, produces only T): writes T_out for every
 * chunk and value head.  k [B,T,Hq,dk], g [B,T,Hv] or NULL, beta [B,T,Hv],
 * T_out [B,T,Hv,C]. */
wyp_status wyp_kkt_solve(const wyp_problem* problem, const void* k, const float* g,
                         const float* beta, const int32_t* cu_seqlens, float* T_out,
                         void* stream);

/* The full preparation step ([Inv] section 1: T is materialised because both W and U reuse
 * it): writes T_out, W_out = T diag(beta) K (T diag(beta exp(G)) K with gates) and
 * U_out = T diag(beta) V in one pass over K and V. */
wyp_status wyp_wy_prepare(const wyp_problem* problem, const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          float* T_out, void* W_out, void* U_out, void* stream);

/* W and U without T in HBM ([Inv] section 1: T exists to be reused for W and U; section 2.4:
 * writing T back costs C values per token, the standalone kernel's bottleneck): the same
 * W_out and U_out as wyp_wy_prepare, bit for bit, with T formed on chip and never written.
 * Arguments as in wyp_wy_prepare without T_out; saves 4 C bytes per token and value head. */
wyp_status wyp_wu_prepare(const wyp_problem* problem, const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          void* W_out, void* U_out, void* stream);

/* One right-hand side, T never formed ([Inv] section 5 (summary), item 10: whether to
 * materialise T depends on how often it is used; used once, the forward substitution is applied
 * straight to the right-hand side).  For every chunk and value head h:
 *     X = A^{-1} diag(beta) R        (A as above, gates included when g is given)
 * where R holds the chunk's rows of rhs for value head h.  With rhs = v, X is U of
 * wyp_wy_prepare (to rounding; a different order of operations).  Computed by block forward
 * substitution over the chunk's 16-row blocks, X_i = L_ii^{-1} (diag(beta_i) R_i -
 * sum_{j<i} A_ij X_j), with only the 16x16 diagonal blocks inverted on chip (fp32 throughout);
 * nothing of T is written or formed beyond those blocks.
 *   rhs    [B, T, Hv, dv]   kv_dtype (dv = 128)
 *   X_out  [B, T, Hv, dv]   kv_dtype
 *   k, g, beta, cu_seqlens, stream   as for wyp_wy_prepare
 * Alignment: k, rhs, X_out 16 bytes; beta, g, cu_seqlens 4 bytes.  rhs and X_out must not
 * overlap.  Supported as wyp_wy_prepare (C in {32, 64, 128}, bf16 or fp32). */
wyp_status wyp_solve_rhs(const wyp_problem* problem, const void* k, const void* rhs,
                         const float* g, const float* beta, const int32_t* cu_seqlens,
                         void* X_out, void* stream);

/* The chunked forward that consumes W and U ([QLA] "FLA GDN Chunked Prefill 面临的主要问题":
 * after the WY step the pipeline carries the state across chunks and forms the output; [QLA]
 * usage: o, final_state = chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
 * output_final_state, cu_seqlens)).  Per sequence and value head h (key / query head
 * h / (Hv/Hq)) it advances the dk x dv state S of the gated delta rule
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t
 * one chunk at a time: with G, Gamma as above and S the state at the chunk start,
 *     V' = U - W S,   O = scale (diag(exp(G)) Q S + (Gamma o tril(Q K^T)) V'),
 *     S <- exp(G_{C-1}) S + K^T diag(exp(G_{C-1} - G)) V'.
 * W and U must be what wyp_wy_prepare / wyp_wu_prepare returned for the same k, beta, g,
 * cu_seqlens and chunk size (g NULL there and here, or the same g in both).
 *   q, k             [B, T, Hq, dk]   kv_dtype
 *   w_in, u_in       [B, T, Hv, dk] / [B, T, Hv, dv]   kv_dtype
 *   g                [B, T, Hv] float32 log gates, or NULL
 *   initial_state    [N, Hv, dk, dv] float32 (row dk, column dv), or NULL for zeros;
 *                    N = num_seqs with cu_seqlens, else B
 *   scale            finite float multiplying every output (dk^-1/2 is the usual choice)
 *   o_out            [B, T, Hv, dv]   kv_dtype
 *   final_state      [N, Hv, dk, dv] float32, or NULL (not written)
 * The state stays fp32 on chip for the whole sequence; its products with W and Q take it
 * rounded to bf16.  Work is split over (sequence, value head, 32- or 64-column slice of dv).
 * chunk_size is the C that W and U were prepared with.
 * Supported: kv_dtype WYP_BF16, chunk_size 32, 64 or 128, dk = dv = 128 (else
 * WYP_ERR_UNSUPPORTED).
 * q, k, w_in, u_in and o_out must be 16-byte aligned; g, the states 4-byte aligned.
 * initial_state and final_state may be the same buffer (an in-place state update): each
 * workgroup reads its own slice of the initial state first and writes only that slice last. */
wyp_status wyp_chunk_fwd(const wyp_problem* problem, const void* q, const void* k,
                         const void* w_in, const void* u_in, const float* g,
                         const float* initial_state, float scale, const int32_t* cu_seqlens,
                         void* o_out, float* final_state, void* stream);

/* The same forward, split along the sequence ([QLA] "兼顾访存开销与序列并行的解法": the state
 * recurrence's kernel has only batch x heads thread blocks; the pages split each sequence and
 * repair the split with a per-segment correction).  The state after a segment of
 * `segment_chunks` chunks is linear in the state before it, S_end = M S_start + A, so the library
 * runs three passes on `stream`: (1) every segment's A (from a zero state) and transition M (the
 * same recurrence with U = 0, from the identity), in parallel; (2) S_start of each segment from
 * the previous one, S_start(s+1) = M_s S_start(s) + A_s, in fp32; (3) wyp_chunk_fwd's work per
 * segment from its S_start, writing o (and the final state from the last segment).  Exact up
 * to rounding (not the pages' gate-decay warm-up approximation).  Pass 2 copies the initial
 * state into the workspace and pass 3 reads it only there, so initial_state and final_state
 * may be the same buffer, as for wyp_chunk_fwd.
 * Arguments as for wyp_chunk_fwd, cu_seqlens included, plus:
 *   segment_chunks   chunks per segment, >= 1.  Segments start at a sequence's first chunk, so a
 *                    sequence of n tokens has ceil(n / (C segment_chunks)) of them (one if it
 *                    is shorter, or empty; such a sequence runs as in wyp_chunk_fwd).  When no
 *                    sequence can have two (batch rows: segment_chunks covers ceil(T / C)
 *                    chunks; packed: C segment_chunks > T), the call is wyp_chunk_fwd itself
 *                    and needs no workspace.
 *   workspace        caller-owned device memory of at least
 *                    wyp_chunk_fwd_cp_workspace_bytes(problem, cu_seqlens, segment_chunks) bytes,
 *                    16-byte aligned; its contents on entry do not matter and on return are
 *                    unspecified.  Calls that share a workspace must not overlap.
 * Supported as wyp_chunk_fwd (bf16, C = 32, 64 or 128, dk = dv = 128). */
wyp_status wyp_chunk_fwd_cp(const wyp_problem* problem, const void* q, const void* k,
                            const void* w_in, const void* u_in, const float* g,
                            const float* initial_state, float scale, const int32_t* cu_seqlens,
                            int32_t segment_chunks, void* workspace, int64_t workspace_bytes,
                            void* o_out, float* final_state, void* stream);

/* Workspace bytes wyp_chunk_fwd_cp needs, with X = C segment_chunks tokens per segment:
 *   batch rows (cu_seqlens NULL): B x Hv x (2 nseg - 1) x dk x dk x 4, nseg = ceil(T / X) (A
 *     and M of every segment but a row's last, and a copy of the initial state); 0 if nseg = 1;
 *   packed (cu_seqlens non-NULL; only whether it is NULL matters, it is not read):
 *     (2 floor(T / X) + N) x Hv x dk x dk x 4, with T the total tokens and N = num_seqs (no
 *     length mix needs more: a sequence's segments after its first number at most its tokens
 *     / X); 0 if T < X.
 * -1 for invalid arguments (segment_chunks < 1, chunk_size other than 32, 64 or 128, NULL
 * problem, batch other than 1 with cu_seqlens). */
int64_t wyp_chunk_fwd_cp_workspace_bytes(const wyp_problem* problem, const int32_t* cu_seqlens,
                                         int32_t segment_chunks);

/* wyp_chunk_fwd_cp for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same passes, results and
 * arguments, without workspace / workspace_bytes.  The workspace is instead a static device array
 * of WYP_CP_SCRATCH_BYTES (32 MiB) inside the library; each GPU the library runs on holds its own
 * copy until the process ends.  The call allocates and frees nothing (no hipMalloc, hipFree or
 * allocating library routine); on its first call on a device it looks up that device's address
 * of the array once.
 *   Limit: wyp_chunk_fwd_cp_workspace_bytes(problem, cu_seqlens, segment_chunks) must not exceed
 *   WYP_CP_SCRATCH_BYTES, else WYP_ERR_UNSUPPORTED (checked on the host, nothing launched).
 *   B = 1, T = 8192, Hv = 16 in 8 segments needs 15 MiB.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different
 *   streams or from different threads without ordering) race and must not be made; calls on one
 *   stream are ordered.  Each call writes every part of the array it reads before reading it,
 *   so nothing has to start at zero and no call sees an earlier call's contents. */
wyp_status wyp_chunk_fwd_cp_noalloc(const wyp_problem* problem, const void* q, const void* k,
                                    const void* w_in, const void* u_in, const float* g,
                                    const float* initial_state, float scale,
                                    const int32_t* cu_seqlens, int32_t segment_chunks,
                                    void* o_out, float* final_state, void* stream);

/* Backward of the preparation step (the training path; [QLA] "反向" (backward): FlashQLA fuses
 * bwd_wy with the other backward kernels).  For upstream gradients dT, dW, dU of wyp_wy_prepare's
 * outputs it returns the gradient of  L = <dT, T> + <dW, W> + <dU, U>  with respect to k, v,
 * beta and g.  With D = diag(beta), E = diag(exp(G)), H = Gamma o K K^T (strict lower part):
 *     X  = strictLower(dT + (dW K^T) D E + (dU V^T) D),   M = strictLower(-T^T X T^T)
 *     dk = D E T^T dW + (R + R^T) K   with R = D (Gamma o M)   (summed over the value heads
 *                                                               that read each key head)
 *     dv = D T^T dU
 *     dbeta_i = sum_d [ (T^T dW)_id e^{G_i} K_id + (T^T dU)_id V_id ] + sum_j M_ij H_ij
 *     dG_i = beta_i e^{G_i} sum_d (T^T dW)_id K_id + sum_j (Z_ij - Z_ji),  Z = M o D H
 *     dg_t = sum of dG_i over the chunk's tokens i >= t.
 * T is recomputed on chip by the same steps as wyp_wy_prepare.
 *   k, v, g, beta, cu_seqlens   as for wyp_wy_prepare (the forward's inputs)
 *   dT      [B, T, Hv, C] float32, or NULL (zero); entries on or right of each chunk's
 *           diagonal are ignored (T is constant there)
 *   dW, dU  [B, T, Hv, dk] / [B, T, Hv, dv]   kv_dtype
 *   dk_out  [B, T, Hq, dk], dv_out [B, T, Hv, dv]   kv_dtype
 *   dbeta_out [B, T, Hv] float32;  dg_out [B, T, Hv] float32, required when g is given (else
 *           ignored)
 * Supported: kv_dtype WYP_BF16, chunk_size 32, 64 or 128, dk = dv = 128 (else
 * WYP_ERR_UNSUPPORTED).  Alignment: k, v, dW, dU, dk_out, dv_out 16 bytes; beta, g, dT, dbeta_out, dg_out 4
 * bytes.  Results are deterministic (fixed reduction order, no atomics). */
wyp_status wyp_wy_backward(const wyp_problem* problem, const void* k, const void* v,
                           const float* g, const float* beta, const int32_t* cu_seqlens,
                           const float* dT, const void* dW, const void* dU, void* dk_out,
                           void* dv_out, float* dbeta_out, float* dg_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WYPREP_H */
