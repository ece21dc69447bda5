// C-ABI front end of libwyprep: argument validation (before any HIP call), status codes and
// the per-thread error text.  The arithmetic lives in the HIP sources (wyprep_kernels.hip,
// chunk_fwd.hip, wy_backward.hip).
#include "wyprep.h"
#include "wyprep_launch.h"

#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

namespace {

thread_local char g_last_error[512] = "";

wyp_status fail(wyp_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host-side checks shared by the entry points.  Touches no HIP API.
wyp_status validate(const wyp_problem* p, const void* k, const void* v, const float* g,
                    const float* beta, const int32_t* cu, const float* T, const void* W,
                    const void* U, bool want_t, bool want_wu, wyp::LaunchArgs* out, bool* empty)
{
    *empty = false;
    if (!p) return fail(WYP_ERR_INVALID_ARGUMENT, "problem is NULL");
    if (p->batch < 1) return fail(WYP_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
    if (p->seqlen < 0) return fail(WYP_ERR_INVALID_ARGUMENT, "seqlen must be >= 0 (got %d)", p->seqlen);
    if (p->num_qk_heads < 1 || p->num_v_heads < 1)
        return fail(WYP_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hv=%d)",
                    p->num_qk_heads, p->num_v_heads);
    if (p->num_v_heads % p->num_qk_heads != 0)
        return fail(WYP_ERR_INVALID_ARGUMENT, "Hv (%d) must be a multiple of Hq (%d)",
                    p->num_v_heads, p->num_qk_heads);
    if (p->kv_dtype != WYP_BF16 && p->kv_dtype != WYP_F32)
        return fail(WYP_ERR_INVALID_ARGUMENT, "kv_dtype %d is not a wyp_dtype", p->kv_dtype);
    if (p->head_dim_k != 128 || (want_wu && p->head_dim_v != 128))
        return fail(WYP_ERR_UNSUPPORTED, "only head_dim_k = head_dim_v = 128 is built (got %d, %d)",
                    p->head_dim_k, p->head_dim_v);
    if (p->chunk_size != 32 && p->chunk_size != 64 && p->chunk_size != 128)
        return fail(WYP_ERR_UNSUPPORTED, "chunk_size must be 32, 64 or 128 (got %d)",
                    p->chunk_size);
    if (cu) {
        if (p->batch != 1)
            return fail(WYP_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1 (got %d)", p->batch);
        if (p->num_seqs < 0)
            return fail(WYP_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", p->num_seqs);
        if (p->num_seqs == 0 && p->seqlen != 0)
            return fail(WYP_ERR_INVALID_ARGUMENT, "num_seqs == 0 with %d tokens", p->seqlen);
        if (!aligned(cu, 4)) return fail(WYP_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    }
    const int64_t C = p->chunk_size;
    const int64_t tokens = static_cast<int64_t>(p->batch) * p->seqlen;
    if (tokens == 0) {  // nothing to read or write; pointers of empty tensors may be NULL
        *empty = true;
        return WYP_OK;
    }
    if (!k || !beta) return fail(WYP_ERR_INVALID_ARGUMENT, "k and beta must be non-NULL");
    if (want_t && !T) return fail(WYP_ERR_INVALID_ARGUMENT, "T_out must be non-NULL");
    if (want_wu && (!v || !W || !U))
        return fail(WYP_ERR_INVALID_ARGUMENT, "v (rhs), W_out and U_out (X_out) must be non-NULL");
    if (!aligned(k, 16) || (want_t && !aligned(T, 16)) ||
        (want_wu && (!aligned(v, 16) || !aligned(W, 16) || !aligned(U, 16))))
        return fail(WYP_ERR_INVALID_ARGUMENT, "k, v, T_out, W_out and U_out must be 16-byte aligned");
    if (!aligned(beta, 4)) return fail(WYP_ERR_INVALID_ARGUMENT, "beta is not 4-byte aligned");
    if (g && !aligned(g, 4)) return fail(WYP_ERR_INVALID_ARGUMENT, "g is not 4-byte aligned");

    int64_t slots;
    // packed: sequence s owns slots [floor(cu[s] / C) + s, floor(cu[s + 1] / C) + s + 1), room for
    // its chunks and at most one empty slot (the kernels skip empty slots)
    if (cu) slots = p->seqlen / C + p->num_seqs;
    else slots = static_cast<int64_t>(p->batch) * ((p->seqlen + C - 1) / C);
    // the launch grid is slots x (Hv or Hq) workgroups, rounded up to a multiple of 8
    const int64_t units = slots * p->num_v_heads;
    if (units + 8 > INT32_MAX)
        return fail(WYP_ERR_UNSUPPORTED, "problem has %lld units, more than one launch holds",
                    static_cast<long long>(units));

    out->k = k;
    out->v = want_wu ? v : nullptr;
    out->beta = beta;
    out->g = g;
    out->cu_seqlens = cu;
    out->T = want_t ? const_cast<float*>(T) : nullptr;
    out->W = want_wu ? const_cast<void*>(W) : nullptr;
    out->U = want_wu ? const_cast<void*>(U) : nullptr;
    out->batch = p->batch;
    out->seqlen = p->seqlen;
    out->num_qk_heads = p->num_qk_heads;
    out->num_v_heads = p->num_v_heads;
    out->num_seqs = cu ? p->num_seqs : p->batch;
    out->chunk_size = p->chunk_size;
    out->kv_dtype = p->kv_dtype;
    out->chunk_slots = slots;
    return WYP_OK;
}

wyp_status run(const wyp_problem* p, const void* k, const void* v, const float* g,
               const float* beta, const int32_t* cu, float* T, void* W, void* U, bool want_t,
               bool want_wu, void* stream)
{
    g_last_error[0] = '\0';
    wyp::LaunchArgs args{};
    bool empty = false;
    const wyp_status st = validate(p, k, v, g, beta, cu, T, W, U, want_t, want_wu, &args, &empty);
    if (st != WYP_OK || empty) return st;
    char msg[256] = "";
    if (wyp::launch(args, stream, msg, sizeof msg) != 0)
        return fail(WYP_ERR_HIP, "kernel launch failed: %s", msg);
    return WYP_OK;
}

wyp_status validate_fwd(const wyp_problem* p, const void* q, const void* k, const void* w,
                        const void* u, const float* g, const float* h0, float scale,
                        const int32_t* cu, const void* o, const float* hT, wyp::FwdArgs* out,
                        bool* empty)
{
    *empty = false;
    if (!p) return fail(WYP_ERR_INVALID_ARGUMENT, "problem is NULL");
    if (p->batch < 1) return fail(WYP_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
    if (p->seqlen < 0) return fail(WYP_ERR_INVALID_ARGUMENT, "seqlen must be >= 0 (got %d)", p->seqlen);
    if (p->num_qk_heads < 1 || p->num_v_heads < 1)
        return fail(WYP_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hv=%d)",
                    p->num_qk_heads, p->num_v_heads);
    if (p->num_v_heads % p->num_qk_heads != 0)
        return fail(WYP_ERR_INVALID_ARGUMENT, "Hv (%d) must be a multiple of Hq (%d)",
                    p->num_v_heads, p->num_qk_heads);
    if (p->kv_dtype != WYP_BF16 && p->kv_dtype != WYP_F32)
        return fail(WYP_ERR_INVALID_ARGUMENT, "kv_dtype %d is not a wyp_dtype", p->kv_dtype);
    if (p->kv_dtype != WYP_BF16)
        return fail(WYP_ERR_UNSUPPORTED, "wyp_chunk_fwd is built for bf16 q, k, W, U only");
    if (p->head_dim_k != 128 || p->head_dim_v != 128)
        return fail(WYP_ERR_UNSUPPORTED, "only head_dim_k = head_dim_v = 128 is built (got %d, %d)",
                    p->head_dim_k, p->head_dim_v);
    if (p->chunk_size != 32 && p->chunk_size != 64 && p->chunk_size != 128)
        return fail(WYP_ERR_UNSUPPORTED, "wyp_chunk_fwd is built for chunk_size 32, 64 and 128 (got %d)",
                    p->chunk_size);
    if (!(scale == scale) || scale == 1.0f / 0.0f || scale == -1.0f / 0.0f)
        return fail(WYP_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (cu) {
        if (p->batch != 1)
            return fail(WYP_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1 (got %d)", p->batch);
        if (p->num_seqs < 0)
            return fail(WYP_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", p->num_seqs);
        if (p->num_seqs == 0 && p->seqlen != 0)
            return fail(WYP_ERR_INVALID_ARGUMENT, "num_seqs == 0 with %d tokens", p->seqlen);
        if (!aligned(cu, 4)) return fail(WYP_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    }
    const int64_t nseq = cu ? p->num_seqs : p->batch;
    const int64_t work = nseq * p->num_v_heads * 4;  // (sequence, value head, dv slice)
    // the grid rounds the (sequence, key head) groups up to a multiple of 8, each group
    // Hv / Hq value heads x up to 8 slices
    const int64_t pad = 64 * static_cast<int64_t>(p->num_v_heads / p->num_qk_heads);
    if (work + pad > INT32_MAX)
        return fail(WYP_ERR_UNSUPPORTED, "problem has %lld work items, more than one launch holds",
                    static_cast<long long>(work));
    const int64_t tokens = static_cast<int64_t>(p->batch) * p->seqlen;
    if (nseq == 0 || (tokens == 0 && !hT)) {  // nothing to read or write
        *empty = true;
        return WYP_OK;
    }
    if (tokens > 0 && (!q || !k || !w || !u || !o))
        return fail(WYP_ERR_INVALID_ARGUMENT, "q, k, W, U and o_out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 16) || !aligned(u, 16) || !aligned(o, 16))
        return fail(WYP_ERR_INVALID_ARGUMENT, "q, k, W, U and o_out must be 16-byte aligned");
    if ((g && !aligned(g, 4)) || (h0 && !aligned(h0, 4)) || (hT && !aligned(hT, 4)))
        return fail(WYP_ERR_INVALID_ARGUMENT, "g, initial_state and final_state must be 4-byte aligned");
    out->q = q;
    out->k = k;
    out->w = w;
    out->u = u;
    out->g = g;
    out->h0 = h0;
    out->cu_seqlens = cu;
    out->o = const_cast<void*>(o);
    out->hT = const_cast<float*>(hT);
    out->scale = scale;
    out->seqlen = p->seqlen;
    out->num_qk_heads = p->num_qk_heads;
    out->num_v_heads = p->num_v_heads;
    out->num_seqs = static_cast<int32_t>(nseq);
    out->chunk_size = p->chunk_size;
    return WYP_OK;
}

wyp_status validate_bwd(const wyp_problem* p, const void* k, const void* v, const float* g,
                        const float* beta, const int32_t* cu, const float* dT, const void* dW,
                        const void* dU, const void* dk, const void* dv, const float* dbeta,
                        const float* dg, wyp::BwdArgs* out, bool* empty)
{
    wyp::LaunchArgs la{};
    // the problem checks of the forward (with W, U standing for dW, dU)
    wyp_status st = validate(p, k, v, g, beta, cu, nullptr, dW, dU, false, true, &la, empty);
    if (st != WYP_OK || *empty) return st;
    if (p->kv_dtype != WYP_BF16)
        return fail(WYP_ERR_UNSUPPORTED, "wyp_wy_backward is built for bf16 k, v only");
    if (!dk || !dv || !dbeta) return fail(WYP_ERR_INVALID_ARGUMENT, "dk, dv and dbeta must be non-NULL");
    if (g && !dg) return fail(WYP_ERR_INVALID_ARGUMENT, "dg must be non-NULL when g is given");
    if (!aligned(dk, 16) || !aligned(dv, 16))
        return fail(WYP_ERR_INVALID_ARGUMENT, "dk and dv must be 16-byte aligned");
    if (!aligned(dbeta, 4) || (dg && !aligned(dg, 4)) || (dT && !aligned(dT, 4)))
        return fail(WYP_ERR_INVALID_ARGUMENT, "dT, dbeta and dg must be 4-byte aligned");
    const int64_t units = la.chunk_slots * p->num_qk_heads;
    if (units > INT32_MAX)
        return fail(WYP_ERR_UNSUPPORTED, "problem has %lld units, more than one launch holds",
                    static_cast<long long>(units));
    out->k = k;
    out->v = v;
    out->beta = beta;
    out->g = g;
    out->cu_seqlens = cu;
    out->dT = dT;
    out->dW = dW;
    out->dU = dU;
    out->dk = const_cast<void*>(dk);
    out->dv = const_cast<void*>(dv);
    out->dbeta = const_cast<float*>(dbeta);
    out->dg = g ? const_cast<float*>(dg) : nullptr;
    out->seqlen = p->seqlen;
    out->num_qk_heads = p->num_qk_heads;
    out->num_v_heads = p->num_v_heads;
    out->num_seqs = la.num_seqs;
    out->chunk_size = p->chunk_size;
    out->chunk_slots = la.chunk_slots;
    return WYP_OK;
}

}  // namespace

extern "C" {

int32_t wyp_abi_version(void) { return WYP_ABI_VERSION; }

const char* wyp_status_string(int32_t status)
{
    switch (status) {
    case WYP_OK: return "WYP_OK";
    case WYP_ERR_INVALID_ARGUMENT: return "WYP_ERR_INVALID_ARGUMENT";
    case WYP_ERR_UNSUPPORTED: return "WYP_ERR_UNSUPPORTED";
    case WYP_ERR_HIP: return "WYP_ERR_HIP";
    default: return "WYP_ERR_UNKNOWN";
    }
}

const char* wyp_last_error(void) { return g_last_error; }

wyp_status wyp_kkt_solve(const wyp_problem* problem, const void* k, const float* g,
                         const float* beta, const int32_t* cu_seqlens, float* T_out, void* stream)
{
    return run(problem, k, nullptr, g, beta, cu_seqlens, T_out, nullptr, nullptr, true, false,
               stream);
}

wyp_status wyp_wy_prepare(const wyp_problem* problem, const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          float* T_out, void* W_out, void* U_out, void* stream)
{
    return run(problem, k, v, g, beta, cu_seqlens, T_out, W_out, U_out, true, true, stream);
}

wyp_status wyp_wu_prepare(const wyp_problem* problem, const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          void* W_out, void* U_out, void* stream)
{
    return run(problem, k, v, g, beta, cu_seqlens, nullptr, W_out, U_out, false, true, stream);
}

wyp_status wyp_solve_rhs(const wyp_problem* problem, const void* k, const void* rhs,
                         const float* g, const float* beta, const int32_t* cu_seqlens,
                         void* X_out, void* stream)
{
    g_last_error[0] = '\0';
    wyp::LaunchArgs args{};
    bool empty = false;
    // the checks of wy_prepare's W / U path, with rhs in v's place and X_out in U's (and W's)
    const wyp_status st = validate(problem, k, rhs, g, beta, cu_seqlens, nullptr, X_out, X_out,
                                   false, true, &args, &empty);
    if (st != WYP_OK || empty) return st;
    args.W = nullptr;
    args.solve = 1;
    char msg[256] = "";
    if (wyp::launch(args, stream, msg, sizeof msg) != 0)
        return fail(WYP_ERR_HIP, "kernel launch failed: %s", msg);
    return WYP_OK;
}

}  // extern "C"

extern "C" wyp_status wyp_chunk_fwd(const wyp_problem* problem, const void* q, const void* k,
                                    const void* w, const void* u, const float* g,
                                    const float* initial_state, float scale,
                                    const int32_t* cu_seqlens, void* o_out, float* final_state,
                                    void* stream)
{
    g_last_error[0] = '\0';
    wyp::FwdArgs args{};
    bool empty = false;
    const wyp_status st = validate_fwd(problem, q, k, w, u, g, initial_state, scale, cu_seqlens,
                                       o_out, final_state, &args, &empty);
    if (st != WYP_OK || empty) return st;
    char msg[256] = "";
    if (wyp::launch_fwd(args, stream, msg, sizeof msg) != 0)
        return fail(WYP_ERR_HIP, "kernel launch failed: %s", msg);
    return WYP_OK;
}

extern "C" wyp_status wyp_wy_backward(const wyp_problem* problem, const void* k, const void* v,
                                      const float* g, const float* beta, const int32_t* cu_seqlens,
                                      const float* dT, const void* dW, const void* dU,
                                      void* dk_out, void* dv_out, float* dbeta_out, float* dg_out,
                                      void* stream)
{
    g_last_error[0] = '\0';
    wyp::BwdArgs args{};
    bool empty = false;
    const wyp_status st = validate_bwd(problem, k, v, g, beta, cu_seqlens, dT, dW, dU, dk_out,
                                       dv_out, dbeta_out, dg_out, &args, &empty);
    if (st != WYP_OK || empty) return st;
    char msg[256] = "";
    if (wyp::launch_bwd(args, stream, msg, sizeof msg) != 0)
        return fail(WYP_ERR_HIP, "kernel launch failed: %s", msg);
    return WYP_OK;
}

namespace {

// Slots of the split forward.  Batch rows: nseg = ceil(chunks / segment_chunks) segments per row,
// B nseg a-slots and B (nseg - 1) m-slots.  Packed sequences (segments aligned to each
// sequence's first chunk, X = C segment_chunks tokens each): floor(T / X) + N a-slots and
// floor(T / X) m-slots, enough for any length mix.  No m-slot means no split.
struct CpPlan {
    int64_t nseg, a_slots, m_slots;
};

bool cp_plan(const wyp_problem* p, bool packed, int32_t segment_chunks, CpPlan* out)
{
    if (!p || segment_chunks < 1 || p->seqlen < 0 || p->num_v_heads < 1) return false;
    if (p->chunk_size != 32 && p->chunk_size != 64 && p->chunk_size != 128) return false;
    const int64_t C = p->chunk_size;
    if (packed) {
        if (p->batch != 1 || p->num_seqs < 0) return false;
        const int64_t e = p->seqlen / (C * segment_chunks);
        out->nseg = 0;
        out->m_slots = e;
        out->a_slots = e > 0 ? e + p->num_seqs : 0;
    } else {
        if (p->batch < 1) return false;
        const int64_t nchunks = (static_cast<int64_t>(p->seqlen) + C - 1) / C;
        const int64_t nseg = nchunks == 0 ? 1 : (nchunks + segment_chunks - 1) / segment_chunks;
        out->nseg = nseg;
        out->m_slots = nseg > 1 ? p->batch * (nseg - 1) : 0;
        out->a_slots = nseg > 1 ? p->batch * nseg : 0;
    }
    return true;
}

// A and M of every segment but a sequence's last, plus its S_start(0): one dk x dv fp32 matrix per
// slot and value head.
int64_t cp_workspace(const wyp_problem* p, const CpPlan& plan)
{
    return (plan.a_slots + plan.m_slots) * p->num_v_heads * 128 * 128 * 4;
}

}  // namespace

extern "C" int64_t wyp_chunk_fwd_cp_workspace_bytes(const wyp_problem* problem, const int32_t* cu_seqlens,
                                                    int32_t segment_chunks)
{
    CpPlan plan;
    if (!cp_plan(problem, cu_seqlens != nullptr, segment_chunks, &plan)) return -1;
    return cp_workspace(problem, plan);
}

namespace {

// The split forward: `workspace` is the caller's (wyp_chunk_fwd_cp) or, when `use_scratch`, the
// library's static scratch (wyp_chunk_fwd_cp_noalloc, which allocates nothing).
wyp_status run_cp(const wyp_problem* problem, const void* q, const void* k, const void* w,
                  const void* u, const float* g, const float* initial_state, float scale,
                  const int32_t* cu_seqlens, int32_t segment_chunks, void* workspace,
                  int64_t workspace_bytes, bool use_scratch, void* o_out, float* final_state,
                  void* stream)
{
    g_last_error[0] = '\0';
    wyp::FwdArgs args{};
    bool empty = false;
    wyp_status st = validate_fwd(problem, q, k, w, u, g, initial_state, scale, cu_seqlens, o_out,
                                 final_state, &args, &empty);
    if (st != WYP_OK) return st;
    CpPlan plan;
    if (!cp_plan(problem, cu_seqlens != nullptr, segment_chunks, &plan))
        return fail(WYP_ERR_INVALID_ARGUMENT, "segment_chunks must be >= 1 (got %d)", segment_chunks);
    if (empty) return WYP_OK;
    char msg[256] = "";
    if (plan.m_slots > 0) {
        const int64_t need = cp_workspace(problem, plan);
        if (use_scratch) {
            if (need > WYP_CP_SCRATCH_BYTES)
                return fail(WYP_ERR_UNSUPPORTED,
                            "the split needs %lld bytes of workspace, more than the %lld-byte scratch "
                            "(use fewer segments or wyp_chunk_fwd_cp)",
                            static_cast<long long>(need), static_cast<long long>(WYP_CP_SCRATCH_BYTES));
        } else {
            if (!workspace || workspace_bytes < need)
                return fail(WYP_ERR_INVALID_ARGUMENT, "workspace of %lld bytes needed (%lld given)",
                            static_cast<long long>(need), static_cast<long long>(workspace_bytes));
            if (!aligned(workspace, 16))
                return fail(WYP_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
        }
        // the largest grid: the combine's or pass 1's 8 blocks per (slot, value head), rounded up
        if (plan.a_slots * problem->num_v_heads * 8 +
                64 * static_cast<int64_t>(problem->num_v_heads / problem->num_qk_heads) > INT32_MAX)
            return fail(WYP_ERR_UNSUPPORTED, "too many segments for one launch");
        if (use_scratch && wyp::cp_scratch(&workspace, msg, sizeof msg) != 0)
            return fail(WYP_ERR_HIP, "%s", msg);
        args.split = 1;
        args.nseg = static_cast<int32_t>(plan.nseg);
        args.seg_chunks = segment_chunks;
        args.a_slots = static_cast<int32_t>(plan.a_slots);
        args.m_slots = static_cast<int32_t>(plan.m_slots);
        args.ws = static_cast<float*>(workspace);
    }
    if (wyp::launch_fwd(args, stream, msg, sizeof msg) != 0)
        return fail(WYP_ERR_HIP, "kernel launch failed: %s", msg);
    return WYP_OK;
}

}  // namespace

extern "C" wyp_status wyp_chunk_fwd_cp(const wyp_problem* problem, const void* q, const void* k,
                                       const void* w, const void* u, const float* g,
                                       const float* initial_state, float scale,
                                       const int32_t* cu_seqlens, int32_t segment_chunks,
                                       void* workspace, int64_t workspace_bytes, void* o_out,
                                       float* final_state, void* stream)
{
    return run_cp(problem, q, k, w, u, g, initial_state, scale, cu_seqlens, segment_chunks,
                  workspace, workspace_bytes, false, o_out, final_state, stream);
}

extern "C" wyp_status wyp_chunk_fwd_cp_noalloc(const wyp_problem* problem, const void* q,
                                               const void* k, const void* w, const void* u,
                                               const float* g, const float* initial_state,
                                               float scale, const int32_t* cu_seqlens,
                                               int32_t segment_chunks, void* o_out,
                                               float* final_state, void* stream)
{
    return run_cp(problem, q, k, w, u, g, initial_state, scale, cu_seqlens, segment_chunks,
                  nullptr, 0, true, o_out, final_state, stream);
}
