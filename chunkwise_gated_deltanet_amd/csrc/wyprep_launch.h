// Internal interface between the C-ABI front end (wyprep_api.cpp) and the HIP kernels
// (wyprep_kernels.hip: preparation; chunk_fwd.hip: chunked forward; wy_backward.hip: backward).
// Not installed; the public boundary is include/wyprep.h.
#pragma once

#include <cstdint>

namespace wyp {

// Validated problem, ready to launch.
struct LaunchArgs {
    const void* k;
    const void* v;            // nullptr for kkt_solve
    const float* beta;
    const float* g;           // nullptr: no gates
    const int32_t* cu_seqlens;  // nullptr: B x T layout
    float* T;                 // nullptr for wu_prepare
    void* W;                  // nullptr for kkt_solve
    void* U;
    int32_t batch;
    int32_t seqlen;
    int32_t num_qk_heads;
    int32_t num_v_heads;
    int32_t num_seqs;
    int32_t chunk_size;
    int32_t kv_dtype;         // 0 bf16, 1 f32
    int64_t chunk_slots;      // chunks (B x T) or an upper bound on them (packed)
    int32_t solve;            // 1: single right-hand side (v holds R, U receives X)
};

// Enqueues the kernel on `stream`.  Returns 0 or the hipError_t value; fills `msg` on error.
int launch(const LaunchArgs& a, void* stream, char* msg, int msg_len);

// Validated chunked forward (state recurrence and output), ready to launch.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* w;
    const void* u;
    const float* g;            // nullptr: no gates
    const float* h0;           // nullptr: zero initial state
    const int32_t* cu_seqlens;
    void* o;
    float* hT;                 // nullptr: final state not written
    float scale;
    int32_t seqlen;
    int32_t num_qk_heads;
    int32_t num_v_heads;
    int32_t num_seqs;          // sequences (cu_seqlens) or batch rows
    int32_t chunk_size;        // C: 32, 64 or 128
    int32_t split;             // 1: the sequence-parallel form (the fields below)
    int32_t nseg;              // batch rows: segments per row
    int32_t seg_chunks;        // chunks per segment
    int32_t a_slots;           // batch rows: B nseg; packed: floor(T / (C seg_chunks)) + N
    int32_t m_slots;           // batch rows: B (nseg - 1); packed: floor(T / (C seg_chunks))
    float* ws;                 // (a_slots + m_slots) x Hv x dk x dk floats
};

int launch_fwd(const FwdArgs& a, void* stream, char* msg, int msg_len);

// Device address of the split forward's static scratch (WYP_CP_SCRATCH_BYTES) on the current
// device.  Returns 0 or the hipError_t value; fills `msg` on error.
int cp_scratch(void** ptr, char* msg, int msg_len);

// Validated backward of the preparation step, ready to launch.
struct BwdArgs {
    const void* k;
    const void* v;
    const float* beta;
    const float* g;            // nullptr: no gates (dg not written)
    const int32_t* cu_seqlens;
    const float* dT;           // nullptr: dT = 0
    const void* dW;
    const void* dU;
    void* dk;
    void* dv;
    float* dbeta;
    float* dg;
    int32_t seqlen;
    int32_t num_qk_heads;
    int32_t num_v_heads;
    int32_t num_seqs;
    int32_t chunk_size;        // C: 32, 64 or 128
    int64_t chunk_slots;
};

int launch_bwd(const BwdArgs& a, void* stream, char* msg, int msg_len);

}  // namespace wyp
