// HIP kernel (gfx950 / CDNA4) for the chunked forward of gated DeltaNet that consumes the WY / UT
// preparation: per sequence and value head it carries the dk x dv state S from chunk to chunk
// and writes the output o.
//
// Pages cited (by title and section):
//   [Inv] "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
//         lower-triangular matrix), section 1: W and U are built so the chunk's C Householder
//         transforms act in one step; section 5, item 12: the gated coefficient.
//   [QLA] The FlashQLA announcement: "FLA GDN Chunked Prefill 面临的主要问题" (the state
//         recurrence's kernel is limited to batch x heads thread blocks; W, U go through HBM),
//         the gate section (the GDN recurrence with alpha_i in (0, 1)), and "使用方式" (usage:
//         o, final_state from q, k, v, g, beta, scale, initial_state [B, Hv, K, V]).
//
// The recurrence S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
// o_t = scale S_t^T q_t, advanced one chunk of C tokens at a time with W and U of that chunk
// (G_i = g_0 + ... + g_i within the chunk, Gamma[i][j] = exp(G_i - G_j), S the state at the
// chunk start):
//   V' = U - W S                                                  (C x dv)
//   O  = scale (diag(exp(G)) Q S + (Gamma o tril(Q K^T)) V')      (causal, diagonal included)
//   S <- exp(G_{C-1}) S + K^T diag(exp(G_{C-1} - G)) V'
// A workgroup owns one (sequence, value head, 32-column slice of dv): the three lines above
// split exactly along dv, so the four slices of a head run as independent workgroups (the
// pages' remedy for the batch x heads limit, "切分 v_head_dim").  The slices of one head sit on
// one XCD, so the Q, K and W rows they all read are served from that XCD's L2.
//
// Per chunk, wave w owns row tile w (16 tokens) of V' and O and dk row tiles 2w, 2w+1 of S:
//   1. V' tile = U - W S^T' (16x16x32 bf16 MFMA; S is read as a bf16 copy S^T kept in LDS);
//      V'^T and its decayed copy are written to LDS (bf16);
//      O tile = exp(G_row) Q S (same form);
//      P^T tiles = K Q^T for the tile's causal columns: the accumulator of P^T is exactly the A
//      operand of the 16x16x16 product P V' below, so P never goes through LDS;
//   2. O tile += (Gamma o P) V'; S tiles = exp(G_last) S + K^T V'_dec (K^T fragments by
//      ds_read_tr16_b64); the new bf16 S^T goes to LDS; O is staged and stored as 16-byte rows.
// The state stays fp32 in the MFMA accumulators for the whole sequence.  Every load of chunk
// c + 1 (K, U, g and this wave's Q and W rows) is issued right after chunk c's first barrier into a
// second register set; the two sets take turns.
//
// Sequence parallelism (wyp_chunk_fwd_cp; [QLA] "兼顾访存开销与序列并行的解法": the state
// kernel's thread blocks number only batch x heads, so the pages split each sequence and fix
// the split up with a correction computed per segment).  The state after a segment is linear in
// the state before it, S_end = M S_start + A, so with segments of L chunks:
//   pass 1 (LOCAL): per (segment but a sequence's last, head), A = the segment's end state from
//          a zero state and M = its transition (the same recurrence with U = 0 from the
//          identity), as twice the slices of a head; no output;
//   pass 2 (combine): S_start(0) = the initial state, copied into the workspace, and S_start of
//          segment s + 1 = M_s S_start(s) + A_s, in fp32, per sequence, head and 16-column slice;
//   pass 3: the kernel above per (segment, head) from its true S_start (for a sequence of two or
//          more segments always read from the workspace, so the initial state may be the
//          final-state buffer), writing o.
// Segments start at each sequence's first chunk, for batch rows and packed sequences alike.
// Exact, not the gate-decay warm-up approximation the pages also describe.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "wyprep.h"
#include "wyprep_launch.h"

// Workspace of wyp_chunk_fwd_cp_noalloc, for callers that cannot allocate: A, M and the
// initial-state copy of every segment, as wyp_chunk_fwd_cp keeps them in its caller's workspace.
// Each GPU holds its own copy of the array for the life of the process.  Host code never passes
// the array's name to a kernel (on the host it only stands in for the device object): it takes
// the device address from hipGetSymbolAddress (cp_scratch below).
static __device__ __align__(256) unsigned char scratch[WYP_CP_SCRATCH_BYTES];

namespace wyp {
namespace fwd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kD = 128;        // dk = dv
constexpr int kThreads = 512;  // the combine's workgroup: one wave per 16-row tile of the state
constexpr int kBufferConfig = 0x00020000;
// Non-temporal policy for what one workgroup alone reads or writes (its U slice, g, o).  Q, K
// and W keep the default policy: the four dv-slice workgroups of a head each read them, and
// the later readers hit the XCD's L2 (with nt W loads the packed Hq=16 Hv=64 workload moved
// 1.71x its algorithmic bytes).
constexpr int kStream = 2;

struct Params {
    const __bf16* q;
    const __bf16* k;
    const __bf16* w;
    const __bf16* u;
    const float* g;
    const float* h0;
    const int32_t* cu;
    __bf16* o;
    float* hT;
    float scale;
    int32_t seqlen;
    int32_t hq;
    int32_t hv;
    int32_t num_seqs;    // sequences (cu_seqlens) or batch rows
    int32_t work;        // work items of this launch: slots x value heads x slices
    int32_t split;       // 1: the sequence-parallel form
    int32_t nseg;        // split batch rows: segments per row
    int32_t seg_chunks;  // split: chunks per segment
    int32_t seg_tokens;  // split: seg_chunks x C tokens per segment
    float* ws_a;         // [a-slot][Hv][dk][dv]: a sequence's first a-slot S_start(0) (pass 2),
                         // a-slot s + 1 A_s (pass 1), then S_start(s + 1) (pass 2)
    float* ws_m;         // [m-slot][Hv][dk][dk]: M_s
};

constexpr int QROW = kD + 8;          // bf16 per K row
constexpr int SROW = kD + 8;          // bf16 per S^T row (one dv column of S)

// A chunk of C tokens is C / 16 row tiles, one per wave: C / 16 waves of 64 threads.  The state's
// 8 dk row tiles are shared out over the waves, 128 / C each.
template <int C>
struct Geo {
    static constexpr int NB = C / 16;        // row tiles per chunk (one per wave)
    static constexpr int THREADS = 4 * C;    // NB waves
    static constexpr int MT = kD / 16 / NB;  // dk row tiles of the state per wave
    static constexpr int NG = C > 64 ? 2 : 1;  // gates per lane of wave 0
    static constexpr int VROW = C + 8;       // bf16 per V'^T row (one dv column of V')
};

// A workgroup owns DVS of its head's dv columns (a slice: 32 or 64).  LDS plan (bytes): only what
// several waves read goes through LDS: K (rows padded by 16 bytes, row stride 272 B, so 16-byte
// reads of one column chunk by 16 consecutive rows spread over the banks), the U slice, the staged
// O slice, the bf16 S^T and V'^T tiles (padded the same way) and G.  Q and W rows of row tile w
// are read by wave w alone, so they go from HBM straight into its MFMA operand registers: this
// halves the LDS traffic of a chunk step.  45.8 KB at DVS = 32 (three workgroups per CU by LDS;
// registers allow three ungated, two gated), 71.8 KB at DVS = 64 (two).
template <int C, int DVS>
struct Slice {
    static constexpr int VROW = Geo<C>::VROW;
    static constexpr int NT = DVS / 16;        // 16-column tiles of the slice
    static constexpr int COUNT = kD / DVS;     // slices per head
    static constexpr int PIECES = DVS / 32;    // 16-byte pieces of the U / O slice per thread
    static constexpr int RPC = DVS / 8;        // 16-byte pieces per row of the slice
    static constexpr int UROW = DVS + 8;       // bf16 per U / O slice row
    static constexpr int OFF_K = 0;
    static constexpr int OFF_U = OFF_K + C * QROW * 2;
    static constexpr int OFF_O = OFF_U + C * UROW * 2;
    static constexpr int OFF_S = OFF_O + C * UROW * 2;
    static constexpr int OFF_VN = OFF_S + DVS * SROW * 2;
    static constexpr int OFF_VD = OFF_VN + DVS * VROW * 2;
    static constexpr int OFF_G = OFF_VD + DVS * VROW * 2;
    static constexpr int LDS_TOTAL = OFF_G + C * 4;
    static_assert(C * RPC == PIECES * Geo<C>::THREADS, "the U / O slice splits evenly over the threads");
    static_assert(LDS_TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
};
static_assert(3 * Slice<64, 32>::LDS_TOTAL <= 160 * 1024, "C = 64: three workgroups per CU by LDS");
static_assert(2 * Slice<64, 64>::LDS_TOTAL <= 160 * 1024, "C = 64: two workgroups per CU by LDS");

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferConfig);
}

// Bytes spanned by rows [0, n) of a row-strided tensor (row stride `stride` bytes, `width` bytes
// read per row); 0 for n <= 0, which puts every access out of range (loads read 0), so loads can
// be issued without branches.
__device__ inline uint32_t row_bytes(int n, uint32_t stride, uint32_t width)
{
    return n > 0 ? static_cast<uint32_t>(n - 1) * stride + width : 0u;
}

// One chunk's data in flight to registers: K (C rows x 256 B: four 16-byte pieces per thread),
// the U slice (C rows x 2 DVS B: DVS / 32 pieces per thread), g (wave 0, one or two per lane), and
// for wave w its own Q and W rows 16 w .. 16 w + 15 as 16x16x32 MFMA operands: lane 16 lg + lr
// holds elements 32 s + 8 lg .. + 7 of row 16 w + lr, s = 0..3.  Rows past the chunk's n tokens
// read as 0 through the buffer range.
template <int C, int DVS>
struct Chunk {
    using F = Slice<C, DVS>;
    static constexpr int THREADS = Geo<C>::THREADS;
    static constexpr int NG = Geo<C>::NG;
    u32x4 q[4], k[4], w[4];
    u32x4 u[F::PIECES];
    float g[NG];

    // This wave's Q and W operands.
    __device__ void issue_qw(const Params& p, int64_t tok0, int n, int hk, int hv, int tid, bool want_q)
    {
        const uint32_t qstride = static_cast<uint32_t>(p.hq) * kD * 2;
        const uint32_t wstride = static_cast<uint32_t>(p.hv) * kD * 2;
        const __amdgpu_buffer_rsrc_t qr = rsrc(p.q + (tok0 * p.hq + hk) * kD, row_bytes(n, qstride, kD * 2));
        const __amdgpu_buffer_rsrc_t wr = rsrc(p.w + (tok0 * p.hv + hv) * kD, row_bytes(n, wstride, kD * 2));
        const int lane = tid & 63, row = 16 * (tid >> 6) + (lane & 15), lg = lane >> 4;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const uint32_t col = (32 * it + 8 * lg) * 2;
            q[it] = want_q ? __builtin_amdgcn_raw_buffer_load_b128(qr, row * qstride + col, 0, 0)
                           : u32x4{0u, 0u, 0u, 0u};
            w[it] = __builtin_amdgcn_raw_buffer_load_b128(wr, row * wstride + col, 0, 0);
        }
    }

    // K, U, g, then Q and W: every load of one chunk, without branches (n = 0: nothing is read).
    template <bool GT>
    __device__ void issue(const Params& p, int64_t tok0, int n, int hk, int hv, int slice, int tid,
                          bool want_q, bool want_u)
    {
        const uint32_t qstride = static_cast<uint32_t>(p.hq) * kD * 2;
        const uint32_t wstride = static_cast<uint32_t>(p.hv) * kD * 2;
        const __amdgpu_buffer_rsrc_t kr = rsrc(p.k + (tok0 * p.hq + hk) * kD, row_bytes(n, qstride, kD * 2));
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int pc = tid + it * THREADS;  // row pc / 16, piece pc % 16
            k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, (pc >> 4) * qstride + (pc & 15) * 16, 0, 0);
        }
        // the transition slices of the sequence-parallel pass read no U: an empty range
        const __amdgpu_buffer_rsrc_t ur = rsrc(p.u + (tok0 * p.hv + hv) * kD + slice * DVS,
                                               want_u ? row_bytes(n, wstride, DVS * 2) : 0u);
#pragma unroll
        for (int it = 0; it < F::PIECES; ++it) {
            const int pc = tid + it * THREADS;  // row pc / RPC, piece pc % RPC
            u[it] = __builtin_amdgcn_raw_buffer_load_b128(ur, (pc / F::RPC) * wstride + (pc % F::RPC) * 16, 0, kStream);
        }
#pragma unroll
        for (int i = 0; i < NG; ++i) g[i] = 0.f;
        if constexpr (GT) {
            // wave 0 only (the other waves get an empty range): lane l takes rows l and 64 + l;
            // rows >= n read as 0
            const __amdgpu_buffer_rsrc_t gr =
                rsrc(p.g + tok0 * p.hv + hv, tid < 64 ? row_bytes(n, p.hv * 4, 4) : 0u);
#pragma unroll
            for (int i = 0; i < NG; ++i)
                g[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                    gr, (64 * i + (tid & 63)) * p.hv * 4, 0, kStream));
        }
        issue_qw(p, tok0, n, hk, hv, tid, want_q);
    }

    // K and U to LDS; wave 0 turns g into the chunk-local inclusive prefix sums G (fp64 shuffle
    // scan, 64 rows at a time, stored as fp32).  Q and W stay in registers.
    template <bool GT>
    __device__ void commit(unsigned char* smem, int tid) const
    {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int pc = tid + it * THREADS;
            *reinterpret_cast<u32x4*>(smem + F::OFF_K + (pc >> 4) * (QROW * 2) + (pc & 15) * 16) = k[it];
        }
#pragma unroll
        for (int it = 0; it < F::PIECES; ++it) {
            const int pc = tid + it * THREADS;
            *reinterpret_cast<u32x4*>(smem + F::OFF_U + (pc / F::RPC) * (F::UROW * 2) + (pc % F::RPC) * 16) = u[it];
        }
        if constexpr (GT) {
            if (tid < 64) {
                double carry = 0.0;  // the sum over the rows of the lanes' earlier blocks
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    double x = static_cast<double>(g[i]);
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const double t = __shfl_up(x, d);
                        if (tid >= d) x += t;
                    }
                    x += carry;
                    reinterpret_cast<float*>(smem + F::OFF_G)[64 * i + tid] = static_cast<float>(x);
                    carry = __shfl(x, 63);
                }
            }
        }
    }
};

// Work item -> (sequence, first token, length).  Packed batches read cu_seqlens directly.
__device__ inline void seq_range(const Params& p, int seq, int64_t* s0, int64_t* s1)
{
    if (p.cu != nullptr) {
        *s0 = p.cu[seq];
        *s1 = p.cu[seq + 1];
    } else {
        *s0 = static_cast<int64_t>(seq) * p.seqlen;
        *s1 = *s0 + p.seqlen;
    }
}

// Where a work item's slot sits.  Unsplit, the slot is the sequence.  Split, a sequence of nseg_n
// segments owns nseg_n consecutive a-slots from abase (the output pass runs segment s in a-slot
// abase + s; the workspace keeps S_start(0) in a-slot abase and A_s, later S_start(s + 1), in
// abase + s + 1) and nseg_n - 1 consecutive m-slots from mbase (pass 1 runs segment s in m-slot
// mbase + s and keeps M_s there).  Batch rows: abase = row x nseg, mbase = row x (nseg - 1).
// Packed sequences, with X = seg_chunks x C tokens per segment and segments aligned to each
// sequence's first chunk: abase = floor(cu[n] / X) + n and mbase = floor(cu[n] / X).  Since
// nseg_n = ceil(len_n / X) <= floor(cu[n + 1] / X) - floor(cu[n] / X) + 1, the ranges of
// consecutive sequences never overlap: floor(T / X) + N a-slots and floor(T / X) m-slots hold
// every packed batch, whatever its length mix.
struct Seg {
    int seq, seg, nseg, abase, mbase;
    bool valid;
};

// Largest n < N with key(n) <= idx, key(n) = floor(cu[n] / X) (+ n for a-slots), which does not
// decrease with n: a 64-ary search (one load per lane per level, two levels for 4096
// sequences).  Every wave runs it; the result is wave-uniform.
template <bool ASLOT>
__device__ inline int packed_owner(const Params& p, int idx, int lane)
{
    const int X = p.seg_tokens;
    int lo = 0, span = p.num_seqs;
    while (span > 1) {  // uniform
        const int step = (span + 63) >> 6;
        bool ok = false;
        if (lane * step < span) {
            const int n = lo + lane * step;
            ok = p.cu[n] / X + (ASLOT ? n : 0) <= idx;
        }
        const unsigned long long b = __ballot(ok);
        const int last = b ? 63 - __clzll(b) : 0;
        lo += last * step;
        span = min(step, span - last * step);
    }
    return uniform(lo);
}

// Segments and slot bases of sequence (or batch row) n of a split launch.
__device__ inline Seg seq_slots(const Params& p, int n)
{
    Seg s;
    s.seq = n;
    s.seg = 0;
    s.valid = true;
    if (p.cu == nullptr) {
        s.nseg = p.nseg;
        s.abase = n * p.nseg;
        s.mbase = n * (p.nseg - 1);
    } else {
        const int X = p.seg_tokens;
        const int c0 = p.cu[n], len = p.cu[n + 1] - c0;
        s.nseg = len > X ? (len + X - 1) / X : 1;
        s.mbase = c0 / X;
        s.abase = s.mbase + n;
    }
    return s;
}

// Unsplit packed batches of 2..64 sequences: the sequence of rank k when they are ordered by length,
// longest first (ties by index), so the longest sequences' workgroups are dispatched first and
// the launch does not end on a long sequence that started late.  One wave ranks all lengths; the
// result is wave-uniform.
__device__ inline int longest_first(const Params& p, int k, int lane)
{
    const int N = p.num_seqs;
    const int len = lane < N ? p.cu[lane + 1] - p.cu[lane] : -1;
    int rank = 0;
    for (int j = 0; j < N; ++j) {  // uniform
        const int lj = __shfl(len, j);
        rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
    }
    const unsigned long long b = __ballot(lane < N && rank == k);
    return b ? uniform(__ffsll(b) - 1) : k;
}

template <bool ASLOT>
__device__ inline Seg locate(const Params& p, int slot, int lane)
{
    Seg s;
    if (!p.split) {
        if (p.cu != nullptr && p.num_seqs > 1 && p.num_seqs <= 64) slot = longest_first(p, slot, lane);
        s.seq = slot;
        s.seg = 0;
        s.nseg = 1;
        s.abase = slot;
        s.mbase = 0;
        s.valid = true;
    } else if (p.cu == nullptr) {
        const int per = ASLOT ? p.nseg : p.nseg - 1;
        s = seq_slots(p, slot / per);
        s.seg = slot % per;
    } else {
        s = seq_slots(p, packed_owner<ASLOT>(p, slot, lane));
        s.seg = slot - (ASLOT ? s.abase : s.mbase);
        s.valid = s.seg >= 0 && s.seg < (ASLOT ? s.nseg : s.nseg - 1);  // else a spare slot
    }
    return s;
}

template <int C, bool GT, bool LOCAL, int DVS>
// Two waves per SIMD for the register allocator: at C = 64 the two register sets of the chunk
// pipeline take 155 (gated: 177) VGPRs; with three the gated instance spills, and the ungated
// one is slower at one workgroup per CU.
__global__ __launch_bounds__(Geo<C>::THREADS) __attribute__((amdgpu_waves_per_eu(2))) void chunk_fwd_kernel(Params p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // item = (slot * Hv + hv) * NSL + slice over the a-slots (unsplit: the sequences), or in
    // pass 1 (LOCAL) over the m-slots with twice the slices (A's, then M's); no pass-1 item for
    // a sequence's last segment
    using F = Slice<C, DVS>;
    constexpr int NT = F::NT;
    constexpr int NB = Geo<C>::NB;
    constexpr int MT = Geo<C>::MT;
    constexpr int VROW = Geo<C>::VROW;
    constexpr int NSL = LOCAL ? 2 * F::COUNT : F::COUNT;
    // Workgroups are dealt round-robin to the 8 XCDs (block b to XCD b mod 8).  A group is one
    // (sequence or segment, key head): its value heads' dv slices read the same Q, K and W rows, so
    // the group stays on one XCD and they meet in its L2.  Consecutive groups go to consecutive
    // XCDs, so every XCD gets an equal share of every sequence (a contiguous range of items per
    // XCD gave each of 8 packed sequences an XCD of its own, and the XCD with the longest one set
    // the time).  The grid is 8 x gsize x ceil(groups / 8) blocks.
    const int gsize = (p.hv / p.hq) * NSL;
    const uint32_t xcd = blockIdx.x & 7u, j = blockIdx.x >> 3;
    const int item = static_cast<int>((8u * (j / static_cast<uint32_t>(gsize)) + xcd) * static_cast<uint32_t>(gsize) +
                                      j % static_cast<uint32_t>(gsize));
    if (item >= p.work) return;  // uniform
    const int slice8 = item % NSL;
    const int hv = (item / NSL) % p.hv;
    const Seg at = locate<!LOCAL>(p, item / NSL / p.hv, threadIdx.x & 63);
    if (!at.valid) return;  // uniform: a spare slot
    const int seg = at.seg, seq = at.seq;
    const int pair = seq * p.hv + hv;
    const bool mcols = LOCAL && slice8 >= F::COUNT;  // a slice of the transition M
    const int slice = slice8 % F::COUNT;
    const int hk = hv / (p.hv / p.hq);
    int64_t s0, s1;
    seq_range(p, seq, &s0, &s1);
    const int nchunks_seq = static_cast<int>((s1 - s0 + C - 1) / C);
    const int c_begin = p.split ? seg * p.seg_chunks : 0;
    const int c_end = p.split ? min(c_begin + p.seg_chunks, nchunks_seq) : nchunks_seq;
    const int64_t slot_floats = static_cast<int64_t>(p.hv) * kD * kD;  // one workspace slot

    int tid = threadIdx.x;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const __bf16* Ks = reinterpret_cast<const __bf16*>(smem + F::OFF_K);
    const __bf16* Us = reinterpret_cast<const __bf16*>(smem + F::OFF_U);
    __bf16* Os = reinterpret_cast<__bf16*>(smem + F::OFF_O);
    __bf16* St = reinterpret_cast<__bf16*>(smem + F::OFF_S);
    __bf16* Vn = reinterpret_cast<__bf16*>(smem + F::OFF_VN);
    __bf16* Vd = reinterpret_cast<__bf16*>(smem + F::OFF_VD);
    const float* Gs = reinterpret_cast<const float*>(smem + F::OFF_G);

    // State tiles of this wave: S[16 mt + 4 lg + r][16 nt + lr], mt = MT wave + m, in fp32.
    // Start: pass 1 from zero (A) or from the identity's columns (M); unsplit, the sequence's
    // initial state (also a split launch's one-segment sequences); split, the S_start the combine
    // left in the workspace (segment 0 too: the combine copied the initial state there before
    // this pass, so the last segment may write the final state over the initial state's buffer).
    f32x4 sacc[MT][NT];
    const float* h0 = nullptr;
    if (!LOCAL) {
        if (at.nseg == 1)
            h0 = p.h0 ? p.h0 + static_cast<int64_t>(pair) * kD * kD : nullptr;
        else if (seg > 0 || p.h0 != nullptr)
            h0 = p.ws_a + (at.abase + seg) * slot_floats + static_cast<int64_t>(hv) * kD * kD;
    }
    if (h0) h0 += slice * DVS;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * (MT * wave + m) + 4 * lg + r, col = 16 * nt + lr;
                sacc[m][nt][r] = h0 ? h0[row * kD + col] : (mcols && row == slice * DVS + col ? 1.f : 0.f);
            }

    // S^T (bf16) for the first chunk's products: row = dv column, 4 consecutive dk per lane
    auto write_st = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                bf16x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = static_cast<__bf16>(sacc[m][nt][r]);
                *reinterpret_cast<bf16x4*>(St + (16 * nt + lr) * SROW + 16 * (MT * wave + m) + 4 * lg) = v;
            }
    };
    write_st();

    // Two register sets take turns (the loop is unrolled by two): chunk c + 1's loads go into the
    // set chunk c does not use, right after chunk c's first barrier, so they have a whole chunk
    // step to arrive, and no register copy makes the compiler wait for them early.
    Chunk<C, DVS> ch0, ch1;
    const bool want_q = !LOCAL, want_u = !mcols;
    {
        const int64_t t0 = s0 + static_cast<int64_t>(c_begin) * C;
        const int n0 = c_begin < c_end ? static_cast<int>(s1 - t0 < C ? s1 - t0 : C) : 0;
        ch0.template issue<GT>(p, t0, n0, hk, hv, slice, tid, want_q, want_u);
        // Each chunk step ends with its O store; the loop is entered after a store too (over an
        // empty range: the hardware drops it), so both ways into the loop have the same memory
        // history and the compiler's waits inside need not cover the youngest store.
        if constexpr (!LOCAL)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, rsrc(p.o, 0u), 0, 0, kStream);
    }
    auto step = [&](int c, const Chunk<C, DVS>& cur, Chunk<C, DVS>& nxt) {
        const int64_t tok0 = s0 + static_cast<int64_t>(c) * C;
        const int n = static_cast<int>(s1 - tok0 < C ? s1 - tok0 : C);
        cur.template commit<GT>(smem, tid);
        // this wave's Q and W operands, straight from the registers they were loaded into
        bf16x8 qa[kD / 32], wa[kD / 32];
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
            qa[s] = __builtin_bit_cast(bf16x8, cur.q[s]);
            wa[s] = __builtin_bit_cast(bf16x8, cur.w[s]);
        }
        __syncthreads();  // B1: the chunk (and the state's S^T) is in LDS
        // every load of the next chunk goes in flight now, into the other register set
        const int64_t nt0 = tok0 + C;
        const int nn = c + 1 < c_end ? static_cast<int>(s1 - nt0 < C ? s1 - nt0 : C) : 0;
        nxt.template issue<GT>(p, nt0, nn, hk, hv, slice, tid, want_q, want_u);
        const int I = wave;  // row tile of V' and O
        const float glast = GT ? Gs[C - 1] : 0.f;
        float grow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) grow[r] = GT ? Gs[16 * I + 4 * lg + r] : 0.f;

        // 1. V' = U - W S and O = exp(G) Q S for row tile I; 16x16x32 bf16 MFMA over dk
        f32x4 vacc[NT], oacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            vacc[nt] = zero4();
            oacc[nt] = zero4();
        }
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 sb = *reinterpret_cast<const bf16x8*>(St + (16 * nt + lr) * SROW + 32 * s + 8 * lg);
                vacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], sb, vacc[nt], 0, 0, 0);
                if constexpr (!LOCAL) oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], sb, oacc[nt], 0, 0, 0);
            }
        }
        // V' = U - W S: element r of lane 16 lg + lr is row 16 I + 4 lg + r, column 16 nt + lr
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            bf16x4 vn, vd;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float uu = static_cast<float>(Us[(16 * I + 4 * lg + r) * F::UROW + 16 * nt + lr]);
                const float x = uu - vacc[nt][r];
                vn[r] = static_cast<__bf16>(x);
                vd[r] = static_cast<__bf16>(GT ? x * __expf(glast - grow[r]) : x);
                if constexpr (GT && !LOCAL) oacc[nt][r] *= __expf(grow[r]);
            }
            if constexpr (!LOCAL) *reinterpret_cast<bf16x4*>(Vn + (16 * nt + lr) * VROW + 16 * I + 4 * lg) = vn;
            *reinterpret_cast<bf16x4*>(Vd + (16 * nt + lr) * VROW + 16 * I + 4 * lg) = vd;
        }
        // P^T tiles K_J Q_I^T, J <= I.  Accumulator element r of lane 16 lg + lr is
        // P[i = 16 I + lr][j = 16 J + 4 lg + r] = q_i . k_j: the A operand of the 16x16x16
        // product with V'.  Causal mask (j <= i) and the decay Gamma[i][j] applied in place.
        bf16x4 pa[NB];
        float gi = 0.f;
        if constexpr (GT) gi = Gs[16 * I + lr];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            if (LOCAL || J > I) break;  // uniform
            f32x4 pt = zero4();
#pragma unroll
            for (int s = 0; s < kD / 32; ++s) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (16 * J + lr) * QROW + 32 * s + 8 * lg);
                pt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qa[s], pt, 0, 0, 0);
            }
            bf16x4 a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J + 4 * lg + r, i = 16 * I + lr;
                float x = j <= i ? pt[r] : 0.f;
                if constexpr (GT) x *= __expf(gi - Gs[j]);
                a[r] = static_cast<__bf16>(x);
            }
            pa[J] = a;
        }
        __syncthreads();  // B2: V'^T and V'_dec^T complete; every read of S^T and U is done

        // 2a. O += (Gamma o P) V' over the causal k tiles (16x16x16 bf16)
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            if (LOCAL || J > I) break;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x4 vb = *reinterpret_cast<const bf16x4*>(Vn + (16 * nt + lr) * VROW + 16 * J + 4 * lg);
                oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, pa[J]), __builtin_bit_cast(i16x4, vb), oacc[nt], 0, 0, 0);
            }
        }
        // 2b. S = exp(G_last) S + K^T V'_dec; K^T fragments by transposed LDS reads: lane
        // 16 lg + L addresses token row 16 kt + 4 lg + L / 4, dk columns 16 mt + 4 (L % 4) .. +3
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mt = MT * wave + m;
            if constexpr (GT) {
                const float e = __expf(glast);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) sacc[m][nt] *= e;
            }
#pragma unroll
            for (int kt = 0; kt < NB; ++kt) {
                const __bf16* p0 = Ks + (16 * kt + 4 * lg + (lr >> 2)) * QROW + 16 * mt + 4 * (lr & 3);
                const i16x4 kfr = __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0)));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16x4 vb = *reinterpret_cast<const bf16x4*>(Vd + (16 * nt + lr) * VROW + 16 * kt + 4 * lg);
                    sacc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kfr, __builtin_bit_cast(i16x4, vb),
                                                                           sacc[m][nt], 0, 0, 0);
                }
            }
        }
        write_st();
        // O rows of tile I, scaled, staged row-major for 16-byte stores
        if constexpr (!LOCAL) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Os[(16 * I + 4 * lg + r) * F::UROW + 16 * nt + lr] = static_cast<__bf16>(p.scale * oacc[nt][r]);
        }
        __syncthreads();  // B3: O staged, the new S^T in place; Q, K, W, U, V' free
        if constexpr (!LOCAL) {
            const uint32_t ostride = static_cast<uint32_t>(p.hv) * kD * 2;
            const __amdgpu_buffer_rsrc_t orr =
                rsrc(p.o + (tok0 * p.hv + hv) * kD + slice * DVS, (n - 1) * ostride + DVS * 2);
#pragma unroll
            for (int it = 0; it < F::PIECES; ++it) {
                const int pc = tid + it * Geo<C>::THREADS;
                const u32x4 val = *reinterpret_cast<const u32x4*>(smem + F::OFF_O + (pc / F::RPC) * (F::UROW * 2) + (pc % F::RPC) * 16);
                __builtin_amdgcn_raw_buffer_store_b128(val, orr, (pc / F::RPC) * ostride + (pc % F::RPC) * 16, 0, kStream);
            }
        }
    };
    for (int c = c_begin; c < c_end; c += 2) {  // uniform
        step(c, ch0, ch1);
        if (c + 1 >= c_end) break;  // uniform
        step(c + 1, ch1, ch0);
    }
    float* out = nullptr;  // where this work item's end state goes
    if (LOCAL)
        out = (mcols ? p.ws_m + (at.mbase + seg) * slot_floats : p.ws_a + (at.abase + seg + 1) * slot_floats) +
              static_cast<int64_t>(hv) * kD * kD + slice * DVS;
    else if (p.hT != nullptr && seg == at.nseg - 1)
        out = p.hT + static_cast<int64_t>(pair) * kD * kD + slice * DVS;
    if (out != nullptr) {
        float* hT = out;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hT[(16 * (MT * wave + m) + 4 * lg + r) * kD + 16 * nt + lr] = sacc[m][nt][r];
    }
}

// Pass 2 of the sequence-parallel forward: per (sequence of two or more segments, value head,
// 16-column dv slice), S_start(0) = the initial state (copied to the sequence's first a-slot)
// and S_start(s + 1) = M_s S_start(s) + A_s for s = 0 .. nseg_n - 2, each written over A_s
// (pass 3 reads them there).  Each step is 128 x 128 x 16 fp32
// multiply-adds on fp32 MFMA 16x16x4.  The steps of one slice form a chain, so the slices are
// 16 columns wide (eight workgroups per head: more chains, each step shorter) and each of the
// eight waves owns one row tile (a chain of 32 dependent MFMAs per step); S^T sits in LDS so
// every B operand is one 16-byte read.  M_{s+1} and A_{s+1} do not depend on S and are in
// flight while step s computes.
constexpr int kCombCols = 16;
constexpr int kCombSlices = kD / kCombCols;

constexpr int kCombTiles = kD / 16 / (kThreads / 64);  // row tiles per wave
static_assert(kCombTiles >= 1 && kCombTiles * (kThreads / 64) * 16 == kD, "the waves cover the state's rows");

struct CombineOperands {
    f32x4 m[kCombTiles][kD / 16];  // M rows 16 mt + lr, columns 16 kt + 4 lg .. + 3 (A operands)
    f32x4 a[kCombTiles];           // A elements [16 mt + 4 lg + r][lr] of the slice (accumulator start)

    // Step s of value head hv of a sequence: A_s sits in a-slot abase + s + 1, M_s in m-slot
    // mbase + s.
    __device__ void load(const Params& p, const Seg& at, int hv, int s, int slice, int wave, int lr, int lg)
    {
        const int64_t head = static_cast<int64_t>(hv) * kD * kD;
        const float* A = p.ws_a + static_cast<int64_t>(at.abase + s + 1) * p.hv * kD * kD + head + slice * kCombCols;
        const float* M = p.ws_m + static_cast<int64_t>(at.mbase + s) * p.hv * kD * kD + head;
#pragma unroll
        for (int mm = 0; mm < kCombTiles; ++mm) {
            const int mt = kCombTiles * wave + mm;
#pragma unroll
            for (int kt = 0; kt < kD / 16; ++kt)
                m[mm][kt] = *reinterpret_cast<const f32x4*>(M + (16 * mt + lr) * kD + 16 * kt + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[mm][r] = A[(16 * mt + 4 * lg + r) * kD + lr];
        }
    }
};

__global__ __launch_bounds__(kThreads) void cp_combine_kernel(Params p)
{
    __shared__ __attribute__((aligned(16))) float St[kCombCols][kD + 4];
    // Workgroups are dealt round-robin to the 8 XCDs: give each XCD a contiguous range of items,
    // so the eight slices of a head read M_s through one L2 (M_s is 64 KB per step).
    // Items are (sequence, value head, slice).  The eight slices of one (sequence, value head)
    // form a group on one XCD (block b runs on XCD b mod 8), so they read M_s through one L2;
    // consecutive groups go to consecutive XCDs, so a few long sequences of a packed batch
    // still spread over every XCD.  The grid is 64 x ceil(groups / 8) blocks.
    const uint32_t xcd = blockIdx.x & 7u, j = blockIdx.x >> 3;
    const int item = static_cast<int>((8u * (j / kCombSlices) + xcd) * kCombSlices + j % kCombSlices);
    const int slice = item % kCombSlices, hv = (item / kCombSlices) % p.hv, seq = item / kCombSlices / p.hv;
    if (seq >= p.num_seqs) return;  // uniform
    const Seg at = seq_slots(p, seq);
    if (at.nseg < 2) return;  // uniform: nothing to chain
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int pair = seq * p.hv + hv;
    const int64_t slot_floats = static_cast<int64_t>(p.hv) * kD * kD;
    const float* h0 = p.h0 ? p.h0 + static_cast<int64_t>(pair) * kD * kD + slice * kCombCols : nullptr;
    float* s0 = p.ws_a + at.abase * slot_floats + static_cast<int64_t>(hv) * kD * kD + slice * kCombCols;
    // Two operand sets take turns (the loop is unrolled by two), so the next step's M and A are
    // loaded straight into the set that step uses, with no register copies that would wait for
    // those loads early.
    CombineOperands ops0, ops1;
    ops0.load(p, at, hv, 0, slice, wave, lr, lg);  // the sequence has two or more segments
    for (int idx = tid; idx < kD * kCombCols; idx += kThreads) {
        const int row = idx / kCombCols, col = idx % kCombCols;
        const float x = h0 ? h0[row * kD + col] : 0.f;
        St[col][row] = x;
        if (h0) s0[row * kD + col] = x;  // pass 3's segment 0 starts from this copy
    }
    __syncthreads();
    auto step = [&](int sg, const CombineOperands& cur, CombineOperands& nxt) {
        // M and A of the next step, in flight during this one.  The last step reloads its own
        // slot (in bounds, unused) so that the issue has no branch: a branch around it makes the
        // compiler's wait for `cur` conservative, and that wait would then cover these loads.
        nxt.load(p, at, hv, sg + 2 < at.nseg ? sg + 1 : sg, slice, wave, lr, lg);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads here, ahead of this step's products
        f32x4 acc[kCombTiles];
#pragma unroll
        for (int mm = 0; mm < kCombTiles; ++mm) {
            acc[mm] = cur.a[mm];
#pragma unroll
            for (int kt = 0; kt < kD / 16; ++kt) {
                const f32x4 b = *reinterpret_cast<const f32x4*>(&St[lr][16 * kt + 4 * lg]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[mm] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.m[mm][kt][q], b[q], acc[mm], 0, 0, 0);
            }
        }
        __syncthreads();  // every read of S_start(s) done
        float* A = s0 + (sg + 1) * slot_floats;
#pragma unroll
        for (int mm = 0; mm < kCombTiles; ++mm) {
            const int mt = kCombTiles * wave + mm;
            *reinterpret_cast<f32x4*>(&St[lr][16 * mt + 4 * lg]) = acc[mm];
#pragma unroll
            for (int r = 0; r < 4; ++r) A[(16 * mt + 4 * lg + r) * kD + lr] = acc[mm][r];
        }
        __syncthreads();
    };
    for (int sg = 0; sg + 1 < at.nseg; sg += 2) {  // uniform
        step(sg, ops0, ops1);
        if (sg + 2 >= at.nseg) break;  // uniform
        step(sg + 1, ops1, ops0);
    }
}

template <int C, bool GT, int DVS>
int launch_t(const FwdArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    using F = Slice<C, DVS>;
    constexpr int THREADS = Geo<C>::THREADS;
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= 64)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            attr_err[device] = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<C, GT, false, DVS>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, F::LDS_TOTAL);
            if (attr_err[device] == hipSuccess)
                attr_err[device] = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<C, GT, true, DVS>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, F::LDS_TOTAL);
        });
        e = attr_err[device];
    }
    if (e == hipSuccess) {
        Params p;
        p.q = static_cast<const __bf16*>(a.q);
        p.k = static_cast<const __bf16*>(a.k);
        p.w = static_cast<const __bf16*>(a.w);
        p.u = static_cast<const __bf16*>(a.u);
        p.g = a.g;
        p.h0 = a.h0;
        p.cu = a.cu_seqlens;
        p.o = static_cast<__bf16*>(a.o);
        p.hT = a.hT;
        p.scale = a.scale;
        p.seqlen = a.seqlen;
        p.hq = a.num_qk_heads;
        p.hv = a.num_v_heads;
        p.num_seqs = a.num_seqs;
        p.split = a.split;
        p.nseg = a.nseg;
        p.seg_chunks = a.seg_chunks;
        p.seg_tokens = a.seg_chunks * C;  // a split has a segment boundary inside T
        p.ws_a = a.ws;
        p.ws_m = a.split ? a.ws + static_cast<int64_t>(a.a_slots) * a.num_v_heads * kD * kD : nullptr;
        const int hv = a.num_v_heads;
        // blocks for `work` items in groups of gsize, dealt to 8 XCDs group by group
        auto grid_of = [&](int work, int nsl) {
            const int gsize = (a.num_v_heads / a.num_qk_heads) * nsl;
            const int groups = work / gsize;
            return static_cast<uint32_t>(8 * gsize * ((groups + 7) / 8));
        };
        if (p.split) {
            p.work = a.m_slots * hv * 2 * F::COUNT;  // pass 1
            hipLaunchKernelGGL((chunk_fwd_kernel<C, GT, true, DVS>), dim3(grid_of(p.work, 2 * F::COUNT)),
                               dim3(THREADS), F::LDS_TOTAL, stream, p);
            e = hipGetLastError();
            if (e == hipSuccess) {  // pass 2
                const int groups = a.num_seqs * hv;
                hipLaunchKernelGGL(cp_combine_kernel, dim3(static_cast<uint32_t>(64 * ((groups + 7) / 8))),
                                   dim3(kThreads), 0, stream, p);
                e = hipGetLastError();
            }
        }
        if (e == hipSuccess) {  // pass 3 (the whole forward when not split)
            p.work = (p.split ? a.a_slots : a.num_seqs) * hv * F::COUNT;
            hipLaunchKernelGGL((chunk_fwd_kernel<C, GT, false, DVS>), dim3(grid_of(p.work, F::COUNT)),
                               dim3(THREADS), F::LDS_TOTAL, stream, p);
            e = hipGetLastError();
        }
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (chunk_fwd, C=%d, gated=%d, split=%d, slice=%d)", hipGetErrorString(e), C,
                      GT ? 1 : 0, a.split, DVS);
        return static_cast<int>(e);
    }
    return 0;
}

// Compute units of the current device, read once per device.
int cu_count(int* out)
{
    static std::once_flag once[64];
    static int cus[64];
    static hipError_t err[64];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= 64)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            err[device] = hipDeviceGetAttribute(&cus[device], hipDeviceAttributeMultiprocessorCount, device);
        });
        e = err[device];
    }
    if (e == hipSuccess) *out = cus[device];
    return static_cast<int>(e);
}

// Slice width per launch.  A 64-column slice reads Q, K, W and the gates once for twice the
// columns and forms P = Q K^T once for them, so it costs about 1.35x a 32-column slice per
// workgroup instead of 2x; it wins once the 64-column workgroups (two per (sequence or segment,
// value head)) give every CU one, and loses below that, where the 32-column grid fills twice as
// many CUs.  Both widths do the same operations per column in the same order, so the results
// are identical bit for bit.  C = 32 keeps 32 columns: its two waves hold four dk row tiles of
// the state each, and the gated 64-column instance would spill.
template <int C, bool GT>
int launch_s(const FwdArgs& a, hipStream_t s, char* msg, int len)
{
    int cus = 0;
    const int e = cu_count(&cus);
    if (e != 0) {
        std::snprintf(msg, len, "%s (compute unit count for chunk_fwd)", hipGetErrorString(static_cast<hipError_t>(e)));
        return e;
    }
    const int64_t items = static_cast<int64_t>(a.split ? a.a_slots : a.num_seqs) * a.num_v_heads;
    if constexpr (C > 32) {
        if (items * Slice<C, 64>::COUNT >= cus) return launch_t<C, GT, 64>(a, s, msg, len);
    }
    return launch_t<C, GT, 32>(a, s, msg, len);
}

}  // namespace
}  // namespace fwd

int cp_scratch(void** ptr, char* msg, int msg_len)
{
    // Looked up once per device, on the first call made with that device current.
    static std::once_flag once[64];
    static void* addr[64];
    static hipError_t err[64];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= 64)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            err[device] = hipGetSymbolAddress(&addr[device], HIP_SYMBOL(scratch));
            if (err[device] == hipSuccess && addr[device] == nullptr) err[device] = hipErrorInvalidSymbol;
        });
        e = err[device];
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (device address of the split forward's scratch)", hipGetErrorString(e));
        return static_cast<int>(e);
    }
    *ptr = addr[device];
    return 0;
}

int launch_fwd(const FwdArgs& a, void* stream, char* msg, int msg_len)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (a.chunk_size) {
    case 32:
        return a.g != nullptr ? fwd::launch_s<32, true>(a, s, msg, msg_len) : fwd::launch_s<32, false>(a, s, msg, msg_len);
    case 64:
        return a.g != nullptr ? fwd::launch_s<64, true>(a, s, msg, msg_len) : fwd::launch_s<64, false>(a, s, msg, msg_len);
    default:
        return a.g != nullptr ? fwd::launch_s<128, true>(a, s, msg, msg_len)
                              : fwd::launch_s<128, false>(a, s, msg, msg_len);
    }
}

}  // namespace wyp
