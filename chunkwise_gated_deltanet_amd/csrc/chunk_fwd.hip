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
// The state stays fp32 in the MFMA accumulators for the whole sequence.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "wyprep_launch.h"

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
constexpr int kC = 64;         // chunk size
constexpr int kNB = kC / 16;   // row tiles per chunk (one per wave)
constexpr int kDVS = 32;       // dv columns per workgroup
constexpr int kSlices = kD / kDVS;
constexpr int kThreads = 256;
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
    int32_t num_seqs;  // sequences (cu_seqlens) or batch rows
    int32_t work;      // num_seqs * hv * kSlices
};

// LDS plan (bytes).  Rows of Q, K, W carry 16 bytes of padding (row stride 272 B) so 16-byte
// reads of one column chunk by 16 consecutive rows spread over the banks; the transposed bf16
// tiles (S^T, V'^T) are padded the same way.
constexpr int QROW = kD + 8;          // bf16 per Q / K / W row
constexpr int UROW = kDVS + 8;        // bf16 per U / O slice row
constexpr int SROW = kD + 8;          // bf16 per S^T row (one dv column of S)
constexpr int VROW = kC + 8;          // bf16 per V'^T row (one dv column of V')
constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + kC * QROW * 2;
constexpr int OFF_W = OFF_K + kC * QROW * 2;
constexpr int OFF_U = OFF_W + kC * QROW * 2;
constexpr int OFF_O = OFF_U + kC * UROW * 2;
constexpr int OFF_S = OFF_O + kC * UROW * 2;
constexpr int OFF_VN = OFF_S + kDVS * SROW * 2;
constexpr int OFF_VD = OFF_VN + kDVS * VROW * 2;
constexpr int OFF_G = OFF_VD + kDVS * VROW * 2;
constexpr int LDS_TOTAL = OFF_G + kC * 4;
static_assert(2 * LDS_TOTAL <= 160 * 1024, "two workgroups per CU");

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferConfig);
}

// One chunk's rows in flight to registers: Q, K, W (64 rows x 256 B: four 16-byte pieces per
// thread each), the U slice (64 rows x 64 B: one piece per thread) and g (wave 0, one per lane).
// Rows past the chunk's n tokens read as 0 through the buffer range.
struct Chunk {
    u32x4 q[4], k[4], w[4];
    u32x4 u;
    float g;

    __device__ void issue(const Params& p, int64_t tok0, int n, int hk, int hv, int slice, int tid)
    {
        const uint32_t qstride = static_cast<uint32_t>(p.hq) * kD * 2;
        const uint32_t wstride = static_cast<uint32_t>(p.hv) * kD * 2;
        const __amdgpu_buffer_rsrc_t qr = rsrc(p.q + (tok0 * p.hq + hk) * kD, (n - 1) * qstride + kD * 2);
        const __amdgpu_buffer_rsrc_t kr = rsrc(p.k + (tok0 * p.hq + hk) * kD, (n - 1) * qstride + kD * 2);
        const __amdgpu_buffer_rsrc_t wr = rsrc(p.w + (tok0 * p.hv + hv) * kD, (n - 1) * wstride + kD * 2);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int pc = tid + it * kThreads;  // row pc / 16, piece pc % 16
            q[it] = __builtin_amdgcn_raw_buffer_load_b128(qr, (pc >> 4) * qstride + (pc & 15) * 16, 0, 0);
            k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, (pc >> 4) * qstride + (pc & 15) * 16, 0, 0);
            w[it] = __builtin_amdgcn_raw_buffer_load_b128(wr, (pc >> 4) * wstride + (pc & 15) * 16, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t ur =
            rsrc(p.u + (tok0 * p.hv + hv) * kD + slice * kDVS, (n - 1) * wstride + kDVS * 2);
        u = __builtin_amdgcn_raw_buffer_load_b128(ur, (tid >> 2) * wstride + (tid & 3) * 16, 0, kStream);
        g = 0.f;
        if (p.g != nullptr && tid < 64) {
            const __amdgpu_buffer_rsrc_t gr = rsrc(p.g + tok0 * p.hv + hv, ((n - 1) * p.hv + 1) * 4);
            g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, tid * p.hv * 4, 0, kStream));
        }
    }

    // Q, K, W, U to LDS; wave 0 turns g into the chunk-local inclusive prefix sums G (fp64
    // shuffle scan, stored as fp32).
    template <bool GT>
    __device__ void commit(unsigned char* smem, int tid) const
    {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int pc = tid + it * kThreads;
            const int off = (pc >> 4) * (QROW * 2) + (pc & 15) * 16;
            *reinterpret_cast<u32x4*>(smem + OFF_Q + off) = q[it];
            *reinterpret_cast<u32x4*>(smem + OFF_K + off) = k[it];
            *reinterpret_cast<u32x4*>(smem + OFF_W + off) = w[it];
        }
        *reinterpret_cast<u32x4*>(smem + OFF_U + (tid >> 2) * (UROW * 2) + (tid & 3) * 16) = u;
        if constexpr (GT) {
            if (tid < 64) {
                double x = static_cast<double>(g);
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const double t = __shfl_up(x, d);
                    if (tid >= d) x += t;
                }
                reinterpret_cast<float*>(smem + OFF_G)[tid] = static_cast<float>(x);
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

template <bool GT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void chunk_fwd_kernel(Params p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // Workgroups are dealt round-robin to the 8 XCDs: give each XCD a contiguous range of work
    // items, so the four dv slices of a head (and the heads sharing a key head) meet in one L2.
    const uint32_t Gsz = gridDim.x;  // a multiple of 8
    const int item = static_cast<int>((blockIdx.x & 7u) * (Gsz >> 3) + (blockIdx.x >> 3));
    if (item >= p.work) return;  // uniform
    const int slice = item % kSlices;
    const int pair = item / kSlices;
    const int hv = pair % p.hv, seq = pair / p.hv;
    const int hk = hv / (p.hv / p.hq);
    int64_t s0, s1;
    seq_range(p, seq, &s0, &s1);

    int tid = threadIdx.x;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const __bf16* Qs = reinterpret_cast<const __bf16*>(smem + OFF_Q);
    const __bf16* Ks = reinterpret_cast<const __bf16*>(smem + OFF_K);
    const __bf16* Ws = reinterpret_cast<const __bf16*>(smem + OFF_W);
    const __bf16* Us = reinterpret_cast<const __bf16*>(smem + OFF_U);
    __bf16* Os = reinterpret_cast<__bf16*>(smem + OFF_O);
    __bf16* St = reinterpret_cast<__bf16*>(smem + OFF_S);
    __bf16* Vn = reinterpret_cast<__bf16*>(smem + OFF_VN);
    __bf16* Vd = reinterpret_cast<__bf16*>(smem + OFF_VD);
    const float* Gs = reinterpret_cast<const float*>(smem + OFF_G);

    // State tiles of this wave: S[16 mt + 4 lg + r][16 nt + lr], mt = 2 wave + m, in fp32.
    f32x4 sacc[2][2];
    const float* h0 = p.h0 ? p.h0 + static_cast<int64_t>(pair) * kD * kD + slice * kDVS : nullptr;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[m][nt][r] = h0 ? h0[(16 * (2 * wave + m) + 4 * lg + r) * kD + 16 * nt + lr] : 0.f;

    // S^T (bf16) for the first chunk's products: row = dv column, 4 consecutive dk per lane
    auto write_st = [&]() {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                bf16x4 v;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = static_cast<__bf16>(sacc[m][nt][r]);
                *reinterpret_cast<bf16x4*>(St + (16 * nt + lr) * SROW + 16 * (2 * wave + m) + 4 * lg) = v;
            }
    };
    write_st();

    const int nchunks = static_cast<int>((s1 - s0 + kC - 1) / kC);
    Chunk cur;
    if (nchunks > 0) cur.issue(p, s0, static_cast<int>(s1 - s0 < kC ? s1 - s0 : kC), hk, hv, slice, tid);
    for (int c = 0; c < nchunks; ++c) {  // uniform
        const int64_t tok0 = s0 + static_cast<int64_t>(c) * kC;
        const int n = static_cast<int>(s1 - tok0 < kC ? s1 - tok0 : kC);
        cur.commit<GT>(smem, tid);
        __syncthreads();  // B1: the chunk (and the state's S^T) is in LDS
        if (c + 1 < nchunks) {
            const int64_t nt0 = tok0 + kC;
            cur.issue(p, nt0, static_cast<int>(s1 - nt0 < kC ? s1 - nt0 : kC), hk, hv, slice, tid);
        }
        const int I = wave;  // row tile of V' and O
        const float glast = GT ? Gs[kC - 1] : 0.f;
        float grow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) grow[r] = GT ? Gs[16 * I + 4 * lg + r] : 0.f;

        // 1. V' = U - W S and O = exp(G) Q S for row tile I; 16x16x32 bf16 MFMA over dk
        f32x4 vacc[2], oacc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            vacc[nt] = zero4();
            oacc[nt] = zero4();
        }
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
            const bf16x8 wa = *reinterpret_cast<const bf16x8*>(Ws + (16 * I + lr) * QROW + 32 * s + 8 * lg);
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (16 * I + lr) * QROW + 32 * s + 8 * lg);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bf16x8 sb = *reinterpret_cast<const bf16x8*>(St + (16 * nt + lr) * SROW + 32 * s + 8 * lg);
                vacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, sb, vacc[nt], 0, 0, 0);
                oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, sb, oacc[nt], 0, 0, 0);
            }
        }
        // V' = U - W S: element r of lane 16 lg + lr is row 16 I + 4 lg + r, column 16 nt + lr
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            bf16x4 vn, vd;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float uu = static_cast<float>(Us[(16 * I + 4 * lg + r) * UROW + 16 * nt + lr]);
                const float x = uu - vacc[nt][r];
                vn[r] = static_cast<__bf16>(x);
                vd[r] = static_cast<__bf16>(GT ? x * __expf(glast - grow[r]) : x);
                if constexpr (GT) oacc[nt][r] *= __expf(grow[r]);
            }
            *reinterpret_cast<bf16x4*>(Vn + (16 * nt + lr) * VROW + 16 * I + 4 * lg) = vn;
            *reinterpret_cast<bf16x4*>(Vd + (16 * nt + lr) * VROW + 16 * I + 4 * lg) = vd;
        }
        // P^T tiles K_J Q_I^T, J <= I.  Accumulator element r of lane 16 lg + lr is
        // P[i = 16 I + lr][j = 16 J + 4 lg + r] = q_i . k_j: the A operand of the 16x16x16
        // product with V'.  Causal mask (j <= i) and the decay Gamma[i][j] applied in place.
        bf16x4 pa[kNB];
        float gi = 0.f;
        if constexpr (GT) gi = Gs[16 * I + lr];
#pragma unroll
        for (int J = 0; J < kNB; ++J) {
            if (J > I) break;  // uniform
            f32x4 pt = zero4();
#pragma unroll
            for (int s = 0; s < kD / 32; ++s) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (16 * J + lr) * QROW + 32 * s + 8 * lg);
                const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Qs + (16 * I + lr) * QROW + 32 * s + 8 * lg);
                pt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, pt, 0, 0, 0);
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
        for (int J = 0; J < kNB; ++J) {
            if (J > I) break;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bf16x4 vb = *reinterpret_cast<const bf16x4*>(Vn + (16 * nt + lr) * VROW + 16 * J + 4 * lg);
                oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(i16x4, pa[J]), __builtin_bit_cast(i16x4, vb), oacc[nt], 0, 0, 0);
            }
        }
        // 2b. S = exp(G_last) S + K^T V'_dec; K^T fragments by transposed LDS reads: lane
        // 16 lg + L addresses token row 16 kt + 4 lg + L / 4, dk columns 16 mt + 4 (L % 4) .. +3
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int mt = 2 * wave + m;
            if constexpr (GT) {
                const float e = __expf(glast);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) sacc[m][nt] *= e;
            }
#pragma unroll
            for (int kt = 0; kt < kNB; ++kt) {
                const __bf16* p0 = Ks + (16 * kt + 4 * lg + (lr >> 2)) * QROW + 16 * mt + 4 * (lr & 3);
                const i16x4 kfr = __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0)));
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const bf16x4 vb = *reinterpret_cast<const bf16x4*>(Vd + (16 * nt + lr) * VROW + 16 * kt + 4 * lg);
                    sacc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kfr, __builtin_bit_cast(i16x4, vb),
                                                                           sacc[m][nt], 0, 0, 0);
                }
            }
        }
        write_st();
        // O rows of tile I, scaled, staged row-major for 16-byte stores
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Os[(16 * I + 4 * lg + r) * UROW + 16 * nt + lr] = static_cast<__bf16>(p.scale * oacc[nt][r]);
        __syncthreads();  // B3: O staged, the new S^T in place; Q, K, W, U, V' free
        {
            const uint32_t ostride = static_cast<uint32_t>(p.hv) * kD * 2;
            const __amdgpu_buffer_rsrc_t orr =
                rsrc(p.o + (tok0 * p.hv + hv) * kD + slice * kDVS, (n - 1) * ostride + kDVS * 2);
            const u32x4 val = *reinterpret_cast<const u32x4*>(smem + OFF_O + (tid >> 2) * (UROW * 2) + (tid & 3) * 16);
            __builtin_amdgcn_raw_buffer_store_b128(val, orr, (tid >> 2) * ostride + (tid & 3) * 16, 0, kStream);
        }
    }
    if (p.hT != nullptr) {
        float* hT = p.hT + static_cast<int64_t>(pair) * kD * kD + slice * kDVS;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hT[(16 * (2 * wave + m) + 4 * lg + r) * kD + 16 * nt + lr] = sacc[m][nt][r];
    }
}

template <bool GT>
int launch_t(const FwdArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    static std::once_flag once[64];
    static hipError_t attr_err[64];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= 64)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            attr_err[device] = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<GT>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS_TOTAL);
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
        p.work = a.num_seqs * a.num_v_heads * kSlices;
        const uint32_t grid = static_cast<uint32_t>((p.work + 7) / 8 * 8);
        hipLaunchKernelGGL(chunk_fwd_kernel<GT>, dim3(grid), dim3(kThreads), LDS_TOTAL, stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (chunk_fwd, gated=%d)", hipGetErrorString(e), GT ? 1 : 0);
        return static_cast<int>(e);
    }
    return 0;
}

}  // namespace
}  // namespace fwd

int launch_fwd(const FwdArgs& a, void* stream, char* msg, int msg_len)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.g != nullptr ? fwd::launch_t<true>(a, s, msg, msg_len) : fwd::launch_t<false>(a, s, msg, msg_len);
}

}  // namespace wyp
