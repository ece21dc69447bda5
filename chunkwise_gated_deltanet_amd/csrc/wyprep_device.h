// Device-side pieces shared by the WY/UT preparation kernel (wyprep_kernels.hip) and its
// backward (wy_backward.hip): vector types, buffer resources, the unit map (a0), the gate
// values parked in staged K rows, the placement of the C x C tile, the Gram fragments, and
// the block inversion of a unit lower-triangular tile (a5: 16x16 substitutions; a6:
// coupling levels).  Step labels a0..a8 are those of wyprep_kernels.hip.
//
// Pages cited (by title and section):
//   [Inv] "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
//         lower-triangular matrix).
//   [QLA] The FlashQLA announcement, section "使用方式" (usage).
//
// MFMA operand convention: for a 16x16 output tile, lane l = 16*g + c holds row/column c and
// k-group g.  In __builtin_amdgcn_mfma_f32_16x16x4f32 sub-step q the lane supplies true
// k = 16*kt + 4*g + q; in __builtin_amdgcn_mfma_f32_16x16x32_bf16 element j supplies true
// k = 32*kt + 8*g + j.  A and B use the same map, so the contraction is exact in any hardware
// k order.  Accumulator element r of lane 16*g + c is D[4*g + r][c]; with the k map above that
// is exactly the B operand a following 16x16x4 product needs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace wyp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kD = 128;        // head dim of k and v
constexpr int kThreads = 256;  // four wave64s
constexpr int kWaves = kThreads / 64;
constexpr int kBufferConfig = 0x00020000;  // gfx9 raw buffer: 32-bit dwords, bounds checked
// Cache policy of the streaming loads and stores: nt (non-temporal).  V, beta, T, W and U
// are touched once per launch, so keeping their lines in L2 / MALL only evicts useful ones
// (B=1 T=8192 H=16 C=64: 41 us per launch with the default policy, 33 us with nt).  K keeps
// the default policy: with grouped value heads every key row is read once per value head of
// its group, by units running side by side on one XCD, and those re-reads hit in L2 (8
// packed sequences, Hq=16 Hv=64 C=64: 1.32 ms with nt K loads, 1.11 ms without).
constexpr int kStream = 2;

struct Params {
    const void* k;
    const void* v;
    const float* beta;
    const float* g;  // log gates, gated instances only
    const int32_t* cu;
    float* T;
    void* W;
    void* U;
    int64_t units;
    int32_t seqlen;
    int32_t hq;
    int32_t hv;
    int32_t num_seqs;
    int32_t group;  // preparation kernel: consecutive units a workgroup takes in turn (divides hv)
};

// Placement of the fp32 C x C tile (A, then T, then T') in LDS; off(r, c) is the float offset
// of entry (r, c).  Up to C = 64 it is row-major with rows padded by 4 floats.  At C = 128 only
// the 36 lower 16x16 tiles (diagonal ones included) are kept, tile (I, J) at position
// I(I+1)/2 + J, each 16 rows of 20 floats: 46 KB instead of 68 KB, so two workgroups share a
// CU.  Every access below stays inside one 16x16 tile, and with either padding the rows of a
// 16-lane group start on different banks.
template <int C, bool TILED = (C > 64)>
struct TLayout {
    static constexpr bool kTiled = false;
    static constexpr int RS = C + 4;  // floats per row
    static constexpr int BYTES = C * RS * 4;
    __device__ static constexpr int off(int r, int c) { return r * RS + c; }
};

template <int C>
struct TLayout<C, true> {
    static constexpr bool kTiled = true;
    static constexpr int RS = 20;  // floats per tile row
    static constexpr int TILE = 16 * RS;
    static constexpr int NB = C / 16;
    static constexpr int BYTES = NB * (NB + 1) / 2 * TILE * 4;
    __device__ static constexpr int off(int r, int c)
    {
        return ((r >> 4) * ((r >> 4) + 1) / 2 + (c >> 4)) * TILE + (r & 15) * RS + (c & 15);
    }
};

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Gate values of token row r of the unit, in the padding after the 128 elements of staged K
// row r: G_r (chunk-local inclusive prefix sum of the log gates, fp64) and exp(G_r) (fp32).
template <int KROW, int ESZ>
struct GateRow {
    __device__ static double* Gp(unsigned char* Kraw, int r)
    {
        return reinterpret_cast<double*>(Kraw + r * (KROW * ESZ) + kD * ESZ);
    }
    __device__ static float* Ep(unsigned char* Kraw, int r)
    {
        return reinterpret_cast<float*>(Kraw + r * (KROW * ESZ) + kD * ESZ + 8);
    }
    __device__ static double G(const unsigned char* Kraw, int r)
    {
        return *reinterpret_cast<const double*>(Kraw + r * (KROW * ESZ) + kD * ESZ);
    }
    __device__ static float E(const unsigned char* Kraw, int r)
    {
        return *reinterpret_cast<const float*>(Kraw + r * (KROW * ESZ) + kD * ESZ + 8);
    }
};

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferConfig);
}

struct Unit {
    int64_t tok0;  // first token (flattened b*T + t)
    int n;         // tokens in the chunk (1..C); 0 = no unit
    int hv;        // value head
};

// a0: logical unit index -> Unit.  logical = slot * Hv + value head.  Batch rows: slot b * cps + c
// is chunk c of row b (cps chunks per row).  Packed sequences: sequence s owns the slots
// [B_s, B_{s+1}) with B_s = floor(cu[s] / C) + s.  B is strictly increasing and leaves room for all
// ceil(len_s / C) chunks of sequence s (B_{s+1} - B_s - ceil(len_s / C) is 0 or 1), so a slot is
// found from cu_seqlens alone, by a search over s, without prefix sums of chunk counts; a slot past
// its sequence's last chunk is empty.  Host side: floor(T / C) + N slots.

// Packed: wave 0 finds the sequence of `slot` by a 64-ary search over B (one round trip to
// cu_seqlens while N <= 64, two while N <= 4096, ...) and returns the chunk's first token and
// length (n = 0 for an empty slot).  With fewer than 64 sequences, lane l may pass cu[min(l, N)]
// in cu_lane (cached = true, loaded once per launch): the search is then one ballot and two
// shuffles, with no memory access.  Every lane of wave 0 gets the same result; other waves must
// not call it.
template <int C>
__device__ inline void find_slot(const Params& p, uint32_t slot, int lane, bool cached, int cu_lane,
                                 int64_t* tok0, int* n)
{
    int lo = 0, hi = p.num_seqs;  // B_lo <= slot (B_0 = 0), and s < hi
    int cu_s = 0, cu_s1 = 0;
    if (cached) {  // uniform
        const bool below = lane < hi && static_cast<uint32_t>(cu_lane / C + lane) <= slot;
        const unsigned long long m = __ballot(below);  // lane 0 is always set
        lo = 63 - __clzll(m);
        cu_s = __shfl(cu_lane, lo);
        cu_s1 = __shfl(cu_lane, lo + 1);
    } else {
        while (true) {  // uniform
            const int span = hi - lo;
            const int step = (span + 63) / 64;
            const int s = lo + lane * step;
            const bool in = s < hi;
            const int c0 = in ? p.cu[s] : 0;
            // in the last round (step 1) each lane also takes its sequence's end
            const int c1 = (in && step == 1) ? p.cu[s + 1] : 0;
            const bool below = in && static_cast<uint32_t>(c0 / C + s) <= slot;
            const unsigned long long m = __ballot(below);  // lane 0 is always set
            const int L = 63 - __clzll(m);
            lo += L * step;
            hi = min(lo + step, hi);
            if (step == 1) {
                cu_s = __shfl(c0, L);
                cu_s1 = __shfl(c1, L);
                break;
            }
        }
    }
    const int c = static_cast<int>(slot) - (cu_s / C + lo);
    const bool valid = c < (cu_s1 - cu_s + C - 1) / C;
    *tok0 = cu_s + static_cast<int64_t>(c) * C;
    *n = valid ? min(C, cu_s1 - (cu_s + c * C)) : 0;
}

// Packed, first half: wave 0 finds the first non-empty unit at logical, logical + stride, ... and
// leaves it in info (info[0] = first token, info[1] = n, 0 past the end, info[2..3] = its
// logical index); the caller's next barrier publishes it.  Nothing to do for batch rows.
template <int C>
__device__ inline void map_search(const Params& p, int* info, int64_t logical, int64_t stride, int tid,
                                  bool cached = false, int cu_lane = 0)
{
    if (p.cu == nullptr || tid >= 64) return;
    int64_t tok0 = 0;
    int n = 0;
    while (logical < p.units) {  // uniform in wave 0
        // units < 2^31 (checked on the host), so 32-bit arithmetic suffices here
        const uint32_t slot = static_cast<uint32_t>(logical) / static_cast<uint32_t>(p.hv);
        find_slot<C>(p, slot, tid, cached, cu_lane, &tok0, &n);
        if (n > 0) break;
        logical += stride;
    }
    if (tid == 0) {
        info[0] = static_cast<int>(tok0);  // packed tokens fit in int32 (the problem's T)
        info[1] = n;
        info[2] = static_cast<int>(logical & 0xffffffff);
        info[3] = static_cast<int>(logical >> 32);
    }
}

// Second half, after that barrier: the unit (n == 0 past the end); `logical` moves to its index.
template <int C>
__device__ inline Unit map_read(const Params& p, const int* info, int64_t& logical)
{
    const uint32_t hvn = static_cast<uint32_t>(p.hv);
    if (p.cu == nullptr) {
        if (logical >= p.units) return Unit{0, 0, 0};
        const uint32_t l32 = static_cast<uint32_t>(logical);
        const uint32_t slot = l32 / hvn;
        const uint32_t cps = static_cast<uint32_t>((p.seqlen + C - 1) / C);
        const uint32_t b = slot / cps, c = slot % cps;
        Unit u;
        u.tok0 = static_cast<int64_t>(b) * p.seqlen + static_cast<int64_t>(c) * C;
        u.n = min(C, p.seqlen - static_cast<int>(c) * C);
        u.hv = static_cast<int>(l32 % hvn);
        return u;
    }
    logical = static_cast<int64_t>(static_cast<uint32_t>(uniform(info[2]))) |
              (static_cast<int64_t>(uniform(info[3])) << 32);
    Unit u;
    u.tok0 = uniform(info[0]);
    u.n = uniform(info[1]);
    u.hv = static_cast<int>(static_cast<uint32_t>(logical) % hvn);
    return u;
}

// Both halves with their own barrier (packed only): the first non-empty unit at logical,
// logical + stride, ...; `logical` moves to its index.
template <int C>
__device__ inline Unit map_unit(const Params& p, int* info, int64_t& logical, int64_t stride, int tid,
                                bool cached = false, int cu_lane = 0)
{
    if (p.cu != nullptr) {
        map_search<C>(p, info, logical, stride, tid, cached, cu_lane);
        __syncthreads();
    }
    return map_read<C>(p, info, logical);
}

// Lower 16x16 tile t (row-major over I >= J) -> (I, J).
__device__ inline void tile_of(int t, int* I, int* J)
{
    int i = 0;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    *I = i;
    *J = t - i * (i + 1) / 2;
}

template <int DT, int KROW>
struct GramFrags {
    static constexpr int NS = DT == 0 ? kD / 32 : kD / 16;
    typedef typename std::conditional<DT == 0, bf16x8, f32x4>::type frag;
    frag a[NS], b[NS];

    __device__ void load(const unsigned char* Kraw, int I, int J, int lr, int lg)
    {
        if constexpr (DT == 0) {
            const __bf16* K = reinterpret_cast<const __bf16*>(Kraw);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                a[s] = *reinterpret_cast<const bf16x8*>(K + (16 * I + lr) * KROW + 32 * s + 8 * lg);
                b[s] = *reinterpret_cast<const bf16x8*>(K + (16 * J + lr) * KROW + 32 * s + 8 * lg);
            }
        } else {
            const float* K = reinterpret_cast<const float*>(Kraw);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                a[s] = *reinterpret_cast<const f32x4*>(K + (16 * I + lr) * KROW + 16 * s + 4 * lg);
                b[s] = *reinterpret_cast<const f32x4*>(K + (16 * J + lr) * KROW + 16 * s + 4 * lg);
            }
        }
    }

    __device__ f32x4 product() const
    {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if constexpr (DT == 0) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s][q], b[s][q], acc, 0, 0, 0);
            }
        }
        return acc;
    }
};

// The right-looking substitution for lane (block, column i).  At step J, X[J][i] is final (1
// for J = i, else -acc[J]; acc holds the negated partial sums, exactly +0 above i), it is
// written back, and every later row k takes acc[k] -= L[k][J] X[J][i].  L[k][J] for k > J is
// row J of the block's upper triangle, where form_a left L^T; all 16 lanes of the block read
// the same row (an LDS broadcast).  Row J is written only at step J, after it has been read, so
// each row can be read D steps ahead, before the writes of the rows in between: its LDS latency
// then overlaps D steps of multiply-adds instead of sitting on the chain (D = 0: read at its
// own step).
template <int RS, int D>
__device__ __attribute__((always_inline)) void substitute(float (&acc)[16], int i, float* blk)
{
    f32x4 rows[D + 1][4];  // rows[J % (D + 1)][c4]: chunks c4 >= (J + 1) / 4 of row J
    auto load_row = [&](int J, f32x4 (&r)[4]) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            if (c4 >= (J + 1) / 4) r[c4] = *reinterpret_cast<const f32x4*>(blk + J * RS + 4 * c4);
    };
#pragma unroll
    for (int J = 0; J < D; ++J) load_row(J, rows[J]);
#pragma unroll
    for (int J = 0; J < 16; ++J) {  // unrolled: every index below is a compile-time constant
        if (J + D < 15) load_row(J + D, rows[(J + D) % (D + 1)]);
        const float x = (J == i) ? 1.f : acc[J];
        blk[J * RS + i] = x;
#pragma unroll
        for (int k = J + 1; k < 16; ++k) acc[k] = __builtin_fmaf(-rows[J % (D + 1)][k / 4][k % 4], x, acc[k]);
    }
}

// a5: invert the C/16 diagonal 16x16 blocks of Ts in place.  Lane (block b, column i) keeps
// column i of X_b = L_b^{-1} in registers, right-looking: after X[j][i] is final, every later
// row k takes its share L[k][j] X[j][i], so one multiply-add per step sits on the dependency
// chain.  Blocks 0-3 run on wave 0, blocks 4-7 on wave 1.  Rows are read two steps ahead from
// C = 64 on; at C = 32 the 32 extra registers would cost resident workgroups (seven to five per
// CU), which the T-only step at C = 32 needs more than the shorter chain.
template <int C, class TL>
__device__ void invert_diagonal_blocks(float* Ts, int tid)
{
    constexpr int NB = C / 16;
    if (tid >= NB * 16) return;
    const int b = tid >> 4, i = tid & 15;
    float* blk = Ts + TL::off(16 * b, 16 * b);
    float acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.f;
    substitute<TL::RS, (C >= 64 ? 2 : 0)>(acc, i, blk);
}

// a6, one level: block size S.  Pair p covers rows/cols [2Sp, 2Sp + 2S); its sub-diagonal
// block L10 (rows 2Sp+S.., cols 2Sp..) is replaced by X10 = -X11 (L10 X00).  Wave w owns pair
// w / (S/16) and 16-column tile w % (S/16) of X10.
template <int C, int S, class TL>
__device__ void coupling_level(float* Ts, int tid)
{
    constexpr int TS = S / 16;
    constexpr int NPAIR = C / (2 * S);
    constexpr int NTASK = NPAIR * TS;
    static_assert(NTASK <= kWaves, "one coupling task per wave");
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const bool active = wave < NTASK;
    const int pr = wave / TS, nc = wave % TS;
    const int base = 2 * S * pr;
    f32x4 res[TS];
    if (active) {
        // tmp[:, nc] = L10 X00[:, nc].  X00 is lower triangular, so k-tiles kt < nc hold
        // zeros.  The row-major layout multiplies them anyway, which keeps every operand load
        // branch-free; the tile-packed layout does not store them and skips them.
        f32x4 tmp[TS];
#pragma unroll
        for (int mr = 0; mr < TS; ++mr) tmp[mr] = zero4();
#pragma unroll
        for (int kt = 0; kt < TS; ++kt) {
            if (TL::kTiled && kt < nc) continue;  // uniform per wave
            float bq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bq[q] = Ts[TL::off(base + 16 * kt + 4 * lg + q, base + 16 * nc + lr)];
#pragma unroll
            for (int mr = 0; mr < TS; ++mr) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(
                    Ts + TL::off(base + S + 16 * mr + lr, base + 16 * kt + 4 * lg));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    tmp[mr] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], bq[q], tmp[mr], 0, 0, 0);
            }
        }
        // X10[:, nc] = -X11 tmp[:, nc]; X11 is lower triangular, so kt <= mr.
#pragma unroll
        for (int mr = 0; mr < TS; ++mr) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kt = 0; kt <= mr; ++kt) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(
                    Ts + TL::off(base + S + 16 * mr + lr, base + S + 16 * kt + 4 * lg));
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], tmp[kt][q], acc, 0, 0, 0);
            }
            res[mr] = -acc;
        }
    }
    __syncthreads();  // every wave has read L10 before any X10 overwrites it
    if (active) {
#pragma unroll
        for (int mr = 0; mr < TS; ++mr)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Ts[TL::off(base + S + 16 * mr + 4 * lg + r, base + 16 * nc + lr)] = res[mr][r];
    }
    __syncthreads();
}

}  // namespace
}  // namespace wyp
