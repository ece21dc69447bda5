// HIP kernels (gfx950 / CDNA4) for the per-chunk WY/UT preparation of chunkwise (Gated)
// DeltaNet.
//
// Pages cited (by title and section):
//   [Inv] "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
//         lower-triangular matrix).
//   [QLA] The FlashQLA announcement, section "使用方式" (usage).
//
// One workgroup of 256 threads (four wave64s) owns one unit = (sequence, chunk, value head):
//   a0  map the workgroup to its unit (packed batches: scan cu_seqlens on the device);
//   a1  stage the chunk's K (n x 128), V (n x 128) and beta (n) in LDS with 16-byte loads;
//       rows n..C-1 of a short chunk are zero with beta = 0 ([Inv] leaves tails open; this is
//       the padded reading: A = blockdiag(A_n, I) so T = blockdiag(T_n, I));
//   a2  Gram G = K K^T, lower 16x16 tiles only, on bf16 MFMA (fp32 MFMA for fp32 inputs);
//   a3  A = I + strictLower(diag(beta) G): beta scales rows, the diagonal is 1 ([Inv] 3.2);
//   a4  the A matrix stays in one fp32 LDS tile; its diagonal 16x16 blocks are inverted in
//       place and each coupling level overwrites its sub-diagonal block ([Inv] 3.3-3.6);
//   a5  C/16 independent 16x16 forward substitutions, one lane per column, 15 dependent
//       steps ([Inv] 2.1 and 3.4);
//   a6  coupling levels s = 16, 32, 64: X10 = -X11 L10 X00 as two fp32 MFMA products, the
//       first product's accumulator feeding the second as its B operand ([Inv] 2.2, 3.5);
//   a7  store T (fp32, upper triangle 0, diagonal 1);
//   a8  T' = T diag(beta) as a hi + lo pair of bf16 values, W = T' K and U = T' V on bf16
//       MFMA (T' is lower triangular, so k-tiles right of the diagonal are skipped), staged
//       in LDS and stored with 16-byte writes.
//
// MFMA operand convention used throughout: for a 16x16 output tile, lane l = 16*g + c holds
// row/column c and k-group g.  In __builtin_amdgcn_mfma_f32_16x16x4f32 sub-step q the lane
// supplies true k = 16*kt + 4*g + q; in __builtin_amdgcn_mfma_f32_16x16x32_bf16 element j
// supplies true k = 32*kt + 8*g + j.  A and B use the same map, so the contraction is exact
// in any hardware k order.  Accumulator element r of lane 16*g + c is D[4*g + r][c]; with the
// k map above that is exactly the B operand a following 16x16x4 product needs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "wyprep_launch.h"

namespace wyp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;        // head dim of k and v
constexpr int kThreads = 256;  // four wave64s
constexpr int kWaves = kThreads / 64;

struct Params {
    const void* k;
    const void* v;
    const float* beta;
    const int32_t* cu;
    float* T;
    void* W;
    void* U;
    int64_t units;
    int32_t seqlen;
    int32_t hq;
    int32_t hv;
    int32_t num_seqs;
};

// LDS plan of one workgroup.  K and V rows carry 16 bytes of padding so that 16-byte reads of
// one column chunk by 16 consecutive rows spread over all banks; T rows carry 4 floats.
template <int C, int DT, bool WU>
struct Lds {
    static constexpr int ESZ = DT == 0 ? 2 : 4;
    static constexpr int KROW = kD + 16 / ESZ;   // elements per staged K / V row
    static constexpr int KBYTES = C * KROW * ESZ;
    static constexpr int TROW = C + 4;           // floats per T row
    static constexpr int TBYTES = C * TROW * 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = KBYTES;
    static constexpr int OFF_T = WU ? 2 * KBYTES : KBYTES;
    static constexpr int OFF_B = OFF_T + TBYTES;
    static constexpr int OFF_INFO = OFF_B + C * 4;
    static constexpr int TOTAL = OFF_INFO + 16;
};

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// a0: unit -> (first token, chunk length, value head).  Returns false for surplus workgroups.
template <int C>
__device__ bool map_unit(const Params& p, int* info, int64_t* tok0, int* n, int* hv)
{
    const uint32_t G = gridDim.x;  // a multiple of 8
    const uint32_t bid = blockIdx.x;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous range of
    // units so that value heads sharing a key head, and neighbouring chunks, meet in one L2.
    const int64_t logical = static_cast<int64_t>(bid & 7u) * (G >> 3) + (bid >> 3);
    if (logical >= p.units) return false;
    *hv = static_cast<int>(logical % p.hv);
    const int64_t slot = logical / p.hv;
    if (p.cu == nullptr) {
        const int64_t cps = (p.seqlen + C - 1) / C;
        const int64_t b = slot / cps, c = slot % cps;
        *tok0 = b * p.seqlen + c * C;
        *n = static_cast<int>(min<int64_t>(C, p.seqlen - c * C));
        return true;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        int64_t run = 0;
        int found_s = -1, found_c = 0;
        for (int base = 0; base < p.num_seqs; base += 64) {
            const int s = base + lane;
            int cnt = 0;
            if (s < p.num_seqs) cnt = (p.cu[s + 1] - p.cu[s] + C - 1) / C;
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(incl, d);
                if (lane >= d) incl += t;
            }
            const int excl = incl - cnt;
            const bool hit = cnt > 0 && slot >= run + excl && slot < run + incl;
            const unsigned long long m = __ballot(hit);
            if (m) {
                const int src = __ffsll(m) - 1;
                found_s = __shfl(s, src);
                found_c = static_cast<int>(slot - run - __shfl(excl, src));
                break;
            }
            run += __shfl(incl, 63);
        }
        if (lane == 0) {
            info[0] = found_s;
            info[1] = found_c;
        }
    }
    __syncthreads();
    const int s = info[0];
    if (s < 0) return false;
    const int64_t s0 = p.cu[s], s1 = p.cu[s + 1];
    *tok0 = s0 + static_cast<int64_t>(info[1]) * C;
    *n = static_cast<int>(min<int64_t>(C, s1 - *tok0));
    return true;
}

// a1: C rows of 128 elements from a [tokens, heads, 128] tensor into LDS (zero rows >= n).
template <int C, int ESZ, int KROW>
__device__ void stage_rows(unsigned char* dst, const void* src, int64_t tok0, int n, int heads,
                           int head)
{
    constexpr int CPR = kD * ESZ / 16;  // 16-byte chunks per row
    constexpr int NIT = C * CPR / kThreads;
    static_assert(C * CPR % kThreads == 0, "row chunks must split evenly");
    const int tid = threadIdx.x;
    const unsigned char* base = static_cast<const unsigned char*>(src);
    uint4 val[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * kThreads;
        const int r = q / CPR, c16 = q % CPR;
        val[it] = uint4{0u, 0u, 0u, 0u};
        if (r < n)
            val[it] = *reinterpret_cast<const uint4*>(
                base + ((tok0 + r) * heads + head) * (kD * ESZ) + c16 * 16);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * kThreads;
        const int r = q / CPR, c16 = q % CPR;
        *reinterpret_cast<uint4*>(dst + r * (KROW * ESZ) + c16 * 16) = val[it];
    }
}

// a2 + a3: A = I + strictLower(diag(beta) K K^T) into Ts (all C x C entries written).
template <int C, int DT, int KROW, int TROW>
__device__ void form_a(const unsigned char* Kraw, float* Ts, const float* bs)
{
    constexpr int NB = C / 16;
    constexpr int NTILE = NB * (NB + 1) / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    for (int t = wave; t < NTILE; t += kWaves) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= t) ++I;
        const int J = t - I * (I + 1) / 2;
        f32x4 acc = zero4();
        if constexpr (DT == 0) {
            const __bf16* K = reinterpret_cast<const __bf16*>(Kraw);
#pragma unroll
            for (int s = 0; s < kD / 32; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + (16 * I + lr) * KROW + 32 * s + 8 * lg);
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(K + (16 * J + lr) * KROW + 32 * s + 8 * lg);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
            }
        } else {
            const float* K = reinterpret_cast<const float*>(Kraw);
#pragma unroll
            for (int s = 0; s < kD / 16; ++s) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(K + (16 * I + lr) * KROW + 16 * s + 4 * lg);
                const f32x4 b = *reinterpret_cast<const f32x4*>(K + (16 * J + lr) * KROW + 16 * s + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], acc, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r, j = 16 * J + lr;
            Ts[i * TROW + j] = (i > j) ? bs[i] * acc[r] : (i == j ? 1.f : 0.f);
        }
    }
    // strictly upper 16x16 tiles
    for (int e = tid; e < C * C; e += kThreads) {
        const int i = e / C, j = e % C;
        if ((j >> 4) > (i >> 4)) Ts[i * TROW + j] = 0.f;
    }
}

// a5: invert the C/16 diagonal 16x16 blocks of Ts in place.  Lane (block b, column i) keeps
// column i of X_b = L_b^{-1} in registers: X[k][i] = -sum_{j<k} L[k][j] X[j][i] for k > i,
// with X[i][i] = 1 and X[j][i] = 0 for j < i.  All reads of a block precede its writes (one
// wave per group of four blocks, LDS operations of a wave complete in order).
template <int C, int TROW>
__device__ void invert_diagonal_blocks(float* Ts)
{
    constexpr int NB = C / 16;
    const int tid = threadIdx.x;
    if (tid >= NB * 16) return;
    const int b = tid >> 4, i = tid & 15;
    float* blk = Ts + 16 * b * TROW + 16 * b;
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = (k == i) ? 1.f : 0.f;
#pragma unroll
    for (int k = 1; k < 16; ++k) {
        float row[16];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(blk + k * TROW + 4 * c4);
            row[4 * c4 + 0] = v[0];
            row[4 * c4 + 1] = v[1];
            row[4 * c4 + 2] = v[2];
            row[4 * c4 + 3] = v[3];
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < k; ++j) s = __builtin_fmaf(row[j], x[j], s);
        x[k] = (k > i) ? -s : x[k];
    }
#pragma unroll
    for (int k = 1; k < 16; ++k)
        if (k > i) blk[k * TROW + i] = x[k];
}

// a6, one level: block size S.  Pair p covers rows/cols [2Sp, 2Sp + 2S); its sub-diagonal
// block L10 (rows 2Sp+S.., cols 2Sp..) is replaced by X10 = -X11 (L10 X00).  Wave w owns pair
// w / (S/16) and 16-column tile w % (S/16) of X10.
template <int C, int S, int TROW>
__device__ void coupling_level(float* Ts)
{
    constexpr int TS = S / 16;
    constexpr int NPAIR = C / (2 * S);
    constexpr int NTASK = NPAIR * TS;
    static_assert(NTASK <= kWaves, "one coupling task per wave");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const bool active = wave < NTASK;
    const int pr = wave / TS, nc = wave % TS;
    const int base = 2 * S * pr;
    f32x4 res[TS];
    if (active) {
        // tmp[:, nc] = L10 X00[:, nc]; X00 is lower triangular, so k-tiles kt < nc vanish.
        f32x4 tmp[TS];
#pragma unroll
        for (int mr = 0; mr < TS; ++mr) {
            f32x4 acc = zero4();
            for (int kt = nc; kt < TS; ++kt) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(
                    Ts + (base + S + 16 * mr + lr) * TROW + base + 16 * kt + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float bq = Ts[(base + 16 * kt + 4 * lg + q) * TROW + base + 16 * nc + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], bq, acc, 0, 0, 0);
                }
            }
            tmp[mr] = acc;
        }
        // X10[:, nc] = -X11 tmp[:, nc]; X11 is lower triangular, so kt <= mr.
#pragma unroll
        for (int mr = 0; mr < TS; ++mr) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kt = 0; kt <= mr; ++kt) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(
                    Ts + (base + S + 16 * mr + lr) * TROW + base + S + 16 * kt + 4 * lg);
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
                Ts[(base + S + 16 * mr + 4 * lg + r) * TROW + base + 16 * nc + lr] = res[mr][r];
    }
    __syncthreads();
}

// a7: T rows [0, n) to T_out[(tok0 + r) * Hv + hv][0:C].
template <int C, int TROW>
__device__ void store_t(const float* Ts, float* Tout, int64_t tok0, int n, int Hv, int hv)
{
    constexpr int TCH = C / 4;
    for (int q = threadIdx.x; q < n * TCH; q += kThreads) {
        const int r = q / TCH, c = q % TCH;
        const f32x4 val = *reinterpret_cast<const f32x4*>(Ts + r * TROW + 4 * c);
        *reinterpret_cast<f32x4*>(Tout + ((tok0 + r) * Hv + hv) * C + 4 * c) = val;
    }
}

// a8 (bf16): W = T' K and U = T' V with T' = T diag(beta).  T' enters the bf16 MFMA as a
// hi + lo pair of bf16 values (T' - hi - lo is below 2^-17 |T'|), so the only rounding left
// in W and U is the final bf16 store.  The B operand (8 consecutive tokens of one K / V
// column) is gathered with two LDS transpose reads: within each 16-lane group, lane i of
// ds_read_tr16_b64 receives element (i mod 4) of the 64-bit rows addressed by lanes
// 4e + i/4, e = 0..3.  16 column tiles of 16 (8 of W, 8 of U); wave w owns tiles w, w+4,
// w+8, w+12.
template <int C, int KROW, int TROW>
__device__ void wu_bf16(unsigned char* Kraw, unsigned char* Vraw, const float* Ts, const float* bs,
                        void* Wout, void* Uout, int64_t tok0, int n, int Hv, int hv)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    constexpr int NB = C / 16;
    constexpr int KT = C / 32;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    bf16x8 ahi[NB][KT], alo[NB][KT];
#pragma unroll
    for (int mi = 0; mi < NB; ++mi)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            if (2 * kt > mi) continue;
            const float* trow = Ts + (16 * mi + lr) * TROW + 32 * kt + 8 * lg;
            const f32x4 t0 = *reinterpret_cast<const f32x4*>(trow);
            const f32x4 t1 = *reinterpret_cast<const f32x4*>(trow + 4);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(bs + 32 * kt + 8 * lg);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(bs + 32 * kt + 8 * lg + 4);
            const float tp[8] = {t0[0] * b0[0], t0[1] * b0[1], t0[2] * b0[2], t0[3] * b0[3],
                                 t1[0] * b1[0], t1[1] * b1[1], t1[2] * b1[2], t1[3] * b1[3]};
            bf16x8 h, l;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                h[j] = static_cast<__bf16>(tp[j]);
                l[j] = static_cast<__bf16>(tp[j] - static_cast<float>(h[j]));
            }
            ahi[mi][kt] = h;
            alo[mi][kt] = l;
        }

    __bf16 out[4][NB][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ct = wave + 4 * c;
        const __bf16* src = reinterpret_cast<const __bf16*>(ct < 8 ? Kraw : Vraw);
        const int ni = ct & 7;
        f32x4 acc[NB];
#pragma unroll
        for (int mi = 0; mi < NB; ++mi) acc[mi] = zero4();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            // lane 16g + L addresses row 32kt + 8g + 4h + L/4, columns 16ni + 4(L%4) .. +3
            const __bf16* p0 = src + (32 * kt + 8 * lg + (lr >> 2)) * KROW + 16 * ni + 4 * (lr & 3);
            const bf16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
            const bf16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * KROW));
            const bf16x8 bfr = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int mi = 0; mi < NB; ++mi)
                if (2 * kt <= mi) {
                    acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[mi][kt], bfr, acc[mi], 0, 0, 0);
                    acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[mi][kt], bfr, acc[mi], 0, 0, 0);
                }
        }
#pragma unroll
        for (int mi = 0; mi < NB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[c][mi][r] = static_cast<__bf16>(acc[mi][r]);
    }
    __syncthreads();  // all waves are done reading K and V; reuse them as output staging
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ct = wave + 4 * c;
        __bf16* dst = reinterpret_cast<__bf16*>(ct < 8 ? Kraw : Vraw);
        const int ni = ct & 7;
#pragma unroll
        for (int mi = 0; mi < NB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * mi + 4 * lg + r) * KROW + 16 * ni + lr] = out[c][mi][r];
    }
    __syncthreads();
    constexpr int CPR = kD * 2 / 16;  // 16 chunks of 16 bytes per output row
    const int per = n * CPR;
    for (int q = tid; q < 2 * per; q += kThreads) {
        const int which = q >= per;
        const int rem = q - which * per;
        const int r = rem / CPR, c16 = rem % CPR;
        const unsigned char* s = (which ? Vraw : Kraw) + r * (KROW * 2) + c16 * 16;
        unsigned char* d = static_cast<unsigned char*>(which ? Uout : Wout) +
                           ((tok0 + r) * Hv + hv) * (kD * 2) + c16 * 16;
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    }
}

// a8 (fp32 inputs): the same products on fp32 MFMA, T' kept in fp32.
template <int C, int KROW, int TROW>
__device__ void wu_f32(unsigned char* Kraw, unsigned char* Vraw, const float* Ts, const float* bs,
                       void* Wout, void* Uout, int64_t tok0, int n, int Hv, int hv)
{
    constexpr int NB = C / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    float out[4][NB][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ct = wave + 4 * c;
        const float* src = reinterpret_cast<const float*>(ct < 8 ? Kraw : Vraw);
        const int ni = ct & 7;
#pragma unroll
        for (int mi = 0; mi < NB; ++mi) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kt = 0; kt <= mi; ++kt) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(Ts + (16 * mi + lr) * TROW + 16 * kt + 4 * lg);
                const f32x4 b = *reinterpret_cast<const f32x4*>(bs + 16 * kt + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float bq = src[(16 * kt + 4 * lg + q) * KROW + 16 * ni + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(t[q] * b[q], bq, acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) out[c][mi][r] = acc[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ct = wave + 4 * c;
        float* dst = reinterpret_cast<float*>(ct < 8 ? Kraw : Vraw);
        const int ni = ct & 7;
#pragma unroll
        for (int mi = 0; mi < NB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * mi + 4 * lg + r) * KROW + 16 * ni + lr] = out[c][mi][r];
    }
    __syncthreads();
    constexpr int CPR = kD * 4 / 16;
    const int per = n * CPR;
    for (int q = tid; q < 2 * per; q += kThreads) {
        const int which = q >= per;
        const int rem = q - which * per;
        const int r = rem / CPR, c16 = rem % CPR;
        const unsigned char* s = (which ? Vraw : Kraw) + r * (KROW * 4) + c16 * 16;
        unsigned char* d = static_cast<unsigned char*>(which ? Uout : Wout) +
                           ((tok0 + r) * Hv + hv) * (kD * 4) + c16 * 16;
        *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    }
}

template <int C, int DT, bool WU>
__global__ __launch_bounds__(kThreads) void wy_prepare_kernel(Params p)
{
    using L = Lds<C, DT, WU>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* Kraw = smem + L::OFF_K;
    unsigned char* Vraw = smem + L::OFF_V;
    float* Ts = reinterpret_cast<float*>(smem + L::OFF_T);
    float* bs = reinterpret_cast<float*>(smem + L::OFF_B);
    int* info = reinterpret_cast<int*>(smem + L::OFF_INFO);

    int64_t tok0;
    int n, hv;
    if (!map_unit<C>(p, info, &tok0, &n, &hv)) return;  // uniform per workgroup
    const int hk = hv / (p.hv / p.hq);

    stage_rows<C, L::ESZ, L::KROW>(Kraw, p.k, tok0, n, p.hq, hk);
    if constexpr (WU) stage_rows<C, L::ESZ, L::KROW>(Vraw, p.v, tok0, n, p.hv, hv);
    if (threadIdx.x < C)
        bs[threadIdx.x] = threadIdx.x < n ? p.beta[(tok0 + threadIdx.x) * p.hv + hv] : 0.f;
    __syncthreads();

    form_a<C, DT, L::KROW, L::TROW>(Kraw, Ts, bs);
    __syncthreads();

    invert_diagonal_blocks<C, L::TROW>(Ts);
    __syncthreads();

    if constexpr (C >= 32) coupling_level<C, 16, L::TROW>(Ts);
    if constexpr (C >= 64) coupling_level<C, 32, L::TROW>(Ts);
    if constexpr (C >= 128) coupling_level<C, 64, L::TROW>(Ts);

    store_t<C, L::TROW>(Ts, p.T, tok0, n, p.hv, hv);

    if constexpr (WU) {
        if constexpr (DT == 0)
            wu_bf16<C, L::KROW, L::TROW>(Kraw, Vraw, Ts, bs, p.W, p.U, tok0, n, p.hv, hv);
        else
            wu_f32<C, L::KROW, L::TROW>(Kraw, Vraw, Ts, bs, p.W, p.U, tok0, n, p.hv, hv);
    }
}

template <int C, int DT, bool WU>
int launch_t(const LaunchArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    using L = Lds<C, DT, WU>;
    static_assert(L::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    Params p;
    p.k = a.k;
    p.v = a.v;
    p.beta = a.beta;
    p.cu = a.cu_seqlens;
    p.T = a.T;
    p.W = a.W;
    p.U = a.U;
    p.units = a.chunk_slots * a.num_v_heads;
    p.seqlen = a.seqlen;
    p.hq = a.num_qk_heads;
    p.hv = a.num_v_heads;
    p.num_seqs = a.num_seqs;
    const int64_t grid = (p.units + 7) / 8 * 8;
    auto kern = wy_prepare_kernel<C, DT, WU>;
    hipError_t e = hipSuccess;
    if (L::TOTAL > 64 * 1024)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), L::TOTAL,
                           stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (C=%d, dtype=%d, wu=%d)", hipGetErrorString(e), C, DT,
                      static_cast<int>(WU));
        return static_cast<int>(e);
    }
    return 0;
}

template <int DT, bool WU>
int launch_c(const LaunchArgs& a, hipStream_t s, char* msg, int len)
{
    switch (a.chunk_size) {
    case 32: return launch_t<32, DT, WU>(a, s, msg, len);
    case 64: return launch_t<64, DT, WU>(a, s, msg, len);
    default:
        if constexpr (DT == 1 && WU) {
            std::snprintf(msg, len, "fp32 wy_prepare at C=128 is not built");
            return static_cast<int>(hipErrorInvalidValue);
        } else {
            return launch_t<128, DT, WU>(a, s, msg, len);
        }
    }
}

}  // namespace

int launch(const LaunchArgs& a, void* stream, char* msg, int msg_len)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool wu = a.W != nullptr;
    if (a.kv_dtype == 0) return wu ? launch_c<0, true>(a, s, msg, msg_len) : launch_c<0, false>(a, s, msg, msg_len);
    return wu ? launch_c<1, true>(a, s, msg, msg_len) : launch_c<1, false>(a, s, msg, msg_len);
}

}  // namespace wyp
