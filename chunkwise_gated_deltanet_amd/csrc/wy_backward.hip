// HIP kernel (gfx950 / CDNA4) for the backward of the per-chunk WY/UT preparation of
// chunkwise (Gated) DeltaNet.
//
// Pages cited (by title and section):
//   [Inv] "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
//         lower-triangular matrix).
//   [QLA] The FlashQLA announcement, sections "使用方式" (usage) and the backward (bwd_wy).
//
// Backward of the preparation step (bf16 k / v, C = 32, 64 and 128): the gradient of
//     L = <dT, T> + <dW, W> + <dU, U>
// with respect to k, v, beta and g.  Forward per chunk and value head (D = diag(beta),
// E = diag(exp(G)), Gamma[i][j] = exp(G_i - G_j), H = Gamma o K K^T on the strict lower
// triangle):  A = I + D H,  T = A^{-1},  W = T D E K,  U = T D V.  Reverse:
//   X  = strictLower(dT + (dW K^T) D E + (dU V^T) D)     (only this part of dT_tot reaches A)
//   Y  = X T^T,  M = strictLower(-T^T Y)                   (the derivative of the inverse)
//   dK = D E (T^T dW) + (R + R^T) K,  R = D (Gamma o M)   (both key rows of each Gram entry)
//   dV = D (T^T dU)
//   dbeta_i = sum_d (T^T dW)_id e^{G_i} K_id + sum_d (T^T dU)_id V_id + sum_j M_ij H_ij
//   dG_i = beta_i e^{G_i} sum_d (T^T dW)_id K_id + sum_j Z_ij - sum_j Z_ji,  Z = M o D H
//   dg_t = sum_{i >= t} dG_i
// A unit is one (chunk, key head); a workgroup handles the value heads of a unit in turn (one
// job each) and sums their dK in registers, so dk is written once, without atomics.  Workgroups
// are persistent and walk a strided list of units; the next job's inputs are loaded while the
// current job computes.  T is recomputed with the forward's own steps (bit-identical to the T
// that wy_prepare returns).  After it the waves split in two halves that run the two
// independent products side by side: Y, M and the elementwise step on one, T^T dW and T^T dU
// with their consumers on the other.  T and R + R^T enter the bf16 products as hi + lo pairs,
// so dbeta and dg keep fp32 accuracy.
//
// Device helpers shared with the forward preparation step (unit map, T-tile layout, Gram
// fragments, block inversion, MFMA operand convention) live in wyprep_device.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "wyprep_device.h"
#include "wyprep_launch.h"

namespace wyp {
namespace {

namespace bwd {

// Workgroup shape and LDS plan per chunk size.  Eight waves at C = 64 (157 KB of LDS, one
// workgroup per CU), four at C = 32 (58 KB, two per CU).  The forward's Gram / substitution /
// coupling steps keep their own wave mapping; after them the waves split in two halves that
// run the two independent products of the reverse step side by side.
template <int C>
struct BG {
    static constexpr int NB = C / 16;
    static constexpr int BT = C == 64 ? 512 : 256;
    static constexpr int BW = BT / 64;
    static constexpr int YW = BW / 2;        // waves [0, YW): Y and M; waves [YW, BW): products over tokens
    static constexpr int ZW = BW - YW;
    static constexpr int CW = kD / 16 / ZW;  // dk column tiles per product wave
    static constexpr int KROW = kD + 8;       // bf16 per staged K / V / dW / dU row
    static constexpr int TRS = C + 4;         // floats per C x C tile row
    static constexpr int KB = C * KROW * 2;
    static constexpr int TB = C * TRS * 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = OFF_K + KB;
    static constexpr int OFF_DW = OFF_V + KB;
    static constexpr int OFF_DU = OFF_DW + KB;
    static constexpr int OFF_T = OFF_DU + KB;           // A -> T (fp32)
    static constexpr int OFF_H = OFF_T + TB;            // H = Gamma o K K^T, with H^T above the diagonal (fp32)
    static constexpr int OFF_X = OFF_H + TB;            // X, lower tiles (fp32)
    static constexpr int OFF_S = OFF_X + TB;            // S = R + R^T as hi / lo chunks
    static constexpr int OFF_B = OFF_S + TB;            // beta (C floats)
    static constexpr int PSTR = C + 16 > 80 ? C + 16 : 80;  // row-partial slot stride (floats; 16 lg + lr banks)
    static constexpr int OFF_PART = OFF_B + C * 4;      // row partials: 2 sums x ZW waves x 4 lane groups
    static constexpr int OFF_PY = OFF_PART + 2 * ZW * 4 * PSTR * 4;  // row / column sums: 2 x YW waves x 4 lane groups
    static constexpr int OFF_GD = OFF_PY + 2 * YW * 4 * PSTR * 4;  // G of the chunk's rows, fp64 (gated)
    static constexpr int OFF_INFO = OFF_GD + C * 8;
    static constexpr int LDS_TOTAL = OFF_INFO + 16;
    static_assert(OFF_X == OFF_H + TB && 2 * TB >= KB, "dk is staged as bf16 rows over H and X");
    static_assert(4 * PSTR >= 16 * 20, "a Y / M wave's row-sum slots hold its 16 x 20 transpose tile");
    static_assert(LDS_TOTAL <= 160 * 1024, "backward LDS plan exceeds 160 KiB");
    static_assert(C != 64 || 2 * ZW * 4 * PSTR >= 4 * 256, "the 32-row coupling's tmp tiles fit over the row partials");
    using TL = TLayout<C>;
    using GR = GateRow<KROW, 2>;
};

struct Params {
    const __bf16* k;
    const __bf16* v;
    const float* beta;
    const float* g;
    const int32_t* cu;
    const float* dT;
    const __bf16* dW;
    const __bf16* dU;
    __bf16* dk;
    __bf16* dv;
    float* dbeta;
    float* dg;
    int64_t units;    // chunk slots x Hq
    int32_t seqlen;
    int32_t hq;
    int32_t hv;
    int32_t num_seqs;
};

// Rows [0, n) of a [tokens, heads, 128] bf16 tensor in flight to registers (two 16-byte pieces
// per thread; rows >= n read as 0 through the buffer range), then into LDS rows of KROW
// elements.  All of a value head's rows are issued before any is waited for.
template <int C>
struct Rows {
    static constexpr int KROW = BG<C>::KROW, kBT = BG<C>::BT;
    static constexpr int NIT = C * 16 / kBT;
    u32x4 x[NIT];

    __device__ void issue(const __bf16* base, int64_t tok0, int n, int heads, int head, int tid)
    {
        const uint32_t stride = static_cast<uint32_t>(heads) * kD * 2;
        // n = 0 (no job): an empty range, every load reads 0 without touching memory
        const __amdgpu_buffer_rsrc_t r =
            rsrc(base + (tok0 * heads + head) * kD, n > 0 ? (n - 1) * stride + kD * 2 : 0u);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kBT;
            x[it] = __builtin_amdgcn_raw_buffer_load_b128(r, (q >> 4) * stride + (q & 15) * 16, 0, kStream);
        }
    }

    __device__ void commit(unsigned char* dst, int tid) const
    {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kBT;
            *reinterpret_cast<u32x4*>(dst + (q >> 4) * (KROW * 2) + (q & 15) * 16) = x[it];
        }
    }
};

// The inputs of one job (one value head hv of a unit: first token tok0, n tokens, key head hk)
// in flight to registers: k (read only for the first value head of a unit), v, dW, dU, beta and
// g.  n = 0 (past the last job) issues loads over empty ranges, so the issue has no branches.
template <int C, bool GT>
struct JobIn {
    Rows<C> k, v, dw, du;
    float b, g;

    __device__ void issue(const Params& p, int64_t tok0, int n, int hk, int hv, bool with_k, int tid)
    {
        k.issue(p.k, tok0, with_k ? n : 0, p.hq, hk, tid);
        v.issue(p.v, tok0, n, p.hv, hv, tid);
        dw.issue(p.dW, tok0, n, p.hv, hv, tid);
        du.issue(p.dU, tok0, n, p.hv, hv, tid);
        const uint32_t bytes = n > 0 ? ((n - 1) * p.hv + 1) * 4 : 0u;
        const __amdgpu_buffer_rsrc_t br = rsrc(p.beta + tok0 * p.hv + hv, bytes);
        b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, (tid & 63) * p.hv * 4, 0, 0));
        g = 0.f;
        if constexpr (GT) {
            const __amdgpu_buffer_rsrc_t gr = rsrc(p.g + tok0 * p.hv + hv, bytes);
            g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, (tid & 63) * p.hv * 4, 0, 0));
        }
    }
};

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest even, two
// values per conversion: hi / lo of x[2p], x[2p + 1] land in 32-bit word p of `hi` / `lo`.
template <int N>
__device__ inline void split_hilo(const float (&x)[N], unsigned (&hi)[N / 2], unsigned (&lo)[N / 2])
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int p = 0; p < N / 2; ++p) {
        const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2 * p], x[2 * p + 1]}, bf16x2));
        const float h0 = __builtin_bit_cast(float, h << 16), h1 = __builtin_bit_cast(float, h & 0xffff0000u);
        hi[p] = h;
        lo[p] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x[2 * p] - h0, x[2 * p + 1] - h1}, bf16x2));
    }
}

// Four values as one 16-byte chunk: hi of x[0..3], then lo of x[0..3].
__device__ inline u32x4 pack_hilo(f32x4 x)
{
    const float v[4] = {x[0], x[1], x[2], x[3]};
    unsigned h[2], l[2];
    split_hilo<4>(v, h, l);
    return u32x4{h[0], h[1], l[0], l[1]};
}

// A fragment of the transposed product over 32 tokens: lane 16 g + c gets column 16 ni + c of
// rows t0 + 8 g .. t0 + 8 g + 7 of the staged bf16 rows (two transposed 4 x 16 LDS reads).
template <int KROW>
__device__ inline bf16x8 tr_frag(const __bf16* base, int t0, int ni, int lr, int lg)
{
    const __bf16* p0 = base + (t0 + 8 * lg + (lr >> 2)) * KROW + 16 * ni + 4 * (lr & 3);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * KROW));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline bf16x8 cat_u32(unsigned a, unsigned b, unsigned c, unsigned d)
{
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8, u32x4v{a, b, c, d});
}

// (R + R^T) K for the dk column tiles ni = zw + ZW c of product wave zw, over 32 tokens per
// bf16 MFMA: acc[c][mi] += sum_t K(t, ni)^T S(t, mi), where the K fragments come from transposed
// LDS reads and S(t, i) is read from the packed hi / lo chunks of row i of `bp` (S is
// symmetric, so its rows are also its columns).  Accumulator element r of lane 16 g + c is
// (.)[16 ni + 4 g + r][16 mi + c].
template <int C>
__device__ inline void tr_products(const unsigned char* src, const float* bp, int zw, int lr, int lg,
                                   f32x4 (&acc)[BG<C>::CW][BG<C>::NB])
{
    using BGC = BG<C>;
    constexpr int kNB = BGC::NB, kZW = BGC::ZW, kCW = BGC::CW;
    constexpr int KROW = BGC::KROW, TRS = BGC::TRS;
    const __bf16* base = reinterpret_cast<const __bf16*>(src);
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
        bf16x8 bh[kNB], bl[kNB];
#pragma unroll
        for (int mi = 0; mi < kNB; ++mi) {
            const float* row = bp + (16 * mi + lr) * TRS + 32 * ks + 8 * lg;
            const u32x4 c0 = *reinterpret_cast<const u32x4*>(row);
            const u32x4 c1 = *reinterpret_cast<const u32x4*>(row + 4);
            bh[mi] = cat_u32(c0[0], c0[1], c1[0], c1[1]);
            bl[mi] = cat_u32(c0[2], c0[3], c1[2], c1[3]);
        }
#pragma unroll
        for (int c = 0; c < kCW; ++c) {
            const bf16x8 xa = tr_frag<KROW>(base, 32 * ks, zw + kZW * c, lr, lg);
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) {
                acc[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh[mi], acc[c][mi], 0, 0, 0);
                acc[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl[mi], acc[c][mi], 0, 0, 0);
            }
        }
    }
}

// T^T dW and T^T dU for the dk column tiles of product wave zw, over 32 tokens per bf16 MFMA:
// aw[c][mi] (au) element r of lane 16 g + c' is (T^T dW)[16 mi + c'][16 ni + 4 g + r].  The B
// fragments of T^T are read as columns of T (fp32, one 4-byte read per row) and split into
// hi / lo bf16 once for both products.  T[t][i] = 0 for t < i, so token steps entirely above
// tile mi are skipped.
template <int C>
__device__ inline void z_products(const unsigned char* dWraw, const unsigned char* dUraw, const float* Ts, int zw,
                                  int lr, int lg, f32x4 (&aw)[BG<C>::CW][BG<C>::NB],
                                  f32x4 (&au)[BG<C>::CW][BG<C>::NB])
{
    using BGC = BG<C>;
    constexpr int kNB = BGC::NB, kZW = BGC::ZW, kCW = BGC::CW;
    constexpr int KROW = BGC::KROW, TRS = BGC::TRS;
    const __bf16* dWb = reinterpret_cast<const __bf16*>(dWraw);
    const __bf16* dUb = reinterpret_cast<const __bf16*>(dUraw);
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
        bf16x8 bh[kNB], bl[kNB];
#pragma unroll
        for (int mi = 0; mi < kNB; ++mi) {
            if (16 * mi > 32 * ks + 31) continue;  // constant after unrolling
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = Ts[(32 * ks + 8 * lg + j) * TRS + 16 * mi + lr];
            unsigned h[4], l[4];
            split_hilo<8>(x, h, l);
            bh[mi] = cat_u32(h[0], h[1], h[2], h[3]);
            bl[mi] = cat_u32(l[0], l[1], l[2], l[3]);
        }
#pragma unroll
        for (int c = 0; c < kCW; ++c) {
            const bf16x8 xw = tr_frag<KROW>(dWb, 32 * ks, zw + kZW * c, lr, lg);
            const bf16x8 xu = tr_frag<KROW>(dUb, 32 * ks, zw + kZW * c, lr, lg);
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) {
                if (16 * mi > 32 * ks + 31) continue;
                aw[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, bh[mi], aw[c][mi], 0, 0, 0);
                au[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xu, bh[mi], au[c][mi], 0, 0, 0);
                aw[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, bl[mi], aw[c][mi], 0, 0, 0);
                au[c][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xu, bl[mi], au[c][mi], 0, 0, 0);
            }
        }
    }
}

// Y = X T^T, M = strictLower(-T^T Y) and the elementwise step for column tile J of M, rows
// I0 .. I1, on one wave with no barrier.  The Y tiles (Mt, J), Mt >= I0, stay in registers,
// where an accumulator's element q of lane 16 g + c (row 4 g + q, column c) is exactly the B
// operand of step q of T^T Y and the A operand of step q of Y^T T; T's columns (fp32) are the
// other operand of both.  So each tile of M comes in two layouts at the cost of its MFMAs alone:
// m (lane 16 g + c holds rows 16 I + 4 g .. + 3 of column 16 J + c) and mt (row 16 I + c,
// columns 16 J + 4 g .. + 3).  From them, with R = D (Gamma o M) and S = R + R^T:
//   - mt gives row i's chunk of S left of the diagonal (R_ij) and the row sum sum_j M_ij H_ij;
//   - m gives row j's chunk of S right of the diagonal (R_ij again, S symmetric) and the column
//     sum sum_i beta_i M_ij H_ij;
// a diagonal tile's chunk takes its lower entries from mt and its upper ones from m.  S goes to
// Ss as hi / lo chunks; the sums accumulate in rowp[I] (row 16 I + c) and colp[J] (row 16 J + c).
template <int C, bool GT, int J, int I0, int I1>
__device__ inline void ym_column(const float* Xs, const float* Ts, const float* Hs, const float* bs, const double* Gd,
                                 float* Ss, float* scratch, int lr, int lg, float (&rowp)[C / 16],
                                 float (&colp)[C / 16])
{
    constexpr int NB = C / 16, TRS = BG<C>::TRS;
    f32x4 y[NB];
#pragma unroll
    for (int Mt = I0; Mt < NB; ++Mt) y[Mt] = zero4();
#pragma unroll
    for (int L = 0; L <= J; ++L) {  // Y(Mt, J) = sum_{L <= J} X(Mt, L) T(J, L)^T
        const f32x4 b = *reinterpret_cast<const f32x4*>(Ts + (16 * J + lr) * TRS + 16 * L + 4 * lg);
#pragma unroll
        for (int Mt = I0; Mt < NB; ++Mt) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(Xs + (16 * Mt + lr) * TRS + 16 * L + 4 * lg);
#pragma unroll
            for (int q = 0; q < 4; ++q) y[Mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], y[Mt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // one k step's operands in registers at a time
    }
    f32x4 m[NB], mt[NB];  // -M in the two layouts
#pragma unroll
    for (int I = I0; I <= I1; ++I) mt[I] = zero4();
#pragma unroll
    for (int Mt = I0; Mt < NB; ++Mt) {  // M(I, J)^T = -sum_{Mt >= I} Y(Mt, J)^T T(Mt, I)
#pragma unroll
        for (int I = I0; I <= I1 && I <= Mt; ++I) {
            f32x4 a;
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] = Ts[(16 * Mt + 4 * lg + q) * TRS + 16 * I + lr];
#pragma unroll
            for (int q = 0; q < 4; ++q) mt[I] = __builtin_amdgcn_mfma_f32_16x16x4f32(y[Mt][q], a[q], mt[I], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // m from mt by a transpose through this wave's own 16 x 20 scratch tile (its LDS operations
    // run in order, so no barrier is needed; 20-float rows keep both sides conflict-free)
#pragma unroll
    for (int I = I0; I <= I1; ++I) {
        *reinterpret_cast<f32x4*>(scratch + lr * 20 + 4 * lg) = mt[I];
#pragma unroll
        for (int r = 0; r < 4; ++r) m[I][r] = scratch[(4 * lg + r) * 20 + lr];
    }
    const int jc = 16 * J + lr;  // the m layout's column
    double gjc = 0.0;
    if constexpr (GT) gjc = Gd[jc];
#pragma unroll
    for (int I = I0; I <= I1; ++I) {
        const int i = 16 * I + lr;  // the mt layout's row
        const float bi = bs[i];
        double gi = 0.0;
        if constexpr (GT) gi = Gd[i];
        // row i, columns 16 J + 4 g ..: H_ij (j < i); row jc, columns 16 I + 4 g ..: H_i'jc (i' > jc)
        const f32x4 hrow = *reinterpret_cast<const f32x4*>(Hs + i * TRS + 16 * J + 4 * lg);
        const f32x4 hcol = *reinterpret_cast<const f32x4*>(Hs + jc * TRS + 16 * I + 4 * lg);
        const f32x4 bcol = *reinterpret_cast<const f32x4*>(bs + 16 * I + 4 * lg);  // beta_i'
        f32x4 slow, sup;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * J + 4 * lg + r;   // mt: M[i][j]
            const int ir = 16 * I + 4 * lg + r;  // m: M[ir][jc]
            const float Mr = -mt[I][r], Mc = -m[I][r];
            float grow = 1.f, gcol = 1.f;
            if constexpr (GT) {  // decay from the earlier to the later token
                grow = __expf(static_cast<float>(gi - Gd[j]));
                gcol = __expf(static_cast<float>(Gd[ir] - gjc));
            }
            const bool lo_ok = I > J || j < i;    // constant for I > J
            const bool up_ok = I > J || ir > jc;
            slow[r] = lo_ok ? bi * grow * Mr : 0.f;
            sup[r] = up_ok ? bcol[r] * gcol * Mc : 0.f;
            rowp[I] += lo_ok ? Mr * hrow[r] : 0.f;
            colp[J] += up_ok ? bcol[r] * Mc * hcol[r] : 0.f;
        }
        if (I > J) {  // constant after unrolling
            *reinterpret_cast<u32x4*>(Ss + i * TRS + 16 * J + 4 * lg) = pack_hilo(slow);
            *reinterpret_cast<u32x4*>(Ss + jc * TRS + 16 * I + 4 * lg) = pack_hilo(sup);
        } else {  // row i = jc: lower entries from mt, upper ones from m, 0 on the diagonal
            *reinterpret_cast<u32x4*>(Ss + i * TRS + 16 * J + 4 * lg) = pack_hilo(slow + sup);
        }
    }
}

// Accumulators of product wave zw (element r of lane 16 g + c = X[16 mi + c][16 ni + 4 g + r])
// as bf16 into its own columns of the staged rows at `dst` (rows of KROW elements).
template <int C>
__device__ inline void stage_rows(unsigned char* dst, const f32x4 (&acc)[BG<C>::CW][BG<C>::NB], int zw, int lr,
                                  int lg)
{
    using BGC = BG<C>;
    constexpr int kNB = BGC::NB, kZW = BGC::ZW, kCW = BGC::CW, KROW = BGC::KROW;
    __bf16* d = reinterpret_cast<__bf16*>(dst);
#pragma unroll
    for (int c = 0; c < kCW; ++c)
#pragma unroll
        for (int mi = 0; mi < kNB; ++mi) {
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(acc[c][mi][r]);
            *reinterpret_cast<bf16x4*>(d + (16 * mi + lr) * KROW + 16 * (zw + kZW * c) + 4 * lg) = o;
        }
}

// Staged rows [0, n) at `src` to a [tokens, heads, 128] tensor, by every thread.
template <int C>
__device__ inline void store_rows(const unsigned char* src, __bf16* out, int64_t tok0, int n, int heads, int head,
                                  int tid)
{
    constexpr int KROW = BG<C>::KROW, kBT = BG<C>::BT;
    const uint32_t stride = static_cast<uint32_t>(heads) * kD * 2;
    const __amdgpu_buffer_rsrc_t r = rsrc(out + (tok0 * heads + head) * kD, (n - 1) * stride + kD * 2);
#pragma unroll
    for (int it = 0; it < Rows<C>::NIT; ++it) {
        const int q = tid + it * kBT;
        const u32x4 val = *reinterpret_cast<const u32x4*>(src + (q >> 4) * (KROW * 2) + (q & 15) * 16);
        __builtin_amdgcn_raw_buffer_store_b128(val, r, (q >> 4) * stride + (q & 15) * 16, 0, kStream);
    }
}

// A = I + strictLower(D H) into Ts exactly as the forward's form_a writes it (diagonal tiles
// keep L^T in their upper triangle for the substitution), and H = Gamma o K K^T into Hs, from one
// Gram per lower tile, over the eight waves.  Hs holds H below the diagonal and its transpose
// above (Hs[j][i] = H[i][j] for i > j; 0 on the diagonal), so row i of Hs lists H_ij for j < i
// and H_ji for j > i: the elementwise step then reads rows only.
template <int C, bool GT>
__device__ void form_a_h(const unsigned char* Kraw, float* Ts, float* Hs, const float* bs, int wave, int lr,
                         int lg)
{
    using BGC = BG<C>;
    constexpr int kC = C, kNB = BGC::NB, kBT = BGC::BT, kBW = BGC::BW, kCW = BGC::CW;
    constexpr int KROW = BGC::KROW, TRS = BGC::TRS;
    using TL = typename BGC::TL;
    using GR = typename BGC::GR;

    constexpr int NTILE = kNB * (kNB + 1) / 2;
    for (int t = wave; t < NTILE; t += kBW) {  // uniform
        int I = 0, J = 0;
        tile_of(t, &I, &J);
        GramFrags<0, KROW> f;
        f.load(Kraw, I, J, lr, lg);
        const f32x4 acc = f.product();
        const f32x4 bet = *reinterpret_cast<const f32x4*>(bs + 16 * I + 4 * lg);
        const float bcol = bs[16 * J + lr];
        double gcol = 0.0;
        if constexpr (GT) gcol = GR::G(Kraw, 16 * J + lr);
        f32x4 hv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr, j = 16 * J + lr;
            float a = acc[rr];
            if constexpr (GT) {
                const double d = GR::G(Kraw, i) - gcol;
                a *= __expf(static_cast<float>(i > j ? d : -d));
            }
            Ts[i * TRS + j] = (i > j) ? bet[rr] * a : (i == j ? 1.f : bcol * a);
            // a diagonal tile above its diagonal holds Gram_ij Gamma_ji = H_ji already
            Hs[i * TRS + j] = i != j ? a : 0.f;
            hv[rr] = a;
        }
        if (I > J)  // uniform: H^T of the tile into the upper tile (J, I), one 16-byte row chunk
            *reinterpret_cast<f32x4*>(Hs + (16 * J + lr) * TRS + 16 * I + 4 * lg) = hv;
    }
    for (int t = wave; t < kNB * (kNB - 1) / 2; t += kBW) {  // strict upper tiles
        int Iu = 0, rem = t;
        while (rem >= kNB - 1 - Iu) {
            rem -= kNB - 1 - Iu;
            ++Iu;
        }
        const int Ju = Iu + 1 + rem;
        *reinterpret_cast<f32x4*>(Ts + (16 * Iu + lr) * TRS + 16 * Ju + 4 * lg) = zero4();
    }
}

// a6 at S = 32 for C = 64 on waves 0-3 (coupling_level runs it on two waves, one of them with 28
// dependent fp32 MFMAs), in two passes: tmp = L10 X00 tile by tile into `tmpb` (one 16-byte
// chunk per lane and tile), barrier, X10 = -X11 tmp over L10, which no wave reads any more.
// Each wave takes one tile of each pass, three MFMA steps in all; every sum runs in
// coupling_level's order (its products with the zero tiles above X00's diagonal skipped), so T
// is the same.
template <int C>
__device__ __attribute__((always_inline)) void coupling32_4w(float* Ts, float* tmpb, int wave, int lane, int lr,
                                                             int lg)
{
    using TL = typename BG<C>::TL;
    static_assert(C == 64, "one 32-row pair");
    constexpr int S = 32, TS = 2;
    if (wave < 4) {  // uniform; pass A: tmp(mr, nc) = sum_{kt >= nc} L10(mr, kt) X00(kt, nc)
        const int mr = wave >> 1, nc = wave & 1;
        f32x4 acc = zero4();
        for (int kt = nc; kt < TS; ++kt) {
            float bq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bq[q] = Ts[TL::off(16 * kt + 4 * lg + q, 16 * nc + lr)];
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + TL::off(S + 16 * mr + lr, 16 * kt + 4 * lg));
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bq[q], acc, 0, 0, 0);
        }
        *reinterpret_cast<f32x4*>(tmpb + (mr * TS + nc) * 256 + 4 * lane) = acc;
    }
    __syncthreads();
    if (wave < 4) {  // uniform; pass B: X10(mr, nc) = -sum_{kt <= mr} X11(mr, kt) tmp(kt, nc)
        const int nc = wave >> 1, mr = wave & 1;
        f32x4 acc = zero4();
        for (int kt = 0; kt <= mr; ++kt) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + TL::off(S + 16 * mr + lr, S + 16 * kt + 4 * lg));
            const f32x4 bv = *reinterpret_cast<const f32x4*>(tmpb + (kt * TS + nc) * 256 + 4 * lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[TL::off(S + 16 * mr + 4 * lg + r, 16 * nc + lr)] = -acc[r];
    }
    __syncthreads();
}

// Batch rows: the units logical, logical + G, logical + 2 G, ... of one workgroup, walked without
// a division per step.  logical = slot * H + head and slot = b * cps + c, so a step of G adds
// G mod H to the head (carrying one slot) and G div H (or one more) slots, split once per
// workgroup into whole rows and chunks.
struct BatchWalk {
    uint32_t head, c, b, H, cps, dhead, dq0, dr0, dq1, dr1;

    __device__ void init(uint32_t logical, uint32_t G, uint32_t heads, uint32_t chunks_per_row)
    {
        H = heads;
        cps = chunks_per_row;
        const uint32_t slot = logical / H;
        head = logical % H;
        b = slot / cps;
        c = slot % cps;
        dhead = G % H;
        const uint32_t dslot = G / H;
        dq0 = dslot / cps;
        dr0 = dslot % cps;
        dq1 = (dslot + 1) / cps;
        dr1 = (dslot + 1) % cps;
    }
    __device__ void step()
    {
        head += dhead;
        const bool carry = head >= H;
        head = carry ? head - H : head;
        c += carry ? dr1 : dr0;
        b += carry ? dq1 : dq0;
        if (c >= cps) {
            c -= cps;
            ++b;
        }
    }
    template <int C>
    __device__ Unit unit(int seqlen, bool valid) const
    {
        Unit u;
        u.tok0 = static_cast<int64_t>(b) * seqlen + static_cast<int64_t>(c) * C;
        u.n = valid ? min(C, seqlen - static_cast<int>(c) * C) : 0;
        u.hv = static_cast<int>(head);
        return u;
    }
};

template <int C, bool GT>
__global__ __launch_bounds__(BG<C>::BT, 2) void wy_backward_kernel(Params p)
{
    using BGC = BG<C>;
    constexpr int kC = C, kNB = BGC::NB, kBT = BGC::BT, kBW = BGC::BW, kCW = BGC::CW;
    constexpr int kYW = BGC::YW, kZW = BGC::ZW;
    constexpr int KROW = BGC::KROW, TRS = BGC::TRS;
    using TL = typename BGC::TL;
    using GR = typename BGC::GR;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* Kraw = smem + BGC::OFF_K;
    unsigned char* Vraw = smem + BGC::OFF_V;
    unsigned char* dWraw = smem + BGC::OFF_DW;
    unsigned char* dUraw = smem + BGC::OFF_DU;
    float* Ts = reinterpret_cast<float*>(smem + BGC::OFF_T);
    float* Hs = reinterpret_cast<float*>(smem + BGC::OFF_H);
    float* Xs = reinterpret_cast<float*>(smem + BGC::OFF_X);
    float* Ss = reinterpret_cast<float*>(smem + BGC::OFF_S);
    float* bs = reinterpret_cast<float*>(smem + BGC::OFF_B);
    float* part = reinterpret_cast<float*>(smem + BGC::OFF_PART);
    float* py = reinterpret_cast<float*>(smem + BGC::OFF_PY);
    double* Gd = reinterpret_cast<double*>(smem + BGC::OFF_GD);
    int* info = reinterpret_cast<int*>(smem + BGC::OFF_INFO);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;

    // unit -> (first token, n, key head): the forward's map with key heads in place of value heads
    wyp::Params mp{};
    mp.cu = p.cu;
    mp.units = p.units;
    mp.seqlen = p.seqlen;
    mp.hq = p.hq;
    mp.hv = p.hq;
    mp.num_seqs = p.num_seqs;
    const int r = p.hv / p.hq;
    // Persistent: the grid holds one resident round, dealt round-robin to the 8 XCDs; each
    // workgroup takes a contiguous range of units per round, so the value heads of a key head
    // and neighbouring chunks meet in one L2.  Jobs (one value head of a unit) run in turn,
    // and the next job's inputs are in flight while the current one computes.
    const uint32_t G = gridDim.x;  // a multiple of 8
    int64_t logical = static_cast<int64_t>(blockIdx.x & 7u) * (G >> 3) + (blockIdx.x >> 3);
    BatchWalk walk{};
    Unit u;
    if (p.cu == nullptr) {  // uniform
        walk.init(static_cast<uint32_t>(logical), G, static_cast<uint32_t>(p.hq),
                  static_cast<uint32_t>((p.seqlen + kC - 1) / kC));
        u = walk.unit<kC>(p.seqlen, logical < p.units);
    } else {
        u = map_unit<kC>(mp, info, logical, G, tid);
    }
    if (u.n <= 0) return;  // uniform
    int hv = u.hv * r;
    bool new_unit = true;
    JobIn<C, GT> in;
    in.issue(p, u.tok0, u.n, u.hv, hv, true, tid);
    f32x4 dk_acc[kCW][kNB];
#pragma unroll
    for (int c = 0; c < kCW; ++c)
#pragma unroll
        for (int mi = 0; mi < kNB; ++mi) dk_acc[c][mi] = zero4();

    auto job = [&]() -> bool {
        // The lane indices are made opaque once per job, so the many per-lane LDS addresses
        // derived from them are formed where they are used instead of being hoisted out of the
        // persistent loop and held in registers across the whole job.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = uniform(tid >> 6);
        const int lr = lane & 15, lg = lane >> 4;
        const int hk = u.hv;
        const int64_t tok0 = u.tok0;
        const int n = u.n;
        // ---- this job's inputs to LDS
        if (new_unit) in.k.commit(Kraw, tid);
        in.v.commit(Vraw, tid);
        in.dw.commit(dWraw, tid);
        in.du.commit(dUraw, tid);
        if (tid < kC) bs[tid] = in.b;
        if constexpr (GT) {
            if (tid < 64) {  // G = inclusive prefix sums of g in fp64 (as the forward)
                double x = static_cast<double>(in.g);  // 0 past the chunk's rows
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const double t = __shfl_up(x, d);
                    if (tid >= d) x += t;
                }
                if (tid < kC) {  // the chunk's C rows
                    *GR::Gp(Kraw, tid) = x;
                    *GR::Ep(Kraw, tid) = __expf(static_cast<float>(x));
                    Gd[tid] = x;
                }
            }
        }
        __syncthreads();
        // ---- the next job (the next value head of this unit, else the first of the next unit).  Its
        // loads are issued where the issuing waves would otherwise wait: the product waves before
        // the coupling levels (which run on waves 0-1), the Y / M waves at the start of their
        // products (they finish well before the product waves).
        Unit nu = u;
        int nhv = hv + 1;
        bool nnew = false;
        if (nhv == (hk + 1) * r) {  // uniform
            logical += G;
            if (p.cu == nullptr) {  // uniform
                walk.step();
                nu = walk.unit<kC>(p.seqlen, logical < p.units);
            } else {
                nu = map_unit<kC>(mp, info, logical, G, tid);
            }
            nhv = nu.hv * r;
            nnew = true;
        }

        // ---- A (into Ts) and H = Gamma o K K^T (strict lower, into Hs)
        form_a_h<C, GT>(Kraw, Ts, Hs, bs, wave, lr, lg);
        __syncthreads();
        // ---- wave 0 inverts the diagonal blocks of A (its substitutions are one long dependency
        // chain); meanwhile the other waves form X, which does not depend on T
        if (wave == 0) {  // uniform
            __builtin_amdgcn_s_setprio(2);  // the chain: its instructions go first on the SIMD
            invert_diagonal_blocks<kC, TL>(Ts, tid);
            __builtin_amdgcn_s_setprio(0);
        } else {
            // ---- X = strictLower(dT + (dW K^T) D E + (dU V^T) D), lower tiles on bf16 MFMA.  The dT
            // reads sit in their own instance of the tile loop: without dT the loop issues no memory
            // operation, so nothing in it waits for the next job's loads in flight.
            {
                auto x_tiles = [&](auto with_dt) {
                    constexpr bool DT = decltype(with_dt)::value;
                    const __amdgpu_buffer_rsrc_t dtr =
                        rsrc(DT ? p.dT + (tok0 * p.hv + hv) * kC : nullptr,
                             DT ? (n - 1) * static_cast<uint32_t>(p.hv) * kC * 4 + kC * 4 : 0u);
                    constexpr int NTILE = kNB * (kNB + 1) / 2;
                    for (int t = wave - 1; t < NTILE; t += kBW - 1) {  // uniform
                        int I = 0, J = 0;
                        tile_of(t, &I, &J);
                        f32x4 pw = zero4(), pu = zero4();
                        const __bf16* dWb = reinterpret_cast<const __bf16*>(dWraw);
                        const __bf16* dUb = reinterpret_cast<const __bf16*>(dUraw);
                        const __bf16* Kb = reinterpret_cast<const __bf16*>(Kraw);
                        const __bf16* Vb = reinterpret_cast<const __bf16*>(Vraw);
#pragma unroll
                        for (int s = 0; s < kD / 32; ++s) {
                            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(dWb + (16 * I + lr) * KROW + 32 * s + 8 * lg);
                            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(Kb + (16 * J + lr) * KROW + 32 * s + 8 * lg);
                            const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(dUb + (16 * I + lr) * KROW + 32 * s + 8 * lg);
                            const bf16x8 b2 = *reinterpret_cast<const bf16x8*>(Vb + (16 * J + lr) * KROW + 32 * s + 8 * lg);
                            pw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, pw, 0, 0, 0);
                            pu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b2, pu, 0, 0, 0);
                        }
                        const int j = 16 * J + lr;
                        const float bj = bs[j];
                        const float ej = GT ? GR::E(Kraw, j) : 1.f;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int i = 16 * I + 4 * lg + rr;
                            float x = 0.f;
                            if (i > j) {
                                float dt = 0.f;
                                if constexpr (DT)
                                    dt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                       dtr, i * p.hv * kC * 4 + j * 4, 0, 0));
                                x = dt + pw[rr] * bj * ej + pu[rr] * bj;
                            }
                            Xs[i * TRS + j] = x;
                        }
                    }
                };
                if (p.dT != nullptr)  // uniform
                    x_tiles(std::true_type{});
                else
                    x_tiles(std::false_type{});
            }
        }
        __syncthreads();
        if (wave >= kYW) in.issue(p, nu.tok0, nu.n, nu.hv, nhv, nnew, tid);  // uniform
        coupling_level<kC, 16, TL>(Ts, tid);
        if constexpr (kC >= 64) coupling32_4w<kC>(Ts, part, wave, lane, lr, lg);  // tmp over the row partials
        const int zw = wave - kYW;
        const bool last_head = hv == (hk + 1) * r - 1;  // uniform

        // ---- Two independent products at once.  Waves [0, YW): Y = X T^T, M = strictLower(-T^T Y)
        // and the elementwise step, by column tiles of M: S = R + R^T into Ss, and the row and
        // column sums into their slots.  Waves [YW, BW): T^T dW and T^T dU with their consumers:
        // dK += D E T^T dW, dV = D T^T dU (staged over dU in the wave's own columns), and the
        // per-row sums for dbeta and dG.
        if (wave < kYW) {  // uniform
            in.issue(p, nu.tok0, nu.n, nu.hv, nhv, nnew, tid);
            float rowp[kNB], colp[kNB];
#pragma unroll
            for (int I = 0; I < kNB; ++I) rowp[I] = colp[I] = 0.f;
            if constexpr (kC == 64) {
                if (wave == 0) {
                    ym_column<64, GT, 0, 0, 1>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                } else if (wave == 1) {
                    ym_column<64, GT, 1, 1, 3>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                } else if (wave == 2) {
                    ym_column<64, GT, 2, 2, 3>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                } else {
                    ym_column<64, GT, 0, 2, 3>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                    ym_column<64, GT, 3, 3, 3>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                }
            } else {
                if (wave == 0)
                    ym_column<32, GT, 0, 0, 1>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
                else
                    ym_column<32, GT, 1, 1, 1>(Xs, Ts, Hs, bs, Gd, Ss, py + wave * 4 * BGC::PSTR, lr, lg, rowp, colp);
            }
            // one slot per (wave, lane group); rows and columns this wave does not touch get 0.  The
            // row-sum slots of this wave served as its transpose scratch above.
#pragma unroll
            for (int I = 0; I < kNB; ++I) {
                py[((0 * kYW + wave) * 4 + lg) * BGC::PSTR + 16 * I + lr] = rowp[I];
                py[((1 * kYW + wave) * 4 + lg) * BGC::PSTR + 16 * I + lr] = colp[I];
            }
        } else {
            const __bf16* Kb = reinterpret_cast<const __bf16*>(Kraw);
            const __bf16* Vb = reinterpret_cast<const __bf16*>(Vraw);
            f32x4 aw[kCW][kNB], au[kCW][kNB];
#pragma unroll
            for (int c = 0; c < kCW; ++c)
#pragma unroll
                for (int mi = 0; mi < kNB; ++mi) aw[c][mi] = au[c][mi] = zero4();
            z_products<C>(dWraw, dUraw, Ts, zw, lr, lg, aw, au);
            // element r of lane 16 g + c: (T^T dW)[i = 16 mi + c][d = 16 ni + 4 g + r]
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) {
                const int i = 16 * mi + lr;
                const float bi = bs[i];
                const float ei = GT ? GR::E(Kraw, i) : 1.f;
                float sk = 0.f;
#pragma unroll
                for (int c = 0; c < kCW; ++c) {
                    const bf16x4 kv = *reinterpret_cast<const bf16x4*>(Kb + i * KROW + 16 * (zw + kZW * c) + 4 * lg);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        sk += aw[c][mi][rr] * static_cast<float>(kv[rr]);
                        dk_acc[c][mi][rr] += bi * ei * aw[c][mi][rr];
                    }
                }
                part[((0 * kZW + zw) * 4 + lg) * BGC::PSTR + i] = sk;  // one slot per lane group
            }
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) {
                const int i = 16 * mi + lr;
                const float bi = bs[i];
                float sv = 0.f;
#pragma unroll
                for (int c = 0; c < kCW; ++c) {
                    const bf16x4 vv = *reinterpret_cast<const bf16x4*>(Vb + i * KROW + 16 * (zw + kZW * c) + 4 * lg);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        sv += au[c][mi][rr] * static_cast<float>(vv[rr]);
                        au[c][mi][rr] *= bi;  // dV
                    }
                }
                part[((1 * kZW + zw) * 4 + lg) * BGC::PSTR + i] = sv;
            }
            // this wave alone reads and writes its columns of dU
            stage_rows<C>(dUraw, au, zw, lr, lg);
        }
        __syncthreads();

        store_rows<C>(dUraw, p.dv, tok0, n, p.hv, hv, tid);  // dV out

        // ---- product waves: (R + R^T) K into dK (bf16 MFMA, S hi / lo; S is symmetric, so its row
        // chunks are also the column chunks the product needs), and after a unit's last value
        // head dk staged over H and X.  Wave 0: dbeta, dG, dg of this value head (lanes past the
        // chunk's C rows hold 0; their stores fall outside the n-row buffer range).
        if (wave >= kYW) {  // uniform
            tr_products<C>(Kraw, Ss, zw, lr, lg, dk_acc);
            if (last_head) {  // uniform
                stage_rows<C>(smem + BGC::OFF_H, dk_acc, zw, lr, lg);
#pragma unroll
                for (int c = 0; c < kCW; ++c)
#pragma unroll
                    for (int mi = 0; mi < kNB; ++mi) dk_acc[c][mi] = zero4();
            }
        } else if (wave == 0) {
            const int i = tid;
            const bool row = i < kC;
            float sk = 0.f, sv = 0.f, mh = 0.f, cz = 0.f;
            if (row) {  // the (wave, lane group) slots in a fixed order
#pragma unroll
                for (int w = 0; w < kZW * 4; ++w) {
                    sk += part[(0 * kZW * 4 + w) * BGC::PSTR + i];
                    sv += part[(1 * kZW * 4 + w) * BGC::PSTR + i];
                }
#pragma unroll
                for (int w = 0; w < kYW * 4; ++w) {
                    mh += py[(0 * kYW * 4 + w) * BGC::PSTR + i];
                    cz += py[(1 * kYW * 4 + w) * BGC::PSTR + i];
                }
            }
            // dbeta_i: sum_d (T^T dW)_id e^{G_i} K_id + sum_d (T^T dU)_id V_id + sum_j M_ij H_ij;
            // dG_i: beta_i e^{G_i} sum_d (T^T dW)_id K_id + sum_j Z_ij - sum_j Z_ji (Z = M o D H)
            const float bi = row ? bs[i] : 0.f;
            const float ei = GT && row ? GR::E(Kraw, i) : 1.f;
            const float db = row ? sk * ei + sv + mh : 0.f;
            float dG = row ? bi * ei * sk + bi * mh - cz : 0.f;
            const __amdgpu_buffer_rsrc_t br = rsrc(p.dbeta + tok0 * p.hv + hv, ((n - 1) * p.hv + 1) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, db), br, i * p.hv * 4, 0, 0);
            if constexpr (GT) {
                // dg_t = sum_{i >= t} dG_i: a reverse inclusive scan over the 64 lanes
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const float t = __shfl_down(dG, d);
                    if (i + d < 64) dG += t;
                }
                const __amdgpu_buffer_rsrc_t gr = rsrc(p.dg + tok0 * p.hv + hv, ((n - 1) * p.hv + 1) * 4);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, dG), gr, i * p.hv * 4, 0, 0);
            }
        }
        // Every read of this value head's K, V, dW, dU, beta and partial sums is done past this
        // barrier, so the next commit may overwrite them; the staged dk (over H and X) is
        // rewritten only after the next job's first barrier.
        __syncthreads();
        if (last_head) store_rows<C>(smem + BGC::OFF_H, p.dk, tok0, n, p.hq, hk, tid);  // uniform
        u = nu;
        hv = nhv;
        new_unit = nnew;
        return u.n > 0;
    };
    // The first job is peeled off the loop: the loop head is then reached only from the end of
    // a job, so the memory-counter waits inside see one issue history.
    if (job()) {
        while (job()) {
        }
    }
}

template <int C, bool GT>
int launch_t(const BwdArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    constexpr int LDS_TOTAL = BG<C>::LDS_TOTAL, kBT = BG<C>::BT;
    // Per device, once: raise the kernel's dynamic LDS limit and count its resident workgroups
    // (occupancy x CUs), so later launches (also under stream capture) make no attribute calls.
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipError_t setup_err[kMaxDevices];
    static int resident[kMaxDevices];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            const void* kern = reinterpret_cast<const void*>(wy_backward_kernel<C, GT>);
            hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_TOTAL);
            int cus = 0, per_cu = 0;
            if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
            if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBT, LDS_TOTAL);
            resident[device] = (per_cu > 0 ? per_cu : 1) * cus;
            setup_err[device] = err;
        });
        e = setup_err[device];
    }
    if (e == hipSuccess) {
        Params p;
        p.k = static_cast<const __bf16*>(a.k);
        p.v = static_cast<const __bf16*>(a.v);
        p.beta = a.beta;
        p.g = a.g;
        p.cu = a.cu_seqlens;
        p.dT = a.dT;
        p.dW = static_cast<const __bf16*>(a.dW);
        p.dU = static_cast<const __bf16*>(a.dU);
        p.dk = static_cast<__bf16*>(a.dk);
        p.dv = static_cast<__bf16*>(a.dv);
        p.dbeta = a.dbeta;
        p.dg = a.dg;
        p.units = a.chunk_slots * a.num_qk_heads;
        p.seqlen = a.seqlen;
        p.hq = a.num_qk_heads;
        p.hv = a.num_v_heads;
        p.num_seqs = a.num_seqs;
        // one resident round (a multiple of 8 workgroups, for the XCD mapping), or fewer
        int64_t grid = (p.units + 7) / 8 * 8;
        const int64_t cap = static_cast<int64_t>(resident[device]) / 8 * 8;
        if (cap >= 8 && grid > cap) grid = cap;
        hipLaunchKernelGGL((wy_backward_kernel<C, GT>), dim3(static_cast<uint32_t>(grid)), dim3(kBT), LDS_TOTAL,
                           stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (wy_backward, C=%d, gated=%d)", hipGetErrorString(e), C, GT ? 1 : 0);
        return static_cast<int>(e);
    }
    return 0;
}


// ---- C = 128 ---------------------------------------------------------------------------------
// The plan above (K, V, dW, dU, T, H, X and S of one job all in LDS) would take about 390 KB at
// C = 128.  Here only K, T and one C x C region stay in LDS.  The region holds X, then Y, then R
// in turn, each hand-over behind a barrier.  V is staged (256-byte rows, 16-byte chunks XOR-
// swizzled by row) over the scratch that later holds the sums and the per-wave panels, for as
// long as X is formed; the rows of dW and dU enter the X tiles straight from memory.  H is not
// kept: the elementwise step forms its tiles again from K.  Once M is known, R and T are written
// once more as bf16 hi / lo tiles (16 x 16, row-major), so that every operand of the products
// over tokens (T^T dW, T^T dU and (R + R^T) K) is one or two LDS reads: a transposed read for 8
// rows of a column, a plain one for 8 entries of a row.  Those products stream each wave's own
// 16 columns of dW and dU through a 32-token panel of that wave.  Eight waves, one workgroup per
// CU; every phase runs on all eight waves, the fp32 Y and M tiles dealt so that the waves (and
// the SIMDs) get equal shares.
namespace c128 {

constexpr int kC = 128;
constexpr int kNB = kC / 16;
constexpr int kBT = 512;
constexpr int kBW = kBT / 64;
constexpr int KROW = kD + 8;  // bf16 per staged K row (and per dv / dk staging row)
using TL = TLayout<kC>;       // the 36 lower 16 x 16 tiles, 16 rows of 20 floats each
using GR = GateRow<KROW, 2>;
constexpr int KB = kC * KROW * 2;
constexpr int OFF_K = 0;
constexpr int OFF_T = OFF_K + KB;             // A -> T (tile-packed fp32); then dv as bf16 rows
constexpr int OFF_XR = OFF_T + TL::BYTES;     // X -> Y -> R (tile-packed); then dk as bf16 rows
constexpr int OFF_B = OFF_XR + TL::BYTES;     // beta
constexpr int OFF_GD = OFF_B + kC * 4;        // G, fp64 (gated)
constexpr int OFF_INFO = OFF_GD + kC * 8;
constexpr int OFF_V = OFF_INFO + 16;          // V rows while X is formed; after that:
constexpr int OFF_QS = OFF_V;                 //   per lower tile of Q = M o H: 16 row and 16 column sums
constexpr int OFF_SUM = OFF_QS + 36 * 32 * 4; //   per wave: sum_d (T^T dW) K and sum_d (T^T dU) V per row
constexpr int OFF_PAN = OFF_SUM + 2 * kBW * kC * 4;  //   per wave: two 16 x 20 transpose tiles; dW / dU panels
constexpr int PAN_BYTES = 2 * 16 * 20 * 4;
constexpr int LDS_TOTAL = OFF_PAN + kBW * PAN_BYTES;
static_assert(LDS_TOTAL - OFF_V >= kC * kD * 2, "V rows fit over the sums and the panels");
static_assert(PAN_BYTES >= 2048, "a wave's dW and dU panels fit its transpose tiles");
static_assert(LDS_TOTAL - OFF_V >= 16 * 1024, "the coupling's tmp tiles fit over the V rows");
static_assert(KB <= TL::BYTES, "dv and dk are staged as bf16 rows over T and XR");
static_assert(OFF_V % 16 == 0 && OFF_PAN % 16 == 0, "16-byte aligned regions");
static_assert(LDS_TOTAL <= 160 * 1024, "C = 128 backward LDS plan exceeds 160 KiB");
static_assert(2 * 36 * 512 <= TL::BYTES, "T and R fit as bf16 hi / lo tiles over their fp32 regions");

// Row sums of the products over tokens: kind 0 = sum_d (T^T dW)_id K_id, 1 = sum_d (T^T dU)_id V_id;
// one row of C floats per (kind, wave).
__device__ inline float* sum_slot(unsigned char* smem, int kind, int wave)
{
    return reinterpret_cast<float*>(smem + OFF_SUM) + (kind * kBW + wave) * kC;
}

// Sums of the lower tile t = I (I + 1) / 2 + J of Q = M o H: [0, 16) row sums sum_j Q_ij over the
// tile's columns, [16, 32) column sums sum_i beta_i Q_ij over its rows.
__device__ inline float* q_slot(unsigned char* smem, int t)
{
    return reinterpret_cast<float*>(smem + OFF_QS) + t * 32;
}

// Lower tiles (Mt, J) of Y = X T^T per wave, as 8 Mt + J (255 ends a list).  Tile (Mt, J) costs
// J + 1 steps of four fp32 MFMAs, so every wave gets 15 steps and each SIMD (waves w and w + 4)
// 30.
__constant__ unsigned char kYTiles[kBW][8] = {
    {63, 54, 255, 255, 255, 255, 255, 255},  // (7,7) (6,6)
    {62, 45, 9, 255, 255, 255, 255, 255},    // (7,6) (5,5) (1,1)
    {53, 61, 17, 0, 255, 255, 255, 255},     // (6,5) (7,5) (2,1) (0,0)
    {36, 44, 52, 255, 255, 255, 255, 255},   // (4,4) (5,4) (6,4)
    {60, 27, 35, 25, 255, 255, 255, 255},    // (7,4) (3,3) (4,3) (3,1)
    {43, 51, 59, 33, 8, 255, 255, 255},      // (5,3) (6,3) (7,3) (4,1) (1,0)
    {18, 26, 34, 41, 49, 16, 24, 255},       // (2,2) (3,2) (4,2) (5,1) (6,1) (2,0) (3,0)
    {42, 50, 58, 57, 32, 40, 48, 56},        // (5,2) (6,2) (7,2) (7,1) (4,0) (5,0) (6,0) (7,0)
};

// Lower tiles (I, J) of M per wave, as 8 I + J (255 ends a list).  Tile (I, J) costs 8 - I steps of
// four fp32 MFMAs plus a fixed cost of about four steps (its Gram, the elementwise step and the
// transposes); four or five tiles per wave, 30 to 34 of these units each.
__constant__ unsigned char kMTiles[kBW][5] = {
    {52, 53, 45, 0, 255},  // (6,4) (6,5) (5,5) (0,0)
    {58, 41, 33, 9, 255},  // (7,2) (5,1) (4,1) (1,1)
    {61, 40, 35, 8, 255},  // (7,5) (5,0) (4,3) (1,0)
    {48, 44, 34, 17, 255}, // (6,0) (5,4) (4,2) (2,1)
    {62, 50, 54, 36, 18},  // (7,6) (6,2) (6,6) (4,4) (2,2)
    {57, 60, 42, 32, 16},  // (7,1) (7,4) (5,2) (4,0) (2,0)
    {59, 63, 43, 24, 27},  // (7,3) (7,7) (5,3) (3,0) (3,3)
    {56, 49, 51, 25, 26},  // (7,0) (6,1) (6,3) (3,1) (3,2)
};

// X tiles while waves 0-1 invert the diagonal blocks: waves 2-7 take row segments (I, J0, J1),
// seven tiles or fewer each (255: none).
__constant__ unsigned char kXSeg[kBW - 2][2][3] = {
    {{7, 0, 3}, {255, 0, 0}}, {{6, 0, 6}, {255, 0, 0}}, {{5, 0, 5}, {0, 0, 0}},
    {{4, 0, 4}, {1, 0, 1}},   {{3, 0, 3}, {2, 0, 2}},   {{7, 4, 7}, {255, 0, 0}},
};

// The next job's K (read only for the first value head of a unit), beta and g in flight.
template <bool GT>
struct Next {
    static constexpr int NIT = kC * 16 / kBT;
    u32x4 k[NIT];
    float b;
    float g[2];  // wave 0 lane l: g of rows l and l + 64

    __device__ __attribute__((always_inline)) void issue(const Params& p, int64_t tok0, int n, int hk, int hv,
                                                         bool with_k, int tid)
    {
        const uint32_t kstride = static_cast<uint32_t>(p.hq) * kD * 2;
        const int nk = with_k ? n : 0;  // n = 0 (no job): empty ranges, every load reads 0
        const __amdgpu_buffer_rsrc_t kr =
            rsrc(p.k + (tok0 * p.hq + hk) * kD, nk > 0 ? (nk - 1) * kstride + kD * 2 : 0u);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kBT;
            k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, (q >> 4) * kstride + (q & 15) * 16, 0, kStream);
        }
        const uint32_t bytes = n > 0 ? ((n - 1) * p.hv + 1) * 4 : 0u;
        const __amdgpu_buffer_rsrc_t br = rsrc(p.beta + tok0 * p.hv + hv, bytes);
        b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, (tid & (kC - 1)) * p.hv * 4, 0, 0));
        g[0] = g[1] = 0.f;
        if constexpr (GT) {
            const __amdgpu_buffer_rsrc_t gr = rsrc(p.g + tok0 * p.hv + hv, bytes);
#pragma unroll
            for (int e = 0; e < 2; ++e)
                g[e] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(gr, ((tid & 63) + 64 * e) * p.hv * 4, 0, 0));
        }
    }

    // K rows (new unit only), beta, and G = inclusive prefix sums of g in fp64 by wave 0, in the
    // forward's order (each half of the chunk scanned, the first half's total added to the second)
    __device__ __attribute__((always_inline)) void commit(unsigned char* Kraw, float* bs, double* Gd, bool with_k,
                                                          int tid) const
    {
        if (with_k) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int q = tid + it * kBT;
                *reinterpret_cast<u32x4*>(Kraw + (q >> 4) * (KROW * 2) + (q & 15) * 16) = k[it];
            }
        }
        if (tid < kC) bs[tid] = b;
        if constexpr (GT) {
            if (tid < 64) {
                double run = 0.0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    double x = static_cast<double>(g[e]);
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const double t = __shfl_up(x, d);
                        if (tid >= d) x += t;
                    }
                    x += run;
                    const int r = tid + 64 * e;
                    *GR::Gp(Kraw, r) = x;
                    *GR::Ep(Kraw, r) = __expf(static_cast<float>(x));
                    Gd[r] = x;
                    run = __shfl(x, 63);
                }
            }
        }
    }
};

// This job's V rows, in flight and then staged: row r's 16-byte chunk q at r * 256 + 16 (q ^ (r & 15)).
struct VRows {
    static constexpr int NIT = kC * 16 / kBT;
    u32x4 x[NIT];

    __device__ __attribute__((always_inline)) void issue(const Params& p, int64_t tok0, int n, int hv, int tid)
    {
        const uint32_t stride = static_cast<uint32_t>(p.hv) * kD * 2;
        const __amdgpu_buffer_rsrc_t vr =
            rsrc(p.v + (tok0 * p.hv + hv) * kD, n > 0 ? (n - 1) * stride + kD * 2 : 0u);  // n = 0: reads 0
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kBT;
            x[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, (q >> 4) * stride + (q & 15) * 16, 0, 0);
        }
    }
    __device__ __attribute__((always_inline)) void commit(unsigned char* dst, int tid) const
    {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kBT;
            const int r = q >> 4, c = q & 15;
            *reinterpret_cast<u32x4*>(dst + r * 256 + 16 * (c ^ (r & 15))) = x[it];
        }
    }
};

// A fragments of rows 16 I .. 16 I + 15 of dW and dU (lane 16 g + c: row 16 I + c, dk 32 s + 8 g
// .. + 7), straight from memory; I < 0 or n = 0 reads nothing.
struct RowFrags {
    bf16x8 w[kD / 32], u[kD / 32];

    __device__ __attribute__((always_inline)) void issue(const Params& p, int64_t tok0, int n, int hv, int I, int lr, int lg)
    {
        const uint32_t stride = static_cast<uint32_t>(p.hv) * kD * 2;
        const uint32_t bytes = I >= 0 && n > 0 ? (n - 1) * stride + kD * 2 : 0u;
        const __amdgpu_buffer_rsrc_t wr = rsrc(p.dW + (tok0 * p.hv + hv) * kD, bytes);
        const __amdgpu_buffer_rsrc_t ur = rsrc(p.dU + (tok0 * p.hv + hv) * kD, bytes);
        const uint32_t off = (16 * (I >= 0 ? I : 0) + lr) * stride + 16 * lg;
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
            w[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, off + 64 * s, 0, 0));
            u[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ur, off + 64 * s, 0, 0));
        }
    }
};

// a2 + a3: A = I + strictLower(D H) into the tile-packed Ts, entry for entry as the forward
// forms it (same Gram fragments and MFMA order, same decay and products), so T is bit-identical.
template <bool GT>
__device__ __attribute__((always_inline)) void form_a(const unsigned char* Kraw, float* Ts, const float* bs, int wave, int lr, int lg)
{
    constexpr int NTILE = kNB * (kNB + 1) / 2;
    for (int t = wave; t < NTILE; t += kBW) {  // uniform
        int I = 0, J = 0;
        tile_of(t, &I, &J);
        GramFrags<0, KROW> f;
        f.load(Kraw, I, J, lr, lg);
        const f32x4 acc = f.product();
        const f32x4 bet = *reinterpret_cast<const f32x4*>(bs + 16 * I + 4 * lg);
        const float bcol = bs[16 * J + lr];
        double gcol = 0.0;
        if constexpr (GT) gcol = GR::G(Kraw, 16 * J + lr);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * lg + r, j = 16 * J + lr;
            float a = acc[r];
            if constexpr (GT) {
                const double d = GR::G(Kraw, i) - gcol;
                a *= __expf(static_cast<float>(i > j ? d : -d));
            }
            Ts[TL::off(i, j)] = (i > j) ? bet[r] * a : (i == j ? 1.f : bcol * a);
        }
    }
}

// X(i, j) = dT_ij + (dW K^T)_ij beta_j e^{G_j} + (dU V^T)_ij beta_j for i > j, 0 otherwise, for
// the tiles (I, J0 .. J1); K rows from LDS, V rows from the swizzled staging.
template <bool GT, bool DT>
__device__ __attribute__((always_inline)) void x_row(const Params& p, const RowFrags& f, int I, int J0, int J1, const unsigned char* Kraw,
                      const unsigned char* Vst, const float* bs, float* Xs, int64_t tok0, int n, int hv, int lr,
                      int lg)
{
    const __bf16* Kb = reinterpret_cast<const __bf16*>(Kraw);
    const __amdgpu_buffer_rsrc_t dtr = rsrc(DT ? p.dT + (tok0 * p.hv + hv) * kC : nullptr,
                                            DT ? (n - 1) * static_cast<uint32_t>(p.hv) * kC * 4 + kC * 4 : 0u);
    for (int J = J0; J <= J1; ++J) {  // uniform
        f32x4 pw = zero4(), pu = zero4();
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
            const bf16x8 bk = *reinterpret_cast<const bf16x8*>(Kb + (16 * J + lr) * KROW + 32 * s + 8 * lg);
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Vst + (16 * J + lr) * 256 + 16 * ((4 * s + lg) ^ lr));
            pw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[s], bk, pw, 0, 0, 0);
            pu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.u[s], bv, pu, 0, 0, 0);
        }
        const int j = 16 * J + lr;
        const float bj = bs[j];
        const float ej = GT ? GR::E(Kraw, j) : 1.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr;
            float x = 0.f;
            if (i > j) {
                float dt = 0.f;
                if constexpr (DT)
                    dt = __builtin_bit_cast(float,
                                            __builtin_amdgcn_raw_buffer_load_b32(dtr, i * p.hv * kC * 4 + j * 4, 0, 0));
                x = dt + pw[rr] * bj * ej + pu[rr] * bj;
            }
            Xs[TL::off(i, j)] = x;
        }
    }
}

// a6 for block size S = 32 or 64 on all eight waves (coupling_level runs a pair's column tile on
// one wave, which at S = 64 makes one wave's chain 104 fp32 MFMAs long).  Two passes, a barrier
// between them: tmp = L10 X00 tile by tile into `tmpb` (one 16-byte chunk per lane and tile),
// then X10 = -X11 tmp written over L10, which no wave reads any more.  Pass A's tile (mr, nc)
// costs TS - nc steps of four MFMAs and pass B's mr + 1, so at S = 64 each wave takes two tiles
// whose costs add up to 5 in each pass, and at S = 32 one tile.  Every tile's sum runs in
// coupling_level's order, so T is bit-identical to it.
template <int S>
__device__ __attribute__((always_inline)) void coupling8(float* Ts, float* tmpb, int wave, int lane, int lr, int lg)
{
    constexpr int TS = S / 16;
    constexpr int PER = TS * TS * (kC / (2 * S)) / kBW;  // tiles per wave and pass
    static_assert((S == 64 && PER == 2) || (S == 32 && PER == 1), "tile dealing below");
#pragma unroll
    for (int t = 0; t < PER; ++t) {  // pass A: tmp(mr, nc) = sum_{kt >= nc} L10(mr, kt) X00(kt, nc)
        const int pr = S == 64 ? 0 : wave >> 2;
        const int mr = S == 64 ? wave >> 1 : (wave >> 1) & 1;
        const int nc = S == 64 ? (t == 0 ? (wave & 1) : 3 - (wave & 1)) : wave & 1;
        const int base = 2 * S * pr;
        f32x4 acc = zero4();
        for (int kt = nc; kt < TS; ++kt) {  // uniform
            float bq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bq[q] = Ts[TL::off(base + 16 * kt + 4 * lg + q, base + 16 * nc + lr)];
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + TL::off(base + S + 16 * mr + lr, base + 16 * kt + 4 * lg));
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bq[q], acc, 0, 0, 0);
        }
        *reinterpret_cast<f32x4*>(tmpb + ((pr * TS + mr) * TS + nc) * 256 + 4 * lane) = acc;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PER; ++t) {  // pass B: X10(mr, nc) = -sum_{kt <= mr} X11(mr, kt) tmp(kt, nc)
        const int pr = S == 64 ? 0 : wave >> 2;
        const int nc = S == 64 ? wave >> 1 : (wave >> 1) & 1;
        const int mr = S == 64 ? (t == 0 ? (wave & 1) : 3 - (wave & 1)) : wave & 1;
        const int base = 2 * S * pr;
        f32x4 acc = zero4();
        for (int kt = 0; kt <= mr; ++kt) {  // uniform
            const f32x4 av =
                *reinterpret_cast<const f32x4*>(Ts + TL::off(base + S + 16 * mr + lr, base + S + 16 * kt + 4 * lg));
            const f32x4 bv = *reinterpret_cast<const f32x4*>(tmpb + ((pr * TS + kt) * TS + nc) * 256 + 4 * lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[TL::off(base + S + 16 * mr + 4 * lg + r, base + 16 * nc + lr)] = -acc[r];
    }
    __syncthreads();
}

// Rows [0, n) of C staged bf16 rows (KROW elements) at `src` to a [tokens, heads, 128] tensor.
__device__ __attribute__((always_inline)) void store_rows(const unsigned char* src, __bf16* out, int64_t tok0, int n, int heads, int head,
                                  int tid)
{
    const uint32_t stride = static_cast<uint32_t>(heads) * kD * 2;
    const __amdgpu_buffer_rsrc_t r = rsrc(out + (tok0 * heads + head) * kD, (n - 1) * stride + kD * 2);
#pragma unroll
    for (int it = 0; it < kC * 16 / kBT; ++it) {
        const int q = tid + it * kBT;
        const u32x4 val = *reinterpret_cast<const u32x4*>(src + (q >> 4) * (KROW * 2) + (q & 15) * 16);
        __builtin_amdgcn_raw_buffer_store_b128(val, r, (q >> 4) * stride + (q & 15) * 16, 0, kStream);
    }
}

// Accumulators acc[mi] of wave ni (element r of lane 16 g + c: row 16 mi + c, column 16 ni + 4 g
// + r) as bf16 into staged rows at `dst`.
__device__ __attribute__((always_inline)) void stage_cols(unsigned char* dst, const f32x4 (&acc)[kNB], int ni, int lr, int lg)
{
    __bf16* d = reinterpret_cast<__bf16*>(dst);
#pragma unroll
    for (int mi = 0; mi < kNB; ++mi) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(acc[mi][r]);
        *reinterpret_cast<bf16x4*>(d + (16 * mi + lr) * KROW + 16 * ni + 4 * lg) = o;
    }
}

// 16 x 16 bf16 tiles with rows of 32 bytes.  tile_col8: lane 16 g + c gets column c of rows
// 8 (g & 1) .. + 7 (two transposed LDS reads); tile_row8: row c, columns 8 (g & 1) .. + 7.
constexpr int kTileBf = 16 * 16 * 2;

__device__ inline bf16x8 tile_col8(const unsigned char* tile, int lr, int lg)
{
    const unsigned char* p0 = tile + (8 * (lg & 1) + (lr >> 2)) * 32 + 8 * (lr & 3);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * 32));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline bf16x8 tile_row8(const unsigned char* tile, int lr, int lg)
{
    return *reinterpret_cast<const bf16x8*>(tile + lr * 32 + 16 * (lg & 1));
}

__device__ inline float sum_lane_groups(float x)
{
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

template <bool GT>
__global__ __launch_bounds__(kBT, 2) void wy_backward128_kernel(Params p)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char* Kraw = smem + OFF_K;
    float* Ts = reinterpret_cast<float*>(smem + OFF_T);
    float* Xs = reinterpret_cast<float*>(smem + OFF_XR);
    float* bs = reinterpret_cast<float*>(smem + OFF_B);
    double* Gd = reinterpret_cast<double*>(smem + OFF_GD);
    int* info = reinterpret_cast<int*>(smem + OFF_INFO);

    const int tid = threadIdx.x;

    wyp::Params mp{};
    mp.cu = p.cu;
    mp.units = p.units;
    mp.seqlen = p.seqlen;
    mp.hq = p.hq;
    mp.hv = p.hq;
    mp.num_seqs = p.num_seqs;
    const int r = p.hv / p.hq;
    // Persistent, one resident round dealt round-robin to the 8 XCDs (as the C = 32 / 64 kernel).
    const uint32_t G = gridDim.x;  // a multiple of 8
    int64_t logical = static_cast<int64_t>(blockIdx.x & 7u) * (G >> 3) + (blockIdx.x >> 3);
    BatchWalk walk{};
    Unit u;
    if (p.cu == nullptr) {  // uniform
        walk.init(static_cast<uint32_t>(logical), G, static_cast<uint32_t>(p.hq),
                  static_cast<uint32_t>((p.seqlen + kC - 1) / kC));
        u = walk.unit<kC>(p.seqlen, logical < p.units);
    } else {
        u = map_unit<kC>(mp, info, logical, G, tid);
    }
    if (u.n <= 0) return;  // uniform
    int hv = u.hv * r;
    bool new_unit = true;
    Next<GT> in;
    in.issue(p, u.tok0, u.n, u.hv, hv, true, tid);
    // The X waves' row segments (fixed per wave).
    int segI[2] = {-1, -1}, segJ0[2] = {0, 0}, segJ1[2] = {0, 0};
    {
        const int wave = uniform(tid >> 6);
        if (wave >= 2) {  // uniform
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int I = kXSeg[wave - 2][s][0];
                segI[s] = I == 255 ? -1 : I;
                segJ0[s] = kXSeg[wave - 2][s][1];
                segJ1[s] = kXSeg[wave - 2][s][2];
            }
        }
    }
    f32x4 dk_acc[kNB];
#pragma unroll
    for (int mi = 0; mi < kNB; ++mi) dk_acc[mi] = zero4();

    // inlined (one call): a call would keep every captured array in scratch memory
    auto job = [&]() __attribute__((always_inline)) -> bool {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // per-lane LDS addresses are formed where used, not held
        const int lane = tid & 63, wave = uniform(tid >> 6);
        const int lr = lane & 15, lg = lane >> 4;
        const int hk = u.hv;
        const int64_t tok0 = u.tok0;
        const int n = u.n;
        const bool last_head = hv == (hk + 1) * r - 1;  // uniform

        in.commit(Kraw, bs, Gd, new_unit, tid);
        __syncthreads();
        Unit nu = u;
        int nhv = hv + 1;
        bool nnew = false;
        if (nhv == (hk + 1) * r) {  // uniform
            logical += G;
            if (p.cu == nullptr) {  // uniform
                walk.step();
                nu = walk.unit<kC>(p.seqlen, logical < p.units);
            } else {
                nu = map_unit<kC>(mp, info, logical, G, tid);
            }
            nhv = nu.hv * r;
            nnew = true;
        }

        // ---- this job's V rows and the X waves' dW / dU fragments in flight; A meanwhile.  (Issued
        // a job ahead instead, from the previous job's end, they measured 3.5% slower: every
        // workgroup then waits for them at the commit of K, and the registers they hold cost the
        // last phases more than the head start gains.)
        VRows vin;
        vin.issue(p, tok0, n, hv, tid);
        RowFrags fa, fb;
        if (wave >= 2) fa.issue(p, tok0, n, hv, segI[0], lr, lg);  // uniform
        if (wave >= 4) fb.issue(p, tok0, n, hv, segI[1], lr, lg);  // uniform: waves 4-6 have a second segment
        form_a<GT>(Kraw, Ts, bs, wave, lr, lg);
        vin.commit(smem + OFF_V, tid);
        __syncthreads();

        // ---- waves 0-1 invert the diagonal blocks (the chain, at raised priority); waves 2-7 form X
        if (wave < 2) {  // uniform
            __builtin_amdgcn_s_setprio(2);
            invert_diagonal_blocks<kC, TL>(Ts, tid);
            __builtin_amdgcn_s_setprio(0);
        } else {
            auto xs = [&](auto with_dt) {
                constexpr bool DT = decltype(with_dt)::value;
                x_row<GT, DT>(p, fa, segI[0], segJ0[0], segJ1[0], Kraw, smem + OFF_V, bs, Xs, tok0, n, hv, lr, lg);
                if (segI[1] >= 0)  // uniform
                    x_row<GT, DT>(p, fb, segI[1], segJ0[1], segJ1[1], Kraw, smem + OFF_V, bs, Xs, tok0, n, hv, lr,
                                  lg);
            };
            if (p.dT != nullptr)  // uniform
                xs(std::true_type{});
            else
                xs(std::false_type{});
        }
        __syncthreads();
        // ---- coupling levels: 16 rows on waves 0-3, 32 and 64 rows on all eight (tmp over the V rows)
        coupling_level<kC, 16, TL>(Ts, tid);
        coupling8<32>(Ts, reinterpret_cast<float*>(smem + OFF_V), wave, lane, lr, lg);
        coupling8<64>(Ts, reinterpret_cast<float*>(smem + OFF_V), wave, lane, lr, lg);

        // ---- Y = X T^T, lower tiles, in registers; then over X as one 16-byte chunk per lane
        f32x4 yt[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            yt[s] = zero4();
            const int code = kYTiles[wave][s];
            if (code != 255) {  // uniform
                const int Mt = code >> 3, J = code & 7;
                for (int L = 0; L <= J; ++L) {  // Y(Mt, J) = sum_{L <= J} X(Mt, L) T(J, L)^T
                    const f32x4 a = *reinterpret_cast<const f32x4*>(Xs + TL::off(16 * Mt + lr, 16 * L + 4 * lg));
                    const f32x4 b = *reinterpret_cast<const f32x4*>(Ts + TL::off(16 * J + lr, 16 * L + 4 * lg));
#pragma unroll
                    for (int q = 0; q < 4; ++q) yt[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], b[q], yt[s], 0, 0, 0);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int code = kYTiles[wave][s];
            if (code != 255)  // uniform
                *reinterpret_cast<f32x4*>(Xs + TL::off(16 * (code >> 3), 16 * (code & 7)) + 4 * lane) = yt[s];
        }
        __syncthreads();

        // ---- M = strictLower(-T^T Y) by tiles, and the elementwise step: R = D (Gamma o M) kept in
        // registers, the row and column sums of Q = M o H (H formed again from K) into this wave's
        // slots.  Tile element r of lane 16 g + c is (16 I + 4 g + r, 16 J + c) (the m layout);
        // R leaves the tile transposed (row 16 I + c, columns 16 J + 4 g ..; a diagonal tile
        // as the symmetric S = R + R^T) and packed into bf16 hi / lo, ready for its row-major
        // store.
        {
            float* scr = reinterpret_cast<float*>(smem + OFF_PAN + wave * PAN_BYTES);  // two 16 x 20 tiles
#pragma unroll
            for (int s = 0; s < 5; ++s) {
                yt[s] = zero4();  // R of this slot
                const int code = kMTiles[wave][s];
                if (code != 255) {  // uniform
                    const int I = code >> 3, J = code & 7;
                    f32x4 acc = zero4();
                    for (int Mt = I; Mt < kNB; ++Mt) {  // (T^T Y)(I, J) = sum_{Mt >= I} T(Mt, I)^T Y(Mt, J)
                        const float* tcol = Ts + TL::off(16 * Mt + 4 * lg, 16 * I + lr);
                        const f32x4 b = *reinterpret_cast<const f32x4*>(Xs + TL::off(16 * Mt, 16 * J) + 4 * lane);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tcol[q * TL::RS], b[q], acc, 0, 0, 0);
                    }
                    GramFrags<0, KROW> gf;
                    gf.load(Kraw, I, J, lr, lg);
                    const f32x4 gr = gf.product();
                    const f32x4 bi = *reinterpret_cast<const f32x4*>(bs + 16 * I + 4 * lg);
                    const int j = 16 * J + lr;
                    double gj = 0.0;
                    if constexpr (GT) gj = Gd[j];
                    f32x4 q4, rm;
                    float colp = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = 16 * I + 4 * lg + rr;
                        const bool ok = I > J || i > j;
                        float gam = 1.f;
                        if constexpr (GT) gam = __expf(static_cast<float>(Gd[i] - gj));
                        const float m = -acc[rr];
                        rm[rr] = ok ? bi[rr] * gam * m : 0.f;
                        q4[rr] = ok ? m * (gam * gr[rr]) : 0.f;
                        colp += bi[rr] * q4[rr];
                    }
                    // both tiles transposed through this wave's scratch (its LDS operations run in order)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        scr[(4 * lg + rr) * 20 + lr] = q4[rr];
                        scr[320 + (4 * lg + rr) * 20 + lr] = rm[rr];
                    }
                    const f32x4 qt = *reinterpret_cast<const f32x4*>(scr + lr * 20 + 4 * lg);
                    f32x4 rt = *reinterpret_cast<const f32x4*>(scr + 320 + lr * 20 + 4 * lg);
                    const float rowp = sum_lane_groups(qt[0] + qt[1] + qt[2] + qt[3]);
                    colp = sum_lane_groups(colp);
                    if (lg == 0) {
                        float* qs = q_slot(smem, I * (I + 1) / 2 + J);
                        qs[lr] = rowp;
                        qs[16 + lr] = colp;
                    }
                    if (I == J) rt += rm;  // uniform: the diagonal tile as S = R + R^T
                    yt[s] = __builtin_bit_cast(f32x4, pack_hilo(rt));
                }
            }
        }
        // ---- the products over tokens read T and R as bf16 hi / lo tiles (16 x 16, rows of 32 bytes,
        // row-major), where a fragment of 8 rows of one column is one transposed LDS read: this
        // thread's share of T in registers now, written over T past the barrier.
        f32x4 tpart[5];
#pragma unroll
        for (int it = 0; it < 5; ++it) {
            const int q = tid + it * kBT;  // 16-byte chunk q of T: tile q >> 6, row (q >> 2) & 15, chunk q & 3
            tpart[it] = q < 36 * 64 ? *reinterpret_cast<const f32x4*>(Ts + (q >> 6) * TL::TILE + ((q >> 2) & 15) * TL::RS + 4 * (q & 3))
                                    : zero4();
        }
        // wave ni's 16 columns of dW and dU for all four 32-token panels, and the V chunks for sv
        const int ni = wave;
        const uint32_t stride = static_cast<uint32_t>(p.hv) * kD * 2;
        const uint32_t bytes = (n - 1) * stride + kD * 2;
        u32x4 pw[kC / 32], pu[kC / 32];
        u32x2 vv[kNB];
        {
            const __amdgpu_buffer_rsrc_t wr = rsrc(p.dW + (tok0 * p.hv + hv) * kD, bytes);
            const __amdgpu_buffer_rsrc_t ur = rsrc(p.dU + (tok0 * p.hv + hv) * kD, bytes);
            const __amdgpu_buffer_rsrc_t vr = rsrc(p.v + (tok0 * p.hv + hv) * kD, bytes);
            const uint32_t poff = (lane >> 1) * stride + (16 * ni + 8 * (lane & 1)) * 2;
#pragma unroll
            for (int ks = 0; ks < kC / 32; ++ks) {
                pw[ks] = __builtin_amdgcn_raw_buffer_load_b128(wr, poff + 32 * ks * stride, 0, kStream);
                pu[ks] = __builtin_amdgcn_raw_buffer_load_b128(ur, poff + 32 * ks * stride, 0, kStream);
            }
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi)
                vv[mi] = __builtin_amdgcn_raw_buffer_load_b64(vr, (16 * mi + lr) * stride + (16 * ni + 4 * lg) * 2, 0,
                                                              kStream);
        }
        __syncthreads();
        {
            unsigned char* Rb = smem + OFF_XR;  // R hi tiles, then R lo tiles (36 x 512 bytes each)
#pragma unroll
            for (int s = 0; s < 5; ++s) {
                const int code = kMTiles[wave][s];
                if (code != 255) {  // uniform
                    const int I = code >> 3, J = code & 7;
                    const int off = (I * (I + 1) / 2 + J) * 512 + lr * 32 + 8 * lg;
                    const u32x4 h = __builtin_bit_cast(u32x4, yt[s]);
                    *reinterpret_cast<u32x2*>(Rb + off) = u32x2{h[0], h[1]};
                    *reinterpret_cast<u32x2*>(Rb + kTileBf * 36 + off) = u32x2{h[2], h[3]};
                }
            }
            unsigned char* Tb = smem + OFF_T;  // T hi tiles, then T lo tiles
#pragma unroll
            for (int it = 0; it < 5; ++it) {
                const int q = tid + it * kBT;
                if (q < 36 * 64) {
                    const u32x4 h = pack_hilo(tpart[it]);
                    const int off = (q >> 6) * 512 + ((q >> 2) & 15) * 32 + 8 * (q & 3);
                    *reinterpret_cast<u32x2*>(Tb + off) = u32x2{h[0], h[1]};
                    *reinterpret_cast<u32x2*>(Tb + kTileBf * 36 + off) = u32x2{h[2], h[3]};
                }
            }
        }
        __syncthreads();

        // ---- wave ni: T^T dW and T^T dU for dk columns 16 ni .. + 15, over the four 32-token panels
        // of its own columns of dW and dU (staged in its own 2 KB); then dK += D E T^T dW,
        // dV = D T^T dU and the per-row sums
        {
            const __bf16* Kb = reinterpret_cast<const __bf16*>(Kraw);
            unsigned char* pan = smem + OFF_PAN + wave * PAN_BYTES;  // [0, 1 KB): dW, [1 KB, 2 KB): dU
            const unsigned char* Tb = smem + OFF_T;
            f32x4 aw[kNB], au[kNB];
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) aw[mi] = au[mi] = zero4();
#pragma unroll
            for (int ks = 0; ks < kC / 32; ++ks) {
                *reinterpret_cast<u32x4*>(pan + (lane >> 1) * 32 + (lane & 1) * 16) = pw[ks];
                *reinterpret_cast<u32x4*>(pan + 1024 + (lane >> 1) * 32 + (lane & 1) * 16) = pu[ks];
                const bf16x8 xw = tr_frag<16>(reinterpret_cast<const __bf16*>(pan), 0, 0, lr, lg);
                const bf16x8 xu = tr_frag<16>(reinterpret_cast<const __bf16*>(pan + 1024), 0, 0, lr, lg);
                const int Tt = 2 * ks + (lg >> 1);  // the 16-row tile of this lane group's 8 tokens
#pragma unroll
                for (int mi = 0; mi <= 2 * ks + 1; ++mi) {
                    // B fragment: T(32 ks + 8 g .. + 7, 16 mi + c), 0 for a tile above the diagonal
                    const bool in = Tt >= mi;
                    const int tile = in ? Tt * (Tt + 1) / 2 + mi : mi * (mi + 1) / 2 + mi;
                    bf16x8 bh = tile_col8(Tb + tile * 512, lr, lg);
                    bf16x8 bl = tile_col8(Tb + kTileBf * 36 + tile * 512, lr, lg);
                    if (!in) bh = bl = bf16x8{};
                    aw[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, bh, aw[mi], 0, 0, 0);
                    au[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xu, bh, au[mi], 0, 0, 0);
                    aw[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, bl, aw[mi], 0, 0, 0);
                    au[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xu, bl, au[mi], 0, 0, 0);
                }
            }
            // element r of lane 16 g + c: (T^T dW)[i = 16 mi + c][d = 16 ni + 4 g + r]
            float* ssk = sum_slot(smem, 0, wave);
            float* ssv = sum_slot(smem, 1, wave);
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) {
                const int i = 16 * mi + lr;
                const float bi = bs[i];
                const float ei = GT ? GR::E(Kraw, i) : 1.f;
                const bf16x4 kv = *reinterpret_cast<const bf16x4*>(Kb + i * KROW + 16 * ni + 4 * lg);
                const bf16x4 vb = __builtin_bit_cast(bf16x4, vv[mi]);
                float sk = 0.f, sv = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    sk += aw[mi][rr] * static_cast<float>(kv[rr]);
                    sv += au[mi][rr] * static_cast<float>(vb[rr]);
                    dk_acc[mi][rr] += bi * ei * aw[mi][rr];
                    au[mi][rr] *= bi;  // dV
                }
                sk = sum_lane_groups(sk);
                sv = sum_lane_groups(sv);
                if (lg == 0) {
                    ssk[i] = sk;
                    ssv[i] = sv;
                }
            }
            __syncthreads();  // every read of T is done
            stage_cols(smem + OFF_T, au, ni, lr, lg);  // dV rows over T
        }

        in.issue(p, nu.tok0, nu.n, nu.hv, nhv, nnew, tid);  // the next job's K, beta and g
        // ---- (R + R^T) K into dK.  S(t, i) is R(t, i) below the diagonal tiles (8 rows of one
        // column of tile (t, i): a transposed read) and R(i, t) above them (8 entries of one row of
        // tile (i, t)); the diagonal tiles hold S itself, read by rows.
        {
            const __bf16* Kb = reinterpret_cast<const __bf16*>(Kraw);
            const unsigned char* Rb = smem + OFF_XR;
#pragma unroll
            for (int ks = 0; ks < kC / 32; ++ks) {
                const bf16x8 xk = tr_frag<KROW>(Kb, 32 * ks, ni, lr, lg);
                const int Tt = 2 * ks + (lg >> 1);
#pragma unroll
                for (int mi = 0; mi < kNB; ++mi) {
                    bf16x8 sh, sl;
                    if (mi < 2 * ks) {  // every lane group below the diagonal: columns of tiles (Tt, mi)
                        const int tile = Tt * (Tt + 1) / 2 + mi;
                        sh = tile_col8(Rb + tile * 512, lr, lg);
                        sl = tile_col8(Rb + kTileBf * 36 + tile * 512, lr, lg);
                    } else if (mi > 2 * ks + 1) {  // every lane group above: rows of tiles (mi, Tt)
                        const int tile = mi * (mi + 1) / 2 + Tt;
                        sh = tile_row8(Rb + tile * 512, lr, lg);
                        sl = tile_row8(Rb + kTileBf * 36 + tile * 512, lr, lg);
                    } else {  // the lane groups of tile mi read rows of the diagonal tile, the others columns
                        const bool below = Tt > mi;
                        const int tc = below ? Tt * (Tt + 1) / 2 + mi : mi * (mi + 1) / 2 + mi;
                        const int tr = mi * (mi + 1) / 2 + (below ? mi : Tt);
                        const bf16x8 ch = tile_col8(Rb + tc * 512, lr, lg);
                        const bf16x8 cl = tile_col8(Rb + kTileBf * 36 + tc * 512, lr, lg);
                        const bf16x8 rh = tile_row8(Rb + tr * 512, lr, lg);
                        const bf16x8 rl = tile_row8(Rb + kTileBf * 36 + tr * 512, lr, lg);
                        sh = below ? ch : rh;
                        sl = below ? cl : rl;
                    }
                    dk_acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xk, sh, dk_acc[mi], 0, 0, 0);
                    dk_acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xk, sl, dk_acc[mi], 0, 0, 0);
                }
            }
        }
        __syncthreads();

        store_rows(smem + OFF_T, p.dv, tok0, n, p.hv, hv, tid);  // dV out
        if (last_head) {  // uniform: dK of the unit staged over R
            stage_cols(smem + OFF_XR, dk_acc, ni, lr, lg);
#pragma unroll
            for (int mi = 0; mi < kNB; ++mi) dk_acc[mi] = zero4();
        }
        if (wave == 0) {
            // dbeta_i = sum_d (T^T dW)_id e^{G_i} K_id + sum_d (T^T dU)_id V_id + sum_j M_ij H_ij;
            // dG_i = beta_i e^{G_i} sum_d (T^T dW)_id K_id + beta_i sum_j M_ij H_ij - sum_j beta_j M_ji H_ji;
            // lane l takes rows l and l + 64
            float dG[2];
            const __amdgpu_buffer_rsrc_t br = rsrc(p.dbeta + tok0 * p.hv + hv, ((n - 1) * p.hv + 1) * 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = lane + 64 * h;
                float sk = 0.f, sv = 0.f, mh = 0.f, cz = 0.f;
#pragma unroll
                for (int w = 0; w < kBW; ++w) {  // the waves' slots in a fixed order
                    sk += sum_slot(smem, 0, w)[i];
                    sv += sum_slot(smem, 1, w)[i];
                }
                const int Ib = i >> 4, ir = i & 15;
                for (int J = 0; J <= Ib; ++J) mh += q_slot(smem, Ib * (Ib + 1) / 2 + J)[ir];  // row i
                for (int I = Ib; I < kNB; ++I) cz += q_slot(smem, I * (I + 1) / 2 + Ib)[16 + ir];  // column i
                const float bi = bs[i];
                const float ei = GT ? GR::E(Kraw, i) : 1.f;
                const float db = sk * ei + sv + mh;
                dG[h] = bi * ei * sk + bi * mh - cz;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, db), br, i * p.hv * 4, 0, 0);
            }
            if constexpr (GT) {
                // dg_t = sum_{i >= t} dG_i: reverse inclusive scans of the two halves, the second
                // half's total added to the first
#pragma unroll
                for (int h = 1; h >= 0; --h) {
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const float t = __shfl_down(dG[h], d);
                        if (lane + d < 64) dG[h] += t;
                    }
                }
                dG[0] += __shfl(dG[1], 0);
                const __amdgpu_buffer_rsrc_t gr = rsrc(p.dg + tok0 * p.hv + hv, ((n - 1) * p.hv + 1) * 4);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, dG[h]), gr,
                                                          (lane + 64 * h) * p.hv * 4, 0, 0);
            }
        }
        // every read of this job's LDS (T, XR, sums, K, beta) is done past this barrier, so the next
        // job's commit and V staging may overwrite them; the staged dk is read below and only
        // rewritten after the next job's second barrier
        __syncthreads();
        if (last_head) store_rows(smem + OFF_XR, p.dk, tok0, n, p.hq, hk, tid);  // uniform
        u = nu;
        hv = nhv;
        new_unit = nnew;
        return u.n > 0;
    };
    while (job()) {
    }
}

template <bool GT>
int launch_t(const BwdArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipError_t setup_err[kMaxDevices];
    static int resident[kMaxDevices];
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess && (device < 0 || device >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) {
        std::call_once(once[device], [&] {
            const void* kern = reinterpret_cast<const void*>(wy_backward128_kernel<GT>);
            hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_TOTAL);
            int cus = 0, per_cu = 0;
            if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
            if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBT, LDS_TOTAL);
            resident[device] = (per_cu > 0 ? per_cu : 1) * cus;
            setup_err[device] = err;
        });
        e = setup_err[device];
    }
    if (e == hipSuccess) {
        Params p;
        p.k = static_cast<const __bf16*>(a.k);
        p.v = static_cast<const __bf16*>(a.v);
        p.beta = a.beta;
        p.g = a.g;
        p.cu = a.cu_seqlens;
        p.dT = a.dT;
        p.dW = static_cast<const __bf16*>(a.dW);
        p.dU = static_cast<const __bf16*>(a.dU);
        p.dk = static_cast<__bf16*>(a.dk);
        p.dv = static_cast<__bf16*>(a.dv);
        p.dbeta = a.dbeta;
        p.dg = a.dg;
        p.units = a.chunk_slots * a.num_qk_heads;
        p.seqlen = a.seqlen;
        p.hq = a.num_qk_heads;
        p.hv = a.num_v_heads;
        p.num_seqs = a.num_seqs;
        int64_t grid = (p.units + 7) / 8 * 8;
        const int64_t cap = static_cast<int64_t>(resident[device]) / 8 * 8;
        if (cap >= 8 && grid > cap) grid = cap;
        hipLaunchKernelGGL((wy_backward128_kernel<GT>), dim3(static_cast<uint32_t>(grid)), dim3(kBT), LDS_TOTAL,
                           stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (wy_backward, C=128, gated=%d)", hipGetErrorString(e), GT ? 1 : 0);
        return static_cast<int>(e);
    }
    return 0;
}

}  // namespace c128

}  // namespace bwd

}  // namespace

int launch_bwd(const BwdArgs& a, void* stream, char* msg, int msg_len)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.chunk_size == 128)
        return a.g != nullptr ? bwd::c128::launch_t<true>(a, s, msg, msg_len) : bwd::c128::launch_t<false>(a, s, msg, msg_len);
    if (a.chunk_size == 32)
        return a.g != nullptr ? bwd::launch_t<32, true>(a, s, msg, msg_len) : bwd::launch_t<32, false>(a, s, msg, msg_len);
    return a.g != nullptr ? bwd::launch_t<64, true>(a, s, msg, msg_len) : bwd::launch_t<64, false>(a, s, msg, msg_len);
}

}  // namespace wyp
