// HIP kernels (gfx950 / CDNA4) for the per-chunk WY/UT preparation of chunkwise (Gated)
// DeltaNet.
//
// Pages cited (by title and section):
//   [Inv] "TileLang 实战：单位下三角矩阵求逆" (TileLang in practice: inverting a unit
//         lower-triangular matrix).
//   [QLA] The FlashQLA announcement, section "使用方式" (usage).
//
// A unit is one (sequence, chunk, value head).  Workgroups of 256 threads (four wave64s) are
// persistent: the grid holds one resident round, and each workgroup walks a strided list of
// units.  While it computes one unit, the next unit's K, V and beta are already in flight
// into registers, so HBM traffic never waits for the arithmetic.  Per unit:
//   a0  map the unit to (first token, length n, value head); packed batches search cu_seqlens
//       on the device (wyprep_device.h);
//   a1  K (n x 128), V (n x 128) and beta (n) arrive through bounded buffer loads: rows
//       n..C-1 of a short chunk read as zero with beta = 0 ([Inv] leaves tails open; this is
//       the padded reading, A = blockdiag(A_n, I), so T = blockdiag(T_n, I)).  K and beta go
//       to LDS at once; V stays in registers until the T tile is free (LDS per unit is
//       K + T, 34 KiB at C = 64, so four workgroups share a CU);
//   a2  Gram G = K K^T, lower 16x16 tiles only, on bf16 MFMA (fp32 MFMA for fp32 inputs);
//   a3  A = I + strictLower(diag(beta) G): beta scales rows, the diagonal is 1 ([Inv] 3.2);
//   a4  A lives in one fp32 LDS tile; its diagonal 16x16 blocks are inverted in place and
//       each coupling level overwrites its sub-diagonal block ([Inv] 3.3-3.6);
//   a5  C/16 independent 16x16 forward substitutions, one lane per column ([Inv] 2.1, 3.4);
//   a6  coupling levels s = 16, 32, 64: X10 = -X11 L10 X00 as two fp32 MFMA products, the
//       first product's accumulator feeding the second as its B operand ([Inv] 2.2, 3.5);
//   a7  store T (fp32; upper triangle 0, diagonal 1), then overwrite the T tile in place with
//       T' = T diag(beta) as a hi + lo pair of bf16 values;
//   a8  W^T = K^T T'^T and U^T = V^T T'^T on bf16 MFMA (16x16x16 at C = 32; from C = 64 on
//       16x16x32, each wave owning two row tiles), hi and lo parts of T' accumulated in turn
//       (T' is lower triangular, so k-tiles right of the diagonal are skipped); the transposed
//       accumulators hold four consecutive output columns per lane, staged in LDS and stored
//       with 16-byte writes.
// Gated instances ([Inv] section 5, item 12: with gating the coefficient is
// diag(beta)(Gamma o K K^T); g [B,T,Hv] is the per-token log gate of [QLA] usage) also read g:
//   a1' wave 0 forms the chunk-local inclusive prefix sums G_i = g_0 + ... + g_i in fp64 (one
//       shuffle scan) and parks G_i and exp(G_i) in the 16 padding bytes of staged K row i;
//   a3' every A entry below the diagonal takes the decay Gamma[i][j] = exp(G_i - G_j);
//   a8' W takes T diag(beta exp(G)): each wave rescales its T' chunks column by column by
//       exp(G_j) in registers (exp(G_j) <= 1 for decaying gates, so nothing overflows) before
//       the W product, and U keeps T' = T diag(beta).
//
// MFMA operand convention: for a 16x16 output tile, lane l = 16*g + c holds row/column c and
// k-group g.  In __builtin_amdgcn_mfma_f32_16x16x4f32 sub-step q the lane supplies true
// k = 16*kt + 4*g + q; in __builtin_amdgcn_mfma_f32_16x16x32_bf16 element j supplies true
// k = 32*kt + 8*g + j.  A and B use the same map, so the contraction is exact in any hardware
// k order.  Accumulator element r of lane 16*g + c is D[4*g + r][c]; with the k map above that
// is exactly the B operand a following 16x16x4 product needs.  The helpers shared with the
// backward (a0, a5, a6, the T-tile layout, Gram fragments) live in wyprep_device.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>
#include <type_traits>

#include "wyprep_device.h"
#include "wyprep_launch.h"

namespace wyp {
namespace {

// What one launch writes: T (kkt_solve, wy_prepare), W and U (wy_prepare, wu_prepare), or X for
// one right-hand side (solve_rhs); and whether it reads log gates g.
constexpr int kModeT = 1;
constexpr int kModeWU = 2;
constexpr int kModeGate = 4;
constexpr int kModeSolve = 8;

// LDS plan of one workgroup.  K and V rows carry 16 bytes of padding and T rows 4 floats, so
// 16-byte reads of one column chunk by 16 consecutive rows spread over all banks.  V never
// has its own region: it waits in registers until the T tile has been read for the last time
// and then takes its place, so one unit needs K + max(T, V) bytes (34 KiB at C = 64: four
// workgroups per CU).  The T tile's placement is TLayout (wyprep_device.h).
template <int C, int DT, bool WU>
struct Lds {
    static constexpr int ESZ = DT == 0 ? 2 : 4;
    // Elements per staged K / V row: 128 plus 16 bytes of padding.  No K / V / W / U access
    // touches the padding; gated instances keep row i's G_i (fp64) and exp(G_i) (fp32) there
    // (see GateRow), so the gates cost no LDS.
    static constexpr int KROW = kD + 16 / ESZ;
    static constexpr int KBYTES = C * KROW * ESZ;
    using TL = TLayout<C>;
    static constexpr int TBYTES = TL::BYTES;
    static constexpr int TVBYTES = WU && KBYTES > TBYTES ? KBYTES : TBYTES;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_T = KBYTES;         // T, later V and the U staging
    static constexpr int OFF_B = OFF_T + TVBYTES;
    static constexpr int OFF_INFO = OFF_B + C * 4;
    static constexpr int TOTAL = OFF_INFO + 16;
};

// Waves per SIMD the LDS plan allows (one wave of each resident workgroup per SIMD); the
// register allocator is held to that budget.
template <int C, int DT, bool WU>
struct WavesPerEu {
    static constexpr int by_lds = (160 * 1024) / Lds<C, DT, WU>::TOTAL;
    static constexpr int value = by_lds < 1 ? 1 : (by_lds > 4 ? 4 : by_lds);
};

// a1: K, V and beta of one unit in flight to registers, then committed to LDS.  K and beta
// are committed at the start of their unit; V only after that unit's T tile has been used.
template <int C, int ESZ, int KROW, bool RV, bool GT>
struct Prefetch {
    static constexpr bool WU = RV;  // V (or the right-hand side) is loaded
    static constexpr int CPR = kD * ESZ / 16;  // 16-byte chunks per row
    static constexpr int NIT = C * CPR / kThreads;
    static constexpr int NG = C > 64 ? 2 : 1;  // log gates per lane of wave 0
    static_assert(C * CPR % kThreads == 0, "row chunks must split evenly");
    u32x4 k[NIT];
    u32x4 v[WU ? NIT : 1];
    float b;
    float g[NG];  // gated: wave 0 lane l holds g of rows l and l + 64

    __device__ static __amdgpu_buffer_rsrc_t rows(const void* base, const Unit& u, int heads, int head)
    {
        const uint32_t stride = static_cast<uint32_t>(heads) * kD * ESZ;
        const unsigned char* p = static_cast<const unsigned char*>(base) + (u.tok0 * heads + head) * (kD * ESZ);
        return rsrc(p, (u.n - 1) * stride + kD * ESZ);
    }

    __device__ void issue_k(const Params& p, const Unit& u, int tid)
    {
        const int hk = u.hv / (p.hv / p.hq);
        const uint32_t kstride = static_cast<uint32_t>(p.hq) * kD * ESZ;
        const __amdgpu_buffer_rsrc_t kr = rows(p.k, u, p.hq, hk);
        // thread tid takes row tid / CPR + it * (kThreads / CPR), chunk tid % CPR: one multiply
        // per thread, then a scalar step per iteration (all of it in the range-checked offset)
        const uint32_t koff = (tid / CPR) * kstride + (tid % CPR) * 16;
        const uint32_t kstep = (kThreads / CPR) * kstride;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
            k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + it * kstep, 0, 0);
        const __amdgpu_buffer_rsrc_t br =
            rsrc(p.beta + u.tok0 * p.hv + u.hv, ((u.n - 1) * p.hv + 1) * 4);
        b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, (tid % C) * p.hv * 4, 0, 0));
        if constexpr (GT) {
            // rows >= n read as 0, so G stays flat over a short chunk's padding
            if (tid < 64) {
                const __amdgpu_buffer_rsrc_t gr =
                    rsrc(p.g + u.tok0 * p.hv + u.hv, ((u.n - 1) * p.hv + 1) * 4);
#pragma unroll
                for (int e = 0; e < NG; ++e)
                    g[e] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(gr, (tid + 64 * e) * p.hv * 4, 0, kStream));
            }
        }
    }

    __device__ void issue_v(const Params& p, const Unit& u, int tid)
    {
        if constexpr (WU) {
            const uint32_t vstride = static_cast<uint32_t>(p.hv) * kD * ESZ;
            const __amdgpu_buffer_rsrc_t vr = rows(p.v, u, p.hv, u.hv);
            const uint32_t voff = (tid / CPR) * vstride + (tid % CPR) * 16;
            const uint32_t vstep = (kThreads / CPR) * vstride;
#pragma unroll
            for (int it = 0; it < NIT; ++it)
                v[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff + it * vstep, 0, kStream);
        }
    }

    __device__ void commit_k(unsigned char* Kraw, float* bs, int tid) const
    {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kThreads;
            *reinterpret_cast<u32x4*>(Kraw + (q / CPR) * (KROW * ESZ) + (q % CPR) * 16) = k[it];
        }
        if (tid < C) bs[tid] = b;
        if constexpr (GT) {
            // a1': G = inclusive prefix sums of g over the chunk, in fp64, by wave 0
            if (tid < 64) {
                const int lane = tid;
                double run = 0.0;
#pragma unroll
                for (int e = 0; e < NG; ++e) {
                    double x = static_cast<double>(g[e]);
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const double t = __shfl_up(x, d);
                        if (lane >= d) x += t;
                    }
                    x += run;
                    const int r = lane + 64 * e;
                    if (r < C) {
                        *GateRow<KROW, ESZ>::Gp(Kraw, r) = x;
                        // fp32 exp: e^G only scales W's columns, whose output is bf16
                        *GateRow<KROW, ESZ>::Ep(Kraw, r) = __expf(static_cast<float>(x));
                    }
                    run = __shfl(x, 63);
                }
            }
        }
    }

    __device__ void commit_v(unsigned char* Vraw, int tid) const
    {
        if constexpr (WU) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int q = tid + it * kThreads;
                *reinterpret_cast<u32x4*>(Vraw + (q / CPR) * (KROW * ESZ) + (q % CPR) * 16) = v[it];
            }
        }
    }
};

// a3 for one lower tile (I, J) of the Gram accumulator acc (element r of lane 16 lg + lr is
// G[16 I + 4 lg + r][16 J + lr]): A below the diagonal, 1 on it.  Diagonal tiles keep L^T in
// their upper triangle (G is symmetric, so entry (i, j), i < j, is beta_j G[j][i] = L[j][i]);
// the substitution reads columns of L there and overwrites it with zeros.
template <int KROW, int ESZ, class TL, bool GT>
__device__ __attribute__((always_inline)) void a_tile_out(const f32x4& acc, const unsigned char* Kraw, float* Ts,
                                                          const float* bs, int I, int J, int lr, int lg)
{
    const f32x4 bet = *reinterpret_cast<const f32x4*>(bs + 16 * I + 4 * lg);
    const float bcol = bs[16 * J + lr];
    double gcol = 0.0;
    if constexpr (GT) gcol = GateRow<KROW, ESZ>::G(Kraw, 16 * J + lr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * lg + r, j = 16 * J + lr;
        float a = acc[r];
        if constexpr (GT) {
            // a3': decay Gamma between the later and the earlier token of the pair
            const double d = GateRow<KROW, ESZ>::G(Kraw, i) - gcol;
            a *= __expf(static_cast<float>(i > j ? d : -d));
        }
        Ts[TL::off(i, j)] = (i > j) ? bet[r] * a : (i == j ? 1.f : bcol * a);
    }
}

// a2 + a3 at C = 128 (bf16 K): wave w forms the lower tiles of row blocks w and 7 - w, nine
// tiles for every wave, one row block after the other.  A row block's K fragments are read once
// for all its tiles, so a unit reads 36 blocks of 16 K rows from LDS instead of the 72 that
// tile-by-tile products read (both blocks of every tile).  Sharing the column blocks between the
// two rows as well (26 reads) measured no faster and holds 16 more registers.
//
// At C = 64 the two row-block pairs (0, 3) and (1, 2) are split over waves p and p + 2 (PART 0
// and 1): wave p forms row p and the first 2 - p tiles of row 3 - p, wave p + 2 the rest of
// row 3 - p (three, three, two and two tiles, as the tile-by-tile order deals them).
template <int C, int KROW, class TL, bool GT, int MA, int PART = -1>
__device__ __attribute__((always_inline)) void form_a_rows_w(const unsigned char* Kraw, float* Ts, const float* bs,
                                                             int lr, int lg)
{
    constexpr int NB = C / 16;
    constexpr int MB = NB - 1 - MA;
    constexpr int NS = kD / 32;
    const __bf16* K = reinterpret_cast<const __bf16*>(Kraw);
    // fragment of row block `blk`: lane 16 g + c holds row 16 blk + c, dk 32 s + 8 g .. + 7
    auto frag = [&](int blk, bf16x8 (&f)[NS]) {
#pragma unroll
        for (int s = 0; s < NS; ++s) f[s] = *reinterpret_cast<const bf16x8*>(K + (16 * blk + lr) * KROW + 32 * s + 8 * lg);
    };
    auto tile = [&](const bf16x8 (&fi)[NS], const bf16x8 (&fj)[NS], int I, int J) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fi[s], fj[s], acc, 0, 0, 0);
        a_tile_out<KROW, 2, TL, GT>(acc, Kraw, Ts, bs, I, J, lr, lg);
        // gated: the fp64 gates each tile's decay reads would otherwise be hoisted out of the
        // unrolled tiles and held all at once
        if constexpr (GT) __builtin_amdgcn_sched_barrier(0);
    };
    // tiles J0 .. J1 of row block I, one row block at a time, so only its fragments and one
    // column block's are live
    auto row = [&](int I, int J0, int J1) {
        bf16x8 fi[NS];
        frag(I, fi);
#pragma unroll
        for (int J = J0; J <= J1; ++J) {  // unrolled: J == I is resolved at compile time
            if (J == I) {
                tile(fi, fi, I, J);
            } else {
                bf16x8 fj[NS];
                frag(J, fj);
                tile(fi, fj, I, J);
            }
        }
    };
    if constexpr (PART < 0) {
        row(MA, 0, MA);
        row(MB, 0, MB);
    } else if constexpr (PART == 0) {
        row(MA, 0, MA);
        row(MB, 0, NB / 2 - 1 - MA);
    } else {
        row(MB, NB / 2 - MA, MB);
    }
}

// a2 + a3: A = I + strictLower(diag(beta) K K^T) into Ts; all C x C entries are written.
// Lower tiles t = 0.. (row-major over I >= J) go to wave t % 4 (with bf16 K at C = 64 and 128:
// by row blocks, form_a_rows_w); upper tiles are zeroed with one 16-byte write per lane.
template <int C, int DT, int KROW, class TL, bool GT>
__device__ __attribute__((always_inline)) void form_a(const unsigned char* Kraw, float* Ts, const float* bs, int tid)
{
    constexpr int ESZ = DT == 0 ? 2 : 4;
    constexpr int NB = C / 16;
    constexpr int NTILE = NB * (NB + 1) / 2;
    constexpr int PER = (NTILE + kWaves - 1) / kWaves;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    if constexpr (C == 128 && DT == 0 && TL::kTiled) {
        static_assert(NB == 2 * kWaves, "one pair of row blocks per wave");
        switch (wave) {  // uniform
        case 0: form_a_rows_w<C, KROW, TL, GT, 0>(Kraw, Ts, bs, lr, lg); break;
        case 1: form_a_rows_w<C, KROW, TL, GT, 1>(Kraw, Ts, bs, lr, lg); break;
        case 2: form_a_rows_w<C, KROW, TL, GT, 2>(Kraw, Ts, bs, lr, lg); break;
        default: form_a_rows_w<C, KROW, TL, GT, 3>(Kraw, Ts, bs, lr, lg); break;
        }
        return;  // the tile-packed layout stores no upper tiles
    }
    if constexpr (C == 64 && DT == 0) {
        switch (wave) {  // uniform
        case 0: form_a_rows_w<C, KROW, TL, GT, 0, 0>(Kraw, Ts, bs, lr, lg); break;
        case 1: form_a_rows_w<C, KROW, TL, GT, 1, 0>(Kraw, Ts, bs, lr, lg); break;
        case 2: form_a_rows_w<C, KROW, TL, GT, 0, 1>(Kraw, Ts, bs, lr, lg); break;
        default: form_a_rows_w<C, KROW, TL, GT, 1, 1>(Kraw, Ts, bs, lr, lg); break;
        }
    } else {
    // Operands are loaded tile by tile: other resident workgroups cover the LDS latency.  A
    // second operand buffer costs 32 registers and measured no faster even at C = 128, where
    // only two workgroups share a CU.
    constexpr int NBUF = 1;
    GramFrags<DT, KROW> f[NBUF];
    int I = 0, J = 0;
    if (wave < NTILE) {
        tile_of(wave, &I, &J);
        f[0].load(Kraw, I, J, lr, lg);
    }
#pragma unroll
    for (int tt = 0; tt < PER; ++tt) {
        const int t = tt * kWaves + wave;
        if (t >= NTILE) break;
        int In = 0, Jn = 0;
        const int tn = t + kWaves;
        if (NBUF == 2 && tt + 1 < PER && tn < NTILE) {
            tile_of(tn, &In, &Jn);
            f[(tt + 1) % NBUF].load(Kraw, In, Jn, lr, lg);
        }
        if (NBUF == 1 && tt > 0) f[0].load(Kraw, I, J, lr, lg);
        a_tile_out<KROW, ESZ, TL, GT>(f[tt % NBUF].product(), Kraw, Ts, bs, I, J, lr, lg);
        if (NBUF == 2) {
            I = In;
            J = Jn;
        } else if (tn < NTILE) {
            tile_of(tn, &I, &J);
        }
    }
    }
    // strictly upper tiles (I < J), enumerated row-major, also dealt round-robin to waves
    // (the tile-packed layout has none)
    if constexpr (!TL::kTiled) {
        constexpr int NUP = NB * (NB - 1) / 2;
#pragma unroll
        for (int tt = 0; tt < (NUP + kWaves - 1) / kWaves; ++tt) {
            const int t = tt * kWaves + wave;
            if (t >= NUP) break;
            int Iu = 0, rem = t;
            while (rem >= NB - 1 - Iu) {
                rem -= NB - 1 - Iu;
                ++Iu;
            }
            const int Ju = Iu + 1 + rem;
            *reinterpret_cast<f32x4*>(Ts + TL::off(16 * Iu + lr, 16 * Ju + 4 * lg)) = zero4();
        }
    }
}

// a7: T rows [0, n) to T_out[(tok0 + r) * Hv + hv][0:C] (with STORE; wu_prepare forms T but
// does not write it); rows >= n fall outside the buffer range and are dropped by the
// hardware.  With PACK, each thread then overwrites the 16-byte
// chunk it just stored with T' = T diag(beta) for the W/U products: four bf16 "hi" values
// followed by four bf16 "lo" values (lo = T' - hi, rounded), i.e. the same bytes per element.
template <int C, class TL, bool PACK, bool STORE>
__device__ void store_t(float* Ts, const float* bs, float* Tout, const Unit& u, int Hv, int tid)
{
    constexpr int TCH = C / 4;                 // 16-byte chunks per row
    constexpr int NIT = C * TCH / kThreads;    // 1 / 4 / 16 for C = 32 / 64 / 128
    static_assert(C * TCH % kThreads == 0, "T rows must split evenly");
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t rstride = static_cast<uint32_t>(Hv) * C * 4;
    const __amdgpu_buffer_rsrc_t tr =
        rsrc(STORE ? Tout + (u.tok0 * Hv + u.hv) * C : nullptr, STORE ? (u.n - 1) * rstride + C * 4 : 0);
    // With more than four chunks per thread (C = 128), the chunks are read in batches of four
    // ahead of the batch's T' writes: the compiler cannot move a read above a write to the same
    // tile, so one chunk at a time would expose every read's latency.
    constexpr int BATCH = NIT > 4 ? 4 : 1;
    // Chunk (row r, 16-byte column chunk c) of thread tid in iteration it.  Row-major tiles: 16
    // consecutive lanes take 16 consecutive chunks of one row, 64 distinct banks.  The
    // tile-packed layout puts the tiles of a row 320 floats apart, on the same banks, so there
    // one wave-wide access covers rows 16 I + rb + {0, 4, 8, 12} and tiles Jb .. Jb + 3 instead:
    // each 16 lanes read one tile's four rows at 20-float pitch (disjoint banks), and every row
    // still gets 256 contiguous bytes of the global store.
    // Wave-wide access n = 4 it + w (w the wave) covers, in the tile-packed layout, row block
    // I = n / 8 = it / 2, rows rb = (n / 2) mod 4 = 2 (it mod 2) + w / 2 plus {0, 4, 8, 12}, tiles
    // jb .. jb + 3; the half of the row (tiles 0-3 or 4-7) alternates with I, so every wave gets
    // as many tiles right of the diagonal (reads and T' writes skipped) as the others.  Written
    // with I and the row step known at compile time, every offset is a per-thread base plus a
    // scalar: no per-chunk multiply.
    const int wv = tid >> 6, lane = tid & 63;
    auto chunk_of = [&](int it, int* r, int* c) {
        if constexpr (TL::kTiled) {
            static_assert(C == 128 && kWaves == 4, "tile-packed T is used at C = 128 only");
            const int I = it >> 1, jb = 4 * ((wv ^ I) & 1);
            *r = 16 * I + 2 * (it & 1) + (wv >> 1) + 4 * ((lane >> 2) & 3);
            *c = 4 * (jb + (lane >> 4)) + (lane & 3);
        } else {
            *r = tid / TCH + it * (kThreads / TCH);
            *c = tid % TCH;
        }
    };
    // global byte offset of chunk (r, c) of iteration it, without a per-chunk multiply
    const uint32_t rowbase = TL::kTiled ? static_cast<uint32_t>((wv >> 1) + 4 * ((lane >> 2) & 3)) * rstride
                                        : static_cast<uint32_t>(tid / TCH) * rstride;
    auto store_off = [&](int it, int c) -> uint32_t {
        const uint32_t rstep = TL::kTiled ? static_cast<uint32_t>(16 * (it >> 1) + 2 * (it & 1))
                                          : static_cast<uint32_t>(it * (kThreads / TCH));
        return rowbase + rstep * rstride + static_cast<uint32_t>(c) * 16;
    };
#pragma unroll
    for (int b0 = 0; b0 < NIT; b0 += BATCH) {
    f32x4 vals[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
        int r, c;
        chunk_of(b0 + j, &r, &c);
        const bool upper = TL::kTiled && (c >> 2) > (r >> 4);
        vals[j] = upper ? zero4() : *reinterpret_cast<const f32x4*>(Ts + TL::off(r, 4 * c));
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
        int r, c;
        chunk_of(b0 + j, &r, &c);
        // tile-packed layout: chunks right of the diagonal tile are zeros that are not stored
        const bool upper = TL::kTiled && (c >> 2) > (r >> 4);
        f32x4* chunk = reinterpret_cast<f32x4*>(Ts + TL::off(r, 4 * c));
        const f32x4 val = vals[j];
        if constexpr (STORE)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), tr, store_off(b0 + j, c), 0, kStream);
        if (PACK && !upper) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(bs + 4 * c);
            bf16x4 h, l;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float tp = val[e] * b[e];
                h[e] = static_cast<__bf16>(tp);
                l[e] = static_cast<__bf16>(tp - static_cast<float>(h[e]));
            }
            const u32x2 hp = __builtin_bit_cast(u32x2, h), lp = __builtin_bit_cast(u32x2, l);
            *reinterpret_cast<u32x4*>(chunk) = u32x4{hp[0], hp[1], lp[0], lp[1]};
        }
    }
    }
}

// Stores n rows of 128 elements staged in LDS (row stride KROW elements) to a
// [tokens, Hv, 128] output.  Rows >= n are dropped by the buffer range.
template <int C, int ESZ, int KROW>
__device__ void store_rows(const unsigned char* src, void* out, const Unit& u, int Hv, int tid)
{
    constexpr int CPR = kD * ESZ / 16;
    constexpr int NIT = C * CPR / kThreads;
    const uint32_t rstride = static_cast<uint32_t>(Hv) * kD * ESZ;
    const __amdgpu_buffer_rsrc_t r_out = rsrc(static_cast<unsigned char*>(out) + (u.tok0 * Hv + u.hv) * (kD * ESZ),
                                              (u.n - 1) * rstride + kD * ESZ);
    // one multiply per thread, then a scalar row step per iteration
    const uint32_t off = (tid / CPR) * rstride + (tid % CPR) * 16, step = (kThreads / CPR) * rstride;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * kThreads;
        const int r = q / CPR, c16 = q % CPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(src + r * (KROW * ESZ) + c16 * 16);
        __builtin_amdgcn_raw_buffer_store_b128(val, r_out, off + it * step, 0, kStream);
    }
}

// a8 (bf16): W^T = K^T T'^T and U^T = V^T T'^T with T' = T diag(beta), read from the T tile
// as packed chunks of four hi and four lo bf16 values (see store_t): one chunk is exactly the
// hi and the lo operand of a 16x16x16 MFMA, and hi + lo carries T' to within 2^-17 |T'|, so
// the only rounding left in W and U is the final bf16 store.  k-tiles of 16 tokens right of
// the diagonal (zeros of T') are skipped.  The K^T / V^T operand (4 consecutive tokens of one
// column) is one LDS transpose read: within each 16-lane group, lane i of ds_read_tr16_b64
// receives element (i mod 4) of the 64-bit rows addressed by lanes 4e + i/4, e = 0..3.  Wave w
// owns column tiles w and w + 4 of W, then of U.  Accumulator element r of lane 16g + c is
// X[16mi + c][16ni + 4g + r]; the result leaves as bf16.  Used at C = 32; from C = 64 on the
// row products below take over.
template <int C, int KROW>
__device__ inline void wu_tiles(const unsigned char* src, const u32x4 (&tp)[C / 16][C / 16], int wave,
                                int lr, int lg, bf16x4 (&out)[2][C / 16])
{
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    constexpr int NB = C / 16;
    const __bf16* base = reinterpret_cast<const __bf16*>(src);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ni = wave + 4 * c;
        f32x4 acc[NB];
#pragma unroll
        for (int mi = 0; mi < NB; ++mi) acc[mi] = zero4();
#pragma unroll
        for (int kt = 0; kt < NB; ++kt) {
            // lane 16g + L addresses row 16kt + 4g + L/4, columns 16ni + 4(L%4) .. +3
            const __bf16* p0 = base + (16 * kt + 4 * lg + (lr >> 2)) * KROW + 16 * ni + 4 * (lr & 3);
            const i16x4 kfr = __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0)));
#pragma unroll
            for (int mi = kt; mi < NB; ++mi) {
                const i16x4 hi = __builtin_bit_cast(i16x4, u32x2{tp[mi][kt][0], tp[mi][kt][1]});
                const i16x4 lo = __builtin_bit_cast(i16x4, u32x2{tp[mi][kt][2], tp[mi][kt][3]});
                acc[mi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kfr, hi, acc[mi], 0, 0, 0);
                acc[mi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kfr, lo, acc[mi], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mi = 0; mi < NB; ++mi) {
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(acc[mi][r]);
            out[c][mi] = o;
        }
    }
}

template <int C, int KROW>
__device__ inline void stage_tiles(unsigned char* dst, const bf16x4 (&out)[2][C / 16], int wave, int lr, int lg)
{
    __bf16* d = reinterpret_cast<__bf16*>(dst);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mi = 0; mi < C / 16; ++mi)
            *reinterpret_cast<bf16x4*>(d + (16 * mi + lr) * KROW + 16 * (wave + 4 * c) + 4 * lg) = out[c][mi];
}

// a8' (gated): one packed T' chunk (four hi bf16, four lo bf16; see store_t) rescaled column
// by column, T' diag(e): hi + lo is T' to within 2^-17 |T'|, the product is rounded once in
// fp32, and the result is split into a new hi / lo pair the same way store_t splits T'.
__device__ inline u32x4 scale_chunk(u32x4 c, f32x4 e)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const bf16x4 h = __builtin_bit_cast(bf16x4, u32x2{c[0], c[1]});
    const bf16x4 l = __builtin_bit_cast(bf16x4, u32x2{c[2], c[3]});
    bf16x4 h2, l2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float f = (static_cast<float>(h[k]) + static_cast<float>(l[k])) * e[k];
        h2[k] = static_cast<__bf16>(f);
        l2[k] = static_cast<__bf16>(f - static_cast<float>(h2[k]));
    }
    const u32x2 hp = __builtin_bit_cast(u32x2, h2), lp = __builtin_bit_cast(u32x2, l2);
    return u32x4{hp[0], hp[1], lp[0], lp[1]};
}

// tp_rows' operands of one k step (columns 32 kt + 8 lg .. + 7) rescaled column by column by
// e^G, T' diag(e^G): hi + lo is rounded once in fp32 and split again, as in scale_chunk
template <int KROW>
__device__ inline void scale_rows(const unsigned char* Kraw, u32x4& hi, u32x4& lo, int kt, int lg)
{
    const bf16x8 h = __builtin_bit_cast(bf16x8, hi), l = __builtin_bit_cast(bf16x8, lo);
    bf16x8 h2, l2;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float f = (static_cast<float>(h[q]) + static_cast<float>(l[q])) *
                        GateRow<KROW, 2>::E(Kraw, 32 * kt + 8 * lg + q);
        h2[q] = static_cast<__bf16>(f);
        l2[q] = static_cast<__bf16>(f - static_cast<float>(h2[q]));
    }
    hi = __builtin_bit_cast(u32x4, h2);
    lo = __builtin_bit_cast(u32x4, l2);
}

// The same products split by rows, from C = 64 on.  At C = 128 all 36 lower T' blocks would take
// 144 registers per lane in every wave, so wave w owns row tiles mA = w and mB = NB - 1 - w (nine
// T' blocks between them, the same count for every wave) across all eight column tiles.  At
// C = 64 waves w and w + 2 own row tiles w and 3 - w (five blocks) and split the column tiles:
// each wave holds half the T' blocks of the all-blocks form and, gated, rescales only those
// (gated C = 64 7% faster, ungated unchanged).  Here k runs in
// steps of 32 tokens on 16x16x32 MFMA (twice the k of 16x16x16 at the same issue cost): element
// j of a lane in group g is token 32 kt + 8 g + j, the K^T / V^T operand is two transposed reads
// (tokens 8 g .. + 3 and 8 g + 4 .. + 7), and the T' operands are tp[2 kt] (hi) and tp[2 kt + 1]
// (lo) as tp_rows lays them out.  Accumulator element r of lane 16g + c is
// X[16m + c][16ni + 4g + r] as above.  The row tiles are template arguments (one instance per
// wave, picked by a uniform switch), so the k loops have fixed bounds and no branches: several
// transposed reads can be in flight together.  (Kept outside: the gate rescale of the operands;
// inside the per-wave instances it raises the register count past two waves per SIMD.)
template <int C, int KROW, int MA, int NI0, int NNI>
__device__ inline void wu_tiles_rows_w(const unsigned char* src, const u32x4 (&tpA)[C / 16],
                                       const u32x4 (&tpB)[C / 16], int lr, int lg, bf16x4 (&out)[NNI][2])
{
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    constexpr int NB = C / 16;
    constexpr int MB = NB - 1 - MA;
    const __bf16* base = reinterpret_cast<const __bf16*>(src);
#pragma unroll
    for (int ni = NI0; ni < NI0 + NNI; ++ni) {
        f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
        for (int kt = 0; kt <= MB / 2; ++kt) {
            const __bf16* p0 = base + (32 * kt + 8 * lg + (lr >> 2)) * KROW + 16 * ni + 4 * (lr & 3);
            const i16x4 f0 = __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0)));
            const i16x4 f1 = __builtin_bit_cast(i16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * KROW)));
            const bf16x8 kfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f0, f1, 0, 1, 2, 3, 4, 5, 6, 7));
            a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, __builtin_bit_cast(bf16x8, tpB[2 * kt]), a1, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, __builtin_bit_cast(bf16x8, tpB[2 * kt + 1]), a1, 0, 0, 0);
            if (kt <= MA / 2) {  // folds away once the loop is unrolled
                a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, __builtin_bit_cast(bf16x8, tpA[2 * kt]), a0, 0, 0, 0);
                a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, __builtin_bit_cast(bf16x8, tpA[2 * kt + 1]), a0, 0, 0, 0);
            }
        }
        bf16x4 o0, o1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o0[r] = static_cast<__bf16>(a0[r]);
            o1[r] = static_cast<__bf16>(a1[r]);
        }
        out[ni - NI0][0] = o0;
        out[ni - NI0][1] = o1;
    }
}

// Output column tiles (of kD / 16) per wave in the row products: all eight at C = 128 (four
// waves, four row-tile pairs); four at C = 64, where waves w and w + 2 share row tiles w and
// 3 - w and take column tiles 0-3 and 4-7.
template <int C>
constexpr int kRowNNI = C == 128 ? kD / 16 : kD / 32;

// T' of row tile m as the B operands of the row products above: for lane (lr, lg), tp[2 kt] holds
// the hi halves and tp[2 kt + 1] the lo halves of row 16 m + lr, columns 32 kt + 8 lg .. + 7, in
// column order.  Each half of a packed chunk (see store_t) is read straight into its place;
// columns in 16x16 blocks right of the diagonal read as zero (the tile-packed layout does not
// store them).
template <int C, class TL>
__device__ inline void tp_rows(const float* Ts, int m, int lr, int lg, u32x4 (&tp)[C / 16])
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int kt = 0; kt < C / 32; ++kt) {
        u32x2 hi[2], lo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = 32 * kt + 8 * lg + 4 * h;
            const float* c = Ts + TL::off(16 * m + lr, col);
            const bool in = (col >> 4) <= m;
            hi[h] = in ? *reinterpret_cast<const u32x2*>(c) : u32x2{0u, 0u};
            lo[h] = in ? *reinterpret_cast<const u32x2*>(c + 2) : u32x2{0u, 0u};
        }
        tp[2 * kt] = u32x4{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
        tp[2 * kt + 1] = u32x4{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
    }
}

template <int C, int KROW>
__device__ inline void wu_tiles_rows(const unsigned char* src, const u32x4 (&tpA)[C / 16], const u32x4 (&tpB)[C / 16],
                                     int wave, int lr, int lg, bf16x4 (&out)[kRowNNI<C>][2])
{
    constexpr int N = kRowNNI<C>;
    static_assert(kWaves == 4 && (C == 128 || C == 64), "four waves; row-tile pairs at C = 64, 128");
    if constexpr (C == 128) {
        switch (wave) {  // uniform
        case 0: wu_tiles_rows_w<C, KROW, 0, 0, N>(src, tpA, tpB, lr, lg, out); break;
        case 1: wu_tiles_rows_w<C, KROW, 1, 0, N>(src, tpA, tpB, lr, lg, out); break;
        case 2: wu_tiles_rows_w<C, KROW, 2, 0, N>(src, tpA, tpB, lr, lg, out); break;
        default: wu_tiles_rows_w<C, KROW, 3, 0, N>(src, tpA, tpB, lr, lg, out); break;
        }
    } else {
        switch (wave) {  // uniform
        case 0: wu_tiles_rows_w<C, KROW, 0, 0, N>(src, tpA, tpB, lr, lg, out); break;
        case 1: wu_tiles_rows_w<C, KROW, 1, 0, N>(src, tpA, tpB, lr, lg, out); break;
        case 2: wu_tiles_rows_w<C, KROW, 0, N, N>(src, tpA, tpB, lr, lg, out); break;
        default: wu_tiles_rows_w<C, KROW, 1, N, N>(src, tpA, tpB, lr, lg, out); break;
        }
    }
}

template <int C, int KROW>
__device__ inline void stage_tiles_rows(unsigned char* dst, const bf16x4 (&out)[kRowNNI<C>][2], int mA, int mB,
                                        int ni0, int lr, int lg)
{
    __bf16* d = reinterpret_cast<__bf16*>(dst);
#pragma unroll
    for (int c = 0; c < kRowNNI<C>; ++c) {
        const int ni = ni0 + c;
        *reinterpret_cast<bf16x4*>(d + (16 * mA + lr) * KROW + 16 * ni + 4 * lg) = out[c][0];
        *reinterpret_cast<bf16x4*>(d + (16 * mB + lr) * KROW + 16 * ni + 4 * lg) = out[c][1];
    }
}

// exp(G_j) of the four T' columns 16 kt + 4 lg + 0..3 that one lane's chunks hold.
template <int KROW>
__device__ inline f32x4 gate_cols(const unsigned char* Kraw, int kt, int lg)
{
    f32x4 e;
#pragma unroll
    for (int q = 0; q < 4; ++q) e[q] = GateRow<KROW, 2>::E(Kraw, 16 * kt + 4 * lg + q);
    return e;
}

// Every wave first takes its T' chunks (lower-triangular 16x16 blocks) into registers; then V,
// waiting in registers, takes the T tile's place.  W is staged over K while U is computed.
// Gated: U is formed first with T' = T diag(beta) and staged over V; the same registers are
// then rescaled column by column to T' diag(exp(G)) for W, whose K rows (and gate values) are
// still in LDS.
template <int C, int KROW, class TL, bool GT, class PF>
__device__ void wu_bf16(unsigned char* Kraw, float* Ts, PF& pf, const Params& p, const Unit& u, int tid)
{
    constexpr int NB = C / 16;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    if constexpr (GT && C >= 64) {
        const int mA = C == 128 ? wave : (wave & 1), mB = NB - 1 - mA;
        const int ni0 = C == 128 ? 0 : (wave >> 1) * kRowNNI<C>;
        u32x4 tpA[NB], tpB[NB];
        tp_rows<C, TL>(Ts, mA, lr, lg, tpA);
        tp_rows<C, TL>(Ts, mB, lr, lg, tpB);
        __syncthreads();  // the T tile is no longer read: V takes its place
        unsigned char* Vraw = reinterpret_cast<unsigned char*>(Ts);
        pf.commit_v(Vraw, tid);
        __syncthreads();
        bf16x4 out[kRowNNI<C>][2];
        wu_tiles_rows<C, KROW>(Vraw, tpA, tpB, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading V: U is staged over it
        stage_tiles_rows<C, KROW>(Vraw, out, mA, mB, ni0, lr, lg);
#pragma unroll
        for (int kt = 0; kt < NB / 2; ++kt) {
            if (2 * kt > mB) continue;  // uniform; a k step wholly right of the diagonal stays zero
            if (2 * kt <= mA) scale_rows<KROW>(Kraw, tpA[2 * kt], tpA[2 * kt + 1], kt, lg);
            scale_rows<KROW>(Kraw, tpB[2 * kt], tpB[2 * kt + 1], kt, lg);
        }
        wu_tiles_rows<C, KROW>(Kraw, tpA, tpB, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading K: W is staged over it
        stage_tiles_rows<C, KROW>(Kraw, out, mA, mB, ni0, lr, lg);
        __syncthreads();
        store_rows<C, 2, KROW>(Kraw, p.W, u, p.hv, tid);
        store_rows<C, 2, KROW>(Vraw, p.U, u, p.hv, tid);
    } else if constexpr (GT) {
        u32x4 tp[NB][NB];
#pragma unroll
        for (int mi = 0; mi < NB; ++mi)
#pragma unroll
            for (int kt = 0; kt <= mi; ++kt)
                tp[mi][kt] = *reinterpret_cast<const u32x4*>(Ts + TL::off(16 * mi + lr, 16 * kt + 4 * lg));
        __syncthreads();  // the T tile is no longer read: V takes its place
        unsigned char* Vraw = reinterpret_cast<unsigned char*>(Ts);
        pf.commit_v(Vraw, tid);
        __syncthreads();
        bf16x4 out[2][NB];
        wu_tiles<C, KROW>(Vraw, tp, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading V: U is staged over it
        stage_tiles<C, KROW>(Vraw, out, wave, lr, lg);
#pragma unroll
        for (int kt = 0; kt < NB; ++kt) {
            const f32x4 e = gate_cols<KROW>(Kraw, kt, lg);
#pragma unroll
            for (int mi = kt; mi < NB; ++mi) tp[mi][kt] = scale_chunk(tp[mi][kt], e);
        }
        wu_tiles<C, KROW>(Kraw, tp, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading K: W is staged over it
        stage_tiles<C, KROW>(Kraw, out, wave, lr, lg);
        __syncthreads();
        store_rows<C, 2, KROW>(Kraw, p.W, u, p.hv, tid);
        store_rows<C, 2, KROW>(Vraw, p.U, u, p.hv, tid);
    } else if constexpr (C >= 64) {
        const int mA = C == 128 ? wave : (wave & 1), mB = NB - 1 - mA;
        const int ni0 = C == 128 ? 0 : (wave >> 1) * kRowNNI<C>;
        u32x4 tpA[NB], tpB[NB];
        tp_rows<C, TL>(Ts, mA, lr, lg, tpA);
        tp_rows<C, TL>(Ts, mB, lr, lg, tpB);
        __syncthreads();  // the T tile is no longer read: V takes its place
        unsigned char* Vraw = reinterpret_cast<unsigned char*>(Ts);
        pf.commit_v(Vraw, tid);
        __syncthreads();
        bf16x4 out[kRowNNI<C>][2];
        wu_tiles_rows<C, KROW>(Kraw, tpA, tpB, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading K: W is staged over it
        stage_tiles_rows<C, KROW>(Kraw, out, mA, mB, ni0, lr, lg);
        wu_tiles_rows<C, KROW>(Vraw, tpA, tpB, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading V: U is staged over it
        stage_tiles_rows<C, KROW>(Vraw, out, mA, mB, ni0, lr, lg);
        __syncthreads();
        store_rows<C, 2, KROW>(Kraw, p.W, u, p.hv, tid);
        store_rows<C, 2, KROW>(Vraw, p.U, u, p.hv, tid);
    } else {
        u32x4 tp[NB][NB];
#pragma unroll
        for (int mi = 0; mi < NB; ++mi)
#pragma unroll
            for (int kt = 0; kt <= mi; ++kt)
                tp[mi][kt] = *reinterpret_cast<const u32x4*>(Ts + TL::off(16 * mi + lr, 16 * kt + 4 * lg));
        __syncthreads();  // the T tile is no longer read: V takes its place
        unsigned char* Vraw = reinterpret_cast<unsigned char*>(Ts);
        pf.commit_v(Vraw, tid);
        __syncthreads();

        bf16x4 out[2][NB];
        wu_tiles<C, KROW>(Kraw, tp, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading K: W is staged over it
        stage_tiles<C, KROW>(Kraw, out, wave, lr, lg);
        wu_tiles<C, KROW>(Vraw, tp, wave, lr, lg, out);
        __syncthreads();  // every wave is done reading V: U is staged over it
        stage_tiles<C, KROW>(Vraw, out, wave, lr, lg);
        __syncthreads();
        store_rows<C, 2, KROW>(Kraw, p.W, u, p.hv, tid);
        store_rows<C, 2, KROW>(Vraw, p.U, u, p.hv, tid);
    }
}

// a8 (fp32 inputs): the same transposed products on fp32 MFMA, T' = T diag(beta) kept in fp32
// registers before V takes the T tile's place.
template <int C, int KROW, class TL, bool GT, class PF>
__device__ void wu_f32(unsigned char* Kraw, float* Ts, const float* bs, PF& pf, const Params& p,
                       const Unit& u, int tid)
{
    constexpr int NB = C / 16;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 tfr[NB][NB];
#pragma unroll
    for (int mi = 0; mi < NB; ++mi)
#pragma unroll
        for (int kt = 0; kt <= mi; ++kt) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(Ts + TL::off(16 * mi + lr, 16 * kt + 4 * lg));
            const f32x4 b = *reinterpret_cast<const f32x4*>(bs + 16 * kt + 4 * lg);
            tfr[mi][kt] = t * b;
        }
    __syncthreads();  // the T tile is no longer read: V takes its place
    unsigned char* Vraw = reinterpret_cast<unsigned char*>(Ts);
    pf.commit_v(Vraw, tid);
    __syncthreads();

    f32x4 out[4][NB];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        // gated: the U tiles (c = 2, 3) first, then T diag(beta) becomes T diag(beta exp(G))
        // in place for the W tiles
        const int c = GT ? (cc + 2) % 4 : cc;
        if (GT && cc == 2) {
#pragma unroll
            for (int kt = 0; kt < NB; ++kt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float e = GateRow<KROW, 4>::E(Kraw, 16 * kt + 4 * lg + q);
#pragma unroll
                    for (int mi = kt; mi < NB; ++mi) tfr[mi][kt][q] *= e;
                }
        }
        const int ct = wave + 4 * c;
        const float* src = reinterpret_cast<const float*>(ct < 8 ? Kraw : Vraw);
        const int ni = ct & 7;
#pragma unroll
        for (int mi = 0; mi < NB; ++mi) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kt = 0; kt <= mi; ++kt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float kq = src[(16 * kt + 4 * lg + q) * KROW + 16 * ni + lr];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kq, tfr[mi][kt][q], acc, 0, 0, 0);
                }
            }
            out[c][mi] = acc;
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
            *reinterpret_cast<f32x4*>(dst + (16 * mi + lr) * KROW + 16 * ni + 4 * lg) = out[c][mi];
    }
    __syncthreads();
    store_rows<C, 4, KROW>(Kraw, p.W, u, p.hv, tid);
    store_rows<C, 4, KROW>(Vraw, p.U, u, p.hv, tid);
}

// The single right-hand side ([Inv] section 5, item 10: T used once is not materialised; the
// substitution is applied to the right-hand side): X = A^{-1} diag(beta) R by block forward
// substitution over the C/16 row blocks,
//     X_i = L_ii^{-1} (diag(beta_i) R_i - sum_{j<i} A_ij X_j),
// with L_ii^{-1} the inverted diagonal blocks (a5) and A_ij the sub-diagonal blocks of A as
// form_a left them; the coupling levels that would fill in T are never run.  Wave w owns the 32
// columns 32 w .. 32 w + 31 of R and X (two column tiles) for every row block, so the waves never
// wait for each other.  The fp32 instance runs both products on fp32 MFMA 16x16x4: the
// accumulator of X_j (element r of lane 16 g + c is X_j[4 g + r][c]) is exactly the B operand the
// later products take, so X stays in registers; the bf16 instance splits the same operands into
// bf16 hi / lo halves for the 16x16x16 bf16 MFMA.  R_i is read from LDS in that layout and X_i
// written back over it (same wave, same columns), as bf16 (or fp32) for the row store.
template <int C, int DT, int KROW, class TL>
__device__ void solve_rhs(unsigned char* Rraw, const float* Ts, const float* bs, int tid)
{
    constexpr int NB = C / 16;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    if constexpr (DT == 0) {
        // bf16 right-hand side and output: the sums A_ij X_j run as three bf16 MFMA 16x16x16
        // products of the hi / lo halves of A_ij and X_j (hi*hi + hi*lo + lo*hi; the dropped
        // lo*lo term is below 2^-17 of the product), a third of the fp32 16x16x4 MFMA time.  The
        // 16x16x16 operands take the same lane layout as the 16x16x4 steps (lane 16 g + c: row or
        // column c, k = 4 g .. 4 g + 3), so X_j's accumulator is split in place once and kept
        // as its two bf16 halves.  The product with L_ii^{-1} stays on fp32 MFMA, so where A is
        // the identity X = diag(beta) R is rounded once.
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        auto split = [](const f32x4& x, i16x4& h, i16x4& l) {
            bf16x4 hb, lb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hb[e] = static_cast<__bf16>(x[e]);
                lb[e] = static_cast<__bf16>(x[e] - static_cast<float>(hb[e]));
            }
            h = __builtin_bit_cast(i16x4, hb);
            l = __builtin_bit_cast(i16x4, lb);
        };
        i16x4 xh[NB][2], xl[NB][2];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int j = 0; j < i; ++j) {
                i16x4 ah, al;
                split(*reinterpret_cast<const f32x4*>(Ts + TL::off(16 * i + lr, 16 * j + 4 * lg)), ah, al);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, xh[j][c], acc[c], 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, xl[j][c], acc[c], 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, xh[j][c], acc[c], 0, 0, 0);
                }
            }
            const f32x4 inv = *reinterpret_cast<const f32x4*>(Ts + TL::off(16 * i + lr, 16 * i + 4 * lg));
            const f32x4 bet = *reinterpret_cast<const f32x4*>(bs + 16 * i + 4 * lg);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int col = 32 * wave + 16 * c + lr;
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i + 4 * lg + r;
                    y[r] = bet[r] * static_cast<float>(reinterpret_cast<const __bf16*>(Rraw)[row * KROW + col]) -
                           acc[c][r];
                }
                f32x4 x = zero4();
#pragma unroll
                for (int q = 0; q < 4; ++q) x = __builtin_amdgcn_mfma_f32_16x16x4f32(inv[q], y[q], x, 0, 0, 0);
                split(x, xh[i][c], xl[i][c]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i + 4 * lg + r;
                    reinterpret_cast<__bf16*>(Rraw)[row * KROW + col] = static_cast<__bf16>(x[r]);
                }
            }
        }
        return;
    }
    f32x4 X[NB][2];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
        for (int j = 0; j < i; ++j) {
            // A_ij row 16 i + lr, columns 16 j + 4 lg .. + 3: the A operand of all four k steps
            const f32x4 a = *reinterpret_cast<const f32x4*>(Ts + TL::off(16 * i + lr, 16 * j + 4 * lg));
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q], X[j][c][q], acc[c], 0, 0, 0);
        }
        const f32x4 inv = *reinterpret_cast<const f32x4*>(Ts + TL::off(16 * i + lr, 16 * i + 4 * lg));
        const f32x4 bet = *reinterpret_cast<const f32x4*>(bs + 16 * i + 4 * lg);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int col = 32 * wave + 16 * c + lr;
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * lg + r;
                y[r] = bet[r] * reinterpret_cast<const float*>(Rraw)[row * KROW + col] - acc[c][r];
            }
            f32x4 x = zero4();
#pragma unroll
            for (int q = 0; q < 4; ++q) x = __builtin_amdgcn_mfma_f32_16x16x4f32(inv[q], y[q], x, 0, 0, 0);
            X[i][c] = x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * lg + r;
                reinterpret_cast<float*>(Rraw)[row * KROW + col] = x[r];
            }
        }
    }
}

// a6 for T alone (kkt_solve) at S = 32 (C = 64) and S = 64 (C = 128).  coupling_level gives a
// pair's column tile to one wave, and that wave's chain (28 and 104 fp32 MFMAs) is the unit's
// longest.  Here every wave takes tiles of both passes: tmp = L10 X00 into `tmpb` (K's region,
// which T alone no longer reads; one 16-byte chunk per lane and tile), a barrier, then
// X10 = -X11 tmp over L10.  Pass A's tile (mr, nc) costs TS - nc steps of four MFMAs and pass B's
// mr + 1: at S = 64 wave w takes row mr = w of pass A and column nc = w of pass B (ten steps
// each), at S = 32 tile (w >> 1, w & 1) of A and (w & 1, w >> 1) of B (three in all).  Each sum
// keeps coupling_level's order (the zero tiles above X00's diagonal skipped), so T is the same.
template <int C, int S, class TL, bool INPLACE>
__device__ void coupling_2pass(float* Ts, float* tmpb, int tid)
{
    constexpr int TS = S / 16;
    constexpr int PER = TS * TS / kWaves;  // tiles per wave and pass: 1 at S = 32, 4 at S = 64
    static_assert(C == 2 * S && kWaves == 4 && (S == 32 || S == 64), "one pair of blocks, four waves");
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    f32x4 acc[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {  // pass A: tmp(mr, nc) = sum_{kt >= nc} L10(mr, kt) X00(kt, nc)
        const int mr = S == 64 ? wave : wave >> 1;
        const int nc = S == 64 ? t : wave & 1;
        acc[t] = zero4();
        for (int kt = nc; kt < TS; ++kt) {  // uniform
            float bq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bq[q] = Ts[TL::off(16 * kt + 4 * lg + q, 16 * nc + lr)];
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + TL::off(S + 16 * mr + lr, 16 * kt + 4 * lg));
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bq[q], acc[t], 0, 0, 0);
        }
        if constexpr (!INPLACE) *reinterpret_cast<f32x4*>(tmpb + (mr * TS + nc) * 256 + 4 * lane) = acc[t];
    }
    if constexpr (INPLACE) {  // tmp over L10, once every wave has read L10 for the last time
        __syncthreads();
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int mr = S == 64 ? wave : wave >> 1;
            const int nc = S == 64 ? t : wave & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ts[TL::off(S + 16 * mr + 4 * lg + r, 16 * nc + lr)] = acc[t][r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PER; ++t) {  // pass B: X10(mr, nc) = -sum_{kt <= mr} X11(mr, kt) tmp(kt, nc)
        const int nc = S == 64 ? wave : wave >> 1;
        const int mr = S == 64 ? t : wave & 1;
        acc[t] = zero4();
        for (int kt = 0; kt <= mr; ++kt) {  // uniform
            const f32x4 av = *reinterpret_cast<const f32x4*>(Ts + TL::off(S + 16 * mr + lr, S + 16 * kt + 4 * lg));
            f32x4 bv;
            if constexpr (INPLACE) {
#pragma unroll
                for (int q = 0; q < 4; ++q) bv[q] = Ts[TL::off(S + 16 * kt + 4 * lg + q, 16 * nc + lr)];
            } else {
                bv = *reinterpret_cast<const f32x4*>(tmpb + (kt * TS + nc) * 256 + 4 * lane);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc[t], 0, 0, 0);
        }
        if constexpr (!INPLACE) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Ts[TL::off(S + 16 * mr + 4 * lg + r, 16 * nc + lr)] = -acc[t][r];
        }
    }
    if constexpr (INPLACE) {  // X10 over tmp, once every wave has read tmp for the last time
        __syncthreads();
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int nc = S == 64 ? wave : wave >> 1;
            const int mr = S == 64 ? t : wave & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ts[TL::off(S + 16 * mr + 4 * lg + r, 16 * nc + lr)] = -acc[t][r];
        }
    }
    __syncthreads();
}

// One unit, from committing its prefetched K to storing its outputs; its own V and the next
// unit's K are issued on the way.  Returns the next unit.
template <int C, int DT, int M, class PF>
__device__ __forceinline__ Unit run_unit(const Params& p, unsigned char* smem, PF& pf, const Unit& cur,
                                         int64_t& next, int64_t stride, bool cached, int cu_lane)
{
    constexpr bool WU = (M & kModeWU) != 0;
    constexpr bool GT = (M & kModeGate) != 0;
    constexpr bool SOLVE = (M & kModeSolve) != 0;
    using L = Lds<C, DT, WU>;
    unsigned char* Kraw = smem + L::OFF_K;
    float* Ts = reinterpret_cast<float*>(smem + L::OFF_T);
    float* bs = reinterpret_cast<float*>(smem + L::OFF_B);
    int* info = reinterpret_cast<int*>(smem + L::OFF_INFO);
    // A fresh copy of the thread index per unit: per-lane addresses are then recomputed for
    // each unit instead of being hoisted out of the loop and held in registers.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    pf.commit_k(Kraw, bs, tid);
    // a0 for the next unit (packed sequences: wave 0 searches cu_seqlens) before this unit's V is
    // issued: loads complete in order, so a search issued behind V would wait for V, and with it,
    // at the barrier, every wave would wait before forming A.
    map_search<C>(p, info, next, stride, tid, cached, cu_lane);
    __syncthreads();
    const Unit nxt = map_read<C>(p, info, next);
    // This unit's V is needed only after its inversion; the next unit's K at the next unit's
    // start.  Issued in that order, a wait for either never waits for the other.  From C = 64
    // on the next K is issued after the diagonal inversions (which one or two of the four waves
    // run), not right behind V, where the two compete for the CU's address units: at C = 128
    // 2-4% faster, at C = 64 3% on the headline, 5% on the packed workload and 7% for T alone.
    pf.issue_v(p, cur, tid);
    if constexpr (C < 64) {
        if (nxt.n > 0) pf.issue_k(p, nxt, tid);
    }

    using TL = typename L::TL;
    form_a<C, DT, L::KROW, TL, GT>(Kraw, Ts, bs, tid);
    __syncthreads();
    // The inversion and the coupling levels are the unit's chain, run by one or two waves while
    // other workgroups' waves share the SIMDs.  With T alone (up to seven workgroups per CU) and
    // at C = 128 (three coupling levels) their raised priority shortens it; with W and U at
    // C <= 64 the other workgroups' product waves should not wait, and it stays even.
    // At C = 64 with four or more value heads per key head (three workgroups per CU) the chain
    // goes first too.
    constexpr bool kChainFirst = !WU || C == 128;
    const bool chain_first = kChainFirst || (C == 64 && p.hv >= 4 * p.hq);  // uniform
    if (chain_first) __builtin_amdgcn_s_setprio(2);
    invert_diagonal_blocks<C, TL>(Ts, tid);
    if constexpr (C >= 64) {
        if (nxt.n > 0) pf.issue_k(p, nxt, tid);
    }
    __syncthreads();
    if constexpr (SOLVE) {
        if (chain_first) __builtin_amdgcn_s_setprio(0);
        // K is no longer read (form_a finished before the last barrier but one): the right-hand
        // side takes its place, and X is staged over it
        pf.commit_v(Kraw, tid);
        __syncthreads();
        solve_rhs<C, DT, L::KROW, TL>(Kraw, Ts, bs, tid);
        __syncthreads();
        store_rows<C, L::ESZ, L::KROW>(Kraw, p.U, cur, p.hv, tid);
        __syncthreads();  // LDS is rewritten by the next unit
        return nxt;
    }
    // Level s writes only rows s and past (the X10 blocks).  Rows at or past n are never stored,
    // and the stored rows of T, W and U depend on T's rows below n alone, so a unit of n <= s
    // rows (a sequence's last chunk, short sequences) skips level s and the ones above it.  Not
    // at C = 64 with W and U: there it gained 5% on short sequences, but the check alone moved
    // the code of the full-chunk case and cost 1.5% on it.
    constexpr bool kSkip = !(C == 64 && WU);
    const int nrows = kSkip ? __builtin_amdgcn_readfirstlane(cur.n) : C;
    if constexpr (C >= 32) {
        if (nrows > 16) coupling_level<C, 16, TL>(Ts, tid);  // uniform
    }
    // The level whose single-wave chain is the longest runs on all four waves in two passes: for
    // T alone with its tmp tiles over K (no longer read), with W and U in place over L10
    if constexpr (C == 64) {
        if (nrows > 32) coupling_2pass<C, 32, TL, WU>(Ts, reinterpret_cast<float*>(Kraw), tid);  // uniform
    }
    if constexpr (C >= 128) {
        if (nrows > 32) coupling_level<C, 32, TL>(Ts, tid);  // uniform
    }
    if constexpr (C == 128) {
        if (nrows > 64) coupling_2pass<C, 64, TL, WU>(Ts, reinterpret_cast<float*>(Kraw), tid);  // uniform
    }
    if (chain_first) __builtin_amdgcn_s_setprio(0);
    store_t<C, TL, DT == 0 && WU, (M & kModeT) != 0>(Ts, bs, p.T, cur, p.hv, tid);
    if constexpr (WU) {
        __syncthreads();  // T (packed T' for bf16) of all threads is in place
        if constexpr (DT == 0)
            wu_bf16<C, L::KROW, TL, GT>(Kraw, Ts, pf, p, cur, tid);
        else
            wu_f32<C, L::KROW, TL, GT>(Kraw, Ts, bs, pf, p, cur, tid);
    }
    __syncthreads();  // LDS is rewritten by the next unit
    return nxt;
}

template <int C, int DT, int M>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEu<C, DT, (M & kModeWU) != 0>::value))) void wy_prepare_kernel(Params p)
{
    constexpr bool WU = (M & kModeWU) != 0;
    using L = Lds<C, DT, WU>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int* info = reinterpret_cast<int*>(smem + L::OFF_INFO);

    // A workgroup takes groups of q = p.group consecutive units (the value heads of one key head
    // of one chunk, or two such at C = 32) one after the other: they read the same key rows and
    // write neighbouring rows of T, W and U.  Its next group is G groups on.  Workgroups are
    // dealt round-robin to the 8 XCDs; in every round each XCD gets a contiguous range of
    // groups.
    const uint32_t G = gridDim.x;  // a multiple of 8
    const int64_t first = static_cast<int64_t>(blockIdx.x & 7u) * (G >> 3) + (blockIdx.x >> 3);
    const int64_t q = p.group;
    const int64_t GS = static_cast<int64_t>(G) * q;  // units from a group to this workgroup's next
    auto next_unit = [q, GS](int64_t l) { return (l + 1) % q != 0 ? l + 1 : l + 1 - q + GS; };

    // Fewer than 64 packed sequences: wave 0 keeps cu_seqlens in registers (lane l: cu[min(l, N)])
    // for the whole launch, so every unit's search is a ballot and two shuffles.
    const bool cached = p.cu != nullptr && p.num_seqs < 64;
    const int cu_lane = cached && threadIdx.x < 64 ? p.cu[min(static_cast<int>(threadIdx.x), p.num_seqs)] : 0;
    // A packed slot past its sequence's end is empty for all its value heads, so the search for a
    // non-empty unit (map_search) starts only at a group's first unit and steps GS at a time.
    int64_t logical = first * q;
    Unit cur = map_unit<C>(p, info, logical, GS, threadIdx.x, cached, cu_lane);
    if (cur.n <= 0) return;  // uniform per workgroup
    __syncthreads();  // every wave has read info before the next unit's search rewrites it
    Prefetch<C, L::ESZ, L::KROW, WU || (M & kModeSolve) != 0, (M & kModeGate) != 0> pf;
    pf.issue_k(p, cur, threadIdx.x);
    // The first unit is peeled off the loop: the loop head is then reached only from the end
    // of a unit, so the memory-counter waits inside see one issue history.
    int64_t next = next_unit(logical);
    cur = run_unit<C, DT, M>(p, smem, pf, cur, next, GS, cached, cu_lane);
    while (cur.n > 0) {  // uniform
        next = next_unit(next);
        cur = run_unit<C, DT, M>(p, smem, pf, cur, next, GS, cached, cu_lane);
    }
}

// Occupancy (resident workgroups per CU) and CU count for one kernel instance, cached per device.
// The first call on a device also raises the instance's dynamic LDS limit where its plan needs
// more than the default 64 KiB, so later launches (including ones under stream capture) make no
// attribute calls.
struct Residency {
    int per_cu, cus;
};

template <int C, int DT, int M>
Residency resident_grid(int device, hipError_t* err)
{
    constexpr int kMaxDevices = 64;
    static Residency cached[kMaxDevices] = {};
    static std::mutex mu;
    if (device < 0 || device >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return Residency{0, 0};
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cached[device].cus == 0) {
        using L = Lds<C, DT, (M & kModeWU) != 0>;
        const void* kern = reinterpret_cast<const void*>(wy_prepare_kernel<C, DT, M>);
        if (L::TOTAL > 64 * 1024) {
            *err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
            if (*err != hipSuccess) return Residency{0, 0};
        }
        int cus = 0, per_cu = 0;
        *err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
        if (*err != hipSuccess) return Residency{0, 0};
        *err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, L::TOTAL);
        if (*err != hipSuccess) return Residency{0, 0};
        cached[device] = Residency{per_cu > 0 ? per_cu : 1, cus};
    }
    return cached[device];
}

template <int C, int DT, int M>
int launch_t(const LaunchArgs& a, hipStream_t stream, char* msg, int msg_len)
{
    using L = Lds<C, DT, (M & kModeWU) != 0>;
    static_assert(L::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    Params p;
    p.k = a.k;
    p.v = a.v;
    p.beta = a.beta;
    p.g = a.g;
    p.cu = a.cu_seqlens;
    p.T = a.T;
    p.W = a.W;
    p.U = a.U;
    p.units = a.chunk_slots * a.num_v_heads;
    p.seqlen = a.seqlen;
    p.hq = a.num_qk_heads;
    p.hv = a.num_v_heads;
    p.num_seqs = a.num_seqs;
    auto kern = wy_prepare_kernel<C, DT, M>;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    Residency res{0, 0};
    if (e == hipSuccess) res = resident_grid<C, DT, M>(device, &e);
    if (e == hipSuccess) {
        const int r = p.hv / p.hq;
        // Resident workgroups per CU.  With W and U, more than four only add HBM streams: at C =
        // 32 (seven fit) four were measured faster, e.g. 29.6 vs 34.6 us at B=1 T=8192 H=16, while
        // T alone gains from all seven.  bf16 W / U with four or more value heads per key head
        // (groups of two key heads, see below) at C = 64 take three, at C = 32 six.  Measured on
        // MI355X against four, one call each, bit-identical: at C = 64 packed 8 sequences
        // Hq=16 Hv=64 1069 -> 1044 us, packed 4 sequences of 8k-24k tokens Hq=16 Hv=64
        // 899 -> 861 us, packed 8 sequences Hq=4 Hv=16 270 -> 251 us, B=4 T=16384 Hq=16 Hv=64
        // unchanged; at C = 32 packed 8 sequences Hq=16 Hv=64 942 -> 840 us.  With one value
        // head per key head both were slower (C = 64: B=1 T=8192 H=16 32.2 -> 33.6 us, 1024
        // short packed sequences 193 -> 220 us; C = 32 with six: B=4 T=4096 H=32 102 -> 113 us,
        // B=1 T=32768 H=8 53 -> 56 us), so they keep four.
        int per_cu = (M & (kModeWU | kModeSolve)) != 0 ? 4 : 1 << 10;
        if (DT == 0 && (M & kModeWU) != 0 && r >= 4) per_cu = C == 64 ? 3 : (C == 32 ? 6 : per_cu);
        if (per_cu > res.per_cu) per_cu = res.per_cu;
        int64_t cap = static_cast<int64_t>(per_cu) * res.cus / 8 * 8;
        // Units in groups: the r = Hv / Hq value heads of one (chunk, key head) in turn on one
        // workgroup.  Measured on MI355X against one unit per workgroup and round: packed 8
        // sequences Hq=16 Hv=64 1132 -> 1073 us, B=4 T=16384 Hq=16 Hv=64 1073 -> 931 us, the same
        // order as before where r = 1.  Two key heads per group, where that still leaves every
        // workgroup two groups, at C = 32 (B=4 T=4096 H=32 108 -> 102 us, B=1 T=32768 H=8
        // 53.7 -> 51.5 us) and for r >= 4 with W and U (the packed workload 1075 -> 1066 us; T
        // alone, at up to seven workgroups per CU, went 432 -> 442 us); for r = 1 at C = 64 and
        // 128 it was 1-3% slower.
        p.group = r;
        if ((C == 32 || (r >= 4 && (M & kModeWU) != 0)) && p.hv % (2 * r) == 0 && p.units / (2 * r) >= 2 * cap)
            p.group = 2 * r;
        int64_t grid = (p.units / p.group + 7) / 8 * 8;
        if (cap >= 8 && grid > cap) grid = cap;
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), L::TOTAL,
                           stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        std::snprintf(msg, msg_len, "%s (C=%d, dtype=%d, mode=%d)", hipGetErrorString(e), C, DT, M);
        return static_cast<int>(e);
    }
    return 0;
}

template <int DT, int M>
int launch_c(const LaunchArgs& a, hipStream_t s, char* msg, int len)
{
    switch (a.chunk_size) {
    case 32: return launch_t<32, DT, M>(a, s, msg, len);
    case 64: return launch_t<64, DT, M>(a, s, msg, len);
    default: return launch_t<128, DT, M>(a, s, msg, len);
    }
}

template <int DT, int G>
int launch_m(const LaunchArgs& a, hipStream_t s, char* msg, int len)
{
    if (a.solve) return launch_c<DT, kModeSolve | G>(a, s, msg, len);
    const bool wu = a.W != nullptr, t = a.T != nullptr;
    if (wu && t) return launch_c<DT, kModeT | kModeWU | G>(a, s, msg, len);
    if (wu) return launch_c<DT, kModeWU | G>(a, s, msg, len);
    return launch_c<DT, kModeT | G>(a, s, msg, len);
}

template <int DT>
int launch_g(const LaunchArgs& a, hipStream_t s, char* msg, int len)
{
    return a.g != nullptr ? launch_m<DT, kModeGate>(a, s, msg, len) : launch_m<DT, 0>(a, s, msg, len);
}

}  // namespace

int launch(const LaunchArgs& a, void* stream, char* msg, int msg_len)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.kv_dtype == 0 ? launch_g<0>(a, s, msg, msg_len) : launch_g<1>(a, s, msg, msg_len);
}

}  // namespace wyp
