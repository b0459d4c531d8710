// The per-key gate's chunk-local decayed Gram products with every decay
// factor at most 1 (exact_key_gram), and the loads they start from
// (load_key_rows).  Used by kda_gram_kernel (gdn_kda_gram.h) and by the
// two-stage kernels' per-key paths (gdn_prepare.h, gdn_scan.h).
//
// For the per-key gate the decay of a pair of rows r > s of a chunk is a
// vector over the key dimension, e^(gcum_r - gcum_s) (per key d, at most 1),
// and it sits inside the sums of the decayed Gram products
//     A[r,s] = beta_r sum_d k_rd k_sd e^(gcum_rd - gcum_sd)     (s < r)
//     P[r,s] =        sum_d q_rd k_sd e^(gcum_rd - gcum_sd)     (s <= r)
// of the TileOPs fused-prepare page (A_g) and of the re-scan's output term on
// the kernel-fun KDA re-scan page.  A matrix-core product can only take it as
// a row factor times a column factor, e^(gcum_r - gcum_m) e^(gcum_m - gcum_s);
// both are decays exactly when the reference row m lies between s and r.  No
// single m does for every pair, so the chunk is halved recursively: at level
// S (S = C, C/2, .., 2) every segment of S rows is split after its middle row
// m = first row + S/2 - 1, the pairs with r in the second half and s in the
// first are formed with the factors about that m, and every pair r > s is
// formed at exactly one level (the first halving that separates r and s).
// At S >= 32 those pairs fill whole 16 x 16 tiles below the diagonal; below
// that they are masked parts of the diagonal tiles.  P's diagonal (r = s, no
// decay) comes from one more product of the raw rows.  Every operand is then
// k or q times a factor in [0, 1]: no gate value can overflow anything, and
// a factor that underflows only drops a contribution below the operands'
// precision.
#pragma once

#include "gdn_buffer.h"

namespace gdn {

// A thread's share of a chunk for the per-key gate: thread t of 256 holds
// rows seg NR .. seg NR + NR - 1 of key columns 4 cg .. 4 cg + 3 (seg =
// t / (K/4), cg = t % (K/4)).
template <int C, int K>
struct KeyRows {
    static constexpr int NSEG = kThreads * 4 / K;
    static constexpr int NR = C / NSEG;
    static_assert(NR >= 2 && NSEG * NR == C, "rows per thread");
};

template <int C, int K, typename OpT>
struct GramLayout {
    static constexpr int LDK = K + Mma<OpT>::kPad;
    static constexpr int LDA = C + 4;
    static constexpr int LDC = C + Mma<OpT>::kPad;
    static constexpr int E = sizeof(OpT);
    static constexpr int NSEG = KeyRows<C, K>::NSEG;
    // region X: the level operands Lk, Lq [C][LDK] while the products run;
    // afterwards the inverse Tm [C][LDA] fp32 and the output tiles Tmb, P
    // [C][LDC] staged for the store
    static constexpr int kXlev = 2 * C * LDK * E;
    static constexpr int kXout = C * LDA * 4 + 2 * C * LDC * E;
    static constexpr int kX = 0;
    static constexpr int kAf = kX + (kXlev > kXout ? kXlev : kXout);   // fp32 [C][LDA] A
    static constexpr int kPf = kAf + C * LDA * 4;                       // fp32 [C][LDA] P
    static constexpr int kSeg = kPf + C * LDA * 4;                      // [NSEG][K] segment totals
    static constexpr int kGend = kSeg + NSEG * K * 4;                   // [NSEG][K] gcum at segment ends
    static constexpr int kBet = kGend + NSEG * K * 4;                   // [C] beta
    static constexpr int kBytes = kBet + C * 4;
};

// Store four operand values of one row (8 bytes fp16, 16 bytes fp32).
__device__ __forceinline__ void store_op4(_Float16 *dst, const float4v &x) {
    half4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)x[e];
    *(half4 *)dst = h;
}
__device__ __forceinline__ void store_op4(float *dst, const float4v &x) { *(float4v *)dst = x; }

// The exact decayed Gram products of one chunk by one workgroup of 256
// threads.  In: this thread's rows (see KeyRows) as gcum (gam), raw k (kv)
// and q (qv); gend[seg][K], gcum at the last row of each thread segment;
// bet[C].  Scratch: Lk, Lq [C][LDK].  Out: Af (WANT_A: strictly lower A,
// rows scaled by beta) and Pf (WANT_P: P, lower including the diagonal),
// fp32 [C][LDA], zero above the diagonal.  Ends with a barrier.
template <int C, int K, typename OpT, bool WANT_A, bool WANT_P>
__device__ void exact_key_gram(const float4v (&gam)[KeyRows<C, K>::NR],
                               const float4v (&kv)[KeyRows<C, K>::NR],
                               const float4v (&qv)[KeyRows<C, K>::NR],
                               const float *gend, const float *bet, OpT *Lk, OpT *Lq,
                               float *Af, float *Pf) {
    typedef GramLayout<C, K, OpT> L;
    constexpr int NR = KeyRows<C, K>::NR, NB = C / 16, LDK = L::LDK, LDA = L::LDA;
    constexpr int NKIND = (WANT_A ? 1 : 0) + (WANT_P ? 1 : 0);
    static_assert(NKIND >= 1, "something to form");
    const int tid = threadIdx.x, wv = wave_id(), l = lane_id();
    const int seg = tid / (K / 4), kc = 4 * (tid % (K / 4));
    const int n = l & 15, g4 = 4 * (l >> 4);

    for (int i = tid; i < C * LDA; i += kThreads) {
        if (WANT_A) Af[i] = 0.f;
        if (WANT_P) Pf[i] = 0.f;
    }

    // Product (kind, block pair) in row layout: lane (g, n) gets row 16 I + n,
    // columns 16 J + 4g + e.  X Y^T with X the k operand rows of block J.
    auto product = [&](bool isA, int I, int J) {
        float4v acc = {0, 0, 0, 0};
        mma_tile<OpT, K>(acc, Lk + 16 * J * LDK, LDK, (isA ? Lk : Lq) + 16 * I * LDK, LDK);
        return acc;
    };
    // diagonal tiles: product index p = kind * NB + block, owned by wave p % 4
    // for every level, accumulated in registers (at most two per wave)
    float4v accD[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    auto diag_owned = [&](int slot, bool &isA, int &I) {
        const int p = wv + 4 * slot;
        isA = WANT_A && p < NB;
        I = isA ? p : p - (WANT_A ? NB : 0);
        return p < NKIND * NB;
    };

#pragma unroll
    for (int S = C; S >= 1; S >>= 1) {
        // ---- this level's operands (S == 1: the raw rows for P's diagonal)
        if (S == 1 && !WANT_P) break;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = seg * NR + i;
            float4v f = {1.f, 1.f, 1.f, 1.f};
            if (S > 1) {
                float4v gs;
                if (S / 2 >= NR) {
                    // the split row ends a thread segment
                    const int js = ((r & ~(S - 1)) + S / 2) / NR - 1;
                    gs = *(const float4v *)(gend + js * K + kc);
                } else {
                    gs = gam[(i & ~(S - 1)) + S / 2 - 1];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = fast_exp(-fabsf(gam[i][e] - gs[e]));
            }
            store_op4(Lk + r * LDK + kc, kv[i] * f);
            if (WANT_P) store_op4(Lq + r * LDK + kc, qv[i] * f);
        }
        __syncthreads();
        // ---- this level's products
        if (S >= 32) {
            // whole tiles (I, J), I > J, with 16 (I ^ J) in [S/2, S)
            constexpr int NT = NB * (NB - 1) / 2;
            int t = 0;
#pragma unroll
            for (int I = 1; I < NB; ++I)
#pragma unroll
                for (int J = 0; J < I; ++J) {
                    if (16 * (I ^ J) >= S / 2 && 16 * (I ^ J) < S) {
#pragma unroll
                        for (int kind = 0; kind < 2; ++kind) {
                            const bool isA = kind == 0;
                            if ((isA && !WANT_A) || (!isA && !WANT_P)) continue;
                            if ((t++ & 3) != wv) continue;
                            const float4v acc = product(isA, I, J);
                            const int r = 16 * I + n, s0 = 16 * J + g4;
                            float *dst = (isA ? Af : Pf) + r * LDA + s0;
                            *(float4v *)dst = isA ? acc * bet[r] : acc;
                        }
                    }
                }
            (void)NT;
        } else {
            // parts of the diagonal tiles: r > s in the same segment of S
            // rows, in different halves (S == 1: r == s)
#pragma unroll
            for (int slot = 0; slot < 2; ++slot) {
                bool isA;
                int I;
                if (!diag_owned(slot, isA, I)) continue;
                if (S == 1 && isA) continue;
                const float4v acc = product(isA, I, I);
                const int r = 16 * I + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * I + g4 + e, x = r ^ s;
                    const bool in = S == 1 ? r == s : (r > s && x < S && x >= S / 2);
                    accD[slot][e] += in ? acc[e] : 0.f;
                }
            }
        }
        __syncthreads();
    }
    // ---- the diagonal tiles
#pragma unroll
    for (int slot = 0; slot < 2; ++slot) {
        bool isA;
        int I;
        if (!diag_owned(slot, isA, I)) continue;
        const int r = 16 * I + n;
        float *dst = (isA ? Af : Pf) + r * LDA + 16 * I + g4;
        *(float4v *)dst = isA ? accD[slot] * bet[r] : accD[slot];
    }
    __syncthreads();
}

// Load one chunk of the per-key gate, k and q in KeyRows order and form the
// chunk-local cumsum: gam[i] = gcum of row seg NR + i (the segment offsets
// are summed in segment order, so the last row's gcum equals the chunk
// total summed that way), gend[seg] = gcum at the segment's last row.  With
// CUM the rows read are the cumsum already (gdn_prepare's gcum).  Rows past
// the stream end read as zero (with CUM a caller's ragged chunk must not
// read gam of those rows).  Ends with a barrier.
template <int C, int K, typename IO, bool CUM = false>
__device__ __forceinline__ void load_key_rows(rsrc_t rg, rsrc_t rk, rsrc_t rq, uint32_t rsK,
                                              uint32_t t0, float *segt, float *gend,
                                              float4v (&gam)[KeyRows<C, K>::NR],
                                              float4v (&kv)[KeyRows<C, K>::NR],
                                              float4v (&qv)[KeyRows<C, K>::NR]) {
    constexpr int NR = KeyRows<C, K>::NR, NSEG = KeyRows<C, K>::NSEG, SIO = sizeof(IO);
    const int tid = threadIdx.x, seg = tid / (K / 4), kc = 4 * (tid % (K / 4));
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const uint32_t row = t0 + (uint32_t)(seg * NR + i);
        gam[i] = __builtin_bit_cast(float4v, bload128(rg, (row * rsK + kc) * 4, 0));
        if constexpr (SIO == 2) {
            const u32x2 wk = __builtin_amdgcn_raw_buffer_load_b64(rk, (row * rsK + kc) * 2, 0, 0);
            const u32x2 wq = __builtin_amdgcn_raw_buffer_load_b64(rq, (row * rsK + kc) * 2, 0, 0);
            kv[i] = float4v{__uint_as_float(wk[0] << 16), __uint_as_float(wk[0] & 0xffff0000u),
                            __uint_as_float(wk[1] << 16), __uint_as_float(wk[1] & 0xffff0000u)};
            qv[i] = float4v{__uint_as_float(wq[0] << 16), __uint_as_float(wq[0] & 0xffff0000u),
                            __uint_as_float(wq[1] << 16), __uint_as_float(wq[1] & 0xffff0000u)};
        } else {
            kv[i] = __builtin_bit_cast(float4v, bload128(rk, (row * rsK + kc) * 4, 0));
            qv[i] = __builtin_bit_cast(float4v, bload128(rq, (row * rsK + kc) * 4, 0));
        }
    }
    if constexpr (!CUM) {
        float4v run = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < NR; ++i) { run += gam[i]; gam[i] = run; }
        *(float4v *)(segt + seg * K + kc) = run;
        __syncthreads();
        float4v off = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NSEG; ++m)
            if (m < seg) off += *(const float4v *)(segt + m * K + kc);
#pragma unroll
        for (int i = 0; i < NR; ++i) gam[i] = off + gam[i];
    }
    *(float4v *)(gend + seg * K + kc) = gam[NR - 1];
    __syncthreads();
}

}  // namespace gdn
