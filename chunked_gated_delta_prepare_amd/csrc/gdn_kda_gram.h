// The per-key gate (Kimi-Delta-Attention): every chunk's exact decayed Gram
// products and the triangular factors the re-scan needs, in a kernel that
// runs over all chunks at once.
//
// kda_gram_kernel forms, for every (stream, chunk, head) in parallel,
//     A[r,s] = beta_r sum_d k_rd k_sd e^(gcum_rd - gcum_sd)     (s < r)
//     P[r,s] =        sum_d q_rd k_sd e^(gcum_rd - gcum_sd)     (s <= r)
// (the TileOPs fused-prepare page's A_g and the kernel-fun KDA re-scan page's
// output term), then the solve tile Tmb (row block b = [Mn_b0 .. | Tb_bb | 0],
// Tb_bb = (I + A_bb)^-1 diag(beta_b), Mn_bj = -(I + A_bb)^-1 A_bj, the block
// solve of forward_kernel) and writes Tmb and P, both [C][C] row-major in the
// operand type (fp16 for bf16 io, fp32 for fp32 io), to a workspace slot per
// (chunk, head).  With bf16 io it also writes the pipelined re-scan's
// operand tiles, referenced to the chunk's start and end (qd = q e^gcum,
// kd = k e^gcum, kg = k e^(gl - gcum), all decays), and e^gl, so that the
// re-scan only copies them (KdaSlotOps).
//
// Every decay inside a product is a decay.  A matrix-core product can take
// e^(gcum_r - gcum_s) only as a row factor times a column factor, and both
// are at most 1 exactly when the reference row lies between s and r.  The
// chunk is halved recursively (level S = C, C/2, .., 2: each segment of S
// rows split after its middle row); every pair r > s is formed at the first
// level that separates it, with the factors about that level's split row m:
// e^(gcum_r - gcum_m) for r in the second half, e^(gcum_m - gcum_s) for s in
// the first.  P's diagonal (r = s) comes from one more product of the raw
// rows.
//
// The factors are products of the per-token decays a_t = e^(g_t) <= 1, never
// exponentials of cumsum differences: e^(gcum_r - gcum_m) = a_(m+1) .. a_r.
// Each thread holds one 16-row block of CW key columns, so the products
// inside a block are running products in registers (one multiply per
// element and level), and a level that crosses blocks multiplies whole-block
// totals from LDS.  Only C x K exponentials are taken per chunk, and every
// partial product lies in [0, 1]: no gate value can overflow anything.
#pragma once

#include "gdn_forward_pipe.h"

namespace gdn {

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct GramParams {
    const void *q, *k;
    const float *beta, *g;
    void *ws;           // [slots][H][2][C][C] operand type: Tmb, then P
    const int *cu;      // packed sequences: B + 1 offsets, else NULL
    int B, T, H;
    int nt;             // chunks per stream (fixed length)
};

// The stream and chunk of workspace slot `slot`: fixed length, slot = b nt + c;
// packed sequences, the slots of sequence b follow those of sequences < b
// (ceil(len / C) each).  Returns false for a slot past the last chunk.
template <int C, bool VL>
__device__ __forceinline__ bool slot_chunk(const GramParams &p, int slot, int &b, int &c,
                                           int &T, int64_t &tok0) {
    if constexpr (VL) {
        int base = 0;
        for (int m = 0; m < p.B; ++m) {
            const int c0 = __builtin_amdgcn_readfirstlane(p.cu[m]);
            const int c1 = __builtin_amdgcn_readfirstlane(p.cu[m + 1]);
            const int bos = min(max(c0, 0), p.T), eos = min(max(c1, bos), p.T);
            const int nc = (eos - bos + C - 1) / C;
            if (slot < base + nc) {
                b = m; c = slot - base; T = eos - bos; tok0 = bos;
                return true;
            }
            base += nc;
        }
        return false;
    } else {
        b = slot / p.nt;
        c = slot - b * p.nt;
        T = p.T;
        tok0 = (int64_t)b * p.T;
        return b < p.B;
    }
}

// Thread map: thread t < NACT holds rows 16 blk .. 16 blk + 15 of key columns
// c0 .. c0 + CW - 1, blk = t / TPB, c0 = CW (t % TPB).  With TPB = 64 a wave
// holds one whole block.
template <int C, int K>
struct GramStrip {
    static constexpr int NB = C / 16;
    static constexpr int CW = (NB * K >= 2 * kThreads) ? 2 : 1;
    static constexpr int TPB = K / CW;
    static constexpr int NACT = NB * TPB;
    static_assert(NACT <= kThreads && CW * TPB == K, "strip map");
};

template <int C, int K, typename OpT>
struct GramLayout2 {
    static constexpr int NB = C / 16;
    static constexpr int LDK = K + Mma<OpT>::kPad;
    static constexpr int LDA = C + 4;
    static constexpr int LDC = C + Mma<OpT>::kPad;
    static constexpr int E = sizeof(OpT);
    // region X: the level operands Lk, Lq [C][LDK] while the products run;
    // afterwards the diagonal inverses Tm [C][LDA] fp32 and the output tiles
    // Tmb, P [C][LDC]
    static constexpr int kXlev = 2 * C * LDK * E;
    static constexpr int kXout = C * LDA * 4 + 2 * C * LDC * E;
    static constexpr int kX = 0;
    static constexpr int kAf = (kXlev > kXout ? kXlev : kXout);    // fp32 [C][LDA] A
    static constexpr int kPf = kAf + C * LDA * 4;                   // fp32 [C][LDA] P
    static constexpr int kBt = kPf + C * LDA * 4;                   // [NB][K] block totals
    static constexpr int kBet = kBt + NB * K * 4;                   // [C] beta
    static constexpr int kBytes = kBet + C * 4;
};

// One row piece (CW columns) of the io dtype: loaded raw into NW dwords,
// unpacked to floats when used.
template <typename IO, int CW>
struct RawPiece {
    static constexpr int NW = (CW * (int)sizeof(IO) + 3) / 4;
    __device__ static void load(rsrc_t r, uint32_t elem, uint32_t (&w)[NW]) {
        if constexpr (sizeof(IO) == 2) {
            w[0] = CW == 2 ? bload32(r, elem * 2, 0) : (uint32_t)bload16(r, elem * 2, 0);
        } else if constexpr (CW == 2) {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 4, 0, 0);
            w[0] = x[0];
            w[1] = x[1];
        } else {
            w[0] = bload32(r, elem * 4, 0);
        }
    }
    __device__ static void load(rsrc_t r, uint32_t elem, float (&x)[CW]) {
        uint32_t w[NW];
        load(r, elem, w);
#pragma unroll
        for (int e = 0; e < CW; ++e) x[e] = __uint_as_float(w[e]);
    }
    __device__ static void unpack(const uint32_t (&w)[NW], float (&x)[CW]) {
        if constexpr (sizeof(IO) == 2) {
            x[0] = __uint_as_float(w[0] << 16);
            if constexpr (CW == 2) x[1] = __uint_as_float(w[0] & 0xffff0000u);
        } else {
#pragma unroll
            for (int e = 0; e < CW; ++e) x[e] = __uint_as_float(w[e]);
        }
    }
};

// Store CW operand values of one row (fp16: 2 or 4 bytes, fp32: 4 or 8).
template <int CW>
__device__ __forceinline__ void store_piece(_Float16 *dst, const float (&x)[CW]) {
    if constexpr (CW == 2) {
        *(h16x2 *)dst = h16x2{(_Float16)x[0], (_Float16)x[1]};
    } else {
        *dst = (_Float16)x[0];
    }
}
template <int CW>
__device__ __forceinline__ void store_piece(float *dst, const float (&x)[CW]) {
    if constexpr (CW == 2) {
        *(f32x2 *)dst = f32x2{x[0], x[1]};
    } else {
        *dst = x[0];
    }
}

template <int C, int K, typename IO, bool VL>
__global__ __launch_bounds__(kThreads) void kda_gram_kernel(GramParams p) {
    typedef typename OpOf<IO>::type OpT;
    typedef GramLayout2<C, K, OpT> L;
    typedef GramStrip<C, K> SM;
    constexpr int NB = C / 16, CW = SM::CW, TPB = SM::TPB, LDK = L::LDK, LDA = L::LDA, LDC = L::LDC;
    constexpr int E = sizeof(OpT), NW = RawPiece<IO, CW>::NW;
    // the diagonal levels need only a block's own rows: when one wave holds
    // them, that wave runs those levels without workgroup barriers
    constexpr bool WAVE_BLOCK = TPB == 64;
    // fp16 operands with wave-held blocks: each block's wave also inverts
    // its diagonal block on the matrix cores, from the registers that hold
    // A_II, and forms its row block of Tmb; P tiles go straight to the
    // output tile.  (fp32 io keeps the fp32 forward substitution.)
    constexpr bool FAST = WAVE_BLOCK && std::is_same<OpT, _Float16>::value;
    // bf16 io: also the pipelined re-scan's operand tiles
    constexpr bool OPS = std::is_same<OpT, _Float16>::value;
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OpT *Lk = (OpT *)(smem + L::kX);
    OpT *Lq = Lk + C * LDK;
    float *Tmf = (float *)(smem + L::kX);
    OpT *Tmb = (OpT *)(smem + L::kX + C * LDA * 4);
    // (fast path: P is written during the levels, into the space of Pf)
    OpT *Ps = FAST ? (OpT *)(smem + L::kPf) : Tmb + C * LDC;
    float *Af = (float *)(smem + L::kAf);
    float *Pf = (float *)(smem + L::kPf);
    float *Bt = (float *)(smem + L::kBt);
    float *bet = (float *)(smem + L::kBet);

    const int tid = threadIdx.x, wv = wave_id(), l = lane_id();
    const int H = p.H;
    const uint32_t rsK = (uint32_t)(H * K);
    const bool act = tid < SM::NACT;
    const int blk = tid / TPB, c0 = CW * (tid % TPB);
    const int n = l & 15, g4 = 4 * (l >> 4);

    const int h = blockIdx.x % H, slot = blockIdx.x / H;
    int b, c, T;
    int64_t tok0;
    if (!slot_chunk<C, VL>(p, slot, b, c, T, tok0)) return;
    const int64_t row0 = tok0 * H + h;                      // (token, head) row of token 0
    const uint32_t t0 = (uint32_t)(c * C);
    {
        {
            const rsrc_t rb = make_rsrc(p.beta + row0, (uint32_t)T * (uint32_t)H * 4);
            if (tid < C) bet[tid] = __uint_as_float(bload32(rb, (t0 + tid) * (uint32_t)H * 4, 0));
        }
        // ---- this thread's 16 rows: the decays a = e^g (rows past the
        // stream end read g = 0, k = q = 0: a = 1, the identity), and k, q
        // in their raw form, unpacked where a level uses them
        float a[16][CW];
        uint32_t kr[16][NW], qr[16][NW];
        if (act) {
            const rsrc_t rg = make_rsrc(p.g + row0 * K, (uint32_t)T * rsK * 4);
            const rsrc_t rk = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)T * rsK * sizeof(IO));
            const rsrc_t rq = make_rsrc((const IO *)p.q + row0 * K, (uint32_t)T * rsK * sizeof(IO));
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t elem = (t0 + (uint32_t)(16 * blk + i)) * rsK + (uint32_t)c0;
                float gx[CW];
                RawPiece<float, CW>::load(rg, elem, gx);
                RawPiece<IO, CW>::load(rk, elem, kr[i]);
                RawPiece<IO, CW>::load(rq, elem, qr[i]);
#pragma unroll
                for (int e = 0; e < CW; ++e) a[i][e] = fast_exp(gx[e]);
            }
        }
        {
            // block totals (the decay across a whole block)
            if (act) {
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    float run = 1.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) run *= a[i][e];
                    Bt[blk * K + c0 + e] = run;
                }
            }
            __syncthreads();

            if constexpr (OPS) {
                // ---- the re-scan's operands of this thread's rows: e^gcum_r
                // = (totals of the blocks before) x a_(16 blk) .. a_r, and
                // e^(gl - gcum_r) = a_(r+1) .. a_(15) x (totals of the
                // blocks after); e^gl once per key column
                if (act) {
                    typedef KdaSlotOps<C, K> SO;
                    const rsrc_t ro = make_rsrc((char *)p.ws + ((int64_t)slot * H + h) * SO::kBytes,
                                                (uint32_t)SO::kBytes);
                    float bpre[CW], run[CW], dn[16][CW];
#pragma unroll
                    for (int e = 0; e < CW; ++e) { bpre[e] = 1.f; run[e] = 1.f; }
                    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                        for (int e = 0; e < CW; ++e) {
                            const float t = Bt[bb * K + c0 + e];
                            if (bb < blk) bpre[e] *= t;
                            if (bb > blk) run[e] *= t;
                        }
#pragma unroll
                    for (int i = 15; i >= 0; --i)
#pragma unroll
                        for (int e = 0; e < CW; ++e) { dn[i][e] = run[e]; run[e] *= a[i][e]; }
                    if (blk == 0) {
                        // (run: the whole chunk's decay)
                        if constexpr (CW == 2)
                            __builtin_amdgcn_raw_buffer_store_b64(
                                u32x2{__float_as_uint(run[0]), __float_as_uint(run[1])}, ro,
                                (uint32_t)(SO::kFl + 4 * c0), 0, 0);
                        else
                            bstore32(__float_as_uint(run[0]), ro, (uint32_t)(SO::kFl + 4 * c0), 0);
                    }
#pragma unroll
                    for (int e = 0; e < CW; ++e) run[e] = bpre[e];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float xq[CW], xk[CW];
                        RawPiece<IO, CW>::unpack(qr[i], xq);
                        RawPiece<IO, CW>::unpack(kr[i], xk);
                        _Float16 hq[CW], hk[CW], hg[CW];
#pragma unroll
                        for (int e = 0; e < CW; ++e) {
                            run[e] *= a[i][e];
                            hq[e] = (_Float16)(xq[e] * run[e]);
                            hk[e] = (_Float16)(xk[e] * run[e]);
                            hg[e] = (_Float16)(xk[e] * dn[i][e]);
                        }
                        const uint32_t off = (uint32_t)swz<K>(16 * blk + i, pcol(c0)) * 2;
                        if constexpr (CW == 2) {
                            auto pk = [](const _Float16 (&x)[CW]) {
                                return (uint32_t)__builtin_bit_cast(uint16_t, x[0]) |
                                       ((uint32_t)__builtin_bit_cast(uint16_t, x[1]) << 16);
                            };
                            bstore32(pk(hq), ro, (uint32_t)SO::kQd + off, 0);
                            bstore32(pk(hk), ro, (uint32_t)SO::kKd + off, 0);
                            bstore32(pk(hg), ro, (uint32_t)SO::kKg + off, 0);
                        } else {
                            bstore16(__builtin_bit_cast(uint16_t, hq[0]), ro, (uint32_t)SO::kQd + off, 0);
                            bstore16(__builtin_bit_cast(uint16_t, hk[0]), ro, (uint32_t)SO::kKd + off, 0);
                            bstore16(__builtin_bit_cast(uint16_t, hg[0]), ro, (uint32_t)SO::kKg + off, 0);
                        }
                    }
                }
            }

            auto put_rows = [&](const float (&f)[16][CW], bool q_upper_only, int S) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float xk[CW], xq[CW];
                    RawPiece<IO, CW>::unpack(kr[i], xk);
                    RawPiece<IO, CW>::unpack(qr[i], xq);
#pragma unroll
                    for (int e = 0; e < CW; ++e) { xk[e] *= f[i][e]; xq[e] *= f[i][e]; }
                    const int r = 16 * blk + i;
                    store_piece<CW>(Lk + r * LDK + c0, xk);
                    // (P takes q rows only from the second half of a segment)
                    if (!q_upper_only || (i & (S / 2)) != 0) store_piece<CW>(Lq + r * LDK + c0, xq);
                }
            };

            // ---- levels that cross blocks (S >= 32): whole 16 x 16 tiles
            // (I, J), I > J, with 16 (I ^ J) in [S/2, S).  A row in the
            // second half of its segment takes the decay from the split to
            // it, one in the first half the decay from it to the split: a
            // running product inside the block times the totals of the whole
            // blocks in between.
#pragma unroll
            for (int S = C; S >= 32; S >>= 1) {
                if (act) {
                    const int mb = (((16 * blk) & ~(S - 1)) + S / 2) / 16 - 1;   // last block of the first half
                    const bool upper = blk > mb;
                    float w[CW], f[16][CW];
#pragma unroll
                    for (int e = 0; e < CW; ++e) w[e] = 1.f;
                    for (int bb = upper ? mb + 1 : blk + 1; bb < (upper ? blk : mb + 1); ++bb)
#pragma unroll
                        for (int e = 0; e < CW; ++e) w[e] *= Bt[bb * K + c0 + e];
#pragma unroll
                    for (int e = 0; e < CW; ++e) {
                        float run = w[e];
                        if (upper) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) { run *= a[i][e]; f[i][e] = run; }
                        } else {
#pragma unroll
                            for (int i = 15; i >= 0; --i) { f[i][e] = run; run *= a[i][e]; }
                        }
                    }
                    put_rows(f, false, S);
                }
                __syncthreads();
                int t = 0;
#pragma unroll
                for (int I = 1; I < NB; ++I)
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        if (16 * (I ^ J) < S / 2 || 16 * (I ^ J) >= S) continue;
#pragma unroll
                        for (int kind = 0; kind < 2; ++kind) {
                            if ((t++ & 3) != wv) continue;
                            float4v acc = {0, 0, 0, 0};
                            mma_tile<OpT, K>(acc, Lk + 16 * J * LDK, LDK, (kind ? Lq : Lk) + 16 * I * LDK, LDK);
                            const int r = 16 * I + n;
                            if (FAST && kind) {
                                store_op4(Ps + r * LDC + 16 * J + g4, acc);
                            } else {
                                float *dst = (kind ? Pf : Af) + r * LDA + 16 * J + g4;
                                *(float4v *)dst = kind ? acc : acc * bet[r];
                            }
                        }
                    }
                __syncthreads();
            }

            // ---- levels inside the blocks (S = 16 .. 2), then the raw rows
            // (S = 1, P's diagonal): the diagonal tiles, masked to the pairs
            // of the level and accumulated in registers.  Owner: with
            // WAVE_BLOCK, wave I holds both tiles of block I; otherwise
            // product p = kind NB + block goes to wave p % 4.
            float4v accD[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
            auto diag_owned = [&](int s2, int &kind, int &I) {
                if constexpr (WAVE_BLOCK) {
                    kind = s2;
                    I = wv;
                    return wv < NB;
                } else {
                    const int q = wv + 4 * s2;
                    kind = q >= NB;
                    I = q - (kind ? NB : 0);
                    return q < 2 * NB;
                }
            };
#pragma unroll
            for (int S = 16; S >= 1; S >>= 1) {
                if (act) {
                    float f[16][CW];
                    if (S == 1) {
#pragma unroll
                        for (int i = 0; i < 16; ++i)
#pragma unroll
                            for (int e = 0; e < CW; ++e) f[i][e] = 1.f;
                    } else {
                        // second half of a segment: a_(m+1) .. a_r; first
                        // half: a_(s+1) .. a_m, with m the segment's middle row
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int m = (i & ~(S - 1)) + S / 2 - 1;
                            if (i > m)
#pragma unroll
                                for (int e = 0; e < CW; ++e) f[i][e] = (i == m + 1) ? a[i][e] : f[i - 1][e] * a[i][e];
                        }
#pragma unroll
                        for (int i = 15; i >= 0; --i) {
                            const int m = (i & ~(S - 1)) + S / 2 - 1;
                            if (i <= m)
#pragma unroll
                                for (int e = 0; e < CW; ++e) f[i][e] = (i == m) ? 1.f : f[i + 1][e] * a[i + 1][e];
                        }
                    }
                    put_rows(f, S > 1, S);
                }
                if constexpr (WAVE_BLOCK) __builtin_amdgcn_wave_barrier();
                else __syncthreads();
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    int kind, I;
                    if (!diag_owned(s2, kind, I)) continue;
                    if (S == 1 && !kind) continue;
                    float4v acc = {0, 0, 0, 0};
                    mma_tile<OpT, K>(acc, Lk + 16 * I * LDK, LDK, (kind ? Lq : Lk) + 16 * I * LDK, LDK);
                    const int r = 16 * I + n;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * I + g4 + e, x = r ^ s;
                        const bool in = S == 1 ? r == s : (r > s && x < S && x >= S / 2);
                        accD[s2][e] += in ? acc[e] : 0.f;
                    }
                }
                if constexpr (WAVE_BLOCK) __builtin_amdgcn_wave_barrier();
                else __syncthreads();
            }

            if constexpr (FAST) {
                // wave I: P_II and the zero tiles right of it into P; T_II =
                // (I + A_II)^-1 in registers (row layout, as accD holds
                // A_II); row block I of Tmb = [-T_II A_I0 .. | T_II diag(beta_I) | 0]
                __syncthreads();                    // every wave is past the level operands
                if (wv < NB) {
                    const int I = wv, r = 16 * I + n;
                    store_op4(Ps + r * LDC + 16 * I + g4, accD[1]);
                    for (int J = I + 1; J < NB; ++J) store_op4(Ps + r * LDC + 16 * J + g4, float4v{0, 0, 0, 0});
                    const float4v ad[2] = {accD[0] * bet[r], float4v{0, 0, 0, 0}};
                    float4v tr[2];
                    diag_inverse_mfma(ad, tr);
                    float4v tb;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Tmf[r * LDA + 16 * I + g4 + e] = tr[0][e];
                        tb[e] = tr[0][e] * bet[16 * I + g4 + e];
                    }
                    store_op4(Tmb + r * LDC + 16 * I + g4, tb);
                    for (int J = I + 1; J < NB; ++J) store_op4(Tmb + r * LDC + 16 * J + g4, float4v{0, 0, 0, 0});
                    __builtin_amdgcn_wave_barrier();
                    for (int J = 0; J < I; ++J) solve_block<LDA, LDC, OpT>(Af, Tmf, Tmb, I, J);
                }
                __syncthreads();
            } else {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    int kind, I;
                    if (!diag_owned(s2, kind, I)) continue;
                    const int r = 16 * I + n;
                    float *dst = (kind ? Pf : Af) + r * LDA + 16 * I + g4;
                    *(float4v *)dst = kind ? accD[s2] : accD[s2] * bet[r];
                }
                __syncthreads();

                // ---- (I + A)^-1 by blocks: diagonal inverses, then Tb and
                // Mn into Tmb; P into its output tile, zero above the
                // diagonal blocks
                if (wv == 0) diag_inverse<LDA>(Af, Tmf, 0, NB);
                for (int i = tid; i < C * LDC; i += kThreads) Tmb[i] = (OpT)0.f;
                for (int i = tid; i < C * C; i += kThreads) {
                    const int r = i / C, s = i % C;
                    Ps[r * LDC + s] = (s / 16 > r / 16) ? (OpT)0.f : Mma<OpT>::cvt(Pf[r * LDA + s]);
                }
                __syncthreads();
                if (wv < NB) emit_diag<LDA, LDC, OpT>(Tmf, Tmb, bet, wv);
                {
                    int t = 0;
#pragma unroll
                    for (int i = 1; i < NB; ++i)
#pragma unroll
                        for (int j = 0; j < i; ++j)
                            if ((t++ & 3) == wv) solve_block<LDA, LDC, OpT>(Af, Tmf, Tmb, i, j);
                }
                __syncthreads();
            }

            // ---- out: Tmb then P, row-major, 8 bytes per store
            const int64_t slot_off = ((int64_t)slot * H + h) * kda_slot_bytes<C, K, IO>();
            const rsrc_t rw = make_rsrc((char *)p.ws + slot_off, (uint32_t)(kda_slot_elems<C>() * E));
            constexpr int PER = 8 / E;                       // elements per 8-byte store
            constexpr int NPIECE = 2 * C * C / PER;
            for (int i = tid; i < NPIECE; i += kThreads) {
                const int e0 = i * PER, tile = e0 / (C * C), rc = e0 % (C * C), row = rc / C, col = rc % C;
                const OpT *src = (tile ? Ps : Tmb) + row * LDC + col;
                const u32x2 w = *(const u32x2 *)src;
                __builtin_amdgcn_raw_buffer_store_b64(w, rw, (uint32_t)(e0 * E), 0, 0);
            }
        }
    }
}

}  // namespace gdn
