// gdn_backward kernels: the gradients of the scalar-gate forward from the
// forward's saved chunk-start states (hck) and per-token deltas (v').
//
// Per chunk of C tokens, with gamma the chunk-local inclusive cumsum of g,
// b = e^gamma, c = e^(gamma_last - gamma), start state h and v' = D:
//   A  = strictly lower  beta_r (k_r . k_s) e^(gamma_r - gamma_s),  T = (I + A)^-1
//   P  = lower (incl.)   (q_r . k_s) e^(gamma_r - gamma_s)
//   o  = diag(b) Q h + P D,   h' = e^gamma_last h + (diag(c) K)^T D
// The state's gradient runs backwards through the chunks (bwd_dh_kernel,
// serial per (batch, head, 64-wide V tile), the same chain as the forward's
// scan run in reverse):
//   dD = P^T dO + diag(c) K dh'                         (dh': the chunk-end gradient)
//   dR = T^T dD                                         (v's gradient is diag(beta) dR)
//   dh = e^gamma_last dh' + (diag(b) Q)^T dO - K^T diag(beta b) dR
// and every chunk's input gradients follow from dR, dh', h and D without
// further recurrence (bwd_grad_kernel, one workgroup per (chunk, head)):
//   dP = lower(dO D^T), dA = -strictly lower(dR D^T),
//   Z = dO h^T, Y = dR h^T, W = D dh'^T,
//   F = dP * E, G = dA * beta_r E (E_rs = e^(gamma_r - gamma_s))
//   dq = diag(b) Z + F K
//   dk = -diag(beta b) Y + diag(c) W + F^T Q + (G + G^T) K
//   dbeta_r = dR_r . v_r - b_r k_r . Y_r + sum_s dA_rs (k_r . k_s) E_rs
//   dgamma_r = b_r q_r . Z_r - beta_r b_r k_r . Y_r - c_r k_r . W_r
//              + (row - column sums of dP * P and dA * A)_r,
//   the last row also taking sum_s c_s k_s . W_s + e^gamma_last <h, dh'>,
//   and dg the reverse cumsum of dgamma within the chunk.
// The kernel_fun KDA re-scan page (module docstring) has the forward re-scan
// save h checkpoints and v_new for exactly this later stage; the stage
// itself is the chain rule through the chunk algebra above.
//
// Matrix products run on bf16 MFMA with fp32 accumulation.  q, k, v, dO and
// the saved h and D are bf16 already and enter as they are; a derived fp32
// operand (dh', dD, dR, T, P, F, G and the decayed rows) enters as bf16 high
// and low parts, about 16 bits, two products per step (three where both
// operands are derived).  Every decay is e^x with x <= 0.
#pragma once

#include "gdn_buffer.h"
#include "gdn_inverse.h"

namespace gdn {

struct BwdParams {
    const void *q, *k, *v, *dout;   // bf16 [B, T, H, K | V]
    const float *beta, *g;          // [B, T, H]
    const float *dhT;               // [B, H, K, V] or NULL
    const void *hck, *vnew;         // bf16 [B, NT, H, K, V], [B, T, H, V]
    float *dq, *dk, *dv, *dbeta, *dg, *dh0;   // dh0 may be NULL
    float *dR;                      // workspace [B, T, H, V]
    float *dhe;                     // workspace [B, NT, H, K, V]: chunk-end gradients
    int B, T, H, V, nvt, NT;
    int swizzle;
};

__device__ __forceinline__ void bf_split(float x, uint16_t &h, uint16_t &l) {
    h = f32_to_bf16_bits(x);
    l = f32_to_bf16_bits(x - __uint_as_float((uint32_t)h << 16));
}
__device__ __forceinline__ void mfma_bf(float4v &acc, const bf16x8 &a, const bf16x8 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// A or Bt fragment, k slots 8 (l/16) .. +7 of the 32-wide step at k0: lane
// (g, i) reads S[m0 + i][k0 + 8g .. +7] (bf16 bits, pitch ld).
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *S, int ld, int m0, int k0) {
    const int l = lane_id();
    return __builtin_bit_cast(bf16x8, *(const u32x4 *)(S + (m0 + (l & 15)) * ld + k0 + 8 * (l >> 4)));
}
// The same with split k slots, matching a B fragment built from two
// accumulator tiles: S[m0 + i][k0 + 4g .. +3] and S[m0 + i][k0 + 16 + 4g .. +3].
__device__ __forceinline__ bf16x8 lds_frag_split(const uint16_t *S, int ld, int m0, int k0) {
    const int l = lane_id();
    const uint16_t *p = S + (m0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
    const u32x2 a = *(const u32x2 *)p, b = *(const u32x2 *)(p + 16);
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
// B fragment (split k slots) from the accumulator tiles of k rows
// [k0, k0 + 16) and [k0 + 16, k0 + 32), as bf16 high and low parts.
__device__ __forceinline__ void acc_frag_split(const float4v &a, const float4v &b, bf16x8 &fh, bf16x8 &fl) {
    uint16_t h[8], lo[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf_split(a[e], h[e], lo[e]);
        bf_split(b[e], h[4 + e], lo[4 + e]);
    }
    fh = __builtin_bit_cast(bf16x8, h);
    fl = __builtin_bit_cast(bf16x8, lo);
}
__device__ __forceinline__ uint16_t half_of(const u32x4 &x, int e) {
    return (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
}

// ---------------------------------------------------------------------------
// bwd_dh_kernel: LDS layout (bf16 planes as uint16_t, pitches padded by 16
// bytes so that the 16 rows of a fragment load fall in distinct banks).
// ---------------------------------------------------------------------------
template <int C, int K> struct BwdScanLayout {
    static constexpr int LK = K + 8, LC = C + 8, LF = C + 4;
    static constexpr int kQr = 0;                          // q   [C][LK]
    static constexpr int kKr = kQr + C * LK * 2;           // k   [C][LK]
    static constexpr int kQT = kKr + C * LK * 2;           // q^T [K][LC]
    static constexpr int kKT = kQT + K * LC * 2;           // k^T [K][LC]
    static constexpr int kDoT = kKT + K * LC * 2;          // dO^T of the V tile [64][LC]
    static constexpr int kPT = kDoT + 64 * LC * 2;         // P^T high, low [2][C][LC]
    static constexpr int kTT = kPT + 2 * C * LC * 2;       // T^T high, low [2][C][LC]
    static constexpr int kAf = kTT + 2 * C * LC * 2;       // A  fp32 [C][LF]
    static constexpr int kTf = kAf + C * LF * 4;           // T  fp32 [C][LF]
    static constexpr int kVec = kTf + C * LF * 4;          // gamma, b, c, beta [C]; e^gamma_last
    static constexpr int kBytes = kVec + (4 * C + 4) * 4;
    static_assert(kBytes <= kLdsBytesMax, "LDS budget");
};

// One chunk's q, k (C x K) and dO tile (C x 64) as 16-byte pieces, piece j of
// this thread covering row (tid + 256 j) % C, columns 8 ((tid + 256 j) / C) ..
// +7, so that the 64 lanes of a wave take 64 rows of one column group (their
// transposed LDS writes then fall in distinct banks); plus g and beta of row
// tid.  Rows at or past T read as zero.
template <int C, int K> struct BwdChunkRegs {
    static constexpr int NQK = C * K / 8 / 256;
    static constexpr int NDO = C * 64 / 8 / 256;
    static_assert(NQK >= 1 && NDO >= 1, "tile too small");
    u32x4 q[NQK], k[NQK], d[NDO];
    float g, beta;
};

template <int C, int K>
__device__ __forceinline__ void bwd_load_chunk(BwdChunkRegs<C, K> &r, rsrc_t rq, rsrc_t rk, rsrc_t rdo,
                                               rsrc_t rg, rsrc_t rb, int t0, uint32_t H, uint32_t rsK,
                                               uint32_t rsV, int vt) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < BwdChunkRegs<C, K>::NQK; ++j) {
        const int pc = tid + 256 * j, row = pc % C, c8 = pc / C;
        const uint32_t off = (row * rsK + 8 * c8) * 2;
        r.q[j] = bload128(rq, off, t0 * rsK * 2);
        r.k[j] = bload128(rk, off, t0 * rsK * 2);
    }
#pragma unroll
    for (int j = 0; j < BwdChunkRegs<C, K>::NDO; ++j) {
        const int pc = tid + 256 * j, row = pc % C, c8 = pc / C;
        r.d[j] = bload128(rdo, (row * rsV + 64 * vt + 8 * c8) * 2, t0 * rsV * 2);
    }
    r.g = 0.f;
    r.beta = 0.f;
    if (tid < C) {
        r.g = __uint_as_float(bload32(rg, tid * H * 4, t0 * H * 4));
        r.beta = __uint_as_float(bload32(rb, tid * H * 4, t0 * H * 4));
    }
}

// The state's gradient, backwards over the chunks: one workgroup per (batch,
// head, 64-wide V tile); wave w owns value columns 16 w .. 16 w + 15 of the
// tile, so the chain (dh' -> dD -> dR -> dh) is wave-local.  Per chunk:
//   phase L  the chunk's q, k, dO tile into LDS (row and transposed forms),
//            the previous chunk's loads issued
//   phase 1  gate cumsum and row factors (wave 0)
//   phase 2  Gram tiles: A into fp32 LDS, P^T as bf16 high and low parts
//   phase 3  T = (I + A)^-1 (fp32), T^T as bf16 parts
//   phase 4  off the chain: P^T dO and (diag(b) Q)^T dO for the wave's columns
//   phase 5  the chain; stores dh' (the chunk-end gradient), dR and dv
// Rows past T load as zero: g = 0, beta = 0, k = q = dO = 0, an identity step
// whose outputs the buffer ranges drop.
template <int C, int K>
__global__ __launch_bounds__(256, 1) void bwd_dh_kernel(BwdParams p) {
    typedef BwdScanLayout<C, K> L;
    constexpr int LK = L::LK, LC = L::LC, LF = L::LF;
    constexpr int NB = C / 16, NS = C / 32, KT16 = K / 16, KS = K / 32;
    constexpr int NQK = BwdChunkRegs<C, K>::NQK, NDO = BwdChunkRegs<C, K>::NDO;
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    uint16_t *Qr = (uint16_t *)(smem + L::kQr), *Kr = (uint16_t *)(smem + L::kKr);
    uint16_t *QT = (uint16_t *)(smem + L::kQT), *KT = (uint16_t *)(smem + L::kKT);
    uint16_t *DoT = (uint16_t *)(smem + L::kDoT);
    uint16_t *PT = (uint16_t *)(smem + L::kPT), *TT = (uint16_t *)(smem + L::kTT);
    float *Af = (float *)(smem + L::kAf), *Tf = (float *)(smem + L::kTf);
    float *gam = (float *)(smem + L::kVec), *bv = gam + C, *cv = bv + C, *betv = cv + C, *glp = betv + C;

    const int tid = threadIdx.x, wv = wave_id(), l = lane_id(), g = l >> 4, n = l & 15;
    int bid = blockIdx.x;
    if (p.swizzle) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
    const int vt = bid % p.nvt, bh = bid / p.nvt, b = bh / p.H, h = bh % p.H;
    const int T = p.T, NT = p.NT, V = p.V;
    const uint32_t H = p.H, rsK = H * K, rsV = H * V;
    const int64_t row0 = (int64_t)b * T * H + h;
    const rsrc_t rq = make_rsrc((const bf16_t *)p.q + row0 * K, (uint32_t)T * rsK * 2);
    const rsrc_t rk = make_rsrc((const bf16_t *)p.k + row0 * K, (uint32_t)T * rsK * 2);
    const rsrc_t rdo = make_rsrc((const bf16_t *)p.dout + row0 * V, (uint32_t)T * rsV * 2);
    const rsrc_t rg = make_rsrc(p.g + row0, (uint32_t)T * H * 4);
    const rsrc_t rb = make_rsrc(p.beta + row0, (uint32_t)T * H * 4);
    const rsrc_t rdR = make_rsrc(p.dR + row0 * V, (uint32_t)T * rsV * 4);
    const rsrc_t rdv = make_rsrc(p.dv + row0 * V, (uint32_t)T * rsV * 4);
    const int col = 64 * vt + 16 * wv;                       // the wave's first value column
    // this lane's (row 4g + 2 (n & 1), column n & ~1) of a 16 x 16 tile
    const uint32_t pr_row = 4 * g + 2 * (n & 1), pr_col = col + (n & ~1);

    // entries never written below stay zero: P^T below its diagonal, T above
    for (int i = tid; i < 2 * C * LC / 2; i += 256) ((uint32_t *)PT)[i] = 0u;
    for (int i = tid; i < C * LF; i += 256) Tf[i] = 0.f;

    // the state's gradient at the end of the last chunk: dhT or zero
    float4v dh[KT16];
#pragma unroll
    for (int kt = 0; kt < KT16; ++kt) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dh[kt][e] = p.dhT ? p.dhT[((int64_t)b * H + h) * K * V + (16 * kt + 4 * g + e) * V + col + n] : 0.f;
    }

    BwdChunkRegs<C, K> cr;
    if (NT > 0) bwd_load_chunk<C, K>(cr, rq, rk, rdo, rg, rb, (NT - 1) * C, H, rsK, rsV, vt);
#pragma unroll 1
    for (int c = NT - 1; c >= 0; --c) {
        const int t0 = c * C;
        __syncthreads();
        // phase L
#pragma unroll
        for (int j = 0; j < NQK; ++j) {
            const int pc = tid + 256 * j, row = pc % C, c8 = pc / C;
            *(u32x4 *)(Qr + row * LK + 8 * c8) = cr.q[j];
            *(u32x4 *)(Kr + row * LK + 8 * c8) = cr.k[j];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                QT[(8 * c8 + e) * LC + row] = half_of(cr.q[j], e);
                KT[(8 * c8 + e) * LC + row] = half_of(cr.k[j], e);
            }
        }
#pragma unroll
        for (int j = 0; j < NDO; ++j) {
            const int pc = tid + 256 * j, row = pc % C, c8 = pc / C;
#pragma unroll
            for (int e = 0; e < 8; ++e) DoT[(8 * c8 + e) * LC + row] = half_of(cr.d[j], e);
        }
        if (tid < C) {
            gam[tid] = cr.g;
            betv[tid] = cr.beta;
        }
        if (c > 0) bwd_load_chunk<C, K>(cr, rq, rk, rdo, rg, rb, t0 - C, H, rsK, rsV, vt);
        __syncthreads();
        // phase 1
        if (wv == 0) {
            float x = l < C ? gam[l] : 0.f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o);
                if (l >= o) x += y;
            }
            const float xl = __shfl(x, C - 1);
            if (l < C) {
                gam[l] = x;
                bv[l] = __expf(x);
                cv[l] = __expf(xl - x);
            }
            if (l == 0) *glp = __expf(xl);
        }
        __syncthreads();
        // phase 2: the lower tiles (i >= j) of k k^T (-> A) and q k^T (-> P^T)
        {
            constexpr int NLT = NB * (NB + 1) / 2;
#pragma unroll 1
            for (int t = wv; t < 2 * NLT; t += 4) {
                const bool isP = t >= NLT;
                int tt = isP ? t - NLT : t, i = 0;
                while (tt > i) {
                    tt -= i + 1;
                    ++i;
                }
                const int j = tt;
                float4v acc = {0, 0, 0, 0};
                const uint16_t *Aop = isP ? Qr : Kr;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    mfma_bf(acc, lds_frag(Aop, LK, 16 * i, 32 * s), lds_frag(Kr, LK, 16 * j, 32 * s));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int R = 16 * i + 4 * g + e, S = 16 * j + n;
                    const float d = __expf(fminf(gam[R] - gam[S], 0.f));
                    if (!isP) {
                        Af[R * LF + S] = S < R ? betv[R] * acc[e] * d : 0.f;
                    } else {
                        uint16_t hh, ll;
                        bf_split(S <= R ? acc[e] * d : 0.f, hh, ll);
                        PT[S * LC + R] = hh;
                        PT[C * LC + S * LC + R] = ll;
                    }
                }
            }
        }
        __syncthreads();
        // phase 3
        tri_inverse<C, LF>(Af, Tf);
        for (int idx = tid; idx < C * C; idx += 256) {
            const int s = idx / C, r = idx % C;
            uint16_t hh, ll;
            bf_split(Tf[s * LF + r], hh, ll);
            TT[r * LC + s] = hh;
            TT[C * LC + r * LC + s] = ll;
        }
        __syncthreads();
        // phase 4: P^T dO (tokens x the wave's columns) and (diag(b) Q)^T dO
        // (keys x the wave's columns)
        float4v pd[NB], qd[KT16];
        {
            bf16x8 bq_h[NS], bq_l[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int s0 = 32 * st + 8 * g;
                const u32x4 raw = *(const u32x4 *)(DoT + (16 * wv + n) * LC + s0);
                uint16_t hh[8], ll[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bf_split(__uint_as_float((uint32_t)half_of(raw, e) << 16) * bv[s0 + e], hh[e], ll[e]);
                bq_h[st] = __builtin_bit_cast(bf16x8, hh);
                bq_l[st] = __builtin_bit_cast(bf16x8, ll);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                pd[i] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    if (32 * st + 31 < 16 * i) continue;      // P^T is zero below its diagonal
                    const bf16x8 bdo = lds_frag(DoT, LC, 16 * wv, 32 * st);
                    mfma_bf(pd[i], lds_frag(PT, LC, 16 * i, 32 * st), bdo);
                    mfma_bf(pd[i], lds_frag(PT + C * LC, LC, 16 * i, 32 * st), bdo);
                }
            }
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt) {
                qd[kt] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const bf16x8 a = lds_frag(QT, LC, 16 * kt, 32 * st);
                    mfma_bf(qd[kt], a, bq_h[st]);
                    mfma_bf(qd[kt], a, bq_l[st]);
                }
            }
        }
        // phase 5: the chain.  dh' is this chunk's end gradient.
        {
            float *he = p.dhe + (((int64_t)b * NT + c) * H + h) * K * V;
            const rsrc_t rhe = make_rsrc(he, (uint32_t)(K * V * 4));
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt)
                store_acc_pairs<float>(dh[kt], rhe, (pr_row * V + pr_col) * 4, V * 4, 16 * kt * V * 4);
        }
        float4v rr[NB];
        {
            bf16x8 bh[KS], bl[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) acc_frag_split(dh[2 * s], dh[2 * s + 1], bh[s], bl[s]);
            float4v dd[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                dd[i] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 a = lds_frag_split(Kr, LK, 16 * i, 32 * s);
                    mfma_bf(dd[i], a, bh[s]);
                    mfma_bf(dd[i], a, bl[s]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) dd[i][e] = cv[16 * i + 4 * g + e] * dd[i][e] + pd[i][e];
            }
            bf16x8 xh[NS], xl[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) acc_frag_split(dd[2 * st], dd[2 * st + 1], xh[st], xl[st]);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                rr[i] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    if (32 * st + 31 < 16 * i) continue;      // T^T is zero below its diagonal
                    const bf16x8 ah = lds_frag_split(TT, LC, 16 * i, 32 * st);
                    const bf16x8 al = lds_frag_split(TT + C * LC, LC, 16 * i, 32 * st);
                    mfma_bf(rr[i], ah, xh[st]);
                    mfma_bf(rr[i], ah, xl[st]);
                    mfma_bf(rr[i], al, xh[st]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint32_t voff = (pr_row * rsV + pr_col) * 4, soff = (t0 + 16 * i) * rsV * 4;
            store_acc_pairs<float>(rr[i], rdR, voff, rsV * 4, soff);
            float4v x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = betv[16 * i + 4 * g + e] * rr[i][e];
            store_acc_pairs<float>(x, rdv, voff, rsV * 4, soff);
        }
        {
            bf16x8 uh[NS], ul[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                float4v x0, x1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r0 = 32 * st + 4 * g + e, r1 = r0 + 16;
                    x0[e] = -betv[r0] * bv[r0] * rr[2 * st][e];
                    x1[e] = -betv[r1] * bv[r1] * rr[2 * st + 1][e];
                }
                acc_frag_split(x0, x1, uh[st], ul[st]);
            }
            const float gl = *glp;
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt) {
                float4v acc = gl * dh[kt] + qd[kt];
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const bf16x8 a = lds_frag_split(KT, LC, 16 * kt, 32 * st);
                    mfma_bf(acc, a, uh[st]);
                    mfma_bf(acc, a, ul[st]);
                }
                dh[kt] = acc;
            }
        }
    }
    if (p.dh0) {
        const rsrc_t rh0 = make_rsrc(p.dh0 + ((int64_t)b * H + h) * K * V, (uint32_t)(K * V * 4));
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt)
            store_acc_pairs<float>(dh[kt], rh0, (pr_row * V + pr_col) * 4, V * 4, 16 * kt * V * 4);
    }
}

// ---------------------------------------------------------------------------
// bwd_grad_kernel: one workgroup per (chunk, head).  LDS holds q and k in
// row and transposed form for the whole chunk, and one region that the
// phases reuse:
//   A   dO, D, dR (bf16 parts)  -> the C x C tiles: k k^T, q k^T, dO D^T, dR D^T
//   A2  F, F^T, G + G^T (bf16 parts)                -> F K, F^T Q, (G + G^T) K
//   B   dO, dR (bf16 parts), h                       -> Z = dO h^T, Y = dR h^T
//   C   D, dh' (bf16 parts)                          -> W = D dh'^T
// Wave w owns key columns 32 w .. 32 w + 31 of dq and dk (all C rows), and
// the lower C x C tiles w, w + 4, ...  Row sums (the gate's and beta's
// gradients) go through per-wave LDS rows, added in a fixed order: the
// results do not depend on scheduling.
// ---------------------------------------------------------------------------
template <int C, int K, int V> struct BwdGradLayout {
    static constexpr int LK = K + 8, LC = C + 8, LV = V + 8;
    static constexpr int kQr = 0;
    static constexpr int kKr = kQr + C * LK * 2;
    static constexpr int kQT = kKr + C * LK * 2;
    static constexpr int kKT = kQT + K * LC * 2;
    static constexpr int kX = kKT + K * LC * 2;
    static constexpr int kA_do = kX, kA_d = kA_do + C * LV * 2, kA_r = kA_d + C * LV * 2;
    static constexpr int kF = kX, kFT = kF + 2 * C * LC * 2, kGs = kFT + 2 * C * LC * 2;
    static constexpr int kB_do = kX, kB_r = kB_do + C * LV * 2, kB_h = kB_r + 2 * C * LV * 2;
    static constexpr int kC_d = kX, kC_dh = kC_d + C * LV * 2;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int kXBytes = cmax(cmax(4 * C * LV * 2, 6 * C * LC * 2),
                                        cmax(3 * C * LV * 2 + K * LV * 2, C * LV * 2 + 2 * K * LV * 2));
    static constexpr int kVec = kX + kXBytes;   // gamma, b, c, beta [C]; pg, pb, pkw [4][C]; hd [4]
    static constexpr int kBytes = kVec + (16 * C + 4) * 4;
    static_assert(kBytes <= kLdsBytesMax, "LDS budget");
};

// rows x X bf16 block of a token-major tensor (row pitch rs elements) into
// LDS [rows][LD], 16 bytes per piece, row-major over the workgroup.
template <int ROWS, int X, int LD>
__device__ __forceinline__ void bwd_rows_to_lds(uint16_t *dst, rsrc_t r, uint32_t rs, uint32_t soff) {
    constexpr int PPR = X / 8, NP = ROWS * PPR;
#pragma unroll
    for (int pc = threadIdx.x; pc < NP; pc += 256) {
        const int row = pc / PPR, c8 = pc % PPR;
        *(u32x4 *)(dst + row * LD + 8 * c8) = bload128(r, (row * rs + 8 * c8) * 2, soff);
    }
}

// rows x X fp32 block (row pitch rs elements) into LDS as bf16 high and low
// planes [2][rows][LD], 16 bytes per piece.  With rv (bf16, same layout and
// pitch rvs) also each row's dot product of the two, reduced over the row's
// pieces (consecutive lanes) and added into acc[row] by the row's first lane.
template <int ROWS, int X, int LD, bool DOT>
__device__ __forceinline__ void bwd_split_to_lds(uint16_t *dst, rsrc_t r, uint32_t rs, uint32_t soff,
                                                 rsrc_t rv, uint32_t rvs, uint32_t vsoff, float *acc) {
    constexpr int PPR = X / 4, NP = ROWS * PPR;
    static_assert(PPR <= 64 && (PPR & (PPR - 1)) == 0, "pieces per row");
#pragma unroll
    for (int pc = threadIdx.x; pc < NP; pc += 256) {
        const int row = pc / PPR, c4 = pc % PPR;
        const u32x4 x = bload128(r, (row * rs + 4 * c4) * 4, soff);
        uint16_t hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bf_split(__uint_as_float(x[e]), hh[e], ll[e]);
        *(u32x2 *)(dst + row * LD + 4 * c4) = __builtin_bit_cast(u32x2, hh);
        *(u32x2 *)(dst + ROWS * LD + row * LD + 4 * c4) = __builtin_bit_cast(u32x2, ll);
        if constexpr (DOT) {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rv, (row * rvs + 4 * c4) * 2, vsoff, 0);
            float d = __uint_as_float(x[0]) * __uint_as_float(w[0] << 16) +
                      __uint_as_float(x[1]) * __uint_as_float(w[0] & 0xffff0000u) +
                      __uint_as_float(x[2]) * __uint_as_float(w[1] << 16) +
                      __uint_as_float(x[3]) * __uint_as_float(w[1] & 0xffff0000u);
#pragma unroll
            for (int o = PPR / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o);
            if (c4 == 0) acc[row] += d;
        }
    }
}

// Sum over the 16 lanes of a lane group (the columns of an accumulator tile).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int C, int K, int V>
__global__ __launch_bounds__(256, 1) void bwd_grad_kernel(BwdParams p) {
    typedef BwdGradLayout<C, K, V> L;
    constexpr int LK = L::LK, LC = L::LC, LV = L::LV;
    constexpr int NB = C / 16, NS = C / 32, KS = K / 32, VS = V / 32, NLT = NB * (NB + 1) / 2;
    constexpr int MT = (NLT + 3) / 4;           // lower C x C tiles per wave (at most)
    constexpr int CT = K / 64;                  // 16-column key tiles per wave
    static_assert(K % 64 == 0, "key tiles");
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    uint16_t *Qr = (uint16_t *)(smem + L::kQr), *Kr = (uint16_t *)(smem + L::kKr);
    uint16_t *QT = (uint16_t *)(smem + L::kQT), *KT = (uint16_t *)(smem + L::kKT);
    float *gam = (float *)(smem + L::kVec), *bv = gam + C, *cv = bv + C, *betv = cv + C;
    float *pg = betv + C, *pb = pg + 4 * C, *pkw = pb + 4 * C, *hd = pkw + 4 * C;

    const int tid = threadIdx.x, wv = wave_id(), l = lane_id(), g = l >> 4, n = l & 15;
    const int NT = p.NT, T = p.T;
    const int c = blockIdx.x % NT, bh = blockIdx.x / NT, b = bh / p.H, h = bh % p.H;
    const int t0 = c * C;
    const uint32_t H = p.H, rsK = H * K, rsV = H * V;
    const int64_t row0 = (int64_t)b * T * H + h;
    const rsrc_t rq = make_rsrc((const bf16_t *)p.q + row0 * K, (uint32_t)T * rsK * 2);
    const rsrc_t rk = make_rsrc((const bf16_t *)p.k + row0 * K, (uint32_t)T * rsK * 2);
    const rsrc_t rv = make_rsrc((const bf16_t *)p.v + row0 * V, (uint32_t)T * rsV * 2);
    const rsrc_t rdo = make_rsrc((const bf16_t *)p.dout + row0 * V, (uint32_t)T * rsV * 2);
    const rsrc_t rD = make_rsrc((const bf16_t *)p.vnew + row0 * V, (uint32_t)T * rsV * 2);
    const rsrc_t rdR = make_rsrc(p.dR + row0 * V, (uint32_t)T * rsV * 4);
    const rsrc_t rg = make_rsrc(p.g + row0, (uint32_t)T * H * 4);
    const rsrc_t rb = make_rsrc(p.beta + row0, (uint32_t)T * H * 4);
    const int64_t kv = (((int64_t)b * NT + c) * H + h) * K * V;
    const rsrc_t rh = make_rsrc((const bf16_t *)p.hck + kv, (uint32_t)(K * V * 2));
    const rsrc_t rdh = make_rsrc(p.dhe + kv, (uint32_t)(K * V * 4));

    // q, k (row and transposed forms); g, beta; per-row partial sums cleared
    {
        constexpr int NP = C * K / 8;
#pragma unroll
        for (int pc = tid; pc < NP; pc += 256) {
            const int row = pc % C, c8 = pc / C;
            const uint32_t off = (row * rsK + 8 * c8) * 2;
            const u32x4 xq = bload128(rq, off, t0 * rsK * 2), xk = bload128(rk, off, t0 * rsK * 2);
            *(u32x4 *)(Qr + row * LK + 8 * c8) = xq;
            *(u32x4 *)(Kr + row * LK + 8 * c8) = xk;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                QT[(8 * c8 + e) * LC + row] = half_of(xq, e);
                KT[(8 * c8 + e) * LC + row] = half_of(xk, e);
            }
        }
        for (int i = tid; i < 12 * C + 4; i += 256) pg[i] = 0.f;
        uint16_t *X = (uint16_t *)(smem + L::kX);
        bwd_rows_to_lds<C, V, LV>(X + (L::kA_do - L::kX) / 2, rdo, rsV, t0 * rsV * 2);
        bwd_rows_to_lds<C, V, LV>(X + (L::kA_d - L::kX) / 2, rD, rsV, t0 * rsV * 2);
        bwd_split_to_lds<C, V, LV, false>(X + (L::kA_r - L::kX) / 2, rdR, rsV, t0 * rsV * 4, rdR, 0, 0, nullptr);
    }
    if (wv == 0) {
        float x = l < C ? __uint_as_float(bload32(rg, l * H * 4, t0 * H * 4)) : 0.f;
        const float bt = l < C ? __uint_as_float(bload32(rb, l * H * 4, t0 * H * 4)) : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o);
            if (l >= o) x += y;
        }
        const float xl = __shfl(x, C - 1);
        if (l < C) {
            gam[l] = x;
            bv[l] = __expf(x);
            cv[l] = __expf(xl - x);
            betv[l] = bt;
        }
    }
    __syncthreads();

    // phase A: lower C x C tiles of this wave
    float4v Fv[MT], Gv[MT];
    {
        const uint16_t *Do = (const uint16_t *)(smem + L::kA_do), *Dm = (const uint16_t *)(smem + L::kA_d);
        const uint16_t *Rh = (const uint16_t *)(smem + L::kA_r), *Rl = Rh + C * LV;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = wv + 4 * m;
            Fv[m] = float4v{0, 0, 0, 0};
            Gv[m] = float4v{0, 0, 0, 0};
            if (t >= NLT) continue;
            int tt = t, i = 0;
            while (tt > i) {
                tt -= i + 1;
                ++i;
            }
            const int j = tt;
            float4v skk = {0, 0, 0, 0}, sqk = {0, 0, 0, 0}, dp = {0, 0, 0, 0}, da = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 kb = lds_frag(Kr, LK, 16 * j, 32 * s);
                mfma_bf(skk, lds_frag(Kr, LK, 16 * i, 32 * s), kb);
                mfma_bf(sqk, lds_frag(Qr, LK, 16 * i, 32 * s), kb);
            }
#pragma unroll
            for (int s = 0; s < VS; ++s) {
                const bf16x8 db = lds_frag(Dm, LV, 16 * j, 32 * s);
                mfma_bf(dp, lds_frag(Do, LV, 16 * i, 32 * s), db);
                mfma_bf(da, lds_frag(Rh, LV, 16 * i, 32 * s), db);
                mfma_bf(da, lds_frag(Rl, LV, 16 * i, 32 * s), db);
            }
            float rs_g[4], rs_b[4], cs = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int R = 16 * i + 4 * g + e, S = 16 * j + n;
                const float E = S <= R ? __expf(gam[R] - gam[S]) : 0.f;
                const float dPm = S <= R ? dp[e] : 0.f, dAm = S < R ? -da[e] : 0.f;
                const float P = sqk[e] * E, kkE = skk[e] * E, A = betv[R] * kkE;
                Fv[m][e] = dPm * E;
                Gv[m][e] = dAm * betv[R] * E;
                const float tg = dPm * P + dAm * A;
                rs_g[e] = tg;
                rs_b[e] = dAm * kkE;
                cs += tg;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rs_g[e] = sum16(rs_g[e]);
                rs_b[e] = sum16(rs_b[e]);
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (n == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pg[wv * C + 16 * i + 4 * g + e] += rs_g[e];
                    pb[wv * C + 16 * i + 4 * g + e] += rs_b[e];
                }
            }
            if (g == 0) pg[wv * C + 16 * j + n] -= cs;
        }
    }
    __syncthreads();
    // phase A2: F, F^T, G + G^T as bf16 parts
    uint16_t *Fp = (uint16_t *)(smem + L::kF), *FTp = (uint16_t *)(smem + L::kFT), *Gp = (uint16_t *)(smem + L::kGs);
    for (int i = tid; i < 6 * C * LC / 2; i += 256) ((uint32_t *)Fp)[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int t = wv + 4 * m;
        if (t >= NLT) continue;
        int tt = t, i = 0;
        while (tt > i) {
            tt -= i + 1;
            ++i;
        }
        const int j = tt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int R = 16 * i + 4 * g + e, S = 16 * j + n;
            uint16_t hh, ll;
            if (S <= R) {
                bf_split(Fv[m][e], hh, ll);
                Fp[R * LC + S] = hh;
                Fp[C * LC + R * LC + S] = ll;
                FTp[S * LC + R] = hh;
                FTp[C * LC + S * LC + R] = ll;
            }
            if (S < R) {
                bf_split(Gv[m][e], hh, ll);
                Gp[R * LC + S] = hh;
                Gp[C * LC + R * LC + S] = ll;
                Gp[S * LC + R] = hh;
                Gp[C * LC + S * LC + R] = ll;
            }
        }
    }
    __syncthreads();
    // phase A3: dq = F K, dk = F^T Q + (G + G^T) K for this wave's key columns
    float4v dq[NB][CT], dk[NB][CT];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int kc = 16 * (CT * wv + ct);
            float4v aq = {0, 0, 0, 0}, ak = {0, 0, 0, 0};
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const bf16x8 kb = lds_frag(KT, LC, kc, 32 * st);
                if (32 * st <= 16 * i + 15) {        // F is zero right of its diagonal
                    mfma_bf(aq, lds_frag(Fp, LC, 16 * i, 32 * st), kb);
                    mfma_bf(aq, lds_frag(Fp + C * LC, LC, 16 * i, 32 * st), kb);
                }
                if (32 * st + 31 >= 16 * i) {        // F^T is zero left of its diagonal
                    const bf16x8 qb = lds_frag(QT, LC, kc, 32 * st);
                    mfma_bf(ak, lds_frag(FTp, LC, 16 * i, 32 * st), qb);
                    mfma_bf(ak, lds_frag(FTp + C * LC, LC, 16 * i, 32 * st), qb);
                }
                mfma_bf(ak, lds_frag(Gp, LC, 16 * i, 32 * st), kb);
                mfma_bf(ak, lds_frag(Gp + C * LC, LC, 16 * i, 32 * st), kb);
            }
            dq[i][ct] = aq;
            dk[i][ct] = ak;
        }
    __syncthreads();
    // phase B: Z = dO h^T, Y = dR h^T; with v . dR into beta's row sums
    {
        uint16_t *X = (uint16_t *)(smem + L::kX);
        bwd_rows_to_lds<C, V, LV>(X + (L::kB_do - L::kX) / 2, rdo, rsV, t0 * rsV * 2);
        bwd_split_to_lds<C, V, LV, true>(X + (L::kB_r - L::kX) / 2, rdR, rsV, t0 * rsV * 4, rv, rsV,
                                         t0 * rsV * 2, pb + wv * C);
        bwd_rows_to_lds<K, V, LV>(X + (L::kB_h - L::kX) / 2, rh, V, 0);
    }
    __syncthreads();
    {
        const uint16_t *Do = (const uint16_t *)(smem + L::kB_do), *Hm = (const uint16_t *)(smem + L::kB_h);
        const uint16_t *Rh = (const uint16_t *)(smem + L::kB_r), *Rl = Rh + C * LV;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            float qz[4] = {0, 0, 0, 0}, ky[4] = {0, 0, 0, 0};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int kc = 16 * (CT * wv + ct);
                float4v z = {0, 0, 0, 0}, y = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < VS; ++s) {
                    const bf16x8 hb = lds_frag(Hm, LV, kc, 32 * s);
                    mfma_bf(z, lds_frag(Do, LV, 16 * i, 32 * s), hb);
                    mfma_bf(y, lds_frag(Rh, LV, 16 * i, 32 * s), hb);
                    mfma_bf(y, lds_frag(Rl, LV, 16 * i, 32 * s), hb);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int R = 16 * i + 4 * g + e, key = kc + n;
                    dq[i][ct][e] += bv[R] * z[e];
                    dk[i][ct][e] -= betv[R] * bv[R] * y[e];
                    qz[e] += __uint_as_float((uint32_t)Qr[R * LK + key] << 16) * z[e];
                    ky[e] += __uint_as_float((uint32_t)Kr[R * LK + key] << 16) * y[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qz[e] = sum16(qz[e]);
                ky[e] = sum16(ky[e]);
            }
            if (n == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int R = 16 * i + 4 * g + e;
                    pg[wv * C + R] += bv[R] * qz[e] - betv[R] * bv[R] * ky[e];
                    pb[wv * C + R] -= bv[R] * ky[e];
                }
            }
        }
    }
    __syncthreads();
    // phase C: W = D dh'^T; with <h, dh'>
    {
        uint16_t *X = (uint16_t *)(smem + L::kX);
        bwd_rows_to_lds<C, V, LV>(X + (L::kC_d - L::kX) / 2, rD, rsV, t0 * rsV * 2);
        float hdp = 0.f;
        constexpr int PPR = V / 4, NP = K * PPR;
        uint16_t *dst = X + (L::kC_dh - L::kX) / 2;
#pragma unroll
        for (int pc = tid; pc < NP; pc += 256) {
            const int row = pc / PPR, c4 = pc % PPR;
            const u32x4 x = bload128(rdh, (row * V + 4 * c4) * 4, 0);
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rh, (row * V + 4 * c4) * 2, 0, 0);
            uint16_t hh[4], ll[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bf_split(__uint_as_float(x[e]), hh[e], ll[e]);
            *(u32x2 *)(dst + row * LV + 4 * c4) = __builtin_bit_cast(u32x2, hh);
            *(u32x2 *)(dst + K * LV + row * LV + 4 * c4) = __builtin_bit_cast(u32x2, ll);
            hdp += __uint_as_float(x[0]) * __uint_as_float(w[0] << 16) +
                   __uint_as_float(x[1]) * __uint_as_float(w[0] & 0xffff0000u) +
                   __uint_as_float(x[2]) * __uint_as_float(w[1] << 16) +
                   __uint_as_float(x[3]) * __uint_as_float(w[1] & 0xffff0000u);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) hdp += __shfl_xor(hdp, o);
        if (l == 0) hd[wv] = hdp;
    }
    __syncthreads();
    {
        const uint16_t *Dm = (const uint16_t *)(smem + L::kC_d);
        const uint16_t *Hh = (const uint16_t *)(smem + L::kC_dh), *Hl = Hh + K * LV;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            float kw[4] = {0, 0, 0, 0};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int kc = 16 * (CT * wv + ct);
                float4v w = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < VS; ++s) {
                    const bf16x8 a = lds_frag(Dm, LV, 16 * i, 32 * s);
                    mfma_bf(w, a, lds_frag(Hh, LV, kc, 32 * s));
                    mfma_bf(w, a, lds_frag(Hl, LV, kc, 32 * s));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int R = 16 * i + 4 * g + e, key = kc + n;
                    dk[i][ct][e] += cv[R] * w[e];
                    kw[e] += __uint_as_float((uint32_t)Kr[R * LK + key] << 16) * w[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) kw[e] = sum16(kw[e]);
            if (n == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) pkw[wv * C + 16 * i + 4 * g + e] += kw[e];
            }
        }
    }
    // dq, dk out
    {
        const rsrc_t rdq = make_rsrc(p.dq + row0 * K, (uint32_t)T * rsK * 4);
        const rsrc_t rdk = make_rsrc(p.dk + row0 * K, (uint32_t)T * rsK * 4);
        const uint32_t pr_row = 4 * g + 2 * (n & 1);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const uint32_t voff = (pr_row * rsK + 16 * (CT * wv + ct) + (n & ~1)) * 4;
                const uint32_t soff = (t0 + 16 * i) * rsK * 4;
                store_acc_pairs<float>(dq[i][ct], rdq, voff, rsK * 4, soff);
                store_acc_pairs<float>(dk[i][ct], rdk, voff, rsK * 4, soff);
            }
    }
    __syncthreads();
    // the gate's and beta's gradients: per-row sums in a fixed order, the
    // last row's extra terms, then the reverse cumsum within the chunk
    if (wv == 0) {
        float dgam = 0.f, db = 0.f, kw = 0.f;
        if (l < C) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dgam += pg[w * C + l];
                db += pb[w * C + l];
                kw += pkw[w * C + l];
            }
        }
        const float ckw = l < C ? cv[l] * kw : 0.f;
        dgam -= ckw;
        float tot = ckw;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        const float gl = __expf(gam[C - 1]);
        if (l == C - 1) dgam += tot + gl * (hd[0] + hd[1] + hd[2] + hd[3]);
        // suffix sum over lanes (lanes >= C hold zero)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_down(dgam, o);
            if (l + o < 64) dgam += y;
        }
        const rsrc_t rdg = make_rsrc(p.dg + row0, (uint32_t)T * H * 4);
        const rsrc_t rdb = make_rsrc(p.dbeta + row0, (uint32_t)T * H * 4);
        if (l < C) {
            bstore32(__float_as_uint(dgam), rdg, l * H * 4, t0 * H * 4);
            bstore32(__float_as_uint(db), rdb, l * H * 4, t0 * H * 4);
        }
    }
}

}  // namespace gdn
