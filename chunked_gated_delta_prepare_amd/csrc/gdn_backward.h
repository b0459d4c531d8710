// gdn_backward kernels: the gradients of the scalar-gate forward from the
// forward's saved chunk-start states (hck) and per-token deltas (v').
//
// Per chunk of C tokens, with gamma the chunk-local inclusive cumsum of g,
// b = e^gamma, c = e^(gamma_last - gamma), start state h and v' = D:
//   A  = strictly lower  beta_r (k_r . k_s) e^(gamma_r - gamma_s),  T = (I + A)^-1
//   P  = lower (incl.)   (q_r . k_s) e^(gamma_r - gamma_s)
//   o  = diag(b) Q h + P D,   h' = e^gamma_last h + (diag(c) K)^T D
// Three launches.  bwd_prep_kernel forms every chunk's P^T, T^T and row
// factors at once (one workgroup per (chunk, head)).  Then the state's
// gradient runs backwards through the chunks (bwd_dh_kernel, serial per
// (batch, head, 64-wide V tile), the forward's chain run in reverse):
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
    void *prep;                     // workspace: the reverse scan's per-chunk slots (BwdSlot)
    float *dpa;                     // workspace, per-key gate: dP, dA [B, NT, H][2][C][C]
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
// A workgroup barrier that orders LDS only: this wave's LDS operations
// complete, then s_barrier.  Global loads in flight (the next phase's
// operands) stay in flight; no wave of these kernels reads global memory
// that another wave of the workgroup writes.
__device__ __forceinline__ void bwd_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint16_t half_of(const u32x4 &x, int e) {
    return (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
}

// ---------------------------------------------------------------------------
// Per-chunk factors of the reverse scan, formed for every (chunk, head) at
// once by bwd_prep_kernel before the serial scan reads them: P^T and T^T
// (C x C, bf16 high and low parts, row-major, pitch C) and the row factors
// b = e^gamma, c = e^(gamma_last - gamma), beta b, beta (fp32 [C]) and
// e^gamma_last.  Slot of chunk c of stream (b, h): (b * NT + c) * H + h.
// ---------------------------------------------------------------------------
template <int C> struct BwdSlot {
    static constexpr int kPTh = 0, kPTl = kPTh + C * C * 2, kTTh = kPTl + C * C * 2,
                         kTTl = kTTh + C * C * 2;
    static constexpr int kVec = kTTl + C * C * 2;      // b, c, beta b, beta [C], e^gamma_last, pad
    static constexpr int kBytes = kVec + (4 * C + 4) * 4;
    static_assert(kBytes % 16 == 0, "slot pieces");
};

template <int C, int K> struct BwdPrepLayout {
    static constexpr int LK = K + 8, LC = C + 8, LF = C + 4;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    // q, k [C][LK] for the Gram products; afterwards A, T fp32 [C][LF] there
    static constexpr int kQr = 0, kKr = kQr + C * LK * 2;
    static constexpr int kAf = 0, kTf = kAf + C * LF * 4;
    static constexpr int kPl = cmax(2 * C * LK * 2, 2 * C * LF * 4);   // P^T h, l, T^T h, l [4][C][LC]
    static constexpr int kVec = kPl + 4 * C * LC * 2;      // gamma, b, c, beta b, beta [C], gl
    static constexpr int kBytes = kVec + (5 * C + 4) * 4;
    static_assert(2 * kBytes <= kLdsBytesMax, "two workgroups per CU");
};

// The reverse scan's per-chunk factors, one workgroup per (chunk, head):
// gate cumsum, the lower tiles of k k^T (-> A) and q k^T (-> P), the
// inverse T = (I + A)^-1 in fp32, then P^T, T^T and the row factors into the
// chunk's slot.  Rows past T load as zero (an identity step).
template <int C, int K>
__global__ __launch_bounds__(256, 2) void bwd_prep_kernel(BwdParams p) {
    typedef BwdPrepLayout<C, K> L;
    typedef BwdSlot<C> SL;
    constexpr int LK = L::LK, LC = L::LC, LF = L::LF;
    constexpr int NB = C / 16, KS = K / 32, NLT = NB * (NB + 1) / 2;
    constexpr int MTP = (2 * NLT + 3) / 4;         // Gram tiles per wave (at most)
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    uint16_t *Qr = (uint16_t *)(smem + L::kQr), *Kr = (uint16_t *)(smem + L::kKr);
    float *Af = (float *)(smem + L::kAf), *Tf = (float *)(smem + L::kTf);
    uint16_t *Pl = (uint16_t *)(smem + L::kPl);          // planes: P^T h, P^T l, T^T h, T^T l
    float *gam = (float *)(smem + L::kVec), *bv = gam + C, *cv = bv + C, *bbv = cv + C, *betv = bbv + C,
          *glp = betv + C;

    const int tid = threadIdx.x, wv = wave_id(), l = lane_id(), g = l >> 4, n = l & 15;
    const int NT = p.NT, T = p.T;
    const int c = blockIdx.x % NT, bh = blockIdx.x / NT, b = bh / p.H, h = bh % p.H;
    const int t0 = c * C;
    const uint32_t H = p.H, rsK = H * K;
    const int64_t row0 = (int64_t)b * T * H + h;
    const rsrc_t rq = make_rsrc((const bf16_t *)p.q + row0 * K, (uint32_t)T * rsK * 2);
    const rsrc_t rk = make_rsrc((const bf16_t *)p.k + row0 * K, (uint32_t)T * rsK * 2);
#pragma unroll
    for (int pc = tid; pc < C * K / 8; pc += 256) {
        const int row = pc / (K / 8), c8 = pc % (K / 8);
        const uint32_t off = (row * rsK + 8 * c8) * 2;
        *(u32x4 *)(Qr + row * LK + 8 * c8) = bload128(rq, off, t0 * rsK * 2);
        *(u32x4 *)(Kr + row * LK + 8 * c8) = bload128(rk, off, t0 * rsK * 2);
    }
    if (wv == 0) {
        const rsrc_t rg = make_rsrc(p.g + row0, (uint32_t)T * H * 4);
        const rsrc_t rb = make_rsrc(p.beta + row0, (uint32_t)T * H * 4);
        float x = l < C ? __uint_as_float(bload32(rg, l * H * 4, t0 * H * 4)) : 0.f;
        const float bt = l < C ? __uint_as_float(bload32(rb, l * H * 4, t0 * H * 4)) : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o);
            if (l >= o) x += y;
        }
        const float xl = __shfl(x, C - 1);
        if (l < C) {
            const float e = __expf(x);
            gam[l] = x;
            bv[l] = e;
            cv[l] = __expf(xl - x);
            bbv[l] = bt * e;
            betv[l] = bt;
        }
        if (l == 0) *glp = __expf(xl);
    }
    __syncthreads();
    // Gram tiles (k k^T for A, q k^T for P) into registers; then, with q and
    // k no longer read, A (fp32) and T's zeros over them, and P^T (bf16 parts)
    float4v gacc[MTP];
#pragma unroll
    for (int m = 0; m < MTP; ++m) {
        const int t = wv + 4 * m;
        gacc[m] = float4v{0, 0, 0, 0};
        if (t >= 2 * NLT) continue;
        const bool isP = t >= NLT;
        int tt = isP ? t - NLT : t, i = 0;
        while (tt > i) {
            tt -= i + 1;
            ++i;
        }
        const int j = tt;
        const uint16_t *Aop = isP ? Qr : Kr;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            mfma_bf(gacc[m], lds_frag(Aop, LK, 16 * i, 32 * s), lds_frag(Kr, LK, 16 * j, 32 * s));
    }
    __syncthreads();
    for (int i = tid; i < C * LF; i += 256) Tf[i] = 0.f;
#pragma unroll
    for (int m = 0; m < MTP; ++m) {
        const int t = wv + 4 * m;
        if (t >= 2 * NLT) continue;
        const bool isP = t >= NLT;
        int tt = isP ? t - NLT : t, i = 0;
        while (tt > i) {
            tt -= i + 1;
            ++i;
        }
        const int j = tt;
        const float4v acc = gacc[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int R = 16 * i + 4 * g + e, S = 16 * j + n;
            const float d = __expf(fminf(gam[R] - gam[S], 0.f));
            if (!isP) {
                Af[R * LF + S] = S < R ? betv[R] * acc[e] * d : 0.f;
            } else {
                uint16_t hh, ll;
                bf_split(S <= R ? acc[e] * d : 0.f, hh, ll);
                Pl[S * LC + R] = hh;
                Pl[C * LC + S * LC + R] = ll;
                if (i != j) {                        // P^T is zero below its diagonal
                    Pl[R * LC + S] = 0;
                    Pl[C * LC + R * LC + S] = 0;
                }
            }
        }
    }
    __syncthreads();
    tri_inverse<C, LF>(Af, Tf);
    for (int idx = tid; idx < C * C; idx += 256) {
        const int s = idx / C, r = idx % C;
        uint16_t hh, ll;
        bf_split(Tf[s * LF + r], hh, ll);
        Pl[2 * C * LC + r * LC + s] = hh;
        Pl[3 * C * LC + r * LC + s] = ll;
    }
    __syncthreads();
    // out: the four planes row by row (8-byte pieces, consecutive lanes on
    // consecutive pieces), then the vectors
    char *slot = (char *)p.prep + (((int64_t)b * NT + c) * H + h) * SL::kBytes;
    const rsrc_t rsl = make_rsrc(slot, (uint32_t)SL::kBytes);
#pragma unroll
    for (int pc = tid; pc < C * C; pc += 256) {
        const int pl = pc / (C * C / 4), rem = pc % (C * C / 4), row = rem / (C / 4), c4 = rem % (C / 4);
        const u32x2 x = *(const u32x2 *)(Pl + pl * C * LC + row * LC + 4 * c4);
        __builtin_amdgcn_raw_buffer_store_b64(x, rsl, (pl * C * C + row * C + 4 * c4) * 2, 0, 0);
    }
    float *sv = (float *)(slot + SL::kVec);
    if (tid < C) {
        sv[tid] = bv[tid];
        sv[C + tid] = cv[tid];
        sv[2 * C + tid] = bbv[tid];
        sv[3 * C + tid] = betv[tid];
    }
    if (tid == 0) sv[4 * C] = *glp;
}

// ---------------------------------------------------------------------------
// bwd_dh_kernel: LDS layout (bf16 planes as uint16_t, pitches padded by 16
// bytes so that the 16 rows of a fragment load fall in distinct banks).
// ---------------------------------------------------------------------------
template <int C, int K> struct BwdScanLayout {
    static constexpr int LK = K + 8, LC = C + 8, LD = 64 + 8;
    static constexpr int kQr = 0;                          // q   [C][LK]
    static constexpr int kKr = kQr + C * LK * 2;           // k   [C][LK]
    static constexpr int kDo = kKr + C * LK * 2;           // dO of the V tile [C][LD]
    static constexpr int kPT = kDo + C * LD * 2;           // P^T high, low [2][C][LC]
    static constexpr int kTT = kPT + 2 * C * LC * 2;       // T^T high, low [2][C][LC]
    static constexpr int kVec = kTT + 2 * C * LC * 2;      // b, c, beta b, beta [C]; e^gamma_last
    static constexpr int kBytes = kVec + (4 * C + 4) * 4;
    static_assert(kBytes <= kLdsBytesMax, "LDS budget");
};

// Transposed fragments of a row-major bf16 block S [k][m] in LDS (pitch ld,
// in elements), read with ds_read_b64_tr_b16 (the f16 helpers move 16-bit
// values and serve bf16 bits alike): lane (g, i) gets S[k0 + 8g + e][m0 + i]
// (standard k slots), or S[k0 + 4g + e][m0 + i] and S[k0 + 16 + 4g + e][m0 + i]
// (split k slots), e = 0 ..
__device__ __forceinline__ bf16x8 lds_frag_T(const uint16_t *S, int ld, int m0, int k0) {
    return __builtin_bit_cast(bf16x8, frag_T((const _Float16 *)S, ld, m0, k0));
}
__device__ __forceinline__ bf16x8 lds_frag_T_split(const uint16_t *S, int ld, int m0, int k0) {
    return __builtin_bit_cast(bf16x8, fragAT_split((const _Float16 *)S, ld, m0, k0));
}

// One chunk's q, k (C x K), dO tile (C x 64) and slot (the four planes and
// the row factors) as 16-byte pieces, row-major over the workgroup (piece j
// of a thread covers row (tid + 256 j) / (width / 8), columns
// 8 ((tid + 256 j) % (width / 8)) .. +7).  Rows at or past T read as zero.
template <int C, int K> struct BwdChunkRegs {
    static constexpr int NQK = C * K / 8 / 256;
    static constexpr int NDO = C * 64 / 8 / 256;
    static constexpr int NPL = 4 * C * C / 8 / 256;       // plane pieces
    static constexpr int NVP = (4 * C + 4) / 4;           // vector pieces (threads < NVP)
    static_assert(NQK >= 1 && NDO >= 1 && NPL >= 1 && NVP <= 256, "tile too small");
    u32x4 q[NQK], k[NQK], d[NDO], pl[NPL], vec;
};

template <int C, int K>
__device__ __forceinline__ void bwd_load_chunk(BwdChunkRegs<C, K> &r, rsrc_t rq, rsrc_t rk, rsrc_t rdo,
                                               rsrc_t rsl, int t0, uint32_t rsK, uint32_t rsV, int vt) {
    typedef BwdChunkRegs<C, K> R;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < R::NQK; ++j) {
        const int pc = tid + 256 * j, row = pc / (K / 8), c8 = pc % (K / 8);
        const uint32_t off = (row * rsK + 8 * c8) * 2;
        r.q[j] = bload128(rq, off, t0 * rsK * 2);
        r.k[j] = bload128(rk, off, t0 * rsK * 2);
    }
#pragma unroll
    for (int j = 0; j < R::NDO; ++j) {
        const int pc = tid + 256 * j, row = pc / 8, c8 = pc % 8;
        r.d[j] = bload128(rdo, (row * rsV + 64 * vt + 8 * c8) * 2, t0 * rsV * 2);
    }
#pragma unroll
    for (int j = 0; j < R::NPL; ++j) r.pl[j] = bload128(rsl, (tid + 256 * j) * 16, 0);
    r.vec = bload128(rsl, BwdSlot<C>::kVec + (tid < R::NVP ? tid : 0) * 16, 0);
}

// The state's gradient, backwards over the chunks: one workgroup per (batch,
// head, 64-wide V tile); wave w owns value columns 16 w .. 16 w + 15 of the
// tile, so the chain (dh' -> dD -> dR -> dh) is wave-local.  Per chunk:
//   phase L  the chunk's q, k, dO tile and its slot (P^T, T^T, the row
//            factors) into LDS; the previous chunk's loads issued
//   phase 4  off the chain: P^T dO and (diag(b) Q)^T dO for the wave's columns
//   phase 5  the chain; stores dh' (the chunk-end gradient), dR and dv
// Rows past T load as zero: an identity step whose outputs the buffer ranges
// drop.
template <int C, int K>
__global__ __launch_bounds__(256, 1) void bwd_dh_kernel(BwdParams p) {
    typedef BwdScanLayout<C, K> L;
    typedef BwdChunkRegs<C, K> CR;
    constexpr int LK = L::LK, LC = L::LC, LD = L::LD;
    constexpr int NB = C / 16, NS = C / 32, KT16 = K / 16, KS = K / 32;
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    uint16_t *Qr = (uint16_t *)(smem + L::kQr), *Kr = (uint16_t *)(smem + L::kKr);
    uint16_t *Do = (uint16_t *)(smem + L::kDo);
    uint16_t *PT = (uint16_t *)(smem + L::kPT), *TT = (uint16_t *)(smem + L::kTT);
    float *bv = (float *)(smem + L::kVec), *cv = bv + C, *bbv = cv + C, *glp = bbv + 2 * C;

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
    const rsrc_t rdR = make_rsrc(p.dR + row0 * V, (uint32_t)T * rsV * 4);
    const int col = 64 * vt + 16 * wv;                       // the wave's first value column
    // this lane's (row 4g + 2 (n & 1), column n & ~1) of a 16 x 16 tile
    const uint32_t pr_row = 4 * g + 2 * (n & 1), pr_col = col + (n & ~1);
    auto slot_rsrc = [&](int c) {
        return make_rsrc((const char *)p.prep + (((int64_t)b * NT + c) * H + h) * BwdSlot<C>::kBytes,
                         (uint32_t)BwdSlot<C>::kBytes);
    };

    // the state's gradient at the end of the last chunk: dhT or zero
    float4v dh[KT16];
    if (p.dhT) {
        // (one branch, then every load in flight together)
        const float *src = p.dhT + ((int64_t)b * H + h) * K * V + col + n;
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dh[kt][e] = src[(16 * kt + 4 * g + e) * V];
    } else {
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) dh[kt] = float4v{0, 0, 0, 0};
    }

    // a chunk's dh' and dR are stored as soon as the chain has them, before
    // the state update and a whole chunk ahead of the next chunk's loads: the
    // wait counter covers loads and stores in issue order, so the waits for
    // those loads then find these stores long done.  (Stored one chunk late,
    // after the next chunk's loads, the loop-head waits covered them instead:
    // 2 ms more over 1024 chunks of 64 heads.)
    float4v dhs[KT16], rrs[NB];
    auto store_stash = [&](int cc) {
        float *he = p.dhe + (((int64_t)b * NT + cc) * H + h) * K * V;
        const rsrc_t rhe = make_rsrc(he, (uint32_t)(K * V * 4));
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt)
            store_acc_pairs<float>(dhs[kt], rhe, (pr_row * V + pr_col) * 4, V * 4, 16 * kt * V * 4);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            store_acc_pairs<float>(rrs[i], rdR, (pr_row * rsV + pr_col) * 4, rsV * 4, (cc * C + 16 * i) * rsV * 4);
    };

    CR cr;
    if (NT > 0) bwd_load_chunk<C, K>(cr, rq, rk, rdo, slot_rsrc(NT - 1), (NT - 1) * C, rsK, rsV, vt);
#pragma unroll 1
    for (int c = NT - 1; c >= 0; --c) {
        const int t0 = c * C;
        bwd_barrier();
        // phase L
#pragma unroll
        for (int j = 0; j < CR::NQK; ++j) {
            const int pc = tid + 256 * j, row = pc / (K / 8), c8 = pc % (K / 8);
            *(u32x4 *)(Qr + row * LK + 8 * c8) = cr.q[j];
            *(u32x4 *)(Kr + row * LK + 8 * c8) = cr.k[j];
        }
#pragma unroll
        for (int j = 0; j < CR::NDO; ++j) {
            const int pc = tid + 256 * j, row = pc / 8, c8 = pc % 8;
            *(u32x4 *)(Do + row * LD + 8 * c8) = cr.d[j];
        }
#pragma unroll
        for (int j = 0; j < CR::NPL; ++j) {
            const int pc = tid + 256 * j, pl = pc / (C * C / 8), rem = pc % (C * C / 8);
            const int row = rem / (C / 8), c8 = rem % (C / 8);
            *(u32x4 *)(PT + pl * C * LC + row * LC + 8 * c8) = cr.pl[j];   // PT, TT planes are adjacent
        }
        if (tid < CR::NVP) *(u32x4 *)(bv + 4 * tid) = cr.vec;
        if (c > 0) bwd_load_chunk<C, K>(cr, rq, rk, rdo, slot_rsrc(c - 1), t0 - C, rsK, rsV, vt);
        bwd_barrier();
        // phase 4: P^T dO (tokens x the wave's columns) and (diag(b) Q)^T dO
        // (keys x the wave's columns)
        float4v pd[NB], qd[KT16];
        {
            bf16x8 bq_h[NS], bq_l[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int s0 = 32 * st + 8 * g;
                const u32x4 raw = __builtin_bit_cast(u32x4, lds_frag_T(Do, LD, 16 * wv, 32 * st));
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
                    const bf16x8 bdo = lds_frag_T(Do, LD, 16 * wv, 32 * st);
                    mfma_bf(pd[i], lds_frag(PT, LC, 16 * i, 32 * st), bdo);
                    mfma_bf(pd[i], lds_frag(PT + C * LC, LC, 16 * i, 32 * st), bdo);
                }
            }
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt) {
                qd[kt] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const bf16x8 a = lds_frag_T(Qr, LK, 16 * kt, 32 * st);
                    mfma_bf(qd[kt], a, bq_h[st]);
                    mfma_bf(qd[kt], a, bq_l[st]);
                }
            }
        }
        // phase 5: the chain.  dh' is this chunk's end gradient.
#pragma unroll
        for (int kt = 0; kt < KT16; ++kt) dhs[kt] = dh[kt];
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
        for (int i = 0; i < NB; ++i) rrs[i] = rr[i];
        store_stash(c);
        {
            bf16x8 uh[NS], ul[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                float4v x0, x1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r0 = 32 * st + 4 * g + e, r1 = r0 + 16;
                    x0[e] = -bbv[r0] * rr[2 * st][e];
                    x1[e] = -bbv[r1] * rr[2 * st + 1][e];
                }
                acc_frag_split(x0, x1, uh[st], ul[st]);
            }
            const float gl = *glp;
#pragma unroll
            for (int kt = 0; kt < KT16; ++kt) {
                float4v acc = gl * dh[kt] + qd[kt];
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const bf16x8 a = lds_frag_T_split(Kr, LK, 16 * kt, 32 * st);
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
// bwd_grad_kernel: one workgroup per (chunk, head).  LDS holds q and k
// (row-major; transposed fragments come from ds_read_b64_tr_b16) for the
// whole chunk, and one region that the phases reuse:
//   A   dO, D, dR (bf16 parts)  -> the C x C tiles: k k^T, q k^T, dO D^T, dR D^T
//   A2  F, F^T, G + G^T (bf16 parts)                -> F K, F^T Q, (G + G^T) K
//   B   dO, dR (bf16 parts), h                       -> Z = dO h^T, Y = dR h^T
//   C   D, dh' (bf16 parts)                          -> W = D dh'^T
// Wave w owns key columns 32 w .. 32 w + 31 of dq and dk (all C rows), and
// the lower C x C tiles w, w + 4, ...  Row sums (the gate's and beta's
// gradients) go through per-wave LDS rows, added in a fixed order: the
// results do not depend on scheduling.
// ---------------------------------------------------------------------------
template <int C, int K, int V, int NW = 4> struct BwdGradLayout {
    static constexpr int LK = K + 8, LC = C + 8, LV = V + 8;
    static constexpr int kQr = 0;
    static constexpr int kKr = kQr + C * LK * 2;
    static constexpr int kX = kKr + C * LK * 2;
    static constexpr int kA_do = kX, kA_d = kA_do + C * LV * 2, kA_r = kA_d + C * LV * 2;
    static constexpr int kF = kX, kFT = kF + 2 * C * LC * 2, kGs = kFT + 2 * C * LC * 2;
    static constexpr int kB_do = kX, kB_r = kB_do + C * LV * 2, kB_h = kB_r + 2 * C * LV * 2;
    static constexpr int kC_d = kX, kC_dh = kC_d + C * LV * 2;
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int kXBytes = cmax(cmax(4 * C * LV * 2, 6 * C * LC * 2),
                                        cmax(3 * C * LV * 2 + K * LV * 2, C * LV * 2 + 2 * K * LV * 2));
    static constexpr int kVec = kX + kXBytes;   // gamma, b, c, beta [C]; pg, pb, pkw [NW][C]; hd [NW]
    static constexpr int kBytes = kVec + (4 * C + 3 * NW * C + NW) * 4;
    static_assert(kBytes <= kLdsBytesMax, "LDS budget");
};

// rows x X bf16 block of a token-major tensor (row pitch rs elements) as
// 16-byte pieces in registers, row-major over the workgroup's NTH threads
// (piece j of a thread: row (tid + NTH j) / (X / 8), columns
// 8 ((tid + NTH j) % (X / 8))).
template <int ROWS, int X, int NTH = 256> struct RowsBf {
    static constexpr int PPR = X / 8, NP = ROWS * PPR / NTH;
    static_assert(NP >= 1 && ROWS * PPR % NTH == 0, "pieces");
    u32x4 v[NP];
    __device__ void load(rsrc_t r, uint32_t rs, uint32_t soff) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = threadIdx.x + NTH * j, row = pc / PPR, c8 = pc % PPR;
            v[j] = bload128(r, (row * rs + 8 * c8) * 2, soff);
        }
    }
    template <int LD> __device__ void put(uint16_t *dst) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = threadIdx.x + NTH * j, row = pc / PPR, c8 = pc % PPR;
            *(u32x4 *)(dst + row * LD + 8 * c8) = v[j];
        }
    }
};

// rows x X fp32 block as 16-byte pieces (four values; piece j of a thread:
// row (tid + NTH j) / (X / 4), columns 4 ((tid + NTH j) % (X / 4)) .. +3),
// put into LDS as bf16 high and low planes [2][ROWS][LD].
template <int ROWS, int X, int NTH = 256> struct RowsF32 {
    static constexpr int PPR = X / 4, NP = ROWS * PPR / NTH;
    static_assert(NP >= 1 && ROWS * PPR % NTH == 0 && PPR <= 32, "pieces");
    u32x4 v[NP];
    __device__ static int row(int j) { return (threadIdx.x + NTH * j) / PPR; }
    __device__ static int c4(int j) { return (threadIdx.x + NTH * j) % PPR; }
    __device__ void load(rsrc_t r, uint32_t rs, uint32_t soff) {
#pragma unroll
        for (int j = 0; j < NP; ++j) v[j] = bload128(r, (row(j) * rs + 4 * c4(j)) * 4, soff);
    }
    template <int LD> __device__ void put_split(uint16_t *dst) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            uint16_t hh[4], ll[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bf_split(__uint_as_float(v[j][e]), hh[e], ll[e]);
            *(u32x2 *)(dst + row(j) * LD + 4 * c4(j)) = __builtin_bit_cast(u32x2, hh);
            *(u32x2 *)(dst + ROWS * LD + row(j) * LD + 4 * c4(j)) = __builtin_bit_cast(u32x2, ll);
        }
    }
};

// Dot product of four fp32 values with four bf16 values (8 bytes).
__device__ __forceinline__ float dot4_bf(const u32x4 &x, const u32x2 &w) {
    return __uint_as_float(x[0]) * __uint_as_float(w[0] << 16) +
           __uint_as_float(x[1]) * __uint_as_float(w[0] & 0xffff0000u) +
           __uint_as_float(x[2]) * __uint_as_float(w[1] << 16) +
           __uint_as_float(x[3]) * __uint_as_float(w[1] & 0xffff0000u);
}

template <int CTRL> __device__ __forceinline__ float dpp_t(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a row (the columns of an accumulator tile), on
// DPP: quad swaps, then the half-row and row mirrors; every lane gets the
// sum, in an order that does not depend on scheduling.
__device__ __forceinline__ float sum16(float x) {
    x += dpp_t<0xB1>(x);
    x += dpp_t<0x4E>(x);
    x += dpp_t<0x141>(x);
    x += dpp_t<0x140>(x);
    return x;
}


// Store four consecutive fp32 values of a row (16 bytes at byte offset off,
// a multiple of 32 for the even lane of a lane pair, the odd lane's piece
// following it) as 8-byte stores: lanes l and l ^ 1 swap halves, so that
// each lane's two stores lie 16 bytes apart.
__device__ __forceinline__ void store_row4_pairs(const float4v &x, rsrc_t r, uint32_t off_even, bool odd) {
    const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
    const float r0 = dpp_t<0xB1>(s0), r1 = dpp_t<0xB1>(s1);
    const u32x2 a = odd ? u32x2{__float_as_uint(r0), __float_as_uint(r1)} : u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])};
    const u32x2 b = odd ? u32x2{__float_as_uint(x[2]), __float_as_uint(x[3])} : u32x2{__float_as_uint(r0), __float_as_uint(r1)};
    __builtin_amdgcn_raw_buffer_store_b64(a, r, off_even + (odd ? 8 : 0), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(b, r, off_even + (odd ? 24 : 16), 0, 0);
}

// NW = 4 or 8 waves.  With eight (two per SIMD, for the larger tiles) the
// key tiles are shared out as with four and each wave takes half of the
// 16-row blocks: wave w has key group w % 4 and row half w / 4.
template <int C, int K, int V, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_grad_kernel(BwdParams p) {
    typedef BwdGradLayout<C, K, V, NW> L;
    constexpr int NTH = 64 * NW, NRH = NW / 4;
    constexpr int LK = L::LK, LC = L::LC, LV = L::LV;
    constexpr int NB = C / 16, NS = C / 32, KS = K / 32, VS = V / 32, NLT = NB * (NB + 1) / 2;
    constexpr int MT = (NLT + NW - 1) / NW;     // lower C x C tiles per wave (at most)
    constexpr int CT = K / 64;                  // 16-column key tiles per wave
    constexpr int NBW = NB / NRH;               // 16-row blocks per wave
    static_assert(K % 64 == 0, "key tiles");
    static_assert((NW == 4 || NW == 8) && NB % NRH == 0, "waves");
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    uint16_t *Qr = (uint16_t *)(smem + L::kQr), *Kr = (uint16_t *)(smem + L::kKr);
    float *gam = (float *)(smem + L::kVec), *bv = gam + C, *cv = bv + C, *betv = cv + C;
    float *pg = betv + C, *pb = pg + NW * C, *pkw = pb + NW * C, *hd = pkw + NW * C;

    const int tid = threadIdx.x, wv = wave_id(), l = lane_id(), g = l >> 4, n = l & 15;
    const int kgrp = wv % 4, rhalf = wv / 4;
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

    // q, k into LDS; dO, D, dR and v into registers (kept until their
    // phases); g, beta; per-row sums cleared
    typedef RowsF32<C, V, NTH> RV;
    RowsBf<C, K, NTH> r_q, r_k;
    r_q.load(rq, rsK, t0 * rsK * 2);
    r_k.load(rk, rsK, t0 * rsK * 2);
    RowsBf<C, V, NTH> r_do, r_D;
    RV r_dR;
    r_do.load(rdo, rsV, t0 * rsV * 2);
    r_D.load(rD, rsV, t0 * rsV * 2);
    r_dR.load(rdR, rsV, t0 * rsV * 4);
    u32x2 r_v[RV::NP];
#pragma unroll
    for (int j = 0; j < RV::NP; ++j)
        r_v[j] = __builtin_amdgcn_raw_buffer_load_b64(rv, (RV::row(j) * rsV + 4 * RV::c4(j)) * 2, t0 * rsV * 2, 0);
    {
        r_q.template put<LK>(Qr);
        r_k.template put<LK>(Kr);
        for (int i = tid; i < 3 * NW * C + NW; i += NTH) pg[i] = 0.f;
        uint16_t *X = (uint16_t *)(smem + L::kX);
        r_do.template put<LV>(X + (L::kA_do - L::kX) / 2);
        r_D.template put<LV>(X + (L::kA_d - L::kX) / 2);
        r_dR.template put_split<LV>(X + (L::kA_r - L::kX) / 2);
    }
    // phase B's h, in flight through phase A
    RowsBf<K, V, NTH> r_h;
    r_h.load(rh, V, 0);
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
    bwd_barrier();

    // phase A: lower C x C tiles of this wave
    float4v Fv[MT], Gv[MT];
    {
        const uint16_t *Do = (const uint16_t *)(smem + L::kA_do), *Dm = (const uint16_t *)(smem + L::kA_d);
        const uint16_t *Rh = (const uint16_t *)(smem + L::kA_r), *Rl = Rh + C * LV;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int t = wv + NW * m;
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
    bwd_barrier();
    // phase A2: F, F^T, G + G^T as bf16 parts
    uint16_t *Fp = (uint16_t *)(smem + L::kF), *FTp = (uint16_t *)(smem + L::kFT), *Gp = (uint16_t *)(smem + L::kGs);
    for (int i = tid; i < 6 * C * LC / 8; i += NTH) ((u32x4 *)Fp)[i] = u32x4{0u, 0u, 0u, 0u};
    bwd_barrier();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int t = wv + NW * m;
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
    bwd_barrier();
    // phase A3: dq = F K, dk = F^T Q + (G + G^T) K for this wave's key
    // columns and row blocks
    float4v dq[NBW][CT], dk[NBW][CT];
#pragma unroll
    for (int ib = 0; ib < NBW; ++ib)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int i = NBW * rhalf + ib, kc = 16 * (CT * kgrp + ct);
            float4v aq = {0, 0, 0, 0}, ak = {0, 0, 0, 0};
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const bf16x8 kb = lds_frag_T(Kr, LK, kc, 32 * st);
                if (32 * st <= 16 * i + 15) {        // F is zero right of its diagonal
                    mfma_bf(aq, lds_frag(Fp, LC, 16 * i, 32 * st), kb);
                    mfma_bf(aq, lds_frag(Fp + C * LC, LC, 16 * i, 32 * st), kb);
                }
                if (32 * st + 31 >= 16 * i) {        // F^T is zero left of its diagonal
                    const bf16x8 qb = lds_frag_T(Qr, LK, kc, 32 * st);
                    mfma_bf(ak, lds_frag(FTp, LC, 16 * i, 32 * st), qb);
                    mfma_bf(ak, lds_frag(FTp + C * LC, LC, 16 * i, 32 * st), qb);
                }
                mfma_bf(ak, lds_frag(Gp, LC, 16 * i, 32 * st), kb);
                mfma_bf(ak, lds_frag(Gp + C * LC, LC, 16 * i, 32 * st), kb);
            }
            dq[ib][ct] = aq;
            dk[ib][ct] = ak;
        }
    bwd_barrier();
    // phase B: Z = dO h^T, Y = dR h^T.  Its operands come from registers;
    // v . dR goes into beta's row sums (a row's pieces are consecutive lanes)
    // and dv = beta dR out; phase C's operands are issued.
    RowsF32<K, V, NTH> r_dh;
    {
        typedef RV RF;
        uint16_t *X = (uint16_t *)(smem + L::kX);
        r_do.template put<LV>(X + (L::kB_do - L::kX) / 2);
        r_dR.template put_split<LV>(X + (L::kB_r - L::kX) / 2);
        r_h.template put<LV>(X + (L::kB_h - L::kX) / 2);
        const rsrc_t rdv = make_rsrc(p.dv + row0 * V, (uint32_t)T * rsV * 4);
#pragma unroll
        for (int j = 0; j < RF::NP; ++j) {
            const int row = RF::row(j), c4 = RF::c4(j);
            float d = sum16(dot4_bf(r_dR.v[j], r_v[j]));
            if (RF::PPR == 32) d += __shfl_xor(d, 16);
            if (c4 == 0) pb[wv * C + row] += d;
            const float bt = betv[row];
            const float4v x = {bt * __uint_as_float(r_dR.v[j][0]), bt * __uint_as_float(r_dR.v[j][1]),
                               bt * __uint_as_float(r_dR.v[j][2]), bt * __uint_as_float(r_dR.v[j][3])};
            store_row4_pairs(x, rdv, ((t0 + row) * rsV + 4 * (c4 & ~1)) * 4, c4 & 1);
        }
        r_dh.load(rdh, V, 0);
    }
    bwd_barrier();
    {
        const uint16_t *Do = (const uint16_t *)(smem + L::kB_do), *Hm = (const uint16_t *)(smem + L::kB_h);
        const uint16_t *Rh = (const uint16_t *)(smem + L::kB_r), *Rl = Rh + C * LV;
#pragma unroll
        for (int ib = 0; ib < NBW; ++ib) {
            const int i = NBW * rhalf + ib;
            float qz[4] = {0, 0, 0, 0}, ky[4] = {0, 0, 0, 0};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int kc = 16 * (CT * kgrp + ct);
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
                    dq[ib][ct][e] += bv[R] * z[e];
                    dk[ib][ct][e] -= betv[R] * bv[R] * y[e];
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
    bwd_barrier();
    // phase C: <h, dh'> from phase B's state tile, still in LDS; then
    // W = D dh'^T over the operands that replace it
    {
        typedef RowsF32<K, V, NTH> RK;
        const uint16_t *Hm = (const uint16_t *)(smem + L::kB_h);
        float hdp = 0.f;
#pragma unroll
        for (int j = 0; j < RK::NP; ++j)
            hdp += dot4_bf(r_dh.v[j], *(const u32x2 *)(Hm + RK::row(j) * LV + 4 * RK::c4(j)));
        hdp = sum16(hdp);
        hdp += __shfl_xor(hdp, 16);
        hdp += __shfl_xor(hdp, 32);
        if (l == 0) hd[wv] = hdp;
    }
    bwd_barrier();
    {
        uint16_t *X = (uint16_t *)(smem + L::kX);
        r_D.template put<LV>(X + (L::kC_d - L::kX) / 2);
        r_dh.template put_split<LV>(X + (L::kC_dh - L::kX) / 2);
    }
    bwd_barrier();
    {
        const uint16_t *Dm = (const uint16_t *)(smem + L::kC_d);
        const uint16_t *Hh = (const uint16_t *)(smem + L::kC_dh), *Hl = Hh + K * LV;
#pragma unroll
        for (int ib = 0; ib < NBW; ++ib) {
            const int i = NBW * rhalf + ib;
            float kw[4] = {0, 0, 0, 0};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int kc = 16 * (CT * kgrp + ct);
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
                    dk[ib][ct][e] += cv[R] * w[e];
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
        for (int ib = 0; ib < NBW; ++ib)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const uint32_t voff = (pr_row * rsK + 16 * (CT * kgrp + ct) + (n & ~1)) * 4;
                const uint32_t soff = (t0 + 16 * (NBW * rhalf + ib)) * rsK * 4;
                store_acc_pairs<float>(dq[ib][ct], rdq, voff, rsK * 4, soff);
                store_acc_pairs<float>(dk[ib][ct], rdk, voff, rsK * 4, soff);
            }
    }
    bwd_barrier();
    // the gate's and beta's gradients: per-row sums in a fixed order, the
    // last row's extra terms, then the reverse cumsum within the chunk
    if (wv == 0) {
        float dgam = 0.f, db = 0.f, kw = 0.f;
        if (l < C) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
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
        float hds = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) hds += hd[w];
        if (l == C - 1) dgam += tot + gl * hds;
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
