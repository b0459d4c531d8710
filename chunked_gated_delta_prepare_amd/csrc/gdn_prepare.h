// gdn_prepare kernel: per-chunk WY factors, one workgroup per (b, h, chunk).
//
// Steps of the TileOPs gated deltanet fused prepare (page "Reuse P as beta
// tiles in gated deltanet fused prepare"): build A_g = strictly lower
// beta * (k k^T * decay), invert I + A_g, then w = inv * (k * beta) and
// u = inv * (v * beta), stored per chunk into [B,T,H,D] slices.  Here the k
// rows of w also carry exp(gcum), which lets the scan use the chunk-start
// state directly.
//
// LDS plan.  The page's lesson is that buffers with disjoint lifetimes must
// share storage or the kernel stops fitting; on gfx950 the budget is 160 KiB
// per CU, and the fp32 gate rows (per-key gate) share one region with the
// Gram/inverse pair, which only comes alive after the operands are built.
// beta lives in LDS, read by every lane of the C x C stages (a value held in
// one lane's registers cannot be read by the others without a shuffle).
#pragma once

#include "gdn_chunk_io.h"
#include "gdn_inverse.h"
#include "gdn_key_gram.h"
#include "gdn_scan.h"

namespace gdn {

struct PrepParams {
    const void *k, *v;
    const float *beta, *g;
    float *w, *u, *gcum;
    int B, T, H, V;
    int nt;         // chunks per sequence
};

constexpr int kMaxVTiles = 2;   // V <= 128 in 64-wide tiles

template <int C, int K, typename IO, bool KEYGATE>
struct PrepLayout {
    typedef typename OpOf<IO>::type OpT;
    static constexpr int LDK = K + Mma<OpT>::kPad;
    static constexpr int LDC = C + Mma<OpT>::kPad;
    static constexpr int LDA = C + 4;                        // fp32 C x C pitch
    static constexpr int E = sizeof(OpT);
    static constexpr int kKs = 0;                            // [C][LDK] k (KDA: exact_key_gram's scratch)
    static constexpr int kKbT = kKs + C * LDK * E;           // [K][LDC] (beta e^g k)^T
    static constexpr int kVbT = kKbT + K * LDC * E;          // [64][LDC] (beta v)^T, one V tile
    static constexpr int kScr = kVbT + 64 * LDC * E;         // shared scratch region
    static constexpr int kA = kScr;                          // fp32 [C][LDA] A
    static constexpr int kTm = kA + C * LDA * 4;             // fp32 [C][LDA] inverse
    static constexpr int kGrows = kScr;                      // KDA: fp32 [C][K] gate rows
    static constexpr int kScrBytes = (2 * C * LDA * 4 > (KEYGATE ? C * K * 4 : 0))
                                         ? 2 * C * LDA * 4 : C * K * 4;
    static constexpr int kGam = kScr + kScrBytes;            // GDN: fp32 gcum[C]
    static constexpr int kBeta = kGam + C * 4;               // fp32 beta[C]
    // KDA: the gate scan's segment totals and segment-end gcum
    static constexpr int NSEG = kThreads * 4 / K;
    static constexpr int kSegt = kBeta + C * 4;
    static constexpr int kGend = kSegt + (KEYGATE ? NSEG * K * 4 : 0);
    static constexpr int kBytes = kGend + (KEYGATE ? NSEG * K * 4 : 0);
};

// Fragment of an fp32 A operand converted to the operand type.
template <typename OpT>
__device__ __forceinline__ typename Mma<OpT>::frag frag_from_f32(const float *p);
template <>
__device__ __forceinline__ Mma<_Float16>::frag frag_from_f32<_Float16>(const float *p) {
    const float4v a = *(const float4v *)p, b = *(const float4v *)(p + 4);
    half8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = (_Float16)a[i]; h[4 + i] = (_Float16)b[i]; }
    return h;
}
template <>
__device__ __forceinline__ Mma<float>::frag frag_from_f32<float>(const float *p) {
    return Mma<float>::load(p);
}

// acc += Tm[16 rows][0..klen) * Bt[16 rows][0..klen)^T with Tm in fp32.
template <typename OpT, int KMAX>
__device__ __forceinline__ void mma_tile_af32(float4v &acc, const float *A, int lda,
                                              const OpT *Bt, int ldb, int klen) {
    typedef Mma<OpT> M;
    const int l = lane_id();
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += 32) {
        if (k0 < klen) {
            const typename M::frag a = frag_from_f32<OpT>(A + (l & 15) * lda + k0 + 8 * (l >> 4));
            const typename M::frag b = M::load(frag_ptr(Bt, ldb, k0));
            M::mma(acc, a, b);
        }
    }
}

template <int C, int K, typename IO, bool KEYGATE>
__global__ __launch_bounds__(kThreads) void prepare_kernel(PrepParams p) {
    typedef PrepLayout<C, K, IO, KEYGATE> L;
    typedef typename L::OpT OpT;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDA = L::LDA;
    constexpr int NCB = C / 16, NKB = K / 16;
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OpT *Ks = (OpT *)(smem + L::kKs);
    OpT *KbT = (OpT *)(smem + L::kKbT);
    OpT *VbT = (OpT *)(smem + L::kVbT);
    float *Af = (float *)(smem + L::kA);
    float *Tm = (float *)(smem + L::kTm);
    float *Gr = (float *)(smem + L::kGrows);
    float *gam = (float *)(smem + L::kGam);
    float *bet = (float *)(smem + L::kBeta);
    float *segt = (float *)(smem + L::kSegt);
    float *gend = (float *)(smem + L::kGend);

    const int pair = blockIdx.x / p.nt, c = blockIdx.x % p.nt;
    const int b = pair / p.H, h = pair - b * p.H;
    const int T = p.T, H = p.H, V = p.V, nvt = V / 64;
    const int t0 = c * C, nvalid = min(C, T - t0);
    const int wv = wave_id(), tid = threadIdx.x, l = lane_id();

    const int64_t row0 = (int64_t)b * T * H + h + (int64_t)t0 * H;   // token-head row of t0
    const int64_t rsK = (int64_t)H * K, rsV = (int64_t)H * V;
    const int64_t rsG = KEYGATE ? rsK : (int64_t)H;

    // ---- S0: loads, gate cumsum, beta
    ChunkRows<IO, C, K> rk;
    rk.load((const IO *)p.k + row0 * K, rsK, nvalid);
    ChunkRows<IO, C, 64> rv[kMaxVTiles];
#pragma unroll
    for (int vt = 0; vt < kMaxVTiles; ++vt)
        if (vt < nvt) rv[vt].load((const IO *)p.v + row0 * V + 64 * vt, rsV, nvalid);
    if (tid < C) bet[tid] = tid < nvalid ? p.beta[(row0 + (int64_t)tid * H)] : 0.f;

    // KDA: the gate, k in exact_key_gram's row order; gcum out and, for the
    // operands below, into Gr
    constexpr int NRK = KEYGATE ? KeyRows<C, K>::NR : 1;
    float4v gamK[NRK], kvK[NRK];
    if constexpr (KEYGATE) {
        const uint32_t rk32 = (uint32_t)rsK;
        const rsrc_t rgs = make_rsrc(p.g + row0 * K, (uint32_t)nvalid * rk32 * 4);
        const rsrc_t rks = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)nvalid * rk32 * sizeof(IO));
        load_key_rows<C, K, IO>(rgs, rks, rks, rk32, 0, segt, gend, gamK, kvK, kvK);
        const int sg = tid / (K / 4), kc = 4 * (tid % (K / 4));
        // gcum out through a range-clamped resource (rows past nvalid fall
        // outside the range and are dropped).  A lane pair holds 8 adjacent
        // columns of one row; it swaps halves so that each lane issues two
        // 8-byte stores 16 bytes apart, which the compiler cannot fuse into
        // one 16-byte store.
        const rsrc_t rgo = make_rsrc(p.gcum + row0 * K, (uint32_t)nvalid * rk32 * 4);
        const bool odd = tid & 1;
#pragma unroll
        for (int i = 0; i < NRK; ++i) {
            const int r = sg * NRK + i;
            *(float4v *)(Gr + r * K + kc) = gamK[i];
            const float s0 = odd ? gamK[i][0] : gamK[i][2], s1 = odd ? gamK[i][1] : gamK[i][3];
            const uint32_t r0 = __builtin_amdgcn_update_dpp(0, __float_as_uint(s0), 0xB1, 0xf, 0xf, false);
            const uint32_t r1 = __builtin_amdgcn_update_dpp(0, __float_as_uint(s1), 0xB1, 0xf, 0xf, false);
            const uint32_t off = ((uint32_t)r * rk32 + (uint32_t)kc) * 4;
            const u32x2 a = odd ? u32x2{r0, r1} : u32x2{__float_as_uint(gamK[i][0]), __float_as_uint(gamK[i][1])};
            const u32x2 b = odd ? u32x2{__float_as_uint(gamK[i][2]), __float_as_uint(gamK[i][3])} : u32x2{r0, r1};
            __builtin_amdgcn_raw_buffer_store_b64(a, rgo, odd ? off - 8 : off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(b, rgo, odd ? off + 8 : off + 16, 0, 0);
        }
    } else {
        if (wv == 0) {
            float x = (l < nvalid) ? p.g[row0 + (int64_t)l * H] : 0.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x, d);
                if (l >= d) x += y;
            }
            if (l < C) {
                gam[l] = x;
                if (l < nvalid) p.gcum[row0 + (int64_t)l * H] = x;
            }
        }
    }
    __syncthreads();

    // ---- S1: operands.  Ks (the scalar gate), KbT = (beta e^gcum k)^T
    {
#pragma unroll
        for (int j = 0; j < ChunkRows<IO, C, K>::kVec; ++j) {
            const int row = ChunkRows<IO, C, K>::row(j), col = ChunkRows<IO, C, K>::col(j);
            const bool ok = row < nvalid;
            float x[8], kb[8];
            rk.get(j, x);
            const float br = bet[row];
            if constexpr (KEYGATE) {
                // (A comes from exact_key_gram below)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    kb[e] = ok ? br * x[e] * fast_exp(Gr[row * K + col + e]) : 0.f;
            } else {
                const float sc = br * fast_exp(gam[row]);
#pragma unroll
                for (int e = 0; e < 8; ++e) kb[e] = x[e] * sc;
                put8(Ks + row * LDK + col, x);
            }
            put8_col(KbT + col * LDC + row, LDC, kb);
        }
    }
    __syncthreads();   // Gr (KDA gate rows) is dead from here: the region is A / Tm

    // ---- S2: A = strictly lower beta * (k k^T * decay); clear Tm
    if constexpr (KEYGATE)
        exact_key_gram<C, K, OpT, true, false>(gamK, kvK, kvK, gend, bet, Ks, Ks, Af, Af);
    for (int i = tid; i < C * LDA; i += kThreads) Tm[i] = 0.f;
    constexpr int NP = KEYGATE ? 0 : NCB * (NCB + 1) / 2;
#pragma unroll
    for (int idx = 0; idx < NP; ++idx) {
        if (idx % kWaves != wv) continue;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= idx) ++I;
        const int J = idx - I * (I + 1) / 2;                 // J <= I
        float4v acc = {0, 0, 0, 0};
        mma_tile<OpT, K>(acc, Ks + 16 * I * LDK, LDK, Ks + 16 * J * LDK, LDK);
        const int cp = 16 * J + acc_col();                  // column s
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int cr = 16 * I + acc_row(r);              // row r
            float val = acc[r] * bet[cr];
            if constexpr (!KEYGATE) val *= fast_exp(gam[cr] - gam[cp]);
            Af[cr * LDA + cp] = cp < cr ? val : 0.f;
        }
    }
    __syncthreads();

    // ---- S3: Tm = (I + A)^-1
    tri_inverse<C, LDA>(Af, Tm);

    // ---- S4: w = Tm (beta e^gcum k) ; u = Tm (beta v)
    {
        constexpr int NT = NCB * NKB;
        float *wout = p.w + row0 * K;
#pragma unroll
        for (int t = wv; t < NT; t += kWaves) {
            const int cb = t / NKB, kbi = t % NKB;
            float4v acc = {0, 0, 0, 0};
            const int klen = 32 * ((16 * (cb + 1) + 31) / 32);
            mma_tile_af32<OpT, C>(acc, Tm + 16 * cb * LDA, LDA, KbT + 16 * kbi * LDC, LDC, klen);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cr = 16 * cb + acc_row(r);
                if (cr < nvalid) wout[cr * rsK + 16 * kbi + acc_col()] = acc[r];
            }
        }
    }
    float *uout = p.u + row0 * V;
#pragma unroll
    for (int vt = 0; vt < kMaxVTiles; ++vt) {
        if (vt >= nvt) break;
#pragma unroll
        for (int j = 0; j < ChunkRows<IO, C, 64>::kVec; ++j) {
            const int row = ChunkRows<IO, C, 64>::row(j), col = ChunkRows<IO, C, 64>::col(j);
            float x[8];
            rv[vt].get(j, x);
            const float br = bet[row];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= br;
            put8_col(VbT + col * LDC + row, LDC, x);
        }
        __syncthreads();
        constexpr int NT = NCB * 4;
#pragma unroll
        for (int t = wv; t < NT; t += kWaves) {
            const int cb = t / 4, vb = t % 4;
            float4v acc = {0, 0, 0, 0};
            const int klen = 32 * ((16 * (cb + 1) + 31) / 32);
            mma_tile_af32<OpT, C>(acc, Tm + 16 * cb * LDA, LDA, VbT + 16 * vb * LDC, LDC, klen);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cr = 16 * cb + acc_row(r);
                if (cr < nvalid) uout[cr * rsV + 64 * vt + 16 * vb + acc_col()] = acc[r];
            }
        }
        __syncthreads();
    }
}

}  // namespace gdn
