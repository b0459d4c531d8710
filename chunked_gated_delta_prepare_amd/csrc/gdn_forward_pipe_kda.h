// gdn_forward for the per-key gate (Kimi-Delta-Attention), pipelined over
// chunks like forward_pipe_kernel (gdn_forward_pipe.h), bf16 io.
//
// The per-chunk algebra is the four-wave kernel's KDA form (gdn_forward.h):
// the decays move into the operands around the chunk's middle row gm,
//     q~ = q e^(gcum - gcum_gm),  k~ = k e^(gcum - gcum_gm),
//     k^ = k e^(gcum_gm - gcum)                      (per key column),
// so that A = strict_lower(diag(beta) k~ k^^T), P = tril_incl(q~ k^^T), and
// the re-scan of the kernel-fun KDA re-scan page becomes
//     X = k~ (e^gcum_gm h),  Y = q~ (e^gcum_gm h),  R' = v - X,
//     v' = (I + A)^-1 diag(beta) R'   (by blocks of 16 tokens, as there),
//     o = Y + P v',  h <- e^gl h + e^(gl - gcum_gm) (k^^T v')   (row-wise).
// The schedule is forward_pipe_kernel's: chain waves 0..3 run the re-scan of
// chunk c with h in MFMA accumulators while prepare waves 4..7 build chunk
// c+1.  What the prepare adds for the per-key gate: the chunk-local cumsum of
// the C x K gate (each thread holds four key columns of C/NSEG rows in
// registers; the segment totals meet in LDS), the per-key factors e^gcum_gm,
// e^gl and e^(gl - gcum_gm) for the chain, and the third operand tile k^.
// The prepare waves also load beta themselves, so chain wave 0 has no gate
// work and the prepare waits for nothing but its own barriers.
#pragma once

#include "gdn_forward_pipe.h"

namespace gdn {

template <int C, int K>
struct PipeKdaLayout {
    static constexpr int NB = C / 16;
    static constexpr int NASP = NB == 4 ? 4 : 0;         // A blocks (2,0) (2,1) (3,0) (3,1)
    static constexpr int kQK = C * K * 2;                // one fp16 C x K tile
    static constexpr int kCC = C * C * 2;                // one fp16 C x C tile
    static constexpr int kVT = C * 64 * 2;               // one bf16 v tile
    static constexpr int kQ = 0;                         // [2] q~
    static constexpr int kK = kQ + 2 * kQK;              // [2] k~
    static constexpr int kH = kK + 2 * kQK;              // [2] k^
    static constexpr int kTmb = kH + 2 * kQK;            // [2] solve blocks (Tb, Mn)
    static constexpr int kP = kTmb + 2 * kCC;            // [2] P
    static constexpr int kV = kP + 2 * kCC;              // [2] raw v tiles
    static constexpr int kAsp = kV + 2 * kVT;            // [NASP][64][8] split A blocks
    static constexpr int kTr = kAsp + NASP * 1024;       // [NB][64][4] fp16 T_bb
    // per-key factors per slot: e^gcum_gm, e^gl, e^(gl - gcum_gm)
    static constexpr int kKf = kTr + NB * 512;           // [2][3K] fp32
    static constexpr int kBet = kKf + 2 * 3 * K * 4;     // [C] beta of the prepared chunk
    // gate cumsum segments: a prepare thread holds 4 key columns of NR rows
    static constexpr int NSEG = 256 * 4 / K;
    static constexpr int NR = C / NSEG;
    static constexpr int kSeg = kBet + C * 4;            // [NSEG][K] segment totals
    static constexpr int kSync = kSeg + NSEG * K * 4;
    static constexpr int kBytes = kSync + 16;
    static_assert(NR >= 1 && NSEG * NR == C, "gate segments tile the chunk");
    static_assert((C / 2) % NR == 0, "the middle row ends a segment");
};

__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

// DQ: the backward's re-scan (the KDA re-scan page's kernel): the chunk-start
// states and v' as with ST, plus dq's chunk-start-state term
// DQ = dO h_c^T (raw) accumulated into p.dq, and no o.  Chunk 64 only: the
// state is staged in the q~ and k~ tiles of the slot the chain has just
// finished with, which hold K x 64 bf16 at C = 64.
template <int C, int K, typename OT, bool ST = false, bool VL = false, bool DQ = false>
__global__ __launch_bounds__(kPipeThreads, 1) void forward_pipe_kda_kernel(FwdParams p) {
    typedef PipeKdaLayout<C, K> L;
    typedef Mma<_Float16> M;
    typedef bf16_t IO;
    constexpr int NB = C / 16, NKB = K / 16;
    constexpr int SIO = 2, SO = sizeof(OT);
    constexpr int NSEG = L::NSEG, NR = L::NR;
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");
    static_assert(NB == 2 || NB == 4, "chunk 32 or 64");
    static_assert(K == 64 || K == 128, "key dim 64 or 128");
    static_assert(!DQ || (ST && C * K * 2 >= K * 64 * 2), "the re-scan saves states; chunk 64");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    _Float16 *Qb = (_Float16 *)(smem + L::kQ);
    _Float16 *Kb = (_Float16 *)(smem + L::kK);
    _Float16 *Hb = (_Float16 *)(smem + L::kH);
    _Float16 *Tmbb = (_Float16 *)(smem + L::kTmb);
    _Float16 *Pb = (_Float16 *)(smem + L::kP);
    uint16_t *Vb = (uint16_t *)(smem + L::kV);
    _Float16 *Asp = (_Float16 *)(smem + L::kAsp);
    _Float16 *Tr = (_Float16 *)(smem + L::kTr);
    float *Kf = (float *)(smem + L::kKf);
    float *bet = (float *)(smem + L::kBet);
    float *segt = (float *)(smem + L::kSeg);
    unsigned *sync_ctr = (unsigned *)(smem + L::kSync);

    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    int pair, vt;
    map_block(blockIdx.x, p.nvt, p.swizzle, pair, vt);
    const int b = pair / p.H, h = pair - b * p.H;
    const StreamRange sr = stream_range<VL>(p, b, h);
    const int T = sr.T, H = p.H, V = p.V;
    const int nt = (T + C - 1) / C;
    const int64_t row0 = sr.row0;
    const uint32_t rsK = (uint32_t)(H * K), rsV = (uint32_t)(H * V);
    WaitCtl wc{p.wait_count, p.wait_limit, p.wait_bias, 0u};

    // the operand tiles above the diagonal are read but stay zero
    for (int i = tid; i < 2 * C * C; i += kPipeThreads) {
        Tmbb[i] = (_Float16)0.f;
        Pb[i] = (_Float16)0.f;
    }
    if (tid == 0) {
        sync_ctr[0] = 0u;                   // prepare waves' barrier
        sync_ctr[1] = 0u;
        sync_ctr[2] = 0u;                   // chain waves' barrier (DQ)
    }
    wg_barrier();

    if (wv < 4) {
        // =====================  chain waves  =============================
        const rsrc_t ro_ = make_rsrc((OT *)p.o + row0 * V, (uint32_t)T * rsV * SO);
        const int g4 = 4 * (l >> 4);
        const int vcol = vt * 64 + 16 * wv + acc_col();
        // o^T tiles: token (l % 16) of a 16-token block, columns 4 (l / 16) .. +3
        const uint32_t o_off = ((uint32_t)(l & 15) * rsV + vt * 64 + 16 * wv + g4) * SO;
        // saved states leave the accumulators as column pairs (store_acc_pairs)
        const rsrc_t rvn_ = make_rsrc(ST ? (OT *)p.vnew + row0 * V : nullptr, ST ? (uint32_t)T * rsV * SO : 0u);
        const uint32_t prow = (uint32_t)(g4 + 2 * (l & 1));
        const uint32_t vn_off = (prow * rsV + (vcol & ~1)) * SO;
        const uint32_t hck_off = (prow * V + (vcol & ~1)) * SO;
        float4v hacc[NKB];
        if (p.h0) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hacc[i][r] = p.h0[((int64_t)pair * K + 16 * i + g4 + r) * V + vcol];
        } else {
#pragma unroll
            for (int i = 0; i < NKB; ++i) hacc[i] = float4v{0, 0, 0, 0};
        }
        // DQ: dq[t] += h_c dO_t for the tokens of chunk n, with h_c in hacc:
        // the state goes to LDS as bf16 high and low parts ([K][64], 16-byte
        // chunks swizzled by row) in the q~ and k~ tiles of slot sl, free
        // then; each wave forms DQ for K/4 key rows over the tile's 64 value
        // columns with bf16 MFMAs (bf16 keeps any dO magnitude in range)
        const rsrc_t rdo_ = make_rsrc(DQ ? (const IO *)p.dout + row0 * V : nullptr, DQ ? (uint32_t)T * rsV * SIO : 0u);
        const uint32_t do_off = ((uint32_t)(l & 15) * rsV + vt * 64 + 8 * (l >> 4)) * SIO;
        unsigned chain_target = 0;
        auto rescan_dq = [&](int n, int sl) {
            const uint32_t t0 = (uint32_t)(n * C);
            uint16_t *Hhi = (uint16_t *)(Qb + sl * C * K), *Hlo = (uint16_t *)(Kb + sl * C * K);
            bf16x8 dof[2][NB];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    dof[s][cb] = __builtin_bit_cast(bf16x8, bload128(rdo_, do_off + 32 * s * SIO,
                                                                     (t0 + 16 * cb) * rsV * SIO));
            prep_barrier(sync_ctr + 2, chain_target, wc);        // every chain wave is past its reads
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i + g4 + r, col = 16 * wv + (l & 15);
                    const uint16_t hb = f32_to_bf16_bits(hacc[i][r]);
                    Hhi[swz<64>(row, col)] = hb;
                    Hlo[swz<64>(row, col)] = f32_to_bf16_bits(hacc[i][r] - __uint_as_float((uint32_t)hb << 16));
                }
            prep_barrier(sync_ctr + 2, chain_target, wc);
            constexpr int NKW = K / 64;                      // 16-row key tiles per wave
            float4v dq[NB][NKW];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int nt = 0; nt < NKW; ++nt) dq[cb][nt] = float4v{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8 bh[NKW], bl[NKW];
#pragma unroll
                for (int nt = 0; nt < NKW; ++nt) {
                    const int row = (K / 4) * wv + 16 * nt + (l & 15), c0 = 32 * s + 8 * (l >> 4);
                    bh[nt] = *(const bf16x8 *)(Hhi + swz<64>(row, c0));
                    bl[nt] = *(const bf16x8 *)(Hlo + swz<64>(row, c0));
                }
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                    for (int nt = 0; nt < NKW; ++nt) {
                        dq[cb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dof[s][cb], bh[nt], dq[cb][nt], 0, 0, 0);
                        dq[cb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dof[s][cb], bl[nt], dq[cb][nt], 0, 0, 0);
                    }
            }
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = (int)t0 + 16 * cb + g4 + r;
                    if (t < T) {
#pragma unroll
                        for (int nt = 0; nt < NKW; ++nt)
                            unsafeAtomicAdd(p.dq + (row0 + (int64_t)t * H) * K + (K / 4) * wv + 16 * nt + (l & 15),
                                            dq[cb][nt][r]);
                    }
                }
        };
        // chunk 0's dq term from h0, staged in slot 1 (not written before the
        // prepare of chunk 1, which starts after the next barrier)
        if constexpr (DQ)
            if (nt > 0) rescan_dq(0, 1);
        wg_barrier();                       // chunk 0 prepared

        for (int c = 0; c < nt; ++c) {
            const int slot = c & 1;
            const _Float16 *Qs = Qb + slot * C * K, *Ks = Kb + slot * C * K, *Hs = Hb + slot * C * K;
            const _Float16 *Tmb = Tmbb + slot * C * C, *Ps = Pb + slot * C * C;
            const uint16_t *Vs = Vb + slot * C * 64;
            const float *fsv = Kf + slot * 3 * K, *flv = fsv + K, *fmv = fsv + 2 * K;
            const uint32_t t0 = (uint32_t)(c * C);

            // h as B fragments over the key dimension, rows scaled by e^gcum_gm
            half8 hf[K / 32];
#pragma unroll
            for (int s = 0; s < K / 32; ++s)
                hf[s] = fragB_acc(hacc[2 * s] * *(const float4v *)(fsv + 32 * s + g4),
                                  hacc[2 * s + 1] * *(const float4v *)(fsv + 32 * s + 16 + g4), _Float16{});
            // X = k~ h', Y^T = h'^T q~^T for this wave's 16 columns
            float4v xa[NB], ya[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                xa[cb] = float4v{0, 0, 0, 0};
                ya[cb] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < K / 32; ++s) {
                    M::mma(xa[cb], frag_sw<K>(Ks, 16 * cb, 32 * s), hf[s]);
                    M::mma(ya[cb], hf[s], frag_sw<K>(Qs, 16 * cb, 32 * s));
                }
            }
            // R' = v - X (the decay is inside X)
            float4v rr[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const u32x2 w = read_T4_sw<64>(Vs, 16 * cb, 16 * wv);
                const float4v vv = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                    __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
                rr[cb] = vv - xa[cb];
            }
            // v' by blocks of 16 tokens (row block b of Tmb: [Mn_b0 .. | Tb_bb | 0])
            float4v da[NB];
            da[0] = float4v{0, 0, 0, 0};
            M::mma(da[0], frag_sw<C>(Tmb, 0, 0), fragB_acc(rr[0], rr[1], _Float16{}));
            da[1] = float4v{0, 0, 0, 0};
            M::mma(da[1], frag_sw<C>(Tmb, 16, 0), fragB_acc(da[0], rr[1], _Float16{}));
            if constexpr (NB == 4) {
                da[2] = float4v{0, 0, 0, 0};
                da[3] = float4v{0, 0, 0, 0};
                M::mma(da[2], frag_sw<C>(Tmb, 32, 32), fragB_acc(rr[2], rr[3], _Float16{}));
                const half8 d01 = fragB_acc(da[0], da[1], _Float16{});
                M::mma(da[2], frag_sw<C>(Tmb, 32, 0), d01);
                M::mma(da[3], frag_sw<C>(Tmb, 48, 0), d01);
                M::mma(da[3], frag_sw<C>(Tmb, 48, 32), fragB_acc(da[2], rr[3], _Float16{}));
            }
            // o^T = v'^T P^T + Y^T: lane (g, j) holds token 16 cb + j, value
            // columns 4g .. 4g+3 of this wave's 16
            half8 df[C / 32];
#pragma unroll
            for (int s = 0; s < C / 32; ++s) df[s] = fragB_acc(da[2 * s], da[2 * s + 1], _Float16{});
            if constexpr (!DQ) {
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    float4v oa = ya[cb];
#pragma unroll
                    for (int s = 0; s < C / 32; ++s)
                        if (32 * s < 16 * (cb + 1)) M::mma(oa, df[s], frag_sw<C>(Ps, 16 * cb, 32 * s));
                    store_o_rows<OT>(oa, ro_, o_off, rsV * SO, (t0 + 16 * cb) * rsV * SO);
                }
            }
            if constexpr (ST) {
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    store_acc_pairs<OT>(da[cb], rvn_, vn_off, rsV * SO, (t0 + 16 * cb) * rsV * SO);
                // the state at the start of this chunk, hck[b, c, h, row, vcol]
                const rsrc_t rh = make_rsrc((OT *)p.hck + (((int64_t)b * nt + c) * H + h) * K * V,
                                            (uint32_t)(K * V * SO));
#pragma unroll
                for (int i = 0; i < NKB; ++i) store_acc_pairs<OT>(hacc[i], rh, hck_off, V * SO, 16 * i * V * SO);
            }
            // h <- e^gl h + e^(gl - gcum_gm) (k^^T v'), row-wise
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                float4v acc = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < C / 32; ++s)
                    M::mma(acc, fragAT_split_p<K>(Hs, 16 * i, 32 * s), df[s]);
                hacc[i] = *(const float4v *)(flv + 16 * i + g4) * hacc[i] +
                          *(const float4v *)(fmv + 16 * i + g4) * acc;
            }
            // the next chunk's dq term from its start state (now in hacc),
            // staged in this chunk's q~ and k~ tiles: the chain is done with
            // them, and the prepare writes this slot only after the barrier
            if constexpr (DQ)
                if (c + 1 < nt) rescan_dq(c + 1, slot);
            wg_barrier();
        }
        if (p.hT) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.hT[((int64_t)pair * K + 16 * i + g4 + r) * V + vcol] = hacc[i][r];
        }
        wait_report(wc);
    } else {
        // =====================  prepare waves  ===========================
        // (unlike the scalar-gate kernel, these keep the default wave
        // priority in the plain forward, where raising it measured 2 %
        // slower, and in the re-scan, 3 % slower; with saved states the
        // chain's store work competes for the SIMDs' issue slots, and a
        // raised priority measured 7 % faster)
        const int pw = wv - 4, pt = tid - 256;
        if constexpr (ST && !DQ) __builtin_amdgcn_s_setprio(3);
        const rsrc_t rq_ = make_rsrc((const IO *)p.q + row0 * K, (uint32_t)T * rsK * SIO);
        const rsrc_t rk_ = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)T * rsK * SIO);
        const rsrc_t rv_ = make_rsrc((const IO *)p.v + row0 * V, (uint32_t)T * rsV * SIO);
        const rsrc_t rg_ = make_rsrc(p.g + row0 * K, (uint32_t)T * rsK * 4);
        const rsrc_t rb_ = make_rsrc(p.beta + row0, (uint32_t)T * (uint32_t)H * 4);

        // thread (seg, cg): rows seg NR .. +NR-1, key columns 4 cg .. 4 cg + 3
        const int cg = pt % (K / 4), seg = pt / (K / 4), kc = 4 * cg;
        const uint32_t qk_off = ((uint32_t)(seg * NR) * rsK + kc) * SIO;
        const uint32_t g_off = ((uint32_t)(seg * NR) * rsK + kc) * 4;
        int qk_lds[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) qk_lds[i] = swz<K>(seg * NR + i, pcol(kc));
        constexpr int NVV = C * 64 / 8 / 256;            // v vectors per thread
        static_assert(NVV >= 1, "tile smaller than the prepare waves");
        uint32_t vv_off[NVV];
        int vv_lds[NVV];
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int i = pt + 256 * j, row = i / 8, ch = i % 8;
            vv_off[j] = ((uint32_t)row * rsV + vt * 64 + 8 * ch) * SIO;
            vv_lds[j] = swz<64>(row, 8 * ch);
        }

        u32x2 rq[NR], rk[NR];
        float4v rg[NR];
        u32x4 rv[NVV];
        float b_pre = 0.f;
        // The loads of chunk n come in pieces, each issued as soon as the
        // registers it fills are free: the CU's memory pipeline takes about a
        // cycle per 64 bytes, and 72 KB per chunk issued at once would stall
        // the issuing waves for most of that time.
        auto load_v_beta = [&](int n) {
            const uint32_t t0 = (uint32_t)(n * C);
#pragma unroll
            for (int j = 0; j < NVV; ++j) rv[j] = bload128(rv_, vv_off[j], t0 * rsV * SIO);
            if (pt < C) b_pre = __uint_as_float(bload32(rb_, (uint32_t)pt * (uint32_t)H * 4, t0 * (uint32_t)H * 4));
        };
        auto load_row = [&](int n, int i) {
            const uint32_t t0 = (uint32_t)(n * C);
            rg[i] = __builtin_bit_cast(float4v, bload128(rg_, g_off, (t0 + i) * rsK * 4));
            rq[i] = bload64(rq_, qk_off, (t0 + i) * rsK * SIO);
            rk[i] = bload64(rk_, qk_off, (t0 + i) * rsK * SIO);
        };
        unsigned sync_target = 0;

        auto prepare = [&](int n) {
            const int slot = n & 1;
            _Float16 *Qs = Qb + slot * C * K, *Ks = Kb + slot * C * K, *Hs = Hb + slot * C * K;
            _Float16 *Tmb = Tmbb + slot * C * C, *Ps = Pb + slot * C * C;
            uint16_t *Vs = Vb + slot * C * 64;
            float *fsv = Kf + slot * 3 * K, *flv = fsv + K, *fmv = fsv + 2 * K;

            // ---- raw v, beta, and the gate cumsum of this thread's rows
#pragma unroll
            for (int j = 0; j < NVV; ++j) *(u32x4 *)(Vs + vv_lds[j]) = rv[j];
            if (pt < C) bet[pt] = b_pre;
            if (n + 1 < nt) load_v_beta(n + 1);
            float4v run = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < NR; ++i) { run += rg[i]; rg[i] = run; }
            *(float4v *)(segt + seg * K + kc) = run;
            prep_barrier(sync_ctr, sync_target, wc);
            // segment offsets in segment order; gcum at the middle row (the
            // end of segment C/2/NR - 1) and at the last row
            float4v off = {0, 0, 0, 0}, gm = {0, 0, 0, 0}, gl = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < NSEG; ++s) {
                const float4v t = *(const float4v *)(segt + s * K + kc);
                if (s < seg) off += t;
                if (s < C / 2 / NR) gm += t;
                gl += t;
            }
            if (seg == 0) {
                float4v e0, e1, e2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    e0[e] = fast_exp(gm[e]);
                    e1[e] = fast_exp(gl[e]);
                    e2[e] = fast_exp(gl[e] - gm[e]);
                }
                *(float4v *)(fsv + kc) = e0;
                *(float4v *)(flv + kc) = e1;
                *(float4v *)(fmv + kc) = e2;
            }
            // ---- operands q~, k~, k^ (fp16) of this thread's rows; the
            // exponent (gcum - gcum_gm) log2 e is one FMA per element on the
            // in-segment cumsum, with the segment's offset folded in
            const float4v dof = (off - gm) * kLog2e;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                float4v d;
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = __builtin_fmaf(rg[i][e], kLog2e, dof[e]);
                half4 hq, hk, hh;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float up = fast_exp2(d[e]), dn = fast_exp2(-d[e]);
                    const uint32_t wq = rq[i][e >> 1], wk = rk[i][e >> 1];
                    const float xq = __uint_as_float((e & 1) ? (wq & 0xffff0000u) : (wq << 16));
                    const float xk = __uint_as_float((e & 1) ? (wk & 0xffff0000u) : (wk << 16));
                    hq[e] = (_Float16)(xq * up);
                    hk[e] = (_Float16)(xk * up);
                    hh[e] = (_Float16)(xk * dn);
                }
                *(half4 *)(Qs + qk_lds[i]) = hq;
                *(half4 *)(Ks + qk_lds[i]) = hk;
                *(half4 *)(Hs + qk_lds[i]) = hh;
                if (n + 1 < nt) load_row(n + 1, i);
            }
            prep_arrive(sync_ctr, sync_target);
            // every prepare wave's operand rows (and beta) are in
            wait_counter(sync_ctr, sync_target, wc);

            // ---- Gram tiles.  A = diag(beta) k~ k^^T and P = q~ k^^T need no
            // decay factor; A tiles get beta of their rows and the strict
            // mask, P tiles the inclusive one.
            auto fac_row = [&](int I, int J, bool isA, const float4v &acc) {
                const int r = 16 * I + (l & 15), s0 = 16 * J + 4 * (l >> 4);
                const float fr = isA ? bet[r] : 1.f;
                float4v a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (isA ? s0 + e < r : s0 + e <= r) ? acc[e] * fr : 0.f;
                return a;
            };
            auto fac_col = [&](int I, int J, const float4v &acc) {      // A blocks only
                const int r0 = 16 * I + 4 * (l >> 4), s = 16 * J + (l & 15);
                const float4v fr = *(const float4v *)(bet + r0);
                float4v a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = s < r0 + e ? acc[e] * fr[e] : 0.f;
                return a;
            };
            auto put_p = [&](int I, int J, const float4v &acc) {
                const float4v a = fac_row(I, J, false, acc);
                half4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = (_Float16)a[e];
                *(half4 *)(Ps + swz<C>(16 * I + (l & 15), pcol(16 * J + 4 * (l >> 4)))) = hv;
            };
            // Two tiles at once.  mma(x, frag of rows X, frag of rows Y) forms
            // X Y^T in col layout: with k^ rows of block J first, P tiles come
            // out in row layout; A tiles (k~ rows of block I first) in col
            // layout.
            auto gram_two = [&](int I0, int J0, bool a0, int I1, int J1, bool a1, bool two, int sl0, int sl1) {
                half8 fa0[K / 32], fb0[K / 32], fa1[K / 32], fb1[K / 32];
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    fa0[k] = frag_sw<K>(Hs, 16 * J0, 32 * k);
                    fb0[k] = frag_sw<K>(a0 ? Ks : Qs, 16 * I0, 32 * k);
                    if (two) {
                        fa1[k] = frag_sw<K>(Hs, 16 * J1, 32 * k);
                        fb1[k] = frag_sw<K>(a1 ? Ks : Qs, 16 * I1, 32 * k);
                    }
                }
                float4v acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    if (a0) M::mma(acc0, fb0[k], fa0[k]); else M::mma(acc0, fa0[k], fb0[k]);
                    if (two) {
                        if (a1) M::mma(acc1, fb1[k], fa1[k]); else M::mma(acc1, fa1[k], fb1[k]);
                    }
                }
                auto put = [&](int I, int J, bool isA, int sl, const float4v &acc) {
                    if (isA)
                        *(half8 *)(Asp + sl * 512 + 8 * l) = split_hi_lo(fac_col(I, J, acc));
                    else
                        put_p(I, J, acc);
                };
                put(I0, J0, a0, sl0, acc0);
                if (two) put(I1, J1, a1, sl1, acc1);
            };
            auto put_mn = [&](int i, int j, const half8 &a_split, const half4 &t) {
                *(half4 *)(Tmb + swz<C>(16 * i + (l & 15), pcol(16 * j + 4 * (l >> 4)))) = solve_block(a_split, t);
            };
            if (pw < NB / 2) {
                // the diagonal pair (pb, pb+1): A_pb,pb, A_pb+1,pb+1 (row
                // layout, for the inverse) and A_pb+1,pb (col layout, for its
                // solve block), kept in registers
                const int pb = 2 * pw;
                half8 f0[K / 32], f1[K / 32], g0[K / 32], g1[K / 32], q0[K / 32], q1[K / 32];
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    f0[k] = frag_sw<K>(Hs, 16 * pb, 32 * k);
                    f1[k] = frag_sw<K>(Hs, 16 * (pb + 1), 32 * k);
                    g0[k] = frag_sw<K>(Ks, 16 * pb, 32 * k);
                    g1[k] = frag_sw<K>(Ks, 16 * (pb + 1), 32 * k);
                }
                if constexpr (NB == 4) {
#pragma unroll
                    for (int k = 0; k < K / 32; ++k) {
                        q0[k] = frag_sw<K>(Qs, 16 * pb, 32 * k);
                        q1[k] = frag_sw<K>(Qs, 16 * (pb + 1), 32 * k);
                    }
                }
                float4v a00 = {0, 0, 0, 0}, a11 = {0, 0, 0, 0}, a10 = {0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    M::mma(a00, f0[k], g0[k]);
                    M::mma(a11, f1[k], g1[k]);
                    M::mma(a10, g1[k], f0[k]);
                }
                const float4v ad[2] = {fac_row(pb, pb, true, a00), fac_row(pb + 1, pb + 1, true, a11)};
                const half8 a10s = split_hi_lo(fac_col(pb + 1, pb, a10));
                float4v tr[2];
                diag_inverse_mfma(ad, tr);
                if constexpr (NB == 4) {
                    // the P tiles of the same 2 x 2 block (their MFMAs fill
                    // the gaps of the inverse's dependent chain)
                    float4v p00 = {0, 0, 0, 0}, p10 = {0, 0, 0, 0}, p11 = {0, 0, 0, 0};
#pragma unroll
                    for (int k = 0; k < K / 32; ++k) {
                        M::mma(p00, f0[k], q0[k]);
                        M::mma(p10, f0[k], q1[k]);
                        M::mma(p11, f1[k], q1[k]);
                    }
                    put_p(pb, pb, p00);
                    put_p(pb + 1, pb, p10);
                    put_p(pb + 1, pb + 1, p11);
                }
                // Tb = T scaled by beta of its columns, and T itself (fp16, row
                // layout) for the other waves' solve blocks
                half4 t16[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int row = 16 * (pb + e) + (l & 15), c4 = 16 * (pb + e) + 4 * (l >> 4);
                    const float4v t = tr[e] * *(const float4v *)(bet + c4);
                    half4 hv;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        hv[q] = (_Float16)t[q];
                        t16[e][q] = (_Float16)tr[e][q];
                    }
                    *(half4 *)(Tmb + swz<C>(row, pcol(c4))) = hv;
                    *(half4 *)(Tr + (pb + e) * 256 + 4 * l) = t16[e];
                }
                put_mn(pb + 1, pb, a10s, t16[1]);
            }
            if constexpr (NB == 4) {
                // prepare wave 2 + J: the A and P tiles (2, J) and (3, J), with
                // the A tiles in slots 2 (I - 2) + J
                if (pw >= 2) {
                    const int J = pw - 2;
                    gram_two(2, J, true, 3, J, true, true, J, 2 + J);
                    gram_two(2, J, false, 3, J, false, true, 0, 0);
                }
            } else {
                // prepare waves 1..3: one P tile each
                if (pw >= 1) {
                    const int t = pw - 1, I = t == 0 ? 0 : 1, J = t == 2 ? 1 : 0;
                    gram_two(I, J, false, 0, 0, false, false, 0, 0);
                }
            }
            if constexpr (NB == 4) {
                // Mn_20, Mn_21, Mn_30, Mn_31 (prepare wave pw takes A block pw):
                // T_22 and T_33 come from wave 1, the A blocks from waves 2, 3
                prep_barrier(sync_ctr, sync_target, wc);
                const int i = 2 + (pw >> 1);
                put_mn(i, pw & 1, *(const half8 *)(Asp + pw * 512 + 8 * l), *(const half4 *)(Tr + i * 256 + 4 * l));
            }
        };

        if (nt > 0) {
            load_v_beta(0);
#pragma unroll
            for (int i = 0; i < NR; ++i) load_row(0, i);
            prepare(0);
        }
        wg_barrier();                       // chunk 0 prepared
        for (int c = 0; c < nt; ++c) {
            if (c + 1 < nt) prepare(c + 1);
            wg_barrier();
        }
        wait_report(wc);
    }
}

}  // namespace gdn
