// gdn_forward for the per-key gate (Kimi-Delta-Attention), pipelined over
// chunks like forward_pipe_kernel (gdn_forward_pipe.h), bf16 io.
//
// kda_gram_kernel (gdn_kda_gram.h) forms, for every chunk in parallel and
// with every decay factor at most 1, the chunk's triangular solve blocks, P,
// and this kernel's operands, and leaves them in a workspace slot per
// (chunk, head).  This kernel is the inter-chunk re-scan of the kernel-fun
// KDA re-scan page with every operand referenced to the chunk's ends, so
// that every factor is a decay:
//     qd = q e^gcum,  kd = k e^gcum,  kg = k e^(gl - gcum)   (per key column;
//                                                           gl: the last row)
//     X = kd h,  Y = qd h,  R' = v - X,
//     v' = (I + A)^-1 diag(beta) R'   (by blocks of 16 tokens from Tmb),
//     o = Y + P v',  h <- e^gl h + kg^T v'   (row-wise by the key vector).
// The schedule is forward_pipe_kernel's: chain waves 0..3 run the re-scan of
// chunk c with h in MFMA accumulators while prepare waves 4..7 copy chunk
// c+1's slot (the operand tiles, already in the chain's LDS layout; Tmb and
// P into that layout; e^gl) and its raw v tile into LDS, and issue the loads
// of chunk c+2.
#pragma once

#include "gdn_forward_pipe.h"
#include "gdn_kda_gram.h"

namespace gdn {

// Prepare waves of the per-key kernel: four, one per SIMD.
template <int C, int K, bool DQ>
constexpr int kda_prep_waves() { return 4; }
template <int C, int K, bool DQ>
constexpr int kda_threads() { return 256 + 64 * kda_prep_waves<C, K, DQ>(); }

template <int C, int K, int NPT = 256>
struct PipeKdaLayout {
    static constexpr int NB = C / 16;
    static constexpr int kQK = C * K * 2;                // one fp16 C x K tile
    static constexpr int kCC = C * C * 2;                // one fp16 C x C tile
    static constexpr int kVT = C * 64 * 2;               // one bf16 v tile
    static constexpr int kQ = 0;                         // [2] qd
    static constexpr int kK = kQ + 2 * kQK;              // [2] kd
    static constexpr int kH = kK + 2 * kQK;              // [2] kg
    static constexpr int kTmb = kH + 2 * kQK;            // [2] solve blocks (Tb, Mn)
    static constexpr int kP = kTmb + 2 * kCC;            // [2] P
    static constexpr int kV = kP + 2 * kCC;              // [2] raw v tiles
    static constexpr int kKf = kV + 2 * kVT;             // [2][K] e^gl per key
    static constexpr int kSync = kKf + 2 * K * 4;
    static constexpr int kBytes = kSync + 16;
    // workspace pieces per chunk: Tmb and P, 16 bytes each
    static constexpr int NWS = 2 * C * C * 2 / 16 / NPT;
    static_assert(NWS >= 1 && NWS * 16 * NPT == 2 * C * C * 2, "workspace pieces per thread");
};

__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

// The raw v tile and the workspace slot of chunk n into registers (see the
// prepare waves of forward_pipe_kda_kernel): v pieces at vv_off plus n
// times v_chunk bytes; the slot's Tmb and P pieces, operand pieces and e^gl
// at n times slot_stride.
template <int NVV, int NWS, int NOP, int NPT>
__device__ __forceinline__ void kda_slot_load(rsrc_t rv_, rsrc_t rw_, const uint32_t (&vv_off)[NVV],
                                              int pt, bool fl_thread, uint32_t v_chunk,
                                              uint32_t slot_stride, int k_ops, int k_fl, int n,
                                              u32x4 (&rv)[NVV], u32x4 (&rw)[NWS], u32x4 (&ro)[NOP],
                                              u32x4 &rf) {
    const uint32_t sv = (uint32_t)n * v_chunk, so = (uint32_t)n * slot_stride;
#pragma unroll
    for (int j = 0; j < NVV; ++j) rv[j] = bload128(rv_, vv_off[j], sv);
#pragma unroll
    for (int j = 0; j < NWS; ++j) rw[j] = bload128(rw_, (uint32_t)(16 * (pt + NPT * j)), so);
#pragma unroll
    for (int j = 0; j < NOP; ++j) ro[j] = bload128(rw_, (uint32_t)(k_ops + 16 * (pt + NPT * j)), so);
    if (fl_thread) rf = bload128(rw_, (uint32_t)(k_fl + 16 * pt), so);
}

// DQ: the backward's re-scan (the KDA re-scan page's kernel): the chunk-start
// states and v' as with ST, plus dq's chunk-start-state term
// DQ = dO h_c^T (raw) accumulated into p.dq, and no o.  At chunk 64 the
// state is staged in the q~ and k~ tiles of the slot the chain has just
// finished with, which hold K x 64 bf16 there; at chunk 32 they are too
// small and it has an LDS array of its own (32 KB at K = 128).
template <int C, int K, typename OT, bool ST = false, bool VL = false, bool DQ = false>
__global__ __launch_bounds__((kda_threads<C, K, DQ>()), 1) void forward_pipe_kda_kernel(FwdParams p) {
    constexpr int NPW = kda_prep_waves<C, K, DQ>(), NPT = 64 * NPW;
    typedef PipeKdaLayout<C, K, NPT> L;
    typedef Mma<_Float16> M;
    typedef bf16_t IO;
    constexpr int NB = C / 16, NKB = K / 16;
    constexpr int SIO = 2, SO = sizeof(OT);
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");
    static_assert(NB == 2 || NB == 4, "chunk 32 or 64");
    static_assert(K == 64 || K == 128, "key dim 64 or 128");
    static_assert(!DQ || ST, "the re-scan saves states");
    constexpr bool kOwnStage = DQ && C * K * 2 < K * 64 * 2;    // chunk 32
    static_assert(L::kBytes + (kOwnStage ? 4 * K * 64 : 0) <= kLdsBytesMax, "LDS budget with the re-scan");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    __shared__ __attribute__((aligned(16))) uint16_t hq_own[kOwnStage ? 2 * K * 64 : 8];
    _Float16 *Qb = (_Float16 *)(smem + L::kQ);
    _Float16 *Kb = (_Float16 *)(smem + L::kK);
    _Float16 *Hb = (_Float16 *)(smem + L::kH);
    _Float16 *Tmbb = (_Float16 *)(smem + L::kTmb);
    _Float16 *Pb = (_Float16 *)(smem + L::kP);
    uint16_t *Vb = (uint16_t *)(smem + L::kV);
    float *Kf = (float *)(smem + L::kKf);
    unsigned *sync_ctr = (unsigned *)(smem + L::kSync);

    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    int pair, vt;
    map_block(blockIdx.x, p.nvt, p.swizzle, pair, vt);
    const int b = pair / p.H, h = pair - b * p.H;
    const StreamRange sr = stream_range<VL>(p, b, h);
    const int T = sr.T, H = p.H, V = p.V;
    const int nt = (T + C - 1) / C;
    const int64_t row0 = sr.row0;
    const uint32_t rsV = (uint32_t)(H * V);
    WaitCtl wc{p.wait_count, p.wait_limit, p.wait_bias, 0u};

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
        // chunks swizzled by row) in the qd and kd tiles of slot sl, free
        // then (chunk 32: in hq_own); each wave forms DQ for K/4 key rows over
        // the tile's 64 value columns with bf16 MFMAs (bf16 keeps any dO
        // magnitude in range)
        const rsrc_t rdo_ = make_rsrc(DQ ? (const IO *)p.dout + row0 * V : nullptr, DQ ? (uint32_t)T * rsV * SIO : 0u);
        const uint32_t do_off = ((uint32_t)(l & 15) * rsV + vt * 64 + 8 * (l >> 4)) * SIO;
        unsigned chain_target = 0;
        auto rescan_dq = [&](int n, int sl) {
            const uint32_t t0 = (uint32_t)(n * C);
            uint16_t *Hhi = kOwnStage ? hq_own : (uint16_t *)(Qb + sl * C * K);
            uint16_t *Hlo = kOwnStage ? hq_own + K * 64 : (uint16_t *)(Kb + sl * C * K);
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
            const float *flv = Kf + slot * K;
            const uint32_t t0 = (uint32_t)(c * C);

            // h as B fragments over the key dimension
            half8 hf[K / 32];
#pragma unroll
            for (int s = 0; s < K / 32; ++s) hf[s] = fragB_acc(hacc[2 * s], hacc[2 * s + 1], _Float16{});
            // X = kd h, Y^T = h^T qd^T for this wave's 16 columns
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
            // R' = v - X (the decay is inside kd)
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
            // h <- e^gl h + kg^T v', the decay row-wise by the key vector
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                float4v acc = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < C / 32; ++s)
                    M::mma(acc, fragAT_split_p<K>(Hs, 16 * i, 32 * s), df[s]);
                hacc[i] = *(const float4v *)(flv + 16 * i + g4) * hacc[i] + acc;
            }
            // the next chunk's dq term from its start state (now in hacc),
            // staged in this chunk's qd and kd tiles: the chain is done with
            // them, and the prepare writes this slot only after the barrier
            if constexpr (DQ)
                if (c + 1 < nt) rescan_dq(c + 1, slot);
            if constexpr (kPoisonLds) {
                // every chain wave is past its reads of this slot, which the
                // prepare rewrites for chunk c + 2
                prep_barrier(sync_ctr + 2, chain_target, wc);
                poison_fill(Qs, C * K * 2, tid, 256);
                poison_fill(Ks, C * K * 2, tid, 256);
                poison_fill(Hs, C * K * 2, tid, 256);
                poison_fill(Tmb, C * C * 2, tid, 256);
                poison_fill(Ps, C * C * 2, tid, 256);
                poison_fill(Vs, C * 64 * 2, tid, 256);
                poison_fill(flv, K * 4, tid, 256);
            }
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
        // priority in the plain forward and the re-scan; with saved states
        // the chain's store work competes for the SIMDs' issue slots, and a
        // raised priority measured 7 % faster)
        const int pt = tid - 256;
        if constexpr (ST && !DQ) __builtin_amdgcn_s_setprio(3);
        const rsrc_t rv_ = make_rsrc((const IO *)p.v + row0 * V, (uint32_t)T * rsV * SIO);
        // this stream's workspace slots (see slot_chunk): chunk n of stream b
        // is slot slot0 + n, each slot H heads of KdaSlotOps
        int slot0 = 0;
        if constexpr (VL) {
            for (int m = 0; m < b; ++m) {
                const int c0 = __builtin_amdgcn_readfirstlane(p.cu[m]);
                const int c1 = __builtin_amdgcn_readfirstlane(p.cu[m + 1]);
                const int bos = min(max(c0, 0), p.T), eos = min(max(c1, bos), p.T);
                slot0 += (eos - bos + C - 1) / C;
            }
        } else {
            slot0 = b * nt;
        }
        typedef KdaSlotOps<C, K> SO;
        constexpr uint32_t kSlotBytes = (uint32_t)SO::kBytes;
        const rsrc_t rw_ = make_rsrc((const char *)p.ws + ((int64_t)slot0 * H + h) * kSlotBytes,
                                     (uint32_t)nt * (uint32_t)H * kSlotBytes);

        constexpr int NVV = C * 64 / 8 / NPT;            // v vectors per thread
        static_assert(NVV >= 1, "tile smaller than the prepare waves");
        uint32_t vv_off[NVV];
        int vv_lds[NVV];
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int i = pt + NPT * j, row = i / 8, ch = i % 8;
            vv_off[j] = ((uint32_t)row * rsV + vt * 64 + 8 * ch) * SIO;
            vv_lds[j] = swz<64>(row, 8 * ch);
        }
        // Tmb and P (row-major in the slot): 16-byte pieces of 8 columns,
        // placed in the swizzled, column-permuted layout of the chain's tiles
        constexpr int NWS = L::NWS;
        int ws_lds[NWS][2];
#pragma unroll
        for (int j = 0; j < NWS; ++j) {
            const int e0 = 8 * (pt + NPT * j), tile = e0 / (C * C), rc = e0 % (C * C);
            const int row = rc / C, col = rc % C;
            const int base = tile ? (L::kP - L::kTmb) / 2 : 0;      // in halves from Tmb slot 0
            ws_lds[j][0] = base + swz<C>(row, pcol(col));
            ws_lds[j][1] = base + swz<C>(row, pcol(col + 4));
        }
        // the operand tiles qd, kd, kg, already in the tiles' layout: 16-byte
        // pieces copied as they are, NOP per thread (piece j of thread pt is
        // byte 16 (pt + NPT j) of the three tiles, tile (pt + NPT j) / (C K / 8))
        constexpr int NOP = 3 * C * K * 2 / 16 / NPT;
        static_assert(NOP * 16 * NPT == 3 * C * K * 2, "operand pieces per thread");
        constexpr int PPT = C * K * 2 / 16;              // pieces per tile
        const bool fl_thread = pt < K / 4;                // e^gl: 16 bytes each

        u32x4 rv[NVV], rw[NWS], ro[NOP], rf = {0, 0, 0, 0};
        // The loads of chunk n + 1 are issued right after chunk n's pieces are
        // in LDS, so they have the chain's whole period to arrive.
        for (int c = -1; c < nt; ++c) {
            const int n = c + 1;
            if (n < nt) {
                if (n == 0)
                    kda_slot_load<NVV, NWS, NOP, NPT>(rv_, rw_, vv_off, pt, fl_thread, rsV * SIO * (uint32_t)C,
                                                      (uint32_t)H * kSlotBytes, SO::kQd, SO::kFl, 0, rv, rw, ro, rf);
                const int slot = n & 1;
                _Float16 *Tmb = Tmbb + slot * C * C;
                uint16_t *Vs = Vb + slot * C * 64;
#pragma unroll
                for (int j = 0; j < NVV; ++j) *(u32x4 *)(Vs + vv_lds[j]) = rv[j];
#pragma unroll
                for (int j = 0; j < NWS; ++j) {
                    *(u32x2 *)(Tmb + ws_lds[j][0]) = u32x2{rw[j][0], rw[j][1]};
                    *(u32x2 *)(Tmb + ws_lds[j][1]) = u32x2{rw[j][2], rw[j][3]};
                }
                // the qd, kd and kg tiles follow each other in LDS, each with
                // its two slots: tile t of slot s starts (2 t + s) C K halves
                // after qd's slot 0
#pragma unroll
                for (int j = 0; j < NOP; ++j) {
                    const int q = pt + NPT * j, tile = q / PPT;
                    *(u32x4 *)(Qb + tile * 2 * C * K + slot * C * K + 8 * (q - tile * PPT)) = ro[j];
                }
                if (fl_thread) *(u32x4 *)(Kf + slot * K + 4 * pt) = rf;
                if (n + 1 < nt)
                    kda_slot_load<NVV, NWS, NOP, NPT>(rv_, rw_, vv_off, pt, fl_thread, rsV * SIO * (uint32_t)C,
                                                      (uint32_t)H * kSlotBytes, SO::kQd, SO::kFl, n + 1, rv, rw, ro, rf);
            }
            wg_barrier();                   // c < 0: chunk 0 prepared; else end of chunk c
        }
        wait_report(wc);
    }
}

}  // namespace gdn
