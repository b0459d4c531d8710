// gdn_scan kernel: the serial inter-chunk scan given the WY factors.
//
// Per-chunk algebra of the kernel_fun KDA forward re-scan (bwd_scan.py,
// KdaB1ScanKernel docstring and SIMT recurrence), plus the output read-out:
//     v'  = u - w h
//     o   = (q * exp(gcum)) h + tril_incl((q k^T) * decay) v'
//     h  <- exp(gcum_last) * h + (k * exp(gcum_last - gcum))^T v'
// One workgroup per (batch, head, 64-wide V tile), serial over chunks, the
// fp32 state tile h [K x BV] resident in accumulator registers.  The page
// splits its CTA into TMA / MMA / SIMT warp roles around TMEM; gfx950 has
// neither, so here all four waves take a share of every product and meet at
// workgroup barriers, with the next chunk's loads in flight in registers.
#pragma once

#include "gdn_chunk_io.h"
#include "gdn_key_gram.h"

namespace gdn {

struct ScanParams {
    const void *q, *k;
    const float *w, *u, *gcum, *h0;
    void *o;
    float *hT;
    int B, T, H, V;
    int nvt;        // V / BV
    int swizzle;    // 1: keep the V tiles of one (b, h) on one XCD
};

template <typename IO> struct OpOf { typedef _Float16 type; };
template <> struct OpOf<float> { typedef float type; };

// Map a linear workgroup id to (pair = b*H + h, V tile).  Workgroups are
// dealt to the 8 XCDs round robin; with the swizzle, ids that land on the
// same XCD cover all V tiles of one head, so q, k and w are fetched into one
// L2 once per head instead of once per tile.
__device__ __forceinline__ void map_block(int bid, int nvt, int swizzle, int &pair, int &vt) {
    if (swizzle) {
        const int xcd = bid & 7, slot = bid >> 3;
        pair = xcd + 8 * (slot / nvt);
        vt = slot % nvt;
    } else {
        pair = bid / nvt;
        vt = bid % nvt;
    }
}

template <int C, int K, int BV, typename IO, bool KEYGATE>
struct ScanLayout {
    typedef typename OpOf<IO>::type OpT;
    static constexpr int LDK = K + Mma<OpT>::kPad;
    static constexpr int LDC = C + Mma<OpT>::kPad;
    static constexpr int E = sizeof(OpT);
    static constexpr int kQ = 0;                              // [C][LDK] q (KDA: q e^g)
    static constexpr int kK = kQ + C * LDK * E;               // [C][LDK] k (KDA: scratch)
    static constexpr int kQr = kK + C * LDK * E;              // [C][LDK] KDA: scratch
    static constexpr int kW = kQr + (KEYGATE ? C * LDK * E : 0);   // [C][LDK] w
    static constexpr int kKT = kW + C * LDK * E;              // [K][LDC] k^T (KDA: kg^T)
    static constexpr int kHT = kKT + K * LDC * E;             // [BV][LDK] h^T
    static constexpr int kP = kHT + BV * LDK * E;             // [C][LDC] masked decayed q k^T
    static constexpr int kDT = kP + C * LDC * E;              // [BV][LDC] v'^T
    static constexpr int kDS = kDT + BV * LDC * E;            // [BV][LDC] GDN: (v' e^(gl-g))^T
    static constexpr int kGam = kDS + (KEYGATE ? 0 : BV * LDC * E);  // fp32 gates
    static constexpr int kGamN = KEYGATE ? K : C;             // KDA: gcum_last[K]; GDN: gcum[C]
    // KDA: P in fp32 from exact_key_gram (whose operand scratch is the k and
    // q tiles kK, kQr), the segment totals and segment-end gcum it reads
    static constexpr int LDA = C + 4;
    static constexpr int kPf = kGam + kGamN * 4;
    static constexpr int NSEG = kThreads * 4 / K;
    static constexpr int kGend = kPf + (KEYGATE ? C * LDA * 4 : 0);
    static constexpr int kBytes = kGend + (KEYGATE ? NSEG * K * 4 : 0);
};

template <int C, int K, int BV, typename IO, typename OT, bool KEYGATE>
__global__ __launch_bounds__(kThreads, 1) void scan_kernel(ScanParams p) {
    typedef ScanLayout<C, K, BV, IO, KEYGATE> L;
    typedef typename L::OpT OpT;
    constexpr int LDK = L::LDK, LDC = L::LDC;
    constexpr int NCB = C / 16, NVB = BV / 16, NKB = K / 16;
    constexpr int NZW = NCB * NVB / kWaves;   // q/w row tiles per wave
    constexpr int NHW = NKB * NVB / kWaves;   // state tiles per wave
    static_assert(NCB * NVB % kWaves == 0 && NKB * NVB % kWaves == 0, "tiling");
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OpT *Qs = (OpT *)(smem + L::kQ);
    OpT *Ks = (OpT *)(smem + L::kK);
    OpT *Qr = (OpT *)(smem + L::kQr);
    OpT *Ws = (OpT *)(smem + L::kW);
    OpT *KT = (OpT *)(smem + L::kKT);
    OpT *HT = (OpT *)(smem + L::kHT);
    OpT *Ps = (OpT *)(smem + L::kP);
    OpT *DT = (OpT *)(smem + L::kDT);
    OpT *DS = KEYGATE ? DT : (OpT *)(smem + L::kDS);
    float *gam = (float *)(smem + L::kGam);
    float *Pf = (float *)(smem + L::kPf);
    float *gend = (float *)(smem + L::kGend);

    int pair, vt;
    map_block(blockIdx.x, p.nvt, p.swizzle, pair, vt);
    const int b = pair / p.H, h = pair - b * p.H;
    const int T = p.T, H = p.H, V = p.V, v0 = vt * BV;
    const int wv = wave_id(), tid = threadIdx.x;
    const int nt = (T + C - 1) / C;

    const int64_t row0 = (int64_t)b * T * H + h;          // token-head row of t = 0
    const IO *qb = (const IO *)p.q + row0 * K;
    const IO *kb = (const IO *)p.k + row0 * K;
    const float *wb = p.w + row0 * K;
    const float *ub = p.u + row0 * V + v0;
    const float *gb = p.gcum + row0 * (KEYGATE ? K : 1);
    OT *ob = (OT *)p.o + row0 * V + v0;
    const int64_t rsK = (int64_t)H * K, rsV = (int64_t)H * V;
    const int64_t rsG = KEYGATE ? (int64_t)H * K : (int64_t)H;

    // ---- state tiles: hacc[i] holds h[16 kb + row][16 vb + col]
    float4v hacc[NHW];
#pragma unroll
    for (int i = 0; i < NHW; ++i) {
        const int t = wv * NHW + i, kbi = t / NVB, vb = t % NVB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kd = 16 * kbi + acc_row(r), vv = v0 + 16 * vb + acc_col();
            hacc[i][r] = p.h0 ? p.h0[((int64_t)pair * K + kd) * V + vv] : 0.f;
        }
        store_tile_T(HT + 16 * vb * LDK + 16 * kbi, LDK, hacc[i]);
    }
    for (int i = tid; i < C * LDC; i += kThreads) Ps[i] = (OpT)0.f;

    // ---- prefetch registers
    ChunkRows<IO, C, K> rq, rk;
    ChunkRows<float, C, K> rw;
    ChunkRows<float, C, K> rg;      // KDA gate rows
    float g_own = 0.f;              // GDN: gcum of row tid (tid < C)
    float gl_own[8];                // KDA: gcum of the chunk's last row
    float4v ureg[NZW];

    auto load_chunk = [&](int c) {
        const int t0 = c * C, nvalid = min(C, T - t0);
        rq.load(qb + t0 * rsK, rsK, nvalid);
        rk.load(kb + t0 * rsK, rsK, nvalid);
        rw.load(wb + t0 * rsK, rsK, nvalid);
        if constexpr (KEYGATE) {
            rg.load(gb + t0 * rsG, rsG, nvalid);
            // every vector of this thread sits in the same column group
            const int col = ChunkRows<float, C, K>::col(0);
            const float *gl = gb + (t0 + nvalid - 1) * rsG + col;
#pragma unroll
            for (int e = 0; e < 8; ++e) gl_own[e] = gl[e];
        } else {
            if (tid < C) g_own = gb[(t0 + min(tid, nvalid - 1)) * rsG];
        }
#pragma unroll
        for (int i = 0; i < NZW; ++i) {
            const int t = wv * NZW + i, cb = t / NVB, vb = t % NVB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cr = 16 * cb + acc_row(r);
                ureg[i][r] = cr < nvalid ? ub[(t0 + cr) * rsV + 16 * vb + acc_col()] : 0.f;
            }
        }
    };
    if (nt > 0) load_chunk(0);

    for (int c = 0; c < nt; ++c) {
        const int t0 = c * C, nvalid = min(C, T - t0);

        // ---- S1: registers -> LDS operands
        if constexpr (KEYGATE) {
            const int col = ChunkRows<float, C, K>::col(0);
            float glast[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) glast[e] = gl_own[e];
            if (tid < K / 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) gam[col + e] = glast[e];
            }
            // q e^gcum and k e^(gl - gcum): decays (P comes from
            // exact_key_gram below)
#pragma unroll
            for (int j = 0; j < ChunkRows<IO, C, K>::kVec; ++j) {
                const int row = ChunkRows<IO, C, K>::row(j);
                const bool ok = row < nvalid;
                float xq[8], xk[8], xw[8], xg[8], a[8], kg[8];
                rq.get(j, xq); rk.get(j, xk); rw.get(j, xw); rg.get(j, xg);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = ok ? xq[e] * fast_exp(xg[e]) : 0.f;
                    kg[e] = ok ? xk[e] * fast_exp(glast[e] - xg[e]) : 0.f;
                }
                put8(Qs + row * LDK + col, a);
                put8(Ws + row * LDK + col, xw);
                put8_col(KT + col * LDC + row, LDC, kg);
            }
        } else {
#pragma unroll
            for (int j = 0; j < ChunkRows<IO, C, K>::kVec; ++j) {
                const int row = ChunkRows<IO, C, K>::row(j), col = ChunkRows<IO, C, K>::col(j);
                float x[8];
                rq.get(j, x);
                put8(Qs + row * LDK + col, x);
                rk.get(j, x);
                put8(Ks + row * LDK + col, x);
                put8_col(KT + col * LDC + row, LDC, x);
                rw.get(j, x);
                put8(Ws + row * LDK + col, x);
            }
            if (tid < C) gam[tid] = g_own;
        }
        // U tiles for this chunk are consumed from registers in S2; keep a copy
        float4v ucur[NZW];
#pragma unroll
        for (int i = 0; i < NZW; ++i) ucur[i] = ureg[i];
        if (c + 1 < nt) load_chunk(c + 1);
        __syncthreads();

        if constexpr (KEYGATE) {
            // P with every decay split at a row between its two tokens: the
            // chunk's gcum, k and q in exact_key_gram's row order (from L2:
            // the ChunkRows copies above have another layout), the k and q
            // tiles as its operand scratch, P in fp32, then into Ps
            constexpr int NR = KeyRows<C, K>::NR;
            const uint32_t rsk = (uint32_t)rsK;
            const rsrc_t rgc = make_rsrc(gb, (uint32_t)T * rsk * 4);
            const rsrc_t rkc = make_rsrc(kb, (uint32_t)T * rsk * sizeof(IO));
            const rsrc_t rqc = make_rsrc(qb, (uint32_t)T * rsk * sizeof(IO));
            float4v gS[NR], kS[NR], qS[NR];
            load_key_rows<C, K, IO, true>(rgc, rkc, rqc, rsk, (uint32_t)t0, nullptr, gend, gS, kS, qS);
            exact_key_gram<C, K, OpT, false, true>(gS, kS, qS, gend, gend, Ks, Qr, Pf, Pf);
            for (int i = tid; i < C * C; i += kThreads)
                Ps[(i / C) * LDC + i % C] = Mma<OpT>::cvt(Pf[(i / C) * L::LDA + i % C]);
            __syncthreads();
        }

        // ---- S2: P = masked decayed q k^T (the scalar gate);  Z = w h,
        // Y = q h;  v' = u - Z
        float gl = 0.f;
        if constexpr (!KEYGATE) gl = gam[nvalid - 1];
        constexpr int NP = KEYGATE ? 0 : NCB * (NCB + 1) / 2;
#pragma unroll
        for (int idx = 0; idx < NP; ++idx) {
            if (idx % kWaves != wv) continue;
            int J = 0;
            while ((J + 1) * (J + 2) / 2 <= idx) ++J;
            const int I = idx - J * (J + 1) / 2;            // I <= J
            float4v acc = {0, 0, 0, 0};
            mma_tile<OpT, K>(acc, Ks + 16 * I * LDK, LDK, Qs + 16 * J * LDK, LDK);
            // acc[r] = P[c = 16J + col][c' = 16I + row(r)]
            const int cc = 16 * J + acc_col();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cp = 16 * I + acc_row(r);
                float val = acc[r];
                if constexpr (!KEYGATE) val *= fast_exp(gam[cc] - gam[cp]);
                acc[r] = cp <= cc ? val : 0.f;
            }
            store_tile_T(Ps + 16 * J * LDC + 16 * I, LDC, acc);
        }
        float4v yacc[NZW];
#pragma unroll
        for (int i = 0; i < NZW; ++i) {
            const int t = wv * NZW + i, cb = t / NVB, vb = t % NVB;
            float4v z = {0, 0, 0, 0};
            yacc[i] = float4v{0, 0, 0, 0};
            mma_tile<OpT, K>(z, Ws + 16 * cb * LDK, LDK, HT + 16 * vb * LDK, LDK);
            mma_tile<OpT, K>(yacc[i], Qs + 16 * cb * LDK, LDK, HT + 16 * vb * LDK, LDK);
            float4v d = ucur[i] - z;
            store_tile_T(DT + 16 * vb * LDC + 16 * cb, LDC, d);
            if constexpr (!KEYGATE) {
#pragma unroll
                for (int r = 0; r < 4; ++r) d[r] *= fast_exp(gl - gam[16 * cb + acc_row(r)]);
                store_tile_T(DS + 16 * vb * LDC + 16 * cb, LDC, d);
            }
        }
        __syncthreads();

        // ---- S3: o = e^g Y + P v';  h = e^gl h + kg^T v'
#pragma unroll
        for (int i = 0; i < NZW; ++i) {
            const int t = wv * NZW + i, cb = t / NVB, vb = t % NVB;
            float4v acc = {0, 0, 0, 0};
            const int klen = 32 * ((16 * (cb + 1) + 31) / 32);
            mma_tile_n<OpT, C>(acc, Ps + 16 * cb * LDC, LDC, DT + 16 * vb * LDC, LDC, klen);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int cr = 16 * cb + acc_row(r);
                float y = yacc[i][r];
                if constexpr (!KEYGATE) y *= fast_exp(gam[cr]);
                if (cr < nvalid)
                    io_traits<OT>::store(ob + (t0 + cr) * rsV + 16 * vb + acc_col(), acc[r] + y);
            }
        }
        const float dl = KEYGATE ? 0.f : fast_exp(gl);
#pragma unroll
        for (int i = 0; i < NHW; ++i) {
            const int t = wv * NHW + i, kbi = t / NVB, vb = t % NVB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (KEYGATE) hacc[i][r] *= fast_exp(gam[16 * kbi + acc_row(r)]);
                else hacc[i][r] *= dl;
            }
            mma_tile<OpT, C>(hacc[i], KT + 16 * kbi * LDC, LDC, DS + 16 * vb * LDC, LDC);
            store_tile_T(HT + 16 * vb * LDK + 16 * kbi, LDK, hacc[i]);
        }
        __syncthreads();
    }

    if (p.hT) {
#pragma unroll
        for (int i = 0; i < NHW; ++i) {
            const int t = wv * NHW + i, kbi = t / NVB, vb = t % NVB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kd = 16 * kbi + acc_row(r), vv = v0 + 16 * vb + acc_col();
                p.hT[((int64_t)pair * K + kd) * V + vv] = hacc[i][r];
            }
        }
    }
}

}  // namespace gdn
