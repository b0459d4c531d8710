// libgdn: gdn_forward_split, the scalar-gate forward with each stream cut
// into two segments that run at the same time (bf16 io, chunk 64).
//
// The state recurrence is affine in the state and acts on every value
// column alike: from a start state h_in, a segment ends in
//     h_out = N + M h_in,    N the end state from a zero start,
//                            M the end state of the identity start with v = 0,
// and its outputs are o_t = o0_t + h_in^T oI_t, with o0 the outputs from the
// zero start and oI_t (a K-vector) those of the identity start.  One launch
// of the SP instance of forward_pipe_kernel runs the first segment from h0
// and, beside it, the second segment as its V tiles from a zero start (o0
// into o, N) and K / 64 more tiles from the identity with v = 0 (oI, M).
// Then h_in is the first segment's end state, and two small kernels finish:
//     split_state_kernel   hT = N + M h_in, and h_in^T in bf16 parts
//     split_out_kernel     o_t += h_in^T oI_t for the second segment's tokens
// This is the chunk-parallel scan of the second segment's transfer; with one
// workgroup per CU the first segment's workgroups and the second's (twice as
// many per head) fill the chip together when the first segment is about
// twice as long as the second.
#include <cstring>
#include <type_traits>

#include "gdn_buffer.h"
#include "gdn_forward.h"
#include "gdn_internal.h"

namespace gdn {

struct SplitParams {
    const void *oI;         // [B, T1, H, K] o dtype
    const float *hin;       // [B, H, K, V] the first segment's end state
    const float *N, *M;     // [B, H, K, V], [B, H, K, K]
    uint16_t *hinT;         // [2][B, H, V, K] h_in^T as bf16 high, then low parts
    void *o;                // [B, T, H, V], tokens from t0 of each row
    float *hT;              // [B, H, K, V] or NULL
    int T, T1, t0, H, B;
};

namespace {

// hT = N + M h_in (fp32; skipped when hT is NULL), and h_in^T as bf16 high
// and low parts for split_out_kernel.  One workgroup per 16 key rows of one
// (batch, head): thread (value column c, row group) holds 16 / (256 / V)
// consecutive key rows of column c; M's 16 rows are staged in LDS and read
// as broadcasts, h_in's rows stream from memory once per workgroup.
constexpr int kStateRows = 16;

template <int K, int V>
__global__ __launch_bounds__(256) void split_state_kernel(SplitParams p) {
    constexpr int RB = kStateRows, CG = 256 / V, RPT = RB / CG;
    static_assert(RPT % 4 == 0, "rows per thread");
    __shared__ float Ms[RB * K];
    const int tid = threadIdx.x, c = tid % V, rg = tid / V;
    const int bh = blockIdx.x / (K / RB), r0 = RB * (blockIdx.x % (K / RB)) + RPT * rg;
    const float *hin = p.hin + (int64_t)bh * K * V;
    {
        // this thread's RPT rows of column c, transposed: RPT consecutive
        // bf16 of row c of h_in^T, stored four at a time
        const int64_t tpos = ((int64_t)bh * V + c) * K + r0, plane = (int64_t)p.B * p.H * V * K;
#pragma unroll
        for (int e4 = 0; e4 < RPT; e4 += 4) {
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const float x0 = hin[(r0 + e4 + e) * V + c], x1 = hin[(r0 + e4 + e + 1) * V + c];
                const uint16_t h0 = f32_to_bf16_bits(x0), h1 = f32_to_bf16_bits(x1);
                const uint16_t l0 = f32_to_bf16_bits(x0 - __uint_as_float((uint32_t)h0 << 16));
                const uint16_t l1 = f32_to_bf16_bits(x1 - __uint_as_float((uint32_t)h1 << 16));
                hw[e / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lw[e / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            *(u32x2 *)(p.hinT + tpos + e4) = u32x2{hw[0], hw[1]};
            *(u32x2 *)(p.hinT + plane + tpos + e4) = u32x2{lw[0], lw[1]};
        }
    }
    if (!p.hT) return;                       // uniform over the grid
    const float *M = p.M + ((int64_t)bh * K + RB * (blockIdx.x % (K / RB))) * K;
    for (int i = tid; i < RB * K; i += 256) Ms[i] = M[i];
    __syncthreads();
    float acc[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) acc[e] = 0.f;
    const float *Mr = Ms + RPT * rg * K;
#pragma unroll 8
    for (int j = 0; j < K; ++j) {
        const float x = hin[j * V + c];
#pragma unroll
        for (int e = 0; e < RPT; ++e) acc[e] += Mr[e * K + j] * x;
    }
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
        const int64_t at = ((int64_t)bh * K + r0 + e) * V + c;
        p.hT[at] = p.N[at] + acc[e];
    }
}

// o_t += h_in^T oI_t for the second segment's tokens, 512 tokens of one
// (batch, head) per workgroup of eight waves.  The product is formed
// transposed, (o^T)[v][t] = sum_k h_in[k][v] oI[t][k]: h_in^T, as bf16 high
// and low parts (about 16 bits of h_in), is staged once into LDS and gives
// the A operand; each wave streams 16-token tiles with the next tile's loads
// in flight.  Every load and store covers whole rows of the head: oI rows
// come in 16 bytes per lane and go to the wave's own LDS tile, from which the
// B fragments are read (fp32 oI as bf16 high and low parts, a third
// product); o rows come in 8 bytes per lane.  The product, in accumulator
// layout, goes back through the same LDS tile as fp32 [token][v] rows, and
// each lane adds its values to its o piece and stores it.  (A first version
// that fed the fragments straight from memory touched 16 token rows with
// every load and store: 291 against 229 us at 65536 tokens, 64 heads.)
// LDS rows hold 16-byte chunks, chunk c of row r at c ^ (r mod 8), so that
// the eight lanes of a 128-byte read phase hit distinct banks.
constexpr int kRowWaves = 8, kRowTiles = 4;

template <int K, int V, typename OT> struct OutRowsLayout {
    static constexpr int CPR = K / 8;                      // 16-byte chunks per At row (bf16)
    static constexpr int CPI = K * (int)sizeof(OT) / 16;   // 16-byte chunks per oI row
    static constexpr int LCT = V + 4;                      // fp32 product row pitch (floats)
    static constexpr int kAt = 2 * V * CPR * 16;           // h_in^T high, low parts
    static constexpr int kTileB = 16 * CPI * 16;           // oI tile [16][K]
    static constexpr int kTileC = 16 * LCT * 4;            // product fp32 [16][LCT]
    static constexpr int kTile = kTileB > kTileC ? kTileB : kTileC;
    static constexpr int kBytes = kAt + kRowWaves * kTile;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

template <int K, int V, typename OT>
__global__ __launch_bounds__(64 * kRowWaves, 1) void split_out_kernel(SplitParams p) {
    typedef OutRowsLayout<K, V, OT> L;
    constexpr bool F32 = sizeof(OT) == 4;
    constexpr int MT = V / 16, NS = K / 32, CPR = L::CPR, CPI = L::CPI, LCT = L::LCT;
    constexpr int RI = 64 / CPI, NI = 16 / RI;     // oI: rows per load, loads per tile
    constexpr int PV = F32 ? 2 : 4;                // o values per 8-byte piece
    constexpr int RO = 64 * PV / V, NO = 16 / RO;  // o: rows per load (and store), loads per tile
    constexpr int TB = 16 * kRowWaves * kRowTiles;
    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    u32x4 *At = (u32x4 *)smem;
    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    u32x4 *Bt = (u32x4 *)(smem + L::kAt + wv * L::kTile);      // chunk c of row r at c ^ (r & 7)
    float *Ct = (float *)(smem + L::kAt + wv * L::kTile);       // the same bytes, after the products
    const int nblk = (p.T1 + TB - 1) / TB;
    const int bid = blockIdx.x;
    const int h = bid % p.H, rest = bid / p.H, blk = rest % nblk, b = rest / nblk;
    const int t_first = TB * blk;
    const int rows = min(TB, p.T1 - t_first);
    const uint32_t HK = (uint32_t)p.H * K, HV = (uint32_t)p.H * V;
    const rsrc_t rI = make_rsrc((const OT *)p.oI + ((int64_t)b * p.T1 + t_first) * HK, (uint32_t)(rows * HK * sizeof(OT)));
    const rsrc_t ro = make_rsrc((OT *)p.o + ((int64_t)b * p.T + p.t0 + t_first) * HV, (uint32_t)(rows * HV * sizeof(OT)));
    const int n = l & 15, g = l >> 4;
    const int ir = l / CPI, ic = l % CPI;            // oI: row ir of each RI, chunk ic
    const int orow = l / (V / PV), oc = l % (V / PV); // o: row orow of each RO, columns PV oc .. +PV-1

    u32x4 bI[NI], bIn[NI];
    u32x2 vo[NO], von[NO];
    auto load = [&](u32x4 *bi, u32x2 *vv, int r0) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            bi[i] = bload128(rI, ((uint32_t)(r0 + RI * i + ir) * HK + (uint32_t)h * K) * sizeof(OT) + 16 * ic, 0);
#pragma unroll
        for (int j = 0; j < NO; ++j)
            vv[j] = __builtin_amdgcn_raw_buffer_load_b64(
                ro, ((uint32_t)(r0 + RO * j + orow) * HV + (uint32_t)h * V + PV * oc) * sizeof(OT), 0, 0);
    };
    load(bI, vo, 16 * wv);
    {
        const int64_t bh = (int64_t)b * p.H + h, plane = (int64_t)p.B * p.H * V * K;
        const u32x4 *hi = (const u32x4 *)(p.hinT + bh * V * K), *lo = (const u32x4 *)(p.hinT + plane + bh * V * K);
#pragma unroll
        for (int i = tid; i < V * CPR; i += 64 * kRowWaves) {
            const int r = i / CPR, c = i % CPR;
            At[r * CPR + (c ^ (r & 7))] = hi[i];
            At[(V + r) * CPR + (c ^ (r & 7))] = lo[i];
        }
    }
    __syncthreads();

#pragma unroll
    for (int it = 0; it < kRowTiles; ++it) {
        const int r0 = 16 * (wv + kRowWaves * it);
        if (it + 1 < kRowTiles) load(bIn, von, r0 + 16 * kRowWaves);
        // this tile's oI rows into the wave's LDS tile (LDS operations of one
        // wave take effect in issue order: no barrier inside the wave's tile)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = RI * i + ir;
            Bt[r * CPI + (ic ^ (r & 7))] = bI[i];
        }
        float4v acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = float4v{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            // lane (n, g): oI[n][32 st + 8 g .. +7]
            bf16x8 bh, bl;
            if constexpr (F32) {
                const u32x4 x0 = Bt[n * CPI + ((8 * st + 2 * g) ^ (n & 7))];
                const u32x4 x1 = Bt[n * CPI + ((8 * st + 2 * g + 1) ^ (n & 7))];
                uint16_t xh[8], xl[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float f = __uint_as_float(j < 4 ? x0[j] : x1[j - 4]);
                    xh[j] = f32_to_bf16_bits(f);
                    xl[j] = f32_to_bf16_bits(f - __uint_as_float((uint32_t)xh[j] << 16));
                }
                bh = __builtin_bit_cast(bf16x8, xh);
                bl = __builtin_bit_cast(bf16x8, xl);
            } else {
                bh = __builtin_bit_cast(bf16x8, Bt[n * CPI + ((4 * st + g) ^ (n & 7))]);
            }
            const int c = (4 * st + g) ^ (n & 7);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int r = 16 * m + n;
                const bf16x8 ah = __builtin_bit_cast(bf16x8, At[r * CPR + c]);
                const bf16x8 al = __builtin_bit_cast(bf16x8, At[(V + r) * CPR + c]);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[m], 0, 0, 0);
                if constexpr (F32) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[m], 0, 0, 0);
            }
        }
        // lane (n, g) holds token n, value columns 16 m + 4 g .. +3; the tile's
        // bytes change type here (the barriers keep the compiler from moving
        // accesses of one view across those of the other)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < MT; ++m) *(float4v *)(Ct + n * LCT + 16 * m + 4 * g) = acc[m];
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int r = RO * j + orow;
            const uint32_t off = ((uint32_t)(r0 + r) * HV + (uint32_t)h * V + PV * oc) * sizeof(OT);
            const u32x2 w = vo[j];
            if constexpr (F32) {
                const float *x = Ct + r * LCT + 2 * oc;
                const float y0 = __uint_as_float(w[0]) + x[0], y1 = __uint_as_float(w[1]) + x[1];
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(y0), __float_as_uint(y1)}, ro, off, 0, 0);
            } else {
                const float4v x = *(const float4v *)(Ct + r * LCT + 4 * oc);
                const float y0 = __uint_as_float(w[0] << 16) + x[0], y1 = __uint_as_float(w[0] & 0xffff0000u) + x[1];
                const float y2 = __uint_as_float(w[1] << 16) + x[2], y3 = __uint_as_float(w[1] & 0xffff0000u) + x[3];
                const uint32_t lo = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_bits(y2) | ((uint32_t)f32_to_bf16_bits(y3) << 16);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, off, 0, 0);
            }
        }
        asm volatile("" ::: "memory");
        if (it + 1 < kRowTiles) {
#pragma unroll
            for (int i = 0; i < NI; ++i) bI[i] = bIn[i];
#pragma unroll
            for (int j = 0; j < NO; ++j) vo[j] = von[j];
        }
    }
}

template <int K, bool F32>
gdn_status launch_split(const gdn_problem *pr, FwdParams &fp, SplitParams &sp, int grid, hipStream_t s) {
    typedef typename std::conditional<F32, float, bf16_t>::type OT;
    gdn_status st = enqueue_forward_pipe_split(K, F32, fp, grid, s);
    if (st != GDN_OK) return st;
    const int V = (int)pr->V;
    const int gst = (int)(pr->B * pr->H * (K / kStateRows));
    const void *fs = V == 64 ? (const void *)&split_state_kernel<K, 64> : (const void *)&split_state_kernel<K, 128>;
    st = launch_kernel(fs, gst, &sp, s, 256);
    if (st != GDN_OK) return st;
    constexpr int TB = 16 * kRowWaves * kRowTiles;
    const int gout = (int)(pr->B * pr->H * ((sp.T1 + TB - 1) / TB));
    const void *fo = V == 64 ? (const void *)&split_out_kernel<K, 64, OT> : (const void *)&split_out_kernel<K, 128, OT>;
    return launch_kernel(fo, gout, &sp, s, 64 * kRowWaves);
}

}  // namespace

int64_t split_workspace_bytes(const gdn_problem *pr, int64_t t_split) {
    const int64_t so = pr->o_dtype == GDN_F32 ? 4 : 2;
    const int64_t bh = pr->B * pr->H, T1 = pr->T - t_split;
    return bh * pr->K * pr->V * 4 * 2 + bh * pr->K * pr->K * 4 + bh * pr->K * pr->V * 2 * 2 +
           pr->B * T1 * pr->H * pr->K * so;
}

gdn_status enqueue_forward_split(const gdn_problem *pr, int64_t t_split, const void *q, const void *k,
                                 const void *v, const float *beta, const float *g, const float *h0,
                                 void *o, float *hT, void *ws, hipStream_t s) {
    const int64_t bh = pr->B * pr->H, T1 = pr->T - t_split;
    char *w = (char *)ws;
    float *hin = (float *)w;
    float *N = hin + bh * pr->K * pr->V;
    float *M = N + bh * pr->K * pr->V;
    uint16_t *hinT = (uint16_t *)(M + bh * pr->K * pr->K);
    void *oI = hinT + 2 * bh * pr->K * pr->V;

    FwdParams fp;
    std::memset(&fp, 0, sizeof(fp));
    fp.q = q; fp.k = k; fp.v = v; fp.beta = beta; fp.g = g; fp.h0 = h0;
    fp.o = o; fp.hT = nullptr;
    fp.B = (int)pr->B; fp.T = (int)pr->T; fp.H = (int)pr->H; fp.V = (int)pr->V;
    fp.nvt = (int)(pr->V / 64);
    fp.swizzle = (bh % 8 == 0) ? 1 : 0;
    wait_params(fp.wait_limit, fp.wait_bias);
    fp.wait_count = wait_count_ptr();
    fp.sp_t = (int)t_split;
    fp.sp_g0 = (int)(bh * fp.nvt);
    fp.sp_oI = oI; fp.sp_h0out = hin; fp.sp_N = N; fp.sp_M = M;
    const int grid = (int)(bh * fp.nvt + bh * (fp.nvt + pr->K / 64));

    SplitParams sp;
    sp.oI = oI; sp.hin = hin; sp.N = N; sp.M = M; sp.hinT = hinT; sp.o = o; sp.hT = hT;
    sp.T = (int)pr->T; sp.T1 = (int)T1; sp.t0 = (int)t_split; sp.H = (int)pr->H; sp.B = (int)pr->B;
    const bool f32 = pr->o_dtype == GDN_F32;
    if (pr->K == 64) return f32 ? launch_split<64, true>(pr, fp, sp, grid, s) : launch_split<64, false>(pr, fp, sp, grid, s);
    return f32 ? launch_split<128, true>(pr, fp, sp, grid, s) : launch_split<128, false>(pr, fp, sp, grid, s);
}

}  // namespace gdn
