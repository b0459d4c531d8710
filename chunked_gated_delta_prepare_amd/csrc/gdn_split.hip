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

// One 16-token tile's operands in registers: oI rows (the B operand, 16
// bytes per 32-key step; fp32 two of them) and the lane's o pieces (four
// value columns per 16-row value tile).
template <int K, int V, typename OT> struct OutTile {
    static constexpr bool F32 = sizeof(OT) == 4;
    static constexpr int NS = K / 32, MT = V / 16;
    u32x4 b[F32 ? 2 * NS : NS];
    u32x4 o[MT];                         // bf16: the first two dwords
};

template <int K, int V, typename OT>
__device__ __forceinline__ void load_out_tile(OutTile<K, V, OT> &t, rsrc_t rI, rsrc_t ro, int row, int h,
                                              int n, int g, uint32_t HK, uint32_t HV) {
    constexpr int NS = K / 32, MT = V / 16;
    const uint32_t ib = ((uint32_t)row * HK + (uint32_t)h * K + 8 * g) * sizeof(OT);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if constexpr (sizeof(OT) == 4) {
            t.b[2 * s] = bload128(rI, ib + 32 * s * 4, 0);
            t.b[2 * s + 1] = bload128(rI, ib + 32 * s * 4 + 16, 0);
        } else {
            t.b[s] = bload128(rI, ib + 32 * s * 2, 0);
        }
    }
    const uint32_t ob = ((uint32_t)row * HV + (uint32_t)h * V + 4 * g) * sizeof(OT);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if constexpr (sizeof(OT) == 4) {
            t.o[m] = bload128(ro, ob + 16 * m * 4, 0);
        } else {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(ro, ob + 16 * m * 2, 0, 0);
            t.o[m] = u32x4{w[0], w[1], 0u, 0u};
        }
    }
}

// o_t += h_in^T oI_t for 64 kOutTiles tokens of one (batch, head) per
// workgroup (512 or 1024 measured no faster than 256).  The
// product is formed transposed, (o^T)[v][t] = sum_k h_in[k][v] oI[t][k]:
// h_in^T, as bf16 high and low parts (about 16 bits of h_in), is staged once
// into LDS and gives the A operand; each wave then streams its own 16-token
// tiles of oI (the B operand: bf16, or fp32 as high and low parts) and o,
// with the next tile's loads in flight while the current one is multiplied.
// A lane's result is four consecutive value columns of one token.  LDS rows
// hold 16-byte chunks, chunk c of row r at c ^ (r mod 8), so that the eight
// lanes of a 128-byte read phase hit distinct banks.
constexpr int kOutTiles = 4;  // 16-token tiles per wave

template <int K, int V, typename OT>
__global__ __launch_bounds__(256, 2) void split_out_kernel(SplitParams p) {
    constexpr bool F32 = sizeof(OT) == 4;
    constexpr int NT = kOutTiles;
    constexpr int TB = 16 * 4 * NT;      // tokens per workgroup
    constexpr int MT = V / 16, NS = K / 32, CPR = K / 8;
    __shared__ __attribute__((aligned(16))) u32x4 At[2 * V * CPR];
    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    const int nblk = (p.T1 + TB - 1) / TB;
    const int bid = blockIdx.x;
    const int h = bid % p.H, rest = bid / p.H, blk = rest % nblk, b = rest / nblk;
    const int t_first = TB * blk;
    const int rows = min(TB, p.T1 - t_first);
    const uint32_t HK = (uint32_t)p.H * K, HV = (uint32_t)p.H * V;
    const rsrc_t rI = make_rsrc((const OT *)p.oI + ((int64_t)b * p.T1 + t_first) * HK, (uint32_t)rows * HK * sizeof(OT));
    const rsrc_t ro = make_rsrc((OT *)p.o + ((int64_t)b * p.T + p.t0 + t_first) * HV, (uint32_t)rows * HV * sizeof(OT));
    const int n = l & 15, g = l >> 4;

    OutTile<K, V, OT> cur, nxt;
    load_out_tile<K, V, OT>(cur, rI, ro, 16 * wv + n, h, n, g, HK, HV);
    {
        const int64_t bh = (int64_t)b * p.H + h, plane = (int64_t)p.B * p.H * V * K;
        const u32x4 *hi = (const u32x4 *)(p.hinT + bh * V * K), *lo = (const u32x4 *)(p.hinT + plane + bh * V * K);
#pragma unroll
        for (int i = tid; i < V * CPR; i += 256) {
            const int r = i / CPR, c = i % CPR;
            At[r * CPR + (c ^ (r & 7))] = hi[i];
            At[(V + r) * CPR + (c ^ (r & 7))] = lo[i];
        }
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int row = 16 * (wv + 4 * i) + n;
        if (i + 1 < NT) load_out_tile<K, V, OT>(nxt, rI, ro, row + 64, h, n, g, HK, HV);
        float4v acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = float4v{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            bf16x8 bh, bl;
            if constexpr (F32) {
                uint16_t x[8], y[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float f = __uint_as_float(j < 4 ? cur.b[2 * s][j] : cur.b[2 * s + 1][j - 4]);
                    x[j] = f32_to_bf16_bits(f);
                    y[j] = f32_to_bf16_bits(f - __uint_as_float((uint32_t)x[j] << 16));
                }
                bh = __builtin_bit_cast(bf16x8, x);
                bl = __builtin_bit_cast(bf16x8, y);
            } else {
                bh = __builtin_bit_cast(bf16x8, cur.b[s]);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int r = 16 * m + n, c = (4 * s + g) ^ (n & 7);
                const bf16x8 ah = __builtin_bit_cast(bf16x8, At[r * CPR + c]);
                const bf16x8 al = __builtin_bit_cast(bf16x8, At[(V + r) * CPR + c]);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[m], 0, 0, 0);
                if constexpr (F32) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[m], 0, 0, 0);
            }
        }
        // lane (g, n): value columns 16 m + 4 g .. +3 of token row
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint32_t col = (uint32_t)h * V + 16 * m + 4 * g;
            if constexpr (!F32) {
                const u32x4 w = cur.o[m];
                const float4v x = float4v{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                          __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)} + acc[m];
                const uint32_t lo = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, ro, ((uint32_t)row * HV + col) * 2, 0, 0);
            } else {
                // lanes of neighbouring tokens swap halves, so that each
                // lane stores two 8-byte pieces a row apart (never one wide
                // store): the even lane columns +0, +1 of its token and the
                // next, the odd lane columns +2, +3 of the previous token
                // and its own
                const float4v x = __builtin_bit_cast(float4v, cur.o[m]) + acc[m];
                const bool odd = n & 1;
                const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
                const float r0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0xB1, 0xf, 0xf, false));
                const float r1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xf, 0xf, false));
                const uint32_t oa = ((uint32_t)(row & ~1) * HV + col) * 4 + 8 * (uint32_t)odd;
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{__float_as_uint(odd ? r0 : x[0]), __float_as_uint(odd ? r1 : x[1])}, ro, oa, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{__float_as_uint(odd ? x[2] : r0), __float_as_uint(odd ? x[3] : r1)}, ro, oa + HV * 4, 0, 0);
            }
        }
        if (i + 1 < NT) cur = nxt;
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
    const int nblk = (sp.T1 + 64 * kOutTiles - 1) / (64 * kOutTiles);
    const int gout = (int)(pr->B * pr->H * nblk);
    const void *fo = V == 64 ? (const void *)&split_out_kernel<K, 64, OT> : (const void *)&split_out_kernel<K, 128, OT>;
    return launch_kernel(fo, gout, &sp, s, 256);
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
