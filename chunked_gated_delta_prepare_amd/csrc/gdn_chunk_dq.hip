// libgdn: dq's chunk-start-state term as a kernel of its own,
//     dq[t] = h_c dO_t     (t in chunk c, h_c = hck[b, c, h], K x V),
// from saved chunk-start states (gdn_forward_states) and dO.  This is the
// product that the kernel-fun KDA re-scan page fuses into its re-scan
// (DQ = dO h^T with a cross-V-tile fp32 reduction); its own measurements
// found the fused form slower, and gdn_rescan_dq and this kernel let the
// two forms be compared here.
//
// One workgroup of four waves per (batch, chunk, head).  The product is
// formed transposed, DQ^T = h_c dO^T, so that both MFMA operands are rows
// read straight from HBM (16 contiguous bytes per lane: a row of h_c and a
// row of dO over 8 value columns) and each lane's result is 4 consecutive
// keys of one token, stored as 8-byte pieces (paired with the next lane's).  Wave w takes key tiles
// [w K/64, (w + 1) K/64) and every token tile, so h_c is read once per
// workgroup and dO (the smaller tile) once per wave, through the cache.
// Tokens past T read zero and their stores are dropped by the buffer
// range.  With fp32 states, h_c enters as bf16 high and low parts (two
// MFMAs), which keeps ~16 bits of it; bf16 states are exact.
#include "gdn_buffer.h"
#include "gdn_internal.h"

namespace gdn {

struct ChunkDqParams {
    const void *dout;
    const void *hck;
    float *dq;
    int T, H, NT;
};

namespace {

template <typename HT> struct HFrag;
template <> struct HFrag<bf16_t> {
    static constexpr int kParts = 1;
    bf16x8 part[1];
    __device__ void load(rsrc_t r, uint32_t voff) { part[0] = __builtin_bit_cast(bf16x8, bload128(r, voff, 0)); }
};
template <> struct HFrag<float> {
    static constexpr int kParts = 2;
    bf16x8 part[2];
    __device__ void load(rsrc_t r, uint32_t voff) {
        const u32x4 a = bload128(r, voff, 0), b = bload128(r, voff + 16, 0);
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = __uint_as_float(j < 4 ? a[j] : b[j - 4]);
            hi[j] = f32_to_bf16_bits(x);
            lo[j] = f32_to_bf16_bits(x - __uint_as_float((uint32_t)hi[j] << 16));
        }
        part[0] = __builtin_bit_cast(bf16x8, hi);
        part[1] = __builtin_bit_cast(bf16x8, lo);
    }
};

template <int C, int K, int V, typename HT>
__global__ __launch_bounds__(256) void chunk_dq_kernel(ChunkDqParams p) {
    constexpr int NTT = C / 16;          // token tiles
    constexpr int MT = K / 64;           // key tiles per wave
    constexpr int NS = V / 32;           // 32-wide steps over the value columns
    const int wv = wave_id(), l = lane_id();
    const int bid = blockIdx.x;
    const int h = bid % p.H, bc = bid / p.H, c = bc % p.NT, b = bc / p.NT;
    const int rows = min(C, p.T - c * C);
    const int64_t tok0 = (int64_t)b * p.T + (int64_t)c * C;
    const uint32_t HV = (uint32_t)p.H * V, HK = (uint32_t)p.H * K;
    const rsrc_t rdo = make_rsrc((const bf16_t *)p.dout + tok0 * HV, (uint32_t)rows * HV * 2);
    const rsrc_t rdq = make_rsrc(p.dq + tok0 * HK, (uint32_t)rows * HK * 4);
    const rsrc_t rh = make_rsrc((const HT *)p.hck + (((int64_t)b * p.NT + c) * p.H + h) * (K * V),
                                (uint32_t)(K * V * sizeof(HT)));
    const int col = 8 * (l >> 4);        // this lane's first value column of a step

    HFrag<HT> a[MT][NS];
    bf16x8 bo[NTT][NS];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            a[m][s].load(rh, (uint32_t)((16 * (MT * wv + m) + (l & 15)) * V + 32 * s + col) * sizeof(HT));
#pragma unroll
    for (int n = 0; n < NTT; ++n)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            bo[n][s] = __builtin_bit_cast(bf16x8, bload128(rdo, ((uint32_t)(16 * n + (l & 15)) * HV +
                                                                 (uint32_t)h * V + 32 * s + col) * 2, 0));
    // every load is in flight before the first product: left to itself the
    // scheduler interleaves them with the MFMAs to save registers, which
    // makes three or four memory round trips of one
    __builtin_amdgcn_sched_barrier(0);
    float4v acc[MT][NTT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NTT; ++n) acc[m][n] = float4v{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NTT; ++n)
#pragma unroll
                for (int q = 0; q < HFrag<HT>::kParts; ++q)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][s].part[q], bo[n][s], acc[m][n], 0, 0, 0);
    // Lane (g, j) holds keys 16 (MT wv + m) + 4 g .. + 3 of token 16 n + j.
    // Neighbouring lanes (tokens j, j ^ 1) swap halves, so that each 8-byte
    // store of a lane pair fills 16 contiguous bytes of one token's row and
    // an instruction writes whole 64-byte pieces of 8 rows: the even lane
    // stores its keys +0, +1 of token j and the odd lane's of token j + 1,
    // the odd lane the even lane's +2, +3 of token j and its own of j + 1.
    const bool odd = l & 1;
    const uint32_t tok_a = (uint32_t)(l & 14), half = 8 * (uint32_t)odd;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NTT; ++n) {
            const float4v x = acc[m][n];
            const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
            const float r0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0xB1, 0xf, 0xf, false));
            const float r1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xf, 0xf, false));
            const uint32_t off = ((uint32_t)(16 * n) + tok_a) * HK * 4 +
                                 ((uint32_t)h * K + 16 * (MT * wv + m) + 4 * (l >> 4)) * 4 + half;
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{__float_as_uint(odd ? r0 : x[0]), __float_as_uint(odd ? r1 : x[1])}, rdq, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{__float_as_uint(odd ? x[2] : r0), __float_as_uint(odd ? x[3] : r1)}, rdq, off + HK * 4, 0, 0);
        }
}

template <int C, int K, int V>
const void *chunk_dq_fn(bool h_f32) {
    return h_f32 ? (const void *)&chunk_dq_kernel<C, K, V, float> : (const void *)&chunk_dq_kernel<C, K, V, bf16_t>;
}

template <int C, int K>
const void *chunk_dq_v(int V, bool h_f32) {
    return V == 64 ? chunk_dq_fn<C, K, 64>(h_f32) : chunk_dq_fn<C, K, 128>(h_f32);
}

}  // namespace

gdn_status enqueue_chunk_dq(const gdn_problem *pr, const void *dout, const void *hck, float *dq,
                            hipStream_t s) {
    ChunkDqParams p;
    p.dout = dout; p.hck = hck; p.dq = dq;
    p.T = (int)pr->T; p.H = (int)pr->H;
    p.NT = (int)((pr->T + pr->chunk - 1) / pr->chunk);
    const bool h_f32 = pr->o_dtype == GDN_F32;
    const int V = (int)pr->V;
    const void *fn = pr->chunk == 32 ? (pr->K == 64 ? chunk_dq_v<32, 64>(V, h_f32) : chunk_dq_v<32, 128>(V, h_f32))
                                     : (pr->K == 64 ? chunk_dq_v<64, 64>(V, h_f32) : chunk_dq_v<64, 128>(V, h_f32));
    const int64_t grid = pr->B * (int64_t)p.NT * pr->H;
    return launch_kernel(fn, (int)grid, &p, s, 256);
}

}  // namespace gdn
