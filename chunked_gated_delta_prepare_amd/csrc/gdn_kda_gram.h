// The per-key gate (Kimi-Delta-Attention): every chunk's exact decayed Gram
// products (exact_key_gram, gdn_key_gram.h) and the triangular factors the
// re-scan needs, in a kernel that runs over all chunks at once.
//
// kda_gram_kernel runs exact_key_gram for every (stream, chunk, head) in
// parallel and finishes what the re-scan needs from the chunk, in the
// re-scan kernels' operand layout: the solve tile Tmb (row block b =
// [Mn_b0 .. | Tb_bb | 0], Tb_bb = (I + A_bb)^-1 diag(beta_b),
// Mn_bj = -(I + A_bb)^-1 A_bj, the block solve of forward_kernel) and P, both
// [C][C] row-major in the operand type (fp16 for bf16 io, fp32 for fp32 io),
// written to a workspace slot per (chunk, head).  The 16 x 16 diagonal
// inverses are fp32 forward substitution here: off the serial path, their
// cost does not matter.
#pragma once

#include "gdn_forward.h"
#include "gdn_key_gram.h"

namespace gdn {

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

template <int C, int K, typename IO, bool VL>
__global__ __launch_bounds__(kThreads) void kda_gram_kernel(GramParams p) {
    typedef typename OpOf<IO>::type OpT;
    typedef GramLayout<C, K, OpT> L;
    constexpr int NR = KeyRows<C, K>::NR, NB = C / 16, LDA = L::LDA, LDC = L::LDC;
    constexpr int SIO = sizeof(IO), E = sizeof(OpT);
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OpT *Lk = (OpT *)(smem + L::kX);
    OpT *Lq = Lk + C * L::LDK;
    float *Tmf = (float *)(smem + L::kX);
    OpT *Tmb = (OpT *)(smem + L::kX + C * LDA * 4);
    OpT *Ps = Tmb + C * LDC;
    float *Af = (float *)(smem + L::kAf);
    float *Pf = (float *)(smem + L::kPf);
    float *segt = (float *)(smem + L::kSeg);
    float *gend = (float *)(smem + L::kGend);
    float *bet = (float *)(smem + L::kBet);

    const int h = blockIdx.x % p.H, slot = blockIdx.x / p.H;
    int b, c, T;
    int64_t tok0;
    if (!slot_chunk<C, VL>(p, slot, b, c, T, tok0)) return;
    const int tid = threadIdx.x, wv = wave_id();
    const int H = p.H;
    const uint32_t rsK = (uint32_t)(H * K);
    const int64_t row0 = tok0 * H + h;                      // (token, head) row of token 0
    const uint32_t t0 = (uint32_t)(c * C);
    const rsrc_t rg = make_rsrc(p.g + row0 * K, (uint32_t)T * rsK * 4);
    const rsrc_t rk = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)T * rsK * SIO);
    const rsrc_t rq = make_rsrc((const IO *)p.q + row0 * K, (uint32_t)T * rsK * SIO);
    const rsrc_t rb = make_rsrc(p.beta + row0, (uint32_t)T * (uint32_t)H * 4);

    if (tid < C) bet[tid] = __uint_as_float(bload32(rb, (t0 + tid) * (uint32_t)H * 4, 0));
    float4v gam[NR], kv[NR], qv[NR];
    load_key_rows<C, K, IO>(rg, rk, rq, rsK, t0, segt, gend, gam, kv, qv);
    exact_key_gram<C, K, OpT, true, true>(gam, kv, qv, gend, bet, Lk, Lq, Af, Pf);

    // ---- (I + A)^-1 by blocks: diagonal inverses, then Tb and Mn into Tmb
    if (wv == 0) diag_inverse<LDA>(Af, Tmf, 0, NB);
    for (int i = tid; i < 2 * C * LDC; i += kThreads) Tmb[i] = (OpT)0.f;
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
    for (int i = tid; i < C * C; i += kThreads) Ps[(i / C) * LDC + (i % C)] = Mma<OpT>::cvt(Pf[(i / C) * LDA + (i % C)]);
    __syncthreads();

    // ---- out: Tmb then P, row-major, 8 bytes per store
    const int64_t slot_off = ((int64_t)slot * H + h) * kda_slot_elems<C>() * E;
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

}  // namespace gdn
