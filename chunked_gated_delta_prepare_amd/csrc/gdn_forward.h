// gdn_forward kernel: prepare and scan fused, one pass over q, k, v.
//
// One workgroup per (batch, head, 64-wide V tile), serial over chunks.  Per
// chunk of C tokens with chunk-start state h (K x 64 slice, fp32 registers):
//   gcum  chunk-local inclusive cumsum of g
//   A     strictly lower beta * (k k^T * decay)           (Gram on the MFMA)
//   Tm    (I + A)^-1: the 16 x 16 diagonal blocks inverted, the rest
//         applied by blocks in the chain (see solve_block)
//   X     k h                     R' = v - e^gcum * X       (GDN)
//   v'    Tm diag(beta) R'        (= u - w h of the WY form, without forming
//                                   w or u: the KDA re-scan page's v')
//   o     e^gcum * (q h) + P v'   P = tril_incl(q k^T * decay)
//   h    <- e^gl h + (k * e^(gl - gcum))^T v'             (gl = last gcum)
// For the per-key gate (KDA) every exponent is per key dimension: the decays
// move into the operands, q e^gcum and k e^gcum (for X and Y) and
// k e^(gl - gcum) (for the state update), all decays, and the chunk's A, its
// inverse by blocks and P (whose decays no row factor alone can carry)
// come from kda_gram_kernel through the workspace.
//
// Work split.  The state update is the serial chain; each wave owns 16 of the
// tile's 64 value columns (its slice of h, v', o), so the chain is wave-local
// and needs no barrier.  The chunk's shared operands (q, k, P, Tm) are built
// cooperatively in phases separated by workgroup barriers:
//   phase 0  registers -> LDS operands; gate cumsum and row factors; the next
//            chunk's loads are issued
//   phase 1  Gram tiles; diagonal 16x16 inverses T_bb and the first solve
//            block by the wave that computed their Gram tiles
//   phase 2  the remaining solve blocks (C = 64)
//   phase 3  the wave-local chain, which finishes the triangular solve by
//            blocks of 16 tokens (see solve_block)
// All HBM traffic is buffer loads/stores; a stream's byte range ends at token
// T, so the rows of a short last chunk read as zero (an identity step: g = 0,
// beta = 0, k = 0) and their outputs are dropped by the hardware.
#pragma once

#include <type_traits>

#include "gdn_buffer.h"
#include "gdn_chunk_io.h"
#include "gdn_inverse.h"
#include "gdn_scan.h"

namespace gdn {

struct FwdParams {
    const void *q, *k, *v;
    const float *beta, *g, *h0;
    void *o;
    float *hT;
    // saved states (o dtype; both NULL unless the states instance runs):
    // hck [B, NT, H, K, V] the state at each chunk start, vnew [B, T, H, V]
    // the delta v' each token writes into the state
    void *hck, *vnew;
    // packed sequences: NULL, or B + 1 token offsets (int32) into a
    // [1, T, H, .] layout, sequence b being tokens [cu[b], cu[b+1])
    const int *cu;
    // backward re-scan: dO [B, T, H, V] (io dtype) in, dq's chunk-start-state
    // term [B, T, H, K] (fp32, accumulated into) out; both NULL otherwise
    const void *dout;
    float *dq;
    // bounded LDS waits of the pipelined kernels (see WaitCtl): a device word
    // that counts waits that gave up (NULL: not counted), the poll limit, and
    // a bias added to every wait target (0; a value no counter reaches makes
    // every wait give up, which the host sets only to test this path)
    unsigned *wait_count;
    unsigned wait_limit, wait_bias;
    // per-key gate: the workspace kda_gram_kernel filled, a slot of Tmb and P
    // ([2][C][C], operand type) per (chunk, head), chunks of stream b from
    // slot b * nt (fixed length) or after those of the sequences before b
    const void *ws;
    int B, T, H, V;
    int nvt;        // V / 64
    int swizzle;
    // sequence split (SP instances of forward_pipe_kernel): each stream is cut
    // at token sp_t; the first sp_g0 workgroups run the first segment from h0
    // (end state to sp_h0out [B, H, K, V]); the rest run the second segment
    // twice in one pass over its chunks, as nvt ordinary V tiles from a zero
    // state (o into o, end state to sp_N [B, H, K, V]) and K / 64 identity
    // tiles with v = 0 and h0 = I (o into sp_oI [B, T - sp_t, H, K], end state
    // to sp_M [B, H, K, K])
    int sp_t, sp_g0;
    void *sp_oI;
    float *sp_h0out, *sp_N, *sp_M;
};

// Workspace slot of one (chunk, head) for the per-key gate.  It starts with
// Tmb then P, [C][C] row-major each in the operand type (kda_slot_elems
// elements).  With bf16 io (fp16 operands) the pipelined re-scan's operand
// tiles follow: qd = q e^gcum, kd = k e^gcum and kg = k e^(gl - gcum), [C][K]
// fp16 each, laid out as that kernel's LDS tiles (16-byte chunks swizzled by
// row, 4-column groups permuted: swz, pcol), then e^gl [K] fp32.
template <int C>
constexpr int64_t kda_slot_elems() { return 2 * (int64_t)C * C; }
template <int C, int K>
struct KdaSlotOps {
    static constexpr int kQd = 2 * C * C * 2;
    static constexpr int kKd = kQd + C * K * 2;
    static constexpr int kKg = kKd + C * K * 2;
    static constexpr int kFl = kKg + C * K * 2;
    static constexpr int kBytes = kFl + K * 4;
};
template <int C, int K, typename IO>
constexpr int64_t kda_slot_bytes() {
    return sizeof(IO) == 4 ? kda_slot_elems<C>() * 4 : (int64_t)KdaSlotOps<C, K>::kBytes;
}

// The tokens of stream b: batch row b, [0, T) of a [B, T, H, .] layout, or
// with VL (cu set) the packed sequence b, tokens [cu[b], cu[b+1]) of a
// [1, T, H, .] layout, the offsets clamped to [0, T] so that no value of cu
// can reach outside the tensors.  row0 is the stream's first (token, head)
// row for head h.
struct StreamRange {
    int T;
    int64_t row0;
};
template <bool VL>
__device__ __forceinline__ StreamRange stream_range(const FwdParams &p, int b, int h) {
    if constexpr (VL) {
        const int c0 = __builtin_amdgcn_readfirstlane(p.cu[b]);
        const int c1 = __builtin_amdgcn_readfirstlane(p.cu[b + 1]);
        const int bos = min(max(c0, 0), p.T);
        const int eos = min(max(c1, bos), p.T);
        return StreamRange{eos - bos, (int64_t)bos * p.H + h};
    } else {
        return StreamRange{p.T, (int64_t)b * p.T * p.H + h};
    }
}

template <int C, int K, typename IO, bool KEYGATE>
struct FwdLayout {
    typedef typename OpOf<IO>::type OpT;
    static constexpr int NB = C / 16;
    static constexpr int LDK = K + Mma<OpT>::kPad;
    static constexpr int LDC = C + Mma<OpT>::kPad;
    static constexpr int LDA = C + 4;
    static constexpr int E = sizeof(OpT);
    static constexpr int kQ = 0;                                   // [C][LDK]
    static constexpr int kK = kQ + C * LDK * E;                    // [C][LDK]
    static constexpr int kKi = kK + C * LDK * E;                   // KDA: [C][LDK]
    static constexpr int kTmb = kKi + (KEYGATE ? C * LDK * E : 0);  // [C][LDC] solve blocks
    static constexpr int kP = kTmb + C * LDC * E;                  // [C][LDC]
    // bf16 io: chunk data is prefetched from HBM straight into LDS: raw q, k
    // in per-thread vector order (each thread later converts the vectors its
    // own lanes fetched), and the v tile row-major [C][64], double buffered
    // because the chain of one chunk reads it while the next one lands.
    // fp32 io prefetches into registers instead.
    static constexpr bool kStage = sizeof(IO) == 2;
    static constexpr int LDV = 64;
    static constexpr int kSq = kP + C * LDC * E;
    static constexpr int kSk = kSq + (kStage ? C * K * 2 : 0);
    static constexpr int kVs = kSk + (kStage ? C * K * 2 : 0);
    static constexpr int kScr = kVs + (kStage ? 2 * C * LDV * 2 : 0);
    // scratch: GDN, fp32 A and Tm of the inverse; KDA, the fp32 gcum rows
    // [C][K] of phase 0 (the KDA chunk's A, inverse and P come from the
    // workspace).  Where that would not fit, the gcum rows share the Tmb / P
    // tiles, which phase 0 fills only after the operands are built.
    static constexpr int kA = kScr;
    static constexpr int kTm = kA + C * LDA * 4;
    static constexpr int kRowN = KEYGATE ? (C + 2 * K + (kThreads * 4 / K) * K) : (5 * C + NB * C + 4);
    static constexpr int kGBytes = C * K * 4;
    static constexpr bool kAliasG = KEYGATE && kScr + kGBytes + kRowN * 4 > kLdsBytesMax &&
                                    2 * C * LDC * E >= kGBytes;
    static constexpr int kGst = kAliasG ? kTmb : kScr;
    static constexpr int kScrBytes = KEYGATE ? (kAliasG ? 0 : kGBytes) : 2 * C * LDA * 4;
    // per-row / per-key fp32 factors
    static constexpr int kRow = kScr + kScrBytes;
    // KDA cumsum segments: a thread holds 4 key columns of C / NSEG rows
    static constexpr int NSEG = kThreads * 4 / K;
    static constexpr int kBytes = kRow + kRowN * 4;
};

// Diagonal 16x16 inverses T_bb = (I + A_bb)^-1 for the blocks in [b0, b0+nb)
// by one wave: lane (blk = l/16, column j = l%16) runs forward substitution
// down its column (each row of A_bb is a broadcast read).  Writes T_bb to Tm.
template <int LDA>
__device__ __forceinline__ void diag_inverse(const float *A, float *Tm, int b0, int nb) {
    const int l = lane_id(), blk = l >> 4, j = l & 15;
    if (blk < nb) {
        const int bb = b0 + blk;
        const float *Ab = A + 16 * bb * LDA + 16 * bb;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float row[16];
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4) {
                if (kk < i) {
                    const float4v a4 = *(const float4v *)(Ab + i * LDA + kk);
                    row[kk] = a4[0]; row[kk + 1] = a4[1]; row[kk + 2] = a4[2]; row[kk + 3] = a4[3];
                }
            }
            float s0 = (i == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
            for (int kk = 0; kk < i; kk += 2) {
                s0 -= row[kk] * t[kk];
                if (kk + 1 < i) s1 -= row[kk + 1] * t[kk + 1];
            }
            t[i] = s0 + s1;
        }
        float *Tb = Tm + 16 * bb * LDA + 16 * bb;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * LDA + j] = t[i];
    }
}

// (I + A)^-1 is never formed whole: the chain solves (I + A) v' = diag(beta) R'
// by blocks of 16 tokens,
//     v'_b = Tb_bb R'_b + sum_{j<b} Mn_bj v'_j,
//     Tb_bb = T_bb diag(beta_b),  Mn_bj = -T_bb A_bj,  T_bb = (I + A_bb)^-1,
// with row block b of the C x C operand tile Tmb holding [Mn_b0 .. | Tb_bb | 0]
// (the TileOPs fused-prepare page's A_g inverse, applied by blocks).  This
// writes Mn_ij (one 16 x 16 product, one wave) into Tmb.
template <int LDA, int LDC, typename OpT>
__device__ __forceinline__ void solve_block(const float *A, const float *Tm, OpT *Tmb,
                                            int i, int j) {
    const int l = lane_id(), g4 = 4 * (l >> 4), col = l & 15;
    float4v a;                      // A_ij in accumulator layout
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = A[(16 * i + g4 + r) * LDA + 16 * j + col];
    float4v y = {0, 0, 0, 0};
    mm16_f32_regB(y, Tm + 16 * i * LDA + 16 * i, LDA, a);
#pragma unroll
    for (int r = 0; r < 4; ++r) Tmb[(16 * i + g4 + r) * LDC + 16 * j + col] = Mma<OpT>::cvt(-y[r]);
}

// Copy a diagonal block of Tm into Tmb scaled by beta of its columns.  (The
// blocks above the diagonal, which the chain's rounded-up k range also reads,
// stay zero from the clear at kernel start.)
template <int LDA, int LDC, typename OpT>
__device__ __forceinline__ void emit_diag(const float *Tm, OpT *Tmb, const float *bet, int b) {
    const int l = lane_id();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = l + 64 * e, row = 16 * b + (idx >> 4), col = 16 * b + (idx & 15);
        Tmb[row * LDC + col] = Mma<OpT>::cvt(Tm[row * LDA + col] * bet[col]);
    }
}

// Four consecutive operand values of one row, one vector store.
__device__ __forceinline__ void store_row4(_Float16 *dst, const float4v &a) {
    half4 h;
    h[0] = (_Float16)a[0]; h[1] = (_Float16)a[1]; h[2] = (_Float16)a[2]; h[3] = (_Float16)a[3];
    *(half4 *)dst = h;
}
__device__ __forceinline__ void store_row4(float *dst, const float4v &a) { *(float4v *)dst = a; }

template <int C, int K, typename IO, typename OT, bool KEYGATE, bool ST = false, bool VL = false>
__global__ __launch_bounds__(kThreads, 1) void forward_kernel(FwdParams p) {
    typedef FwdLayout<C, K, IO, KEYGATE> L;
    typedef typename L::OpT OpT;
    typedef Mma<OpT> M;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDA = L::LDA;
    constexpr int NB = C / 16, NKB = K / 16;
    constexpr int SIO = sizeof(IO), SO = sizeof(OT);
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");
    static_assert(NB == 2 || NB == 4, "chunk 32 or 64");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OpT *Qs = (OpT *)(smem + L::kQ);      // GDN q; KDA q e^gcum
    OpT *Ks = (OpT *)(smem + L::kK);      // GDN k; KDA k e^gcum
    OpT *Ki = KEYGATE ? (OpT *)(smem + L::kKi) : Ks;   // KDA k e^(gl - gcum)
    OpT *Tmb = (OpT *)(smem + L::kTmb);
    OpT *Ps = (OpT *)(smem + L::kP);
    uint16_t *Sq = (uint16_t *)(smem + L::kSq);
    uint16_t *Sk = (uint16_t *)(smem + L::kSk);
    uint16_t *Vs = (uint16_t *)(smem + L::kVs);
    float *Af = (float *)(smem + L::kA);
    float *Tmf = (float *)(smem + L::kTm);
    float *Gst = (float *)(smem + L::kGst);
    float *rowf = (float *)(smem + L::kRow);
    // GDN row factors (gcv: gcum itself)
    float *gcv = rowf, *eg = rowf + C, *egl = rowf + 2 * C, *bet = rowf + 3 * C;
    float *einv = rowf + 4 * C, *efac = rowf + 5 * C, *misc = rowf + 5 * C + NB * C;
    // KDA key factors (beta takes the first C slots)
    float *kbet = rowf, *flv = rowf + C, *glv = rowf + C + K, *segt = rowf + C + 2 * K;
    float *betp = KEYGATE ? kbet : bet;

    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    const int g4 = 4 * (l >> 4);                 // first accumulator row of this lane

    int pair, vt;
    map_block(blockIdx.x, p.nvt, p.swizzle, pair, vt);
    const int b = pair / p.H, h = pair - b * p.H;
    const StreamRange sr = stream_range<VL>(p, b, h);
    const int T = sr.T, H = p.H, V = p.V;
    const int vcol = vt * 64 + 16 * wv + acc_col();          // this lane's value column
    const int nt = (T + C - 1) / C;
    // per-key gate: this stream's first workspace slot (chunk n: slot0 + n)
    int slot0 = 0;
    if constexpr (KEYGATE) {
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
    }

    // ---- buffer descriptors: each covers this (b, h) stream up to token T
    const int64_t row0 = sr.row0;
    const uint32_t rsK = (uint32_t)(H * K), rsV = (uint32_t)(H * V);
    const uint32_t rsG = KEYGATE ? rsK : (uint32_t)H;
    const rsrc_t rq_ = make_rsrc((const IO *)p.q + row0 * K, (uint32_t)T * rsK * SIO);
    const rsrc_t rk_ = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)T * rsK * SIO);
    const rsrc_t rv_ = make_rsrc((const IO *)p.v + row0 * V, (uint32_t)T * rsV * SIO);
    const rsrc_t ro_ = make_rsrc((OT *)p.o + row0 * V, (uint32_t)T * rsV * SO);
    const rsrc_t rg_ = make_rsrc(p.g + row0 * (KEYGATE ? K : 1), (uint32_t)T * rsG * 4);
    const rsrc_t rb_ = make_rsrc(p.beta + row0, (uint32_t)T * (uint32_t)H * 4);

    // per-thread constant offsets
    constexpr int NVEC = C * K / 8 / kThreads;               // q/k vectors per thread
    uint32_t qk_off[NVEC];
#pragma unroll
    for (int j = 0; j < NVEC; ++j) {
        const int i = tid + kThreads * j, row = i / (K / 8), col = 8 * (i % (K / 8));
        qk_off[j] = ((uint32_t)row * rsK + col) * SIO;
    }
    const uint32_t v_off = ((uint32_t)g4 * rsV + vcol) * SIO;
    constexpr int NVV = L::kStage ? C * 64 / 8 / kThreads : 1;   // v vectors per thread
    uint32_t vv_off[NVV];
#pragma unroll
    for (int j = 0; j < NVV; ++j) {
        const int i = tid + kThreads * j, row = i / 8, col = 8 * (i % 8);
        vv_off[j] = ((uint32_t)row * rsV + vt * 64 + col) * SIO;
    }
    const uint32_t o_off = ((uint32_t)g4 * rsV + vcol) * SO;
    const rsrc_t rvn_ = make_rsrc(ST ? (OT *)p.vnew + row0 * V : nullptr, ST ? (uint32_t)T * rsV * SO : 0u);
    // saved states leave the accumulators as column pairs (store_acc_pairs)
    const uint32_t prow = (uint32_t)(g4 + 2 * (l & 1));
    const uint32_t vn_off = (prow * rsV + (vcol & ~1)) * SO;
    const uint32_t hck_off = (prow * V + (vcol & ~1)) * SO;
    // KDA gate: thread (kseg, cg) holds rows kseg NR .. +NR-1 of the four key
    // columns 4 cg .. 4 cg + 3, one 16-byte load per row (one load per lane
    // per row would take four times the vector-memory instructions, and the
    // waves stall at issue while the loads of a chunk queue up)
    constexpr int NR = KEYGATE ? C * K / (4 * kThreads) : 1;
    const int kseg = KEYGATE ? tid / (K / 4) : 0, kcol = KEYGATE ? 4 * (tid % (K / 4)) : 0;
    const uint32_t g_off = KEYGATE ? ((uint32_t)(kseg * NR) * rsG + kcol) * 4
                                   : (uint32_t)l * rsG * 4;

    // ---- state: hacc[i][r] = h[16 i + 4 (l/16) + r][vcol]
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
    // the operand tiles above the diagonal are read but stay zero
    for (int i = tid; i < C * LDC; i += kThreads) {
        Tmb[i] = (OpT)0.f;
        Ps[i] = (OpT)0.f;
    }

    // ---- prefetch registers
    constexpr int NRQ = L::kStage ? 1 : NVEC;
    Raw8B<IO> rq[NRQ], rk[NRQ];         // fp32 io: q, k rows
    float vreg[L::kStage ? 1 : NB][4];  // fp32 io: v in accumulator layout
    float g_own[KEYGATE ? 1 : NR];
    float4v gk4[KEYGATE ? NR : 1];      // KDA: gates of four key columns per row
    float b_own = 0.f;
    // (the gate and beta loads go first: the staged loads are then the last
    // memory operations of a chunk before its outputs are stored)
    // The loads of a chunk come in parts (kLd*), so that the staged path can
    // spread them over the previous chunk: the CU's memory pipeline takes
    // about a cycle per 64 bytes, and a wave that issues more loads than it
    // queues stalls at issue until they drain.
    enum { kLdG = 1, kLdQ = 2, kLdK = 4, kLdV = 8, kLdAll = 15 };
    auto load_gate_rows = [&](int c, int i0, int n) {      // KDA gate rows i0 .. i0+n-1
        const uint32_t t0 = (uint32_t)(c * C);
#pragma unroll
        for (int i = i0; i < i0 + n; ++i)
            gk4[i] = __builtin_bit_cast(float4v, bload128(rg_, g_off, (t0 + i) * rsG * 4));
    };
    auto load_beta = [&](int c) {
        const uint32_t t0 = (uint32_t)(c * C);
        b_own = __uint_as_float(bload32(rb_, (uint32_t)l * (uint32_t)H * 4, t0 * (uint32_t)H * 4));
    };
    auto load_chunk = [&](int c, int parts) {
        const uint32_t t0 = (uint32_t)(c * C);
        if (parts & kLdG) {
            if constexpr (KEYGATE) load_gate_rows(c, 0, NR);
            else g_own[0] = __uint_as_float(bload32(rg_, g_off, t0 * rsG * 4));
            load_beta(c);
        }
        if constexpr (L::kStage) {
#if defined(__HIP_DEVICE_COMPILE__)
            // (device pass only: seen by the host pass, this builtin makes it
            // drop the kernel's launch stub without a diagnostic)
            // LDS destination of lane l: base + 16 l, base uniform per wave
            typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                const int blk = (j * kThreads + wv * 64) * 8;     // in 16-bit elements
                if (parts & kLdQ)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq_, (lds_void *)(Sq + blk), 16,
                                                             qk_off[j], t0 * rsK * SIO, 0, 0);
                if (parts & kLdK)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk_, (lds_void *)(Sk + blk), 16,
                                                             qk_off[j], t0 * rsK * SIO, 0, 0);
            }
            uint16_t *vdst = Vs + (c & 1) * C * L::LDV;
            if (parts & kLdV) {
#pragma unroll
                for (int j = 0; j < NVV; ++j)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv_, (lds_void *)(vdst + (j * kThreads + wv * 64) * 8),
                                                             16, vv_off[j], t0 * rsV * SIO, 0, 0);
            }
#endif
        } else {
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                rq[j].load(rq_, qk_off[j], t0 * rsK * SIO);
                rk[j].load(rk_, qk_off[j], t0 * rsK * SIO);
            }
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vreg[cb][r] = BufElem<IO>::load(rv_, v_off, (t0 + 16 * cb + r) * rsV * SIO);
        }
    };
    if (nt > 0) load_chunk(0, kLdAll);
    // staged path: the parts of chunk c+1 issued during chunk c
    //   KDA gate rows and beta   phase 0, two rows per operand vector, once
    //                            the gate scan of chunk c is done with them
    //   (scalar gate and beta)   phase 1
    //   q                        phase 1        k   phase 2 (C = 64) or 3
    //   v                        phase 3
    constexpr int kLdP1 = kLdQ | (KEYGATE ? 0 : kLdG);
    constexpr int kLdP2 = NB == 4 ? kLdK : 0;
    constexpr int kLdP3 = kLdV | (NB == 4 ? 0 : kLdK);

    for (int c = 0; c < nt; ++c) {
        const uint32_t t0 = (uint32_t)(c * C);

        // ================= phase 0: operands into LDS =======================
        float vcur[NB][4];
        if constexpr (L::kStage) {
            // this chunk's staged loads were issued a chunk ago; only the
            // previous chunk's output stores may still be in flight after them
            if (c == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB * 4));
        } else {
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) vcur[cb][r] = vreg[cb][r];
        }
        if (wv == 1 && l < C) betp[l] = b_own;
        if constexpr (!KEYGATE) {
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                const int i = tid + kThreads * j, row = i / (K / 8), col = 8 * (i % (K / 8));
                if constexpr (L::kStage) {
                    Raw8B<IO> xq, xk;
                    stage_get(xq, Sq + i * 8);
                    stage_get(xk, Sk + i * 8);
                    put_raw8(Qs + row * LDK + col, xq);
                    put_raw8(Ks + row * LDK + col, xk);
                } else {
                    put_raw8(Qs + row * LDK + col, rq[j]);
                    put_raw8(Ks + row * LDK + col, rk[j]);
                }
            }
            if (wv == 0) {
                // inclusive scan of the gate down the chunk, then row factors
                float x = l < C ? g_own[0] : 0.f;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const float y = __shfl_up(x, d);
                    if (l >= d) x += y;
                }
                // Every factor a product uses is at most 1 for any g <= 0:
                // off-diagonal Gram tiles (I > J) split e^(gcum_r - gcum_s)
                // at the end of block J, einv[s] = e^(gend_J - gcum_s) and
                // efac[J][r] = e^(gcum_r - gend_J); diagonal tiles take each
                // entry's decay from gcum directly.
                // gl: gcum at the chunk's last token (not a padded row's,
                // which the scan sums in another order), so that token's
                // e^(gl - gcum) is exactly 1
                const float gl = __shfl(x, min(C, T - (int)t0) - 1);
                const float gref = __shfl(x, l | 15);       // gcum at the end of l's block
                float ef[NB];
#pragma unroll
                for (int J = 0; J < NB; ++J) ef[J] = __shfl(x, 16 * J + 15);
                if (l < C) {
                    gcv[l] = x;
                    eg[l] = fast_exp(x);
                    egl[l] = fast_exp(gl - x);
                    einv[l] = fast_exp(gref - x);
#pragma unroll
                    for (int J = 0; J < NB; ++J) efac[J * C + l] = fast_exp(fminf(x - ef[J], 0.f));
                }
                if (l == 0) misc[0] = fast_exp(gl);
            }
            if constexpr (!L::kStage)
                if (c + 1 < nt) load_chunk(c + 1, kLdAll);
            __syncthreads();
        } else {
            // gcum down each key column: thread (seg, cg) holds NR rows of
            // four columns; segment totals are added in segment order
            float4v run = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < NR; ++i) { run += gk4[i]; gk4[i] = run; }
            *(float4v *)(segt + kseg * K + kcol) = run;
            __syncthreads();
            // (gl, the chunk total, sums the segment totals in the same
            // order as the offsets, so it equals gcum at the last token)
            float4v off = {0, 0, 0, 0}, gtot = {0, 0, 0, 0};
#pragma unroll
            for (int sgi = 0; sgi < L::NSEG; ++sgi) {
                const float4v t = *(const float4v *)(segt + sgi * K + kcol);
                if (sgi < kseg) off += t;
                gtot += t;
            }
#pragma unroll
            for (int i = 0; i < NR; ++i)
                *(float4v *)(Gst + (kseg * NR + i) * K + kcol) = off + gk4[i];
            if (kseg == 0) *(float4v *)(glv + kcol) = gtot;
            __syncthreads();
            if (tid < K) flv[tid] = fast_exp(glv[tid]);
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                const int i = tid + kThreads * j, row = i / (K / 8), col = 8 * (i % (K / 8));
                float xq[8], xk[8], a[8], bq[8], bk[8];
                if constexpr (L::kStage) {
                    Raw8B<IO> sq, sk;
                    stage_get(sq, Sq + i * 8);
                    stage_get(sk, Sk + i * 8);
                    unpack_raw8(sq, xq);
                    unpack_raw8(sk, xk);
                } else {
                    unpack_raw8(rq[j], xq);
                    unpack_raw8(rk[j], xk);
                }
                // qd = q e^gcum, kd = k e^gcum, kg = k e^(gl - gcum): decays
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float gr = Gst[row * K + col + e];
                    const float up = fast_exp(gr), dn = fast_exp(glv[col + e] - gr);
                    a[e] = xq[e] * up;
                    bq[e] = xk[e] * up;
                    bk[e] = xk[e] * dn;
                }
                put8(Qs + row * LDK + col, a);
                put8(Ks + row * LDK + col, bq);
                put8(Ki + row * LDK + col, bk);
                if constexpr (L::kStage) {
                    // the next chunk's gate rows (NR = 2 NVEC), spread over
                    // the loop; this chunk's are in Gst by now
                    static_assert(NR == 2 * NVEC, "two gate rows per operand vector");
                    if (c + 1 < nt) {
                        load_gate_rows(c + 1, 2 * j, 2);
                        if (j == 0) load_beta(c + 1);
                    }
                }
            }
            if constexpr (!L::kStage)
                if (c + 1 < nt) load_chunk(c + 1, kLdAll);
            __syncthreads();
            // this chunk's Tmb and P, formed by kda_gram_kernel, from the
            // workspace (their tiles may have held the gcum rows until the
            // barrier above)
            {
                const OpT *src = (const OpT *)((const char *)p.ws +
                                               ((int64_t)(slot0 + c) * H + h) * kda_slot_bytes<C, K, IO>());
                constexpr int PER = 16 / L::E;
                for (int i = tid; i < 2 * C * C / PER; i += kThreads) {
                    const int e0 = i * PER, tile = e0 / (C * C), rc = e0 % (C * C);
                    const u32x4 w = *(const u32x4 *)(src + e0);
                    *(u32x4 *)((tile ? Ps : Tmb) + (rc / C) * LDC + rc % C) = w;
                }
            }
            __syncthreads();
        }

        // ================= phase 1: Gram, diagonal inverses, first solve block
        // Staged prefetch of the next chunk: issued here, after the barrier
        // that retires this chunk's staging reads, so that a whole phase of
        // work separates it from the next barrier (which waits for it).
        if constexpr (L::kStage)
            if (c + 1 < nt) load_chunk(c + 1, kLdP1);
        // Tile (I, J) is computed transposed (rows s of block J against rows
        // r of block I), so lane (l/16, j) ends up with row r = 16 I + j and
        // four consecutive columns s = 16 J + 4 (l/16) + e: one vector store.
        // (The per-key gate has its A, inverse and P from the workspace.)
        if constexpr (!KEYGATE) {
            auto gram_put = [&](int I, int J, bool isA, const float4v &acc) {
                const int r = 16 * I + acc_col(), s0 = 16 * J + g4;
                float4v fac = {1.f, 1.f, 1.f, 1.f};
                if constexpr (!KEYGATE) {
                    if (I == J) {
                        const float gr = gcv[r];
                        const float4v gs = *(const float4v *)(gcv + s0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) fac[e] = fast_exp(fminf(gr - gs[e], 0.f));
                    } else {
                        fac = *(const float4v *)(einv + s0) * efac[J * C + r];
                    }
                }
                if (isA) {
                    const float br = betp[r];
                    float4v a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = (s0 + e < r) ? acc[e] * fac[e] * br : 0.f;
                    *(float4v *)(Af + r * LDA + s0) = a;
                } else {
                    float4v a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = (s0 + e <= r) ? acc[e] * fac[e] : 0.f;
                    store_row4(Ps + r * LDC + s0, a);
                }
            };
            // Several tiles at once (a wave-uniform list): every fragment
            // load first, then the accumulations interleaved, so that one
            // wave per SIMD keeps the matrix pipe busy instead of waiting out
            // each tile's load and dependent accumulate latency in turn.
            auto gram_batch = [&](auto n_c, const int *tI, const int *tJ, const bool *tA) {
                constexpr int N = decltype(n_c)::value;
                typename M::frag fa[N][K / 32], fb[N][K / 32];
#pragma unroll
                for (int u = 0; u < N; ++u)
#pragma unroll
                    for (int k = 0; k < K / 32; ++k) {
                        fa[u][k] = M::load(frag_ptr(Ki + 16 * tJ[u] * LDK, LDK, 32 * k));
                        fb[u][k] = M::load(frag_ptr((tA[u] ? Ks : Qs) + 16 * tI[u] * LDK, LDK, 32 * k));
                    }
                float4v acc[N];
#pragma unroll
                for (int u = 0; u < N; ++u) acc[u] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int k = 0; k < K / 32; ++k)
#pragma unroll
                    for (int u = 0; u < N; ++u) M::mma(acc[u], fa[u][k], fb[u][k]);
#pragma unroll
                for (int u = 0; u < N; ++u) gram_put(tI[u], tJ[u], tA[u], acc[u]);
            };
            // tiles per batch: fp32 fragments are twice the registers
            constexpr int BATCH = sizeof(OpT) == 2 ? 4 : 1;
            const int pb = 2 * wv;          // diagonal pair (pb, pb+1) for waves 0 .. NB/2-1
            if (wv < NB / 2) {
                const int tI[3] = {pb, pb + 1, pb + 1}, tJ[3] = {pb, pb + 1, pb};
                const bool tA[3] = {true, true, true};
                if constexpr (BATCH >= 3) {
                    gram_batch(std::integral_constant<int, 3>{}, tI, tJ, tA);
                } else {
#pragma unroll
                    for (int u = 0; u < 3; ++u)
                        gram_batch(std::integral_constant<int, 1>{}, tI + u, tJ + u, tA + u);
                }
                if constexpr (sizeof(OpT) == 2) {
                    // fp16 operands: the two diagonal inverses on the matrix
                    // cores (block doubling), into Tm's fp32 rows
                    const int n = l & 15;
                    float4v ad[2], tr[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        ad[e] = *(const float4v *)(Af + (16 * (pb + e) + n) * LDA + 16 * (pb + e) + g4);
                    diag_inverse_mfma(ad, tr);
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        *(float4v *)(Tmf + (16 * (pb + e) + n) * LDA + 16 * (pb + e) + g4) = tr[e];
                } else {
                    diag_inverse<LDA>(Af, Tmf, pb, 2);
                }
                emit_diag<LDA, LDC, OpT>(Tmf, Tmb, betp, pb);
                emit_diag<LDA, LDC, OpT>(Tmf, Tmb, betp, pb + 1);
                solve_block<LDA, LDC, OpT>(Af, Tmf, Tmb, pb + 1, pb);
            }
            // the other tiles, round robin over the waves that hold no pair
            constexpr int NA_REST = (NB == 4) ? 4 : 0;    // A (2,0) (2,1) (3,0) (3,1)
            constexpr int NP = NB * (NB + 1) / 2;
            constexpr int NREST = NA_REST + NP;
            constexpr int W0 = NB / 2, NW = kWaves - NB / 2;
            constexpr int PER = NREST / NW;               // tiles t = (wv - W0) + NW u
            static_assert(NREST % NW == 0, "the other tiles split evenly over their waves");
            if (wv >= W0) {
                int tI[PER], tJ[PER];
                bool tA[PER];
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int t = (wv - W0) + NW * u;
                    if (t < NA_REST) {
                        tI[u] = 2 + t / 2; tJ[u] = t % 2; tA[u] = true;
                    } else {
                        const int idx = t - NA_REST;
                        int I = 0;
                        while ((I + 1) * (I + 2) / 2 <= idx) ++I;
                        tI[u] = I; tJ[u] = idx - I * (I + 1) / 2; tA[u] = false;
                    }
                }
#pragma unroll
                for (int u0 = 0; u0 < PER; u0 += BATCH) {
                    if constexpr (PER % BATCH == 0) {
                        gram_batch(std::integral_constant<int, BATCH>{}, tI + u0, tJ + u0, tA + u0);
                    } else {
                        if (u0 + BATCH <= PER)
                            gram_batch(std::integral_constant<int, BATCH>{}, tI + u0, tJ + u0, tA + u0);
                        else
                            gram_batch(std::integral_constant<int, PER % BATCH>{}, tI + u0, tJ + u0, tA + u0);
                    }
                }
            }
        }
        __syncthreads();

        // ================= phase 2: remaining solve blocks (C = 64) ==========
        if constexpr (L::kStage && kLdP2 != 0)
            if (c + 1 < nt) load_chunk(c + 1, kLdP2);
        if constexpr (NB == 4 && !KEYGATE) {
            // Mn_20, Mn_21, Mn_30, Mn_31: T_22 and T_33 from the pair waves,
            // the A blocks from the tile waves
            solve_block<LDA, LDC, OpT>(Af, Tmf, Tmb, 2 + (wv >> 1), wv & 1);
            __syncthreads();
        }

        // ================= phase 3: the wave-local chain =====================
        if constexpr (L::kStage)
            if (c + 1 < nt) load_chunk(c + 1, kLdP3);
        // Every intermediate (h, R', v') stays in registers: the accumulator
        // of one product is the B fragment of the next (see fragB_acc), the
        // shared operands come from LDS with matching split k slots.
        {
            if constexpr (ST) {
                // the state at the start of this chunk: hck[b, c, h, row, vcol]
                const rsrc_t rh = make_rsrc((OT *)p.hck + (((int64_t)b * nt + c) * H + h) * K * V,
                                            (uint32_t)(K * V * SO));
#pragma unroll
                for (int i = 0; i < NKB; ++i) store_acc_pairs<OT>(hacc[i], rh, hck_off, V * SO, 16 * i * V * SO);
            }
            float4v eg4[NB], egl4[NB];
            float el = 1.f;
            if constexpr (!KEYGATE) {
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    eg4[cb] = *(const float4v *)(eg + 16 * cb + g4);
                    egl4[cb] = *(const float4v *)(egl + 16 * cb + g4);
                }
                el = misc[0];
            }
            // h as B fragments over the key dimension
            typename M::frag hf[K / 32];
#pragma unroll
            for (int s = 0; s < K / 32; ++s) hf[s] = fragB_acc(hacc[2 * s], hacc[2 * s + 1], OpT{});
            // X = k h, Y = q h for this wave's 16 columns
            float4v xa[NB], ya[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                xa[cb] = float4v{0, 0, 0, 0};
                ya[cb] = float4v{0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < K / 32; ++s) {
                    M::mma(xa[cb], fragA_split(Ks, LDK, 16 * cb, 32 * s), hf[s]);
                    M::mma(ya[cb], fragA_split(Qs, LDK, 16 * cb, 32 * s), hf[s]);
                }
            }
            // R' = v - e^gcum X  (KDA: the decay is inside X already)
            if constexpr (L::kStage) {
                // v[16 cb + 4 (l/16) + e][this lane's column] for e = 0..3
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    const u32x2 w = read_T4(Vs + (c & 1) * C * L::LDV + 16 * cb * L::LDV, L::LDV, 16 * wv);
                    vcur[cb][0] = __uint_as_float(w[0] << 16);
                    vcur[cb][1] = __uint_as_float(w[0] & 0xffff0000u);
                    vcur[cb][2] = __uint_as_float(w[1] << 16);
                    vcur[cb][3] = __uint_as_float(w[1] & 0xffff0000u);
                }
            }
            float4v rr[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const float4v vv = {vcur[cb][0], vcur[cb][1], vcur[cb][2], vcur[cb][3]};
                if constexpr (KEYGATE) rr[cb] = vv - xa[cb];
                else rr[cb] = vv - eg4[cb] * xa[cb];
            }
            // v' solves (I + A) v' = diag(beta) R' by blocks of 16 tokens
            // (see solve_block): row block b of Tmb is [Mn_b0 .. | Tb_bb | 0],
            // so each step is a 32-wide k step over a [v' ; R'] fragment pair
            float4v da[NB];
            da[0] = float4v{0, 0, 0, 0};
            M::mma(da[0], fragA_split(Tmb, LDC, 0, 0), fragB_acc(rr[0], rr[1], OpT{}));
            da[1] = float4v{0, 0, 0, 0};
            M::mma(da[1], fragA_split(Tmb, LDC, 16, 0), fragB_acc(da[0], rr[1], OpT{}));
            if constexpr (NB == 4) {
                da[2] = float4v{0, 0, 0, 0};
                da[3] = float4v{0, 0, 0, 0};
                M::mma(da[2], fragA_split(Tmb, LDC, 32, 32), fragB_acc(rr[2], rr[3], OpT{}));
                const typename M::frag d01 = fragB_acc(da[0], da[1], OpT{});
                M::mma(da[2], fragA_split(Tmb, LDC, 32, 0), d01);
                M::mma(da[3], fragA_split(Tmb, LDC, 48, 0), d01);
                M::mma(da[3], fragA_split(Tmb, LDC, 48, 32), fragB_acc(da[2], rr[3], OpT{}));
            }
            if constexpr (ST) {
                // v' of this chunk's tokens (dropped past token T by the range)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    store_acc_pairs<OT>(da[cb], rvn_, vn_off, rsV * SO, (t0 + 16 * cb) * rsV * SO);
            }
            // o = e^gcum Y + P v'
            typename M::frag df[C / 32];
#pragma unroll
            for (int s = 0; s < C / 32; ++s) df[s] = fragB_acc(da[2 * s], da[2 * s + 1], OpT{});
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                float4v oa = {0, 0, 0, 0};
#pragma unroll
                for (int s = 0; s < C / 32; ++s)
                    if (32 * s < 16 * (cb + 1))
                        M::mma(oa, fragA_split(Ps, LDC, 16 * cb, 32 * s), df[s]);
                if constexpr (KEYGATE) oa = oa + ya[cb];
                else oa = oa + eg4[cb] * ya[cb];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    BufElem<OT>::store(oa[r], ro_, o_off, (t0 + 16 * cb + r) * rsV * SO);
            }
            // h <- e^gl h + kg^T v'
            if constexpr (!KEYGATE) {
#pragma unroll
                for (int s = 0; s < C / 32; ++s)
                    df[s] = fragB_acc(da[2 * s] * egl4[2 * s], da[2 * s + 1] * egl4[2 * s + 1], OpT{});
#pragma unroll
                for (int i = 0; i < NKB; ++i) {
                    hacc[i] = hacc[i] * el;
#pragma unroll
                    for (int s = 0; s < C / 32; ++s)
                        M::mma(hacc[i], fragAT_split(Ks, LDK, 16 * i, 32 * s), df[s]);
                }
            } else {
                // h = e^gl h + (k e^(gl - gcum))^T v', the decay row-wise
#pragma unroll
                for (int i = 0; i < NKB; ++i) {
                    float4v acc = {0, 0, 0, 0};
#pragma unroll
                    for (int s = 0; s < C / 32; ++s)
                        M::mma(acc, fragAT_split(Ki, LDK, 16 * i, 32 * s), df[s]);
                    hacc[i] = *(const float4v *)(flv + 16 * i + g4) * hacc[i] + acc;
                }
            }
        }
        __syncthreads();
    }

    if (p.hT) {
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.hT[((int64_t)pair * K + 16 * i + g4 + r) * V + vcol] = hacc[i][r];
    }
}

}  // namespace gdn
