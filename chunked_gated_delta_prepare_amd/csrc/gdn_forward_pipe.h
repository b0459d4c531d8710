// gdn_forward, pipelined over chunks (scalar gate per head, bf16 io).
//
// The per-chunk algebra is the one of forward_kernel (gdn_forward.h): the
// WY prepare of the TileOPs fused-prepare page (gate cumsum, decayed Gram,
// (I + A)^-1) and the inter-chunk re-scan of the kernel-fun KDA re-scan page
// (v' = (I + A)^-1 diag(beta) (v - e^gcum k h), o = e^gcum q h + P v', h
// update).  (I + A)^-1 is never formed whole: the prepare provides the
// inverted 16 x 16 diagonal blocks and the blocks -T_bb A_bj, and the chain
// finishes the triangular solve by blocks of 16 tokens.
//
// What changes is the schedule.  Only the re-scan depends on the state h;
// the prepare of a chunk needs nothing but that chunk's q, k, g and beta.  So
// the workgroup has eight waves in two roles:
//   chain waves 0..3   the re-scan of chunk c: h in MFMA accumulators, each
//                      wave owns 16 of the tile's 64 value columns
//   prepare waves 4..7 chunk c+1: fp16 q/k tiles, Gram tiles, the inverted
//                      diagonal blocks and the solve blocks, P; they also
//                      issue the loads of chunk c+2
// Chain wave 0 also computes chunk c+1's gate cumsum and row factors at the
// start of chunk c and signals the prepare waves through an LDS counter.
// and one workgroup barrier per chunk hands the prepared buffers over.  The
// shared operands, the raw v tile included, are double buffered (slot c & 1).
// The prepare waves hold the next chunk's q, k, v, g and beta in registers
// (loaded a chunk ahead) and order their own phases with an LDS arrival
// counter, so the chain waves never wait on them mid-chunk.
//
// q/k/Tm/P tiles are stored without padding, 16-byte chunks XOR-swizzled by
// row (see swz), which keeps the fragment reads free of bank conflicts and
// the transposed (ds_read_b64_tr_b16) reads at their minimum inside the
// 160 KB budget.
#pragma once

#include "gdn_forward.h"

namespace gdn {

constexpr int kPipeThreads = 512;

// Element (row, col) of an fp16 tile with rows of LD halves: the 16-byte
// chunk j of row r sits at chunk position j ^ s(r).  For 64- and 32-half
// rows s(r) = r mod LD/8.  The 128-half q/k tiles are read two ways, as
// 16-byte row fragments (16 rows, one chunk each) and by transposed 8-byte
// reads (four rows, the same half of four chunks each); s is then the
// GF(2)-linear map of r mod 16 with s(1) = 14, s(2) = 1, s(4) = 11,
// s(8) = 8, picked by measurement among the maps that keep the fragment
// reads free of bank conflicts: it leaves the transposed reads at the
// two-way minimum that the permuted columns allow (the plain map r mod 16
// costs four-way).
template <int LD>
__device__ __forceinline__ int swz(int row, int col) {
    constexpr int NC = LD / 8;
    if constexpr (NC == 16) {
        const int s = ((row & 1) ? 14 : 0) ^ ((row & 2) ? 1 : 0) ^ ((row & 4) ? 11 : 0) ^ ((row & 8) ? 8 : 0);
        return row * LD + (((col >> 3) ^ s) << 3) + (col & 7);
    }
    return row * LD + (((col >> 3) ^ (row & (NC - 1))) << 3) + (col & 7);
}

// Operand tiles keep their columns permuted within each 32-column group:
// the 4-column group a (columns 4a .. 4a+3) sits at slot 2a for a < 4 and
// at slot 2(a-4)+1 otherwise.  Lane group q's split k slots {4q .. 4q+3} and
// {16+4q .. 16+4q+3} (see fragA_split) are then the one 16-byte chunk at
// slots 2q, 2q+1, so every A fragment is a single aligned read.  Any
// product over the permuted columns pairs equal positions on both sides, so
// Gram tiles read the permuted tiles as they are.
__device__ __forceinline__ int pcol(int col) {
    const int a = (col >> 2) & 7;
    const int slot = a < 4 ? 2 * a : 2 * a - 7;
    return (col & ~31) | (slot << 2) | (col & 3);
}

// Debug builds (GDN_POISON_LDS=1, the library libgdn_poison.so) fill each LDS
// stage of the pipelined kernels with NaN once its last reader is done with
// it, so that a read which runs ahead of the write it should wait for gets
// NaN instead of the previous chunk's values.  All-ones bits are a NaN in
// fp16, bf16 and fp32 alike.  Production builds contain none of this code.
#ifndef GDN_POISON_LDS
#define GDN_POISON_LDS 0
#endif
constexpr bool kPoisonLds = GDN_POISON_LDS != 0;

// bytes (a multiple of 16) from a 16-byte aligned p, by threads t of n
__device__ __forceinline__ void poison_fill(const void *p, int bytes, int t, int n) {
    for (int i = t; i < bytes / 16; i += n) ((u32x4 *)p)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
}

// The 16 x 16 blocks (I, J <= I) of a swizzled, column-permuted C x C tile:
// the blocks that the prepare rewrites every chunk (those above stay zero).
template <int C>
__device__ __forceinline__ void poison_lower(const _Float16 *S, int t, int n) {
    constexpr int NB = C / 16;
    for (int i = t; i < NB * NB * 64; i += n) {
        const int blk = i / 64, I = blk / NB, J = blk % NB, r = (i % 64) / 4, cg = i % 4;
        if (J <= I) *(u32x2 *)(S + swz<C>(16 * I + r, pcol(16 * J + 4 * cg))) = u32x2{~0u, ~0u};
    }
}

// Lane (q, i): row r0 + i, stored columns k0 + 8q .. +7 (one 16-byte read).
// On a permuted tile this is the split-slot A fragment of logical columns
// k0 .. k0+31.
template <int LD>
__device__ __forceinline__ half8 frag_sw(const _Float16 *S, int r0, int k0) {
    const int l = lane_id();
    return *(const half8 *)(S + swz<LD>(r0 + (l & 15), k0 + 8 * (l >> 4)));
}

// Accumulator-layout transposed read (see read_T4): lane (g, j) gets
// S[k0 + 4g + e][m0 + j], e = 0..3.
template <int LD>
__device__ __forceinline__ u32x2 read_T4_sw(const void *S, int k0, int m0) {
    const int l = lane_id(), L = l & 15;
    const _Float16 *p = (const _Float16 *)S + swz<LD>(k0 + 4 * (l >> 4) + (L >> 2), m0 + 4 * (L & 3));
    typedef __fp16 v4fp16 __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16 *)p));
}

// Split-slot A fragment of S^T (see fragAT_split) for a column-permuted S:
// lane (g, L) fetches logical columns m0 + 4 (L % 4) .. +3, which are stored
// contiguously at pcol(m0 + 4 (L % 4)).
template <int LD>
__device__ __forceinline__ half4 read_T4_p(const _Float16 *S, int k0, int m0) {
    const int l = lane_id(), L = l & 15;
    const _Float16 *p = S + swz<LD>(k0 + 4 * (l >> 4) + (L >> 2), pcol(m0 + 4 * (L & 3)));
    typedef __fp16 v4fp16 __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;
    return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16 *)p));
}
template <int LD>
__device__ __forceinline__ half8 fragAT_split_p(const _Float16 *S, int m0, int k0) {
    const half4 a = read_T4_p<LD>(S, k0, m0);
    const half4 b = read_T4_p<LD>(S, k0 + 16, m0);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup barrier that waits only for this wave's LDS operations: vector
// memory loads in flight (the prefetch of later chunks) stay in flight.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Bounded LDS waits.  A wave polls an LDS counter (s_sleep between polls);
// a normal wait ends after a few thousand cycles.  One that polls `limit`
// times without its condition coming true gives up and the wave goes on, so
// a stalled partner can never hang the kernel.  Each wave counts its
// give-ups (`missed`, wave-uniform) and adds them, once, at its end, to
// *count: a device word the host reads back (gdn_wait_timeouts) to learn
// that the launch's results are not to be trusted.  `bias` is added to
// every target: 0, or a value no counter reaches, with which every wait
// gives up (only to test this path; every kernel still ends normally).
struct WaitCtl {
    unsigned *count;
    unsigned limit, bias;
    unsigned missed;
};

__device__ __forceinline__ void wait_report(const WaitCtl &wc) {
    if (wc.missed && wc.count && lane_id() == 0)
        __hip_atomic_fetch_add(wc.count, wc.missed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until an LDS counter reaches target.
__device__ __forceinline__ void wait_counter(const unsigned *ctr, unsigned target, WaitCtl &wc) {
    asm volatile("" ::: "memory");
    const unsigned t = target + wc.bias;
    for (unsigned it = 0;; ++it) {
        const unsigned v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((unsigned)__builtin_amdgcn_readfirstlane((int)v) >= t) break;
        if (it >= wc.limit) { ++wc.missed; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Barrier of N waves (the four prepare waves by default): an LDS arrival
// counter that only grows (N arrivals per barrier), with a bounded wait.
template <unsigned N = 4>
__device__ __forceinline__ void prep_barrier(unsigned *ctr, unsigned &target, WaitCtl &wc) {
    target += N;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (lane_id() == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wait_counter(ctr, target, wc);
}

// The arrival half of prep_barrier, for a wave that has other work to issue
// before it waits (wait_two below).
__device__ __forceinline__ void prep_arrive(unsigned *ctr, unsigned &target) {
    target += 4;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (lane_id() == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

// Wait until ctr[0] >= t0 and ctr[1] >= t1, both read by one 8-byte LDS load
// per poll (bounded like wait_counter).
__device__ __forceinline__ void wait_two(const unsigned *ctr, unsigned t0, unsigned t1, WaitCtl &wc) {
    asm volatile("" ::: "memory");
    const unsigned u0 = t0 + wc.bias, u1 = t1 + wc.bias;
    for (unsigned it = 0;; ++it) {
        const uint64_t v = __hip_atomic_load((const uint64_t *)ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const unsigned a = (unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
        const unsigned b = (unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
        if (a >= u0 && b >= u1) break;
        if (it >= wc.limit) { ++wc.missed; break; }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Lane-shifted copy within rows of 16 lanes (DPP row_shr), zero where the
// source lane falls before the row start.
template <int CTRL>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Four consecutive output values of one token: one 8-byte (bf16) or 16-byte
// (fp32) buffer store.
__device__ __forceinline__ void store4(const float4v &x, rsrc_t r, uint32_t voff, uint32_t soff) {
    const uint32_t lo = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, voff, soff, 0);
}
template <typename OT>
__device__ __forceinline__ void store4(const float4v &x, rsrc_t r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ void store4<bf16_t>(const float4v &x, rsrc_t r, uint32_t voff, uint32_t soff) {
    store4(x, r, voff, soff);
}
// (two 8-byte stores, not one 16-byte store: for vector-memory stores of
// more than 8 bytes the compiler does not hold back a following write of the
// data registers, and lanes then store the overwritten value)
template <>
__device__ __forceinline__ void store4<float>(const float4v &x, rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{u[0], u[1]}, r, voff, soff, 0);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{u[2], u[3]}, r, voff + 8, soff, 0);
}

// o^T tiles: lane (g, j) holds 4 consecutive columns of token j (voff is
// that token's byte offset, row_bytes the token pitch).  bf16: one 8-byte
// store.  fp32: the neighbouring lanes (tokens j, j ^ 1) swap halves by DPP
// so that each lane pair fills 16 contiguous bytes of one token with its two
// 8-byte stores (an instruction then writes 64-byte pieces of 8 rows instead
// of 8-byte pieces of 16 rows with gaps between them).
template <typename OT>
__device__ __forceinline__ void store_o_rows(const float4v &x, rsrc_t r, uint32_t voff,
                                             uint32_t row_bytes, uint32_t soff) {
    if constexpr (sizeof(OT) == 2) {
        store4<bf16_t>(x, r, voff, soff);
    } else {
        const bool odd = lane_id() & 1;
        const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
        const float r0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0xB1, 0xf, 0xf, false));
        const float r1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xf, 0xf, false));
        // token j & ~1 at columns +2 odd, then token j | 1
        const uint32_t va = odd ? voff - row_bytes + 8 : voff;
        __builtin_amdgcn_raw_buffer_store_b64(
            u32x2{__float_as_uint(odd ? r0 : x[0]), __float_as_uint(odd ? r1 : x[1])}, r, va, soff, 0);
        __builtin_amdgcn_raw_buffer_store_b64(
            u32x2{__float_as_uint(odd ? x[2] : r0), __float_as_uint(odd ? x[3] : r1)}, r, va + row_bytes, soff, 0);
    }
}

// Inclusive scan of a chunk's scalar gate (lane l holds g of row l) and
// the row factors the chunk needs, written by one wave: e^gcum, e^(gl-gcum),
// e^gl for the chain; beta, gcum itself, e^(gend_J - gcum) and
// e^(gcum - gend_J) for the Gram tiles, where gend_J is gcum at the last row
// of 16-row block J.  Every factor a product uses is at most 1 for any g <= 0:
// an off-diagonal tile (I > J) splits its decay e^(gcum_r - gcum_s) at the
// boundary after block J, which lies between r and s; a diagonal tile takes
// the decay of each entry directly (gate_decay_diag).  (Within rows of 16
// lanes by DPP shifts, then the row totals.)
// nvalid is the chunk's number of tokens (C except in a short last chunk):
// gl is gcum at its last token, so that e^(gl - gcum) of that token is
// exactly 1 (the padded rows' gcum, summed in another order by the scan,
// can differ from it by an ulp of |gcum|).
template <int C>
__device__ __forceinline__ void gate_factors(float g_own, float b_own, float *eg, float *bet, int nvalid) {
    constexpr int NB = C / 16;
    float *egl = eg + C, *einv = bet + C, *efac = bet + 2 * C, *gcp = bet + (2 + NB) * C;
    const int l = lane_id();
    float x = l < C ? g_own : 0.f;
    x += dpp_row_shr<0x111>(x);
    x += dpp_row_shr<0x112>(x);
    x += dpp_row_shr<0x114>(x);
    x += dpp_row_shr<0x118>(x);
    const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
    const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
    const int rw = l >> 4;
    x += (rw >= 1 ? t0 : 0.f) + (rw >= 2 ? t1 : 0.f) + (rw >= 3 ? t2 : 0.f);
    float gend[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J) gend[J] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16 * J + 15));
    const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), nvalid - 1));
    if (l < C) {
        eg[l] = fast_exp(x);
        egl[l] = fast_exp(gl - x);
        bet[l] = b_own;
        gcp[l] = x;
        float gref = gend[0];
#pragma unroll
        for (int J = 1; J < NB; ++J)
            if ((l >> 4) == J) gref = gend[J];
        einv[l] = fast_exp(gref - x);
        // (rows of block J and before get a growth factor here, which no
        // product reads: efac[J] multiplies rows of later blocks only)
#pragma unroll
        for (int J = 0; J < NB; ++J) efac[J * C + l] = fast_exp(fminf(x - gend[J], 0.f));
    }
    if (l == 0) eg[2 * C] = fast_exp(gl);
}

// The decays e^(gcum_r - gcum_s) of a diagonal Gram tile entry by entry, for
// row r against the columns s0 .. s0+3 (1 where s > r: those entries are
// masked out).
__device__ __forceinline__ float4v gate_decay_diag(const float *gcp, int r, int s0) {
    const float gr = gcp[r];
    const float4v gs = *(const float4v *)(gcp + s0);
    float4v f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = fast_exp(fminf(gr - gs[e], 0.f));
    return f;
}

// Count one arrival on an LDS counter once this wave's LDS writes are done.
__device__ __forceinline__ void signal_counter(unsigned *ctr) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (lane_id() == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
}

// A 16 x 16 block of A in col layout as an MFMA operand of k = 32: its fp16
// high parts (k = 8g .. 8g+3) and low parts (k = 8g+4 .. 8g+7), so that one
// product with an fp16 right operand keeps A to about 22 bits.
__device__ __forceinline__ half8 split_hi_lo(const float4v &x) {
    half8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (_Float16)x[e];
        h[4 + e] = (_Float16)(x[e] - (float)h[e]);
    }
    return h;
}

// The solve block Mn = -T_ii A_ij, in row layout (lane (g, n): row n, columns
// 4g .. 4g+3), from A_ij split by split_hi_lo and T_ii in row layout, fp16:
// (A_ij^T T_ii^T) with T_ii^T's rows repeated for the low parts.
__device__ __forceinline__ half4 solve_block(const half8 &a_split, const half4 &t) {
    const half8 tt = __builtin_shufflevector(t, t, 0, 1, 2, 3, 0, 1, 2, 3);
    const float4v x = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_split, tt, float4v{0, 0, 0, 0}, 0, 0, 0);
    half4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)(-x[e]);
    return h;
}

template <int C, int K>
struct PipeLayout {
    static constexpr int NB = C / 16;
    static constexpr int NASP = NB == 4 ? 4 : 0;         // A blocks (2,0) (2,1) (3,0) (3,1)
    static constexpr int kQK = C * K * 2;                // one fp16 q or k tile
    static constexpr int kCC = C * C * 2;                // one fp16 C x C tile
    static constexpr int kVT = C * 64 * 2;               // one bf16 v tile
    static constexpr int kQ = 0;                         // [2] q tiles
    static constexpr int kK = kQ + 2 * kQK;              // [2] k tiles
    static constexpr int kTmb = kK + 2 * kQK;            // [2] solve blocks (Tb, Mn)
    static constexpr int kP = kTmb + 2 * kCC;            // [2] P
    static constexpr int kV = kP + 2 * kCC;              // [2] raw v tiles
    // A blocks of the later solve blocks, split fp16, one half8 per lane
    static constexpr int kAsp = kV + 2 * kVT;            // [NASP][64][8]
    // the diagonal inverses T_bb in row layout, fp16, one half4 per lane
    static constexpr int kTr = kAsp + NASP * 1024;       // [NB][64][4]
    // chain-side row factors per slot: e^gcum, e^(gl - gcum), e^gl
    static constexpr int kRowCN = 2 * C + 4;
    static constexpr int kRowC = kTr + NB * 512;         // [2][kRowCN]
    // prepare-side row factors: beta, e^(gend_J(s) - gcum_s), e^(gcum - gend_J),
    // gcum (gend_J: gcum at the last row of block J)
    static constexpr int kRowP = kRowC + 2 * kRowCN * 4; // [C + C + NB C + C]
    static constexpr int kSync = kRowP + (3 * C + NB * C) * 4;
    static constexpr int kBytes = kSync + 16;
    static_assert(kSync % 8 == 0, "the two sync counters are read as one 8-byte word");
};

// DQ: the backward's re-scan (the KDA re-scan page's kernel): the chunk-start
// states and v' as with ST, plus dq's chunk-start-state term
// DQ = dO h_c^T (raw) accumulated into p.dq, and no o.
// SP: the sequence-split instance (see FwdParams): the stream's first
// segment, or its second one as ordinary tiles from a zero state and as
// identity tiles (v = 0, h0 = I), whose outputs are the second segment's
// correction basis (gdn_forward_split).
template <int C, int K, typename OT, bool ST = false, bool VL = false, bool DQ = false, bool SP = false>
__global__ __launch_bounds__(kPipeThreads, 1) void forward_pipe_kernel(FwdParams p) {
    typedef PipeLayout<C, K> L;
    typedef Mma<_Float16> M;
    typedef bf16_t IO;
    constexpr int NB = C / 16, NKB = K / 16;
    constexpr int SIO = 2, SO = sizeof(OT);
    static_assert(L::kBytes <= kLdsBytesMax, "LDS budget");
    static_assert(NB == 2 || NB == 4, "chunk 32 or 64");
    static_assert(K == 64 || K == 128, "key dim 64 or 128");
    static_assert(!DQ || ST, "the re-scan also saves the states");
    static_assert(L::kBytes + (DQ ? 4 * K * 64 : 0) <= kLdsBytesMax, "LDS budget with the re-scan");

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    // DQ: h_c as bf16 high and low parts, [K][64] (key row, tile column),
    // 16-byte chunks XOR-swizzled by row (swz<64>)
    __shared__ __attribute__((aligned(16))) uint16_t hq_lds[DQ ? 2 * K * 64 : 8];
    _Float16 *Qb = (_Float16 *)(smem + L::kQ);
    _Float16 *Kb = (_Float16 *)(smem + L::kK);
    _Float16 *Tmbb = (_Float16 *)(smem + L::kTmb);
    _Float16 *Pb = (_Float16 *)(smem + L::kP);
    uint16_t *Vb = (uint16_t *)(smem + L::kV);
    _Float16 *Asp = (_Float16 *)(smem + L::kAsp);
    _Float16 *Tr = (_Float16 *)(smem + L::kTr);
    float *rowC = (float *)(smem + L::kRowC);
    float *bet = (float *)(smem + L::kRowP);
    float *einv = bet + C, *efac = bet + 2 * C, *gcp = bet + (2 + NB) * C;
    unsigned *sync_ctr = (unsigned *)(smem + L::kSync);

    const int wv = wave_id(), l = lane_id(), tid = threadIdx.x;
    int pair, vt, seg = 0;
    bool ident = false;             // SP: an identity tile of the second segment
    if (SP && (int)blockIdx.x >= p.sp_g0) {
        seg = 1;
        map_block((int)blockIdx.x - p.sp_g0, p.nvt + K / 64, p.swizzle, pair, vt);
        ident = vt >= p.nvt;
    } else {
        map_block(blockIdx.x, p.nvt, p.swizzle, pair, vt);
    }
    const int b = pair / p.H, h = pair - b * p.H;
    StreamRange sr = stream_range<VL>(p, b, h);
    if constexpr (SP) {
        sr.T = seg ? p.T - p.sp_t : p.sp_t;
        sr.row0 = ((int64_t)b * p.T + (seg ? p.sp_t : 0)) * p.H + h;
    }
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
        sync_ctr[1] = 0u;                   // chunks whose row factors are written
        sync_ctr[2] = 0u;                   // chain waves' barrier (DQ)
    }
    wg_barrier();

    if (wv < 4) {
        // =====================  chain waves  =============================
        // (SP identity tiles: o rows K wide in sp_oI, columns from 64 (vt - nvt))
        const uint32_t rsO = ident ? rsK : rsV;
        const int ocol = (ident ? vt - p.nvt : vt) * 64;
        const rsrc_t ro_ = ident ? make_rsrc((OT *)p.sp_oI + ((int64_t)b * T * H + h) * K, (uint32_t)T * rsK * SO)
                                 : make_rsrc((OT *)p.o + row0 * V, (uint32_t)T * rsV * SO);
        const int g4 = 4 * (l >> 4);
        const int vcol = vt * 64 + 16 * wv + acc_col();
        // o^T tiles: token (l % 16) of a 16-token block, columns 4 (l / 16) .. +3
        const uint32_t o_off = ((uint32_t)(l & 15) * rsO + ocol + 16 * wv + g4) * SO;
        // saved states: v' and h leave the accumulators as column pairs
        // (store_acc_pairs): this lane's first row 4 (l / 16) + 2 (l & 1)
        // of a 16-row block (tokens for v', key rows for h), columns
        // vcol & ~1 and vcol | 1
        const rsrc_t rvn_ = make_rsrc(ST ? (OT *)p.vnew + row0 * V : nullptr, ST ? (uint32_t)T * rsV * SO : 0u);
        const uint32_t prow = (uint32_t)(g4 + 2 * (l & 1));
        const uint32_t vn_off = (prow * rsV + (vcol & ~1)) * SO;
        const uint32_t hck_off = (prow * V + (vcol & ~1)) * SO;
        // DQ: dO rows as bf16 A fragments, lane (q, i): row i of a 16-token
        // block, columns 8q .. 8q+7 of a 32-column half of the tile
        const rsrc_t rdo_ = make_rsrc(DQ ? (const IO *)p.dout + row0 * V : nullptr, DQ ? (uint32_t)T * rsV * SIO : 0u);
        const uint32_t do_off = ((uint32_t)(l & 15) * rsV + vt * 64 + 8 * (l >> 4)) * SIO;
        unsigned chain_target = 0;
        float4v hacc[NKB];
        if (ident) {
            // h0 = I: this lane's column ocol + 16 wv + (l % 16) of the K x K identity
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) hacc[i][r] = (16 * i + g4 + r == ocol + 16 * wv + acc_col()) ? 1.f : 0.f;
        } else if (p.h0 && seg == 0) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hacc[i][r] = p.h0[((int64_t)pair * K + 16 * i + g4 + r) * V + vcol];
        } else {
#pragma unroll
            for (int i = 0; i < NKB; ++i) hacc[i] = float4v{0, 0, 0, 0};
        }
        // Chain wave 0 also scans the gate: chunk c+1's row factors at the
        // start of chunk c (the prepare waves are converting operands
        // meanwhile), from gate and beta loaded a chunk earlier.
        const rsrc_t rg_ = make_rsrc(p.g + row0, (uint32_t)T * (uint32_t)H * 4);
        const rsrc_t rb_ = make_rsrc(p.beta + row0, (uint32_t)T * (uint32_t)H * 4);
        const uint32_t gb_off = (uint32_t)l * (uint32_t)H * 4;
        float g_nx = 0.f, b_nx = 0.f;
        auto gload = [&](int n) {
            const uint32_t so = (uint32_t)(n * C) * (uint32_t)H * 4;
            g_nx = __uint_as_float(bload32(rg_, gb_off, so));
            b_nx = __uint_as_float(bload32(rb_, gb_off, so));
        };
        if (wv == 0 && nt > 0) {
            gload(0);
            gate_factors<C>(g_nx, b_nx, rowC, bet, min(C, T));
            signal_counter(sync_ctr + 1);
            if (nt > 1) gload(1);
        }
        asm volatile("" : "+v"(g_nx), "+v"(b_nx));     // (see the o stores below)
        wg_barrier();                       // chunk 0 prepared

        for (int c = 0; c < nt; ++c) {
            const int slot = c & 1;
            const _Float16 *Qs = Qb + slot * C * K, *Ks = Kb + slot * C * K;
            const _Float16 *Tmb = Tmbb + slot * C * C, *Ps = Pb + slot * C * C;
            const uint16_t *Vs = Vb + slot * C * 64;
            const float *eg = rowC + slot * L::kRowCN, *egl = eg + C;
            const uint32_t t0 = (uint32_t)(c * C);
            if (wv == 0 && c + 1 < nt) {
                gate_factors<C>(g_nx, b_nx, rowC + (slot ^ 1) * L::kRowCN, bet, min(C, T - (c + 1) * C));
                signal_counter(sync_ctr + 1);
                if (c + 2 < nt) gload(c + 2);
            }
            const float el = eg[2 * C];
            if constexpr (DQ) {
                // h_c into LDS as bf16 high and low parts (RNE), then each
                // wave forms DQ for its K/4 key rows over the tile's 64
                // value columns: DQ[t][key] = sum_v dO[t][v] h_c[key][v], two
                // bf16 MFMAs per step (the split keeps h_c to ~16 bits;
                // bf16 keeps any dO magnitude in range)
                uint16_t *Hhi = hq_lds, *Hlo = hq_lds + K * 64;
                // this chunk's dO fragments first: their latency then runs
                // under the LDS writes and the barrier below
                bf16x8 dof[2][NB];
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int cb = 0; cb < NB; ++cb)
                        dof[s][cb] = __builtin_bit_cast(bf16x8, bload128(rdo_, do_off + 32 * s * SIO,
                                                                         (t0 + 16 * cb) * rsV * SIO));
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
                constexpr int NKW = K / 64;                  // 16-row key tiles per wave
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
                    for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
                        for (int nt = 0; nt < NKW; ++nt) {
                            dq[cb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dof[s][cb], bh[nt], dq[cb][nt], 0, 0, 0);
                            dq[cb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dof[s][cb], bl[nt], dq[cb][nt], 0, 0, 0);
                        }
                    }
                }
                // accumulate into dq (the V tiles of a head add up there)
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
            }

            float4v eg4[NB], egl4[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                eg4[cb] = *(const float4v *)(eg + 16 * cb + g4);
                egl4[cb] = *(const float4v *)(egl + 16 * cb + g4);
            }
            half8 hf[K / 32];
#pragma unroll
            for (int s = 0; s < K / 32; ++s) hf[s] = fragB_acc(hacc[2 * s], hacc[2 * s + 1], _Float16{});
            // X = k h, Y = q h for this wave's 16 columns
            // (Y is formed transposed, Y^T = h^T q^T: the same fragments with
            // the operands swapped, so a lane ends up with four consecutive
            // value columns of one token)
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
            // R' = v - e^gcum X
            float4v rr[NB];
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const u32x2 w = read_T4_sw<64>(Vs, 16 * cb, 16 * wv);
                const float4v vv = {__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                    __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
                rr[cb] = vv - eg4[cb] * xa[cb];
            }
            // v' solves (I + A) v' = diag(beta) R' by blocks of 16 tokens:
            //   v'_b = Tb_bb R'_b + sum_{j<b} Mn_bj v'_j,
            //   Tb_bb = (I + A_bb)^-1 diag(beta_b),  Mn_bj = -(I + A_bb)^-1 A_bj.
            // Row block b of the C x C operand tile holds [Mn_b0 .. | Tb_bb | 0],
            // so each step is a 32-wide k step over a [v' ; R'] fragment pair.
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
            // o^T = v'^T P^T + Y^T diag(e^gcum): lane (g, j) holds token
            // 16 cb + j, value columns 4g .. 4g+3 of this wave's 16
            half8 df[C / 32];
#pragma unroll
            for (int s = 0; s < C / 32; ++s) df[s] = fragB_acc(da[2 * s], da[2 * s + 1], _Float16{});
            if constexpr (!DQ) {
#pragma unroll
                for (int cb = 0; cb < NB; ++cb) {
                    float4v oa = eg[16 * cb + (l & 15)] * ya[cb];
#pragma unroll
                    for (int s = 0; s < C / 32; ++s)
                        if (32 * s < 16 * (cb + 1)) M::mma(oa, df[s], frag_sw<C>(Ps, 16 * cb, 32 * s));
                    store_o_rows<OT>(oa, ro_, o_off, rsO * SO, (t0 + 16 * cb) * rsO * SO);
                }
            }
            if constexpr (ST) {
                // v' of this chunk's tokens (dropped past token T by the range)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    store_acc_pairs<OT>(da[cb], rvn_, vn_off, rsV * SO, (t0 + 16 * cb) * rsV * SO);
                // the state at the start of this chunk, hck[b, c, h, row, vcol]:
                // issued late in the chunk, after the prepare waves' loads of
                // the chunk after next, which would otherwise queue behind it
                const rsrc_t rh = make_rsrc((OT *)p.hck + (((int64_t)b * nt + c) * H + h) * K * V,
                                            (uint32_t)(K * V * SO));
#pragma unroll
                for (int i = 0; i < NKB; ++i) store_acc_pairs<OT>(hacc[i], rh, hck_off, V * SO, 16 * i * V * SO);
            }
            // h <- e^gl h + (k e^(gl - gcum))^T v'
#pragma unroll
            for (int s = 0; s < C / 32; ++s)
                df[s] = fragB_acc(da[2 * s] * egl4[2 * s], da[2 * s + 1] * egl4[2 * s + 1], _Float16{});
#pragma unroll
            for (int i = 0; i < NKB; ++i) {
                hacc[i] = hacc[i] * el;
#pragma unroll
                for (int s = 0; s < C / 32; ++s)
                    M::mma(hacc[i], fragAT_split_p<K>(Ks, 16 * i, 32 * s), df[s]);
            }
            if constexpr (kPoisonLds) {
                // every chain wave is past its reads of this slot, which the
                // prepare rewrites for chunk c + 2
                prep_barrier(sync_ctr + 2, chain_target, wc);
                poison_fill(Qs, C * K * 2, tid, 256);
                poison_fill(Ks, C * K * 2, tid, 256);
                poison_fill(Vs, C * 64 * 2, tid, 256);
                poison_fill(eg, L::kRowCN * 4, tid, 256);
                poison_lower<C>(Tmb, tid, 256);
                poison_lower<C>(Ps, tid, 256);
            }
            // (chain wave 0 has the gate and beta of chunk c + 2 in flight:
            // they are taken into registers here, where the wait counts the
            // o stores issued since, so the next chunk's factor scan does not
            // wait for those stores)
            asm volatile("" : "+v"(g_nx), "+v"(b_nx));
            wg_barrier();
        }
        // (SP: the first segment's end state, or the second's zero-state
        // end N or its transfer M, K wide)
        float *hTp = p.hT;
        int hcols = V, hcol = vcol;
        if constexpr (SP) {
            hTp = seg == 0 ? p.sp_h0out : (ident ? p.sp_M : p.sp_N);
            hcols = ident ? K : V;
            hcol = ident ? ocol + 16 * wv + acc_col() : vcol;
        }
        if (hTp) {
#pragma unroll
            for (int i = 0; i < NKB; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hTp[((int64_t)pair * K + 16 * i + g4 + r) * hcols + hcol] = hacc[i][r];
        }
        wait_report(wc);
    } else {
        // =====================  prepare waves  ===========================
        // The prepare is the longer of the two roles per chunk: its waves
        // win instruction arbitration over the chain waves sharing a SIMD.
        // (Not in the chunk-64 re-scan with dq, whose chain carries the dq
        // products: there the default priority measured 6 % faster; at
        // chunk 32 the raised one is 5 % faster.)
        if constexpr (!(DQ && C == 64)) __builtin_amdgcn_s_setprio(3);
        const int pw = wv - 4, pt = tid - 256;
        const rsrc_t rq_ = make_rsrc((const IO *)p.q + row0 * K, (uint32_t)T * rsK * SIO);
        const rsrc_t rk_ = make_rsrc((const IO *)p.k + row0 * K, (uint32_t)T * rsK * SIO);
        // (SP identity tiles read v = 0: an empty range)
        const rsrc_t rv_ = make_rsrc((const IO *)p.v + row0 * V, ident ? 0u : (uint32_t)T * rsV * SIO);

        constexpr int NVEC = C * K / 8 / 256;            // q/k vectors per thread
        constexpr int NVV = C * 64 / 8 / 256;            // v vectors per thread
        static_assert(NVEC >= 1 && NVV >= 1, "tile smaller than the prepare waves");
        uint32_t qk_off[NVEC];
        int qk_lds[NVEC][2];        // stored positions of the two 4-column halves
#pragma unroll
        for (int j = 0; j < NVEC; ++j) {
            const int i = pt + 256 * j, row = i / (K / 8), ch = i % (K / 8);
            qk_off[j] = ((uint32_t)row * rsK + 8 * ch) * SIO;
            qk_lds[j][0] = swz<K>(row, pcol(8 * ch));
            qk_lds[j][1] = swz<K>(row, pcol(8 * ch + 4));
        }
        uint32_t vv_off[NVV];
        int vv_lds[NVV];
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int i = pt + 256 * j, row = i / 8, ch = i % 8;
            vv_off[j] = ((uint32_t)row * rsV + vt * 64 + 8 * ch) * SIO;
            vv_lds[j] = swz<64>(row, 8 * ch);
        }

        u32x4 rq[NVEC], rk[NVEC], rv[NVV];
        auto issue_loads = [&](int n) {
            const uint32_t t0 = (uint32_t)(n * C);
#pragma unroll
            for (int j = 0; j < NVV; ++j) rv[j] = bload128(rv_, vv_off[j], t0 * rsV * SIO);
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                rq[j] = bload128(rq_, qk_off[j], t0 * rsK * SIO);
                rk[j] = bload128(rk_, qk_off[j], t0 * rsK * SIO);
            }
        };
        unsigned sync_target = 0;

        auto prepare = [&](int n) {
            const int slot = n & 1;
            _Float16 *Qs = Qb + slot * C * K, *Ks = Kb + slot * C * K;
            _Float16 *Tmb = Tmbb + slot * C * C, *Ps = Pb + slot * C * C;
            uint16_t *Vs = Vb + slot * C * 64;

            // ---- operands (the row factors come from chain wave 0)
#pragma unroll
            for (int j = 0; j < NVV; ++j) *(u32x4 *)(Vs + vv_lds[j]) = rv[j];
#pragma unroll
            for (int j = 0; j < NVEC; ++j) {
                half8 hq, hk;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // bf16 -> fp16 is exact here (|q|, |k| <= 1)
                    hq[2 * e] = (_Float16)__uint_as_float(rq[j][e] << 16);
                    hq[2 * e + 1] = (_Float16)__uint_as_float(rq[j][e] & 0xffff0000u);
                    hk[2 * e] = (_Float16)__uint_as_float(rk[j][e] << 16);
                    hk[2 * e + 1] = (_Float16)__uint_as_float(rk[j][e] & 0xffff0000u);
                }
                *(half4 *)(Qs + qk_lds[j][0]) = __builtin_shufflevector(hq, hq, 0, 1, 2, 3);
                *(half4 *)(Qs + qk_lds[j][1]) = __builtin_shufflevector(hq, hq, 4, 5, 6, 7);
                *(half4 *)(Ks + qk_lds[j][0]) = __builtin_shufflevector(hk, hk, 0, 1, 2, 3);
                *(half4 *)(Ks + qk_lds[j][1]) = __builtin_shufflevector(hk, hk, 4, 5, 6, 7);
            }
            prep_arrive(sync_ctr, sync_target);
            if (n + 1 < nt) issue_loads(n + 1);
            // every prepare wave's q/k rows and chunk n's row factors are in
            wait_two(sync_ctr, sync_target, (unsigned)(n + 1), wc);

            // ---- Gram tiles.  Tile (I, J) of a P or A block, with its decay
            // e^(gcum_r - gcum_s) (and beta_r for A): off the diagonal
            // efac[J][r] einv[s], split at the end of block J; on it entry by
            // entry.  Row layout (lane (g, n): row 16 I + n, columns
            // 16 J + 4g + e) or col layout (rows 16 I + 4g + e, column
            // 16 J + n).
            auto fac_row = [&](int I, int J, bool isA, const float4v &acc) {
                const int r = 16 * I + (l & 15), s0 = 16 * J + 4 * (l >> 4);
                const float fr = isA ? bet[r] : 1.f;
                const float4v fs = I == J ? gate_decay_diag(gcp, r, s0)
                                          : *(const float4v *)(einv + s0) * efac[J * C + r];
                float4v a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (isA ? s0 + e < r : s0 + e <= r) ? acc[e] * fs[e] * fr : 0.f;
                return a;
            };
            auto fac_col = [&](int I, int J, const float4v &acc) {      // A blocks only
                const int r0 = 16 * I + 4 * (l >> 4), s = 16 * J + (l & 15);
                const float4v fr = *(const float4v *)(efac + J * C + r0) * *(const float4v *)(bet + r0);
                const float fs = einv[s];
                float4v a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = s < r0 + e ? acc[e] * fs * fr[e] : 0.f;
                return a;
            };
            auto put_p = [&](int I, int J, const float4v &acc) {
                const float4v a = fac_row(I, J, false, acc);
                half4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = (_Float16)a[e];
                *(half4 *)(Ps + swz<C>(16 * I + (l & 15), pcol(16 * J + 4 * (l >> 4)))) = h;
            };
            // Two tiles at once: every fragment load first, then the two
            // accumulations interleaved.  mma(x, frag of rows X, frag of rows
            // Y) forms X Y^T in col layout: P tiles (rows of block J first)
            // come out in row layout, A tiles (block I first) in col layout.
            auto gram_two = [&](int I0, int J0, bool a0, int I1, int J1, bool a1, bool two, int sl0, int sl1) {
                half8 fa0[K / 32], fb0[K / 32], fa1[K / 32], fb1[K / 32];
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    fa0[k] = frag_sw<K>(Ks, 16 * J0, 32 * k);
                    fb0[k] = frag_sw<K>(a0 ? Ks : Qs, 16 * I0, 32 * k);
                    if (two) {
                        fa1[k] = frag_sw<K>(Ks, 16 * J1, 32 * k);
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
                half8 f0[K / 32], f1[K / 32], q0[K / 32], q1[K / 32];
#pragma unroll
                for (int k = 0; k < K / 32; ++k) {
                    f0[k] = frag_sw<K>(Ks, 16 * pb, 32 * k);
                    f1[k] = frag_sw<K>(Ks, 16 * (pb + 1), 32 * k);
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
                    M::mma(a00, f0[k], f0[k]);
                    M::mma(a11, f1[k], f1[k]);
                    M::mma(a10, f1[k], f0[k]);
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
                    half4 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[q] = (_Float16)t[q];
                        t16[e][q] = (_Float16)tr[e][q];
                    }
                    *(half4 *)(Tmb + swz<C>(row, pcol(c4))) = h;
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
            if constexpr (kPoisonLds) {
                // every prepare wave is past its reads of the row factors
                // (rewritten for chunk n + 1 by chain wave 0), the split A
                // blocks and the fp16 T_bb
                prep_barrier(sync_ctr, sync_target, wc);
                poison_fill(bet, (3 + NB) * C * 4, pt, 256);
                poison_fill(Asp, L::NASP * 1024, pt, 256);
                poison_fill(Tr, NB * 512, pt, 256);
            }
        };

        if (nt > 0) {
            issue_loads(0);
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
