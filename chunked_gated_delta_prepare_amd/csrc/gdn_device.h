// Device building blocks for the gfx950 kernels: matrix-core operand traits,
// LDS fragment loads, global row loads and dtype conversions.
//
// Matrix-core conventions used throughout (wave64, 16x16 output tiles):
//   * Every product is written "NT": C[m][n] = sum_k A[m][k] * Bt[n][k], with
//     both A and Bt stored in LDS as [rows][k], k contiguous, row pitch padded
//     by 16 bytes so the 16 rows a fragment load touches fall in distinct
//     bank groups.
//   * Lane l supplies row (l % 16) of A and of Bt, and the k slots
//     8*(l/16) .. 8*(l/16)+7 of the current 32-wide k step.  Any bijection of
//     k slots onto the instruction's k positions gives the same sum, as long
//     as A and Bt use the same one -- they do, since both come from the same
//     lane and slot.
//   * The accumulator of a 16x16 tile holds C[4*(l/16) + r][l % 16] in
//     element r (r = 0..3) of lane l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLdsBytesMax = 160 * 1024;

struct bf16_t { uint16_t bits; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename T> struct io_traits;
template <> struct io_traits<float> {
    static constexpr int bytes = 4;
    __device__ static float load(const float *p) { return *p; }
    __device__ static void store(float *p, float x) { *p = x; }
};
template <> struct io_traits<bf16_t> {
    static constexpr int bytes = 2;
    __device__ static float load(const bf16_t *p) { return bf16_bits_to_f32(p->bits); }
    __device__ static void store(bf16_t *p, float x) { p->bits = f32_to_bf16_bits(x); }
};

// Load 8 consecutive io elements (16- or 32-byte aligned) as floats.
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4v a = *(const float4v *)p;
    const float4v b = *(const float4v *)(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
__device__ __forceinline__ void load8(const bf16_t *p, float (&x)[8]) {
    const u32x4 a = *(const u32x4 *)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(a[i] << 16);
        x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core operand traits.  OpT is the element type operands are held in
// (in LDS): _Float16 for bf16 io, float for fp32 io.
// ---------------------------------------------------------------------------
template <typename OpT> struct Mma;

template <> struct Mma<_Float16> {
    static constexpr int kPad = 8;               // 16 bytes per row
    typedef half8 frag;
    __device__ static frag load(const _Float16 *p) { return *(const half8 *)p; }
    __device__ static void mma(float4v &acc, const frag &a, const frag &b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    __device__ static _Float16 cvt(float x) { return (_Float16)x; }
};

template <> struct Mma<float> {
    static constexpr int kPad = 4;               // 16 bytes per row
    struct frag { float4v lo, hi; };
    __device__ static frag load(const float *p) {
        frag f;
        f.lo = *(const float4v *)p;
        f.hi = *(const float4v *)(p + 4);
        return f;
    }
    // Eight 16x16x4 steps; step s takes slot s of every lane's 8 k slots.
    __device__ static void mma(float4v &acc, const frag &a, const frag &b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
    }
    __device__ static float cvt(float x) { return x; }
};

// Pointer to this lane's fragment of a 16-row operand block whose row 0 is
// at `base` (pitch `ld` elements), for the k step starting at column k0.
template <typename OpT>
__device__ __forceinline__ const OpT *frag_ptr(const OpT *base, int ld, int k0) {
    const int l = lane_id();
    return base + (l & 15) * ld + k0 + 8 * (l >> 4);
}

// acc += A[16 x klen] * Bt[16 x klen]^T for klen a multiple of 32.
template <typename OpT, int KLEN>
__device__ __forceinline__ void mma_tile(float4v &acc, const OpT *A, int lda,
                                         const OpT *Bt, int ldb) {
    typedef Mma<OpT> M;
#pragma unroll
    for (int k0 = 0; k0 < KLEN; k0 += 32) {
        const typename M::frag a = M::load(frag_ptr(A, lda, k0));
        const typename M::frag b = M::load(frag_ptr(Bt, ldb, k0));
        M::mma(acc, a, b);
    }
}

// Same with a run-time k length (multiple of 32, at most KMAX).
template <typename OpT, int KMAX>
__device__ __forceinline__ void mma_tile_n(float4v &acc, const OpT *A, int lda,
                                           const OpT *Bt, int ldb, int klen) {
    typedef Mma<OpT> M;
#pragma unroll
    for (int k0 = 0; k0 < KMAX; k0 += 32) {
        if (k0 < klen) {
            const typename M::frag a = M::load(frag_ptr(A, lda, k0));
            const typename M::frag b = M::load(frag_ptr(Bt, ldb, k0));
            M::mma(acc, a, b);
        }
    }
}

// Store an accumulator tile transposed: dst[n][m] (m contiguous) for the tile
// whose C[m][n] the accumulator holds; each lane writes 4 consecutive m.
template <typename OpT>
__device__ __forceinline__ void store_tile_T(OpT *dst, int ld, const float4v &acc) {
    const int l = lane_id();
    OpT *p = dst + (l & 15) * ld + 4 * (l >> 4);
    p[0] = Mma<OpT>::cvt(acc[0]);
    p[1] = Mma<OpT>::cvt(acc[1]);
    p[2] = Mma<OpT>::cvt(acc[2]);
    p[3] = Mma<OpT>::cvt(acc[3]);
}

// Row index (within a 16x16 tile) of accumulator element r, and the column.
__device__ __forceinline__ int acc_row(int r) { return 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// 2^x on the transcendental unit (v_exp_f32), for arguments already scaled
// by log2(e) (one multiply shared by e^d and e^-d).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace gdn
