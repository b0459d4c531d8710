// Unit lower triangular inverse Tm = (I + A)^-1 of a C x C strictly lower A,
// in fp32, on one workgroup.
//
// The TileOPs fused prepare page reaches the inverse by a Neumann series on
// a C x C buffer (about log2(C) squarings of the whole matrix).  Here the
// same inverse is formed exactly and with far fewer flops, by blocks of 16:
//   1. each 16 x 16 diagonal block T_ii = (I + A_ii)^-1 by forward
//      substitution, one lane per column (wave 0, 16 lanes per block);
//   2. sub-diagonals outward, Tm_ij = -T_ii * sum_{k=j}^{i-1} A_ik Tm_kj,
//      one wave per block of a sub-diagonal, on the fp32 matrix cores.
// A and Tm are fp32 [C][LDA] in LDS; Tm must start zeroed above the diagonal
// blocks (the caller clears it), A is read only strictly below the diagonal.
#pragma once

#include "gdn_device.h"

namespace gdn {

// Diagonal 16 x 16 inverses T = (I + A)^-1 of two blocks by one wave, on the
// matrix cores.  The inverse is built by doubling the block size s = 1, 2, 4,
// 8: with B the block-diagonal inverse at size s and L the (2,1) blocks of
// size s inside each 2s-block of A, the inverse at size 2s is B - B L B (the
// inverse of a 2 x 2 block lower-triangular matrix).  Every factor is bounded
// (|A| < 1 entrywise, the partial inverses are O(1)), so fp16 operands with
// fp32 accumulation keep T within a few fp16 roundings of the exact inverse,
// the precision at which the chain uses it anyway.
//
// Two layouts of a 16 x 16 matrix M in lane (g, n) = (l / 16, l % 16):
//   col layout  M[4g + r][n], r = 0..3: the MFMA B operand and its result
//   row layout  M[n][4g + r]:           the MFMA A operand
// X Y takes X in row and Y in col layout; Y^T X^T takes the same registers
// with the roles swapped and returns X Y in row layout.
// In: a[j], block j of A (strictly lower) in row layout.  Out: t[j], T of
// block j in row layout (row n, columns 4g .. 4g+3), fp32.
__device__ __forceinline__ void diag_inverse_mfma(const float4v (&a)[2], float4v (&t)[2]) {
    const int l = lane_id(), g = l >> 4, n = l & 15;
    float4v Bc[2], Br[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        // s = 1: B = I minus the subdiagonal entries A[i][i-1] at odd rows i.
        // In col layout lane (g, 4g) needs A[4g+1][4g] and lane (g, 4g+2)
        // needs A[4g+3][4g+2]: row-layout entries of the next lane.
        const float sub1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a[j][0]), 0x101, 0xf, 0xf, true));
        const float sub3 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a[j][2]), 0x101, 0xf, 0xf, true));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float ca = (r & 1) && n == i - 1 ? (r == 1 ? sub1 : sub3) : 0.f;   // A[i][i-1]
            const float rb = (n & 1) && i == n - 1 ? a[j][r] : 0.f;                  // A[n][n-1]
            Bc[j][r] = (i == n ? 1.f : 0.f) - ca;
            Br[j][r] = (i == n ? 1.f : 0.f) - rb;
        }
    }
#pragma unroll
    for (int s = 2; s <= 8; s *= 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            half4 Lr, Bch, Brh;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g + r;
                const bool inL = (n / (2 * s)) == (i / (2 * s)) && (n & s) && !(i & s);
                Lr[r] = (_Float16)(inL ? a[j][r] : 0.f);
                Bch[r] = (_Float16)Bc[j][r];
                Brh[r] = (_Float16)Br[j][r];
            }
            const float4v x = __builtin_amdgcn_mfma_f32_16x16x16f16(Lr, Bch, float4v{0, 0, 0, 0}, 0, 0, 0);
            half4 xn;
#pragma unroll
            for (int r = 0; r < 4; ++r) xn[r] = (_Float16)(-x[r]);
            if (s < 8) Bc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(Brh, xn, Bc[j], 0, 0, 0);
            Br[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(xn, Brh, Br[j], 0, 0, 0);
        }
    }
    t[0] = Br[0];
    t[1] = Br[1];
}

// acc += A16 * B16 for 16 x 16 fp32 blocks (both row-major in LDS).
// Instruction k index g of step s stands for contraction index 4g + s.
__device__ __forceinline__ void mm16_f32(float4v &acc, const float *A, int lda,
                                         const float *B, int ldb) {
    const int l = lane_id(), g = l >> 4, i = l & 15;
    const float4v a = *(const float4v *)(A + i * lda + 4 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], B[(4 * g + s) * ldb + i], acc, 0, 0, 0);
}

// acc += A16 * X where X is another product's accumulator (lane (g, col)
// holds X[4g + r][col]), which is exactly the B operand layout above.
__device__ __forceinline__ void mm16_f32_regB(float4v &acc, const float *A, int lda,
                                              const float4v &X) {
    const int l = lane_id(), g = l >> 4, i = l & 15;
    const float4v a = *(const float4v *)(A + i * lda + 4 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], X[s], acc, 0, 0, 0);
}

template <int C, int LDA>
__device__ void tri_inverse(const float *A, float *Tm) {
    constexpr int NB = C / 16;
    const int wv = wave_id(), l = lane_id();
    // 1. diagonal blocks
    if (wv == 0) {
        const int blk = l >> 4, j = l & 15;
        if (blk < NB) {
            const float *Ab = A + 16 * blk * LDA + 16 * blk;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) s -= Ab[i * LDA + kk] * t[kk];
                t[i] = s;
            }
            float *Tb = Tm + 16 * blk * LDA + 16 * blk;
#pragma unroll
            for (int i = 0; i < 16; ++i) Tb[i * LDA + j] = t[i];
        }
    }
    __syncthreads();
    // 2. sub-diagonal s: blocks (j + s, j), block j on wave j
#pragma unroll
    for (int s = 1; s < NB; ++s) {
        const int j = wv, i = wv + s;
        if (i < NB) {
            float4v x = {0, 0, 0, 0};
            for (int k = j; k < i; ++k)
                mm16_f32(x, A + 16 * i * LDA + 16 * k, LDA, Tm + 16 * k * LDA + 16 * j, LDA);
            x = -x;
            float4v y = {0, 0, 0, 0};
            mm16_f32_regB(y, Tm + 16 * i * LDA + 16 * i, LDA, x);
            float *dst = Tm + 16 * i * LDA + 16 * j;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[acc_row(r) * LDA + acc_col()] = y[r];
        }
        __syncthreads();
    }
}

}  // namespace gdn
