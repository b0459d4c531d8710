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
