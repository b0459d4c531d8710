// Chunk-granular global<->register<->LDS movement shared by the kernels.
#pragma once

#include "gdn_device.h"

namespace gdn {

// Eight raw io elements as loaded from HBM (kept raw until written to LDS so
// the prefetch registers hold bf16 bits, not widened floats).
template <typename IO> struct Raw8;
template <> struct Raw8<bf16_t> { u32x4 v; };
template <> struct Raw8<float> { float4v a, b; };

__device__ __forceinline__ void gload8(Raw8<bf16_t> &r, const bf16_t *p) {
    r.v = *(const u32x4 *)p;
}
__device__ __forceinline__ void gload8(Raw8<float> &r, const float *p) {
    r.a = *(const float4v *)p;
    r.b = *(const float4v *)(p + 4);
}
__device__ __forceinline__ void zero8(Raw8<bf16_t> &r) { r.v = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void zero8(Raw8<float> &r) {
    r.a = float4v{0, 0, 0, 0};
    r.b = float4v{0, 0, 0, 0};
}
__device__ __forceinline__ void unpack8(const Raw8<bf16_t> &r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r.v[i] << 16);
        x[2 * i + 1] = __uint_as_float(r.v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack8(const Raw8<float> &r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = r.a[i];
        x[4 + i] = r.b[i];
    }
}

// A [C][D] block of rows of a [.., rows, .., D] tensor (row pitch `rs`
// elements), loaded 8 elements per vector, vectors spread over the workgroup:
// vector i = tid + 256*j covers row i / (D/8), columns 8*(i % (D/8)) .. +7.
// Rows at or beyond `nvalid` read as zero.
template <typename IO, int C, int D>
struct ChunkRows {
    static constexpr int kVecPerRow = D / 8;
    static constexpr int kVec = C * D / 8 / kThreads;
    static_assert(kVec >= 1 && (C * D / 8) % kThreads == 0, "tile too small");
    Raw8<IO> r[kVec];

    __device__ static int row(int j) { return (threadIdx.x + kThreads * j) / kVecPerRow; }
    __device__ static int col(int j) { return 8 * ((threadIdx.x + kThreads * j) % kVecPerRow); }

    __device__ void load(const IO *base, int64_t rs, int nvalid) {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int rr = row(j);
            if (rr < nvalid) gload8(r[j], base + rr * rs + col(j));
            else zero8(r[j]);
        }
    }
    __device__ void get(int j, float (&x)[8]) const { unpack8(r[j], x); }
};

// Write 8 floats as operands at dst[0..7] (16-byte aligned).
template <typename OpT>
__device__ __forceinline__ void put8(OpT *dst, const float (&x)[8]);
template <>
__device__ __forceinline__ void put8<_Float16>(_Float16 *dst, const float (&x)[8]) {
    half8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
    *(half8 *)dst = h;
}
template <>
__device__ __forceinline__ void put8<float>(float *dst, const float (&x)[8]) {
    *(float4v *)dst = float4v{x[0], x[1], x[2], x[3]};
    *(float4v *)(dst + 4) = float4v{x[4], x[5], x[6], x[7]};
}

// Write 8 floats down a column: dst[i * ld] = x[i].
template <typename OpT>
__device__ __forceinline__ void put8_col(OpT *dst, int ld, const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i * ld] = Mma<OpT>::cvt(x[i]);
}

}  // namespace gdn
