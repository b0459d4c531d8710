// Buffer-resource loads and stores (MUBUF): a 128-bit descriptor in SGPRs
// holds the base and the byte range, each access adds a 32-bit VGPR offset
// and a uniform SGPR offset.  Accesses past the range read zero and drop
// stores in hardware, which is how the kernels handle a sequence end that
// falls inside a chunk: the range of a (batch, head) stream ends at token T.
#pragma once

#include "gdn_device.h"

namespace gdn {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// dword 3 of a raw buffer descriptor on gfx9-family parts
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void bstore32(uint32_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, voff, soff, 0);
}
__device__ __forceinline__ void bstore16(uint16_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(x, r, voff, soff, 0);
}

// One io element as float (buffer path).
template <typename IO> struct BufElem;
template <> struct BufElem<float> {
    __device__ static float load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __uint_as_float(bload32(r, voff, soff));
    }
    __device__ static void store(float x, rsrc_t r, uint32_t voff, uint32_t soff) {
        bstore32(__float_as_uint(x), r, voff, soff);
    }
};
template <> struct BufElem<bf16_t> {
    __device__ static float load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __uint_as_float((uint32_t)bload16(r, voff, soff) << 16);
    }
    __device__ static void store(float x, rsrc_t r, uint32_t voff, uint32_t soff) {
        bstore16(f32_to_bf16_bits(x), r, voff, soff);
    }
};

// Store one 16 x 16 accumulator tile x of a row-major matrix (lane (g, j)
// holds rows 4g .. 4g+3 of column j) as runs of two columns: lanes j and
// j ^ 1 swap halves (DPP quad_perm [1,0,3,2]), so that the even lane holds
// rows 4g, 4g+1 and the odd lane rows 4g+2, 4g+3 of columns j & ~1 and
// j | 1, and each lane issues two stores of two elements (4 bytes bf16,
// 8 bytes fp32) instead of four of one.  voff is the byte offset of this
// lane's (row 4g + 2 (j & 1), column j & ~1); row_bytes the row pitch;
// soff the uniform offset of the tile's row 0.
template <typename OT>
__device__ __forceinline__ void store_acc_pairs(const float4v &x, rsrc_t r, uint32_t voff,
                                                uint32_t row_bytes, uint32_t soff) {
    const bool odd = lane_id() & 1;
    const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
    const float r0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0xB1, 0xf, 0xf, false));
    const float r1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xf, 0xf, false));
    const float a0 = odd ? r0 : x[0], b0 = odd ? x[2] : r0;     // row 2 odd + 0
    const float a1 = odd ? r1 : x[1], b1 = odd ? x[3] : r1;     // row 2 odd + 1
    if constexpr (sizeof(OT) == 2) {
        bstore32((uint32_t)f32_to_bf16_bits(a0) | ((uint32_t)f32_to_bf16_bits(b0) << 16), r, voff, soff);
        bstore32((uint32_t)f32_to_bf16_bits(a1) | ((uint32_t)f32_to_bf16_bits(b1) << 16), r, voff,
                 soff + row_bytes);
    } else {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(a0), __float_as_uint(b0)}, r, voff, soff, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(a1), __float_as_uint(b1)}, r, voff,
                                              soff + row_bytes, 0);
    }
}

// Eight raw io elements (16 bytes of bf16, 32 bytes of fp32).
template <typename IO> struct Raw8B;
template <> struct Raw8B<bf16_t> {
    u32x4 v;
    __device__ void load(rsrc_t r, uint32_t voff, uint32_t soff) { v = bload128(r, voff, soff); }
};
template <> struct Raw8B<float> {
    u32x4 a, b;
    __device__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
        a = bload128(r, voff, soff);
        b = bload128(r, voff + 16, soff);
    }
};

// Raw io elements -> operand type, written as one 16-byte (f16) or two
// 16-byte (fp32) LDS stores.  Optional per-element scale.
__device__ __forceinline__ void put_raw8(_Float16 *dst, const Raw8B<bf16_t> &r) {
    half8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[2 * i] = (_Float16)__uint_as_float(r.v[i] << 16);
        h[2 * i + 1] = (_Float16)__uint_as_float(r.v[i] & 0xffff0000u);
    }
    *(half8 *)dst = h;
}
__device__ __forceinline__ void put_raw8(float *dst, const Raw8B<float> &r) {
    *(u32x4 *)dst = r.a;
    *(u32x4 *)(dst + 4) = r.b;
}
__device__ __forceinline__ void unpack_raw8(const Raw8B<bf16_t> &r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r.v[i] << 16);
        x[2 * i + 1] = __uint_as_float(r.v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack_raw8(const Raw8B<float> &r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = __uint_as_float(r.a[i]);
        x[4 + i] = __uint_as_float(r.b[i]);
    }
}

// Transposed A fragment: lane l supplies A[m0 + l%16][k0 + 8 (l/16) .. +7]
// where A = S^T for a row-major S [k][m] in LDS (pitch ld): the eight values
// walk down a column of S.  For f16 this is two ds_read_b64_tr_b16: within a
// 16-lane group, lane i receives element (i % 4) of the 64-bit words fetched
// by lanes 4e + i/4 (e = 0..3), so lane L fetches row k0 + 8q + L/4, columns
// m0 + 4 (L % 4) .. +3.
__device__ __forceinline__ half8 frag_T(const _Float16 *S, int ld, int m0, int k0) {
    const int l = lane_id(), q = l >> 4, L = l & 15;
    const _Float16 *p = S + (k0 + 8 * q + (L >> 2)) * ld + m0 + 4 * (L & 3);
    typedef __fp16 v4fp16 __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;
    // (the f16-typed form: element-wise repacking of the i16-typed form has
    // been seen to compile into a lane-replicating permute)
    const half4 a = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16 *)p));
    const half4 b = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16 *)(p + 4 * ld)));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Mma<float>::frag frag_T(const float *S, int ld, int m0, int k0) {
    const int l = lane_id(), q = l >> 4, m = m0 + (l & 15);
    Mma<float>::frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.lo[e] = S[(k0 + 8 * q + e) * ld + m];
        f.hi[e] = S[(k0 + 8 * q + 4 + e) * ld + m];
    }
    return f;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8]).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm0 = waitcnt_vm(0);
constexpr int kWaitLgkm0 = (15) | (3 << 14) | (7 << 4);   // lgkmcnt(0), vmcnt/expcnt max

// Raw staged vector (16 bytes) back from LDS.
__device__ __forceinline__ void stage_get(Raw8B<bf16_t> &r, const uint16_t *p) {
    r.v = *(const u32x4 *)p;
}

// Accumulator-layout read of a row-major 16-bit matrix S (pitch ld): lane
// (g = l/16, j = l%16) gets S[4g + e][m0 + j] for e = 0..3 (one
// ds_read_b64_tr_b16; lane L of each 16-lane group fetches row 4g + L/4,
// columns m0 + 4 (L % 4) .. +3).
__device__ __forceinline__ u32x2 read_T4(const uint16_t *S, int ld, int m0) {
    const int l = lane_id(), L = l & 15;
    const uint16_t *p = S + (4 * (l >> 4) + (L >> 2)) * ld + m0 + 4 * (L & 3);
    typedef __fp16 v4fp16 __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16 *)p));
}

// ---------------------------------------------------------------------------
// Register-chained products.  The accumulator of a 16x16 tile C gives lane
// (q = l/16, j = l%16) the rows 4q .. 4q+3 of column j.  Two such tiles that
// cover rows 0..15 and 16..31 of a 32-wide k step therefore hand lane group q
// eight distinct k values, {4q + e} and {16 + 4q + e} (e = 0..3), and column
// j: exactly a B fragment, if the A fragment uses the same "split" k slots.
// Products chained this way keep their intermediate in registers.
// ---------------------------------------------------------------------------

// B fragment from the accumulators of the k rows [k0, k0+16) and [k0+16, k0+32).
__device__ __forceinline__ half8 fragB_acc(const float4v &lo, const float4v &hi, _Float16) {
    half8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (_Float16)lo[e];
        h[4 + e] = (_Float16)hi[e];
    }
    return h;
}
__device__ __forceinline__ Mma<float>::frag fragB_acc(const float4v &lo, const float4v &hi, float) {
    Mma<float>::frag f;
    f.lo = lo;
    f.hi = hi;
    return f;
}

// A fragment with split k slots from a row-major S[m][k] (pitch ld): lane
// (q, i) reads S[m0 + i][k0 + 4q .. +3] and S[m0 + i][k0 + 16 + 4q .. +3].
__device__ __forceinline__ half8 fragA_split(const _Float16 *S, int ld, int m0, int k0) {
    const int l = lane_id();
    const _Float16 *p = S + (m0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
    const half4 a = *(const half4 *)p, b = *(const half4 *)(p + 16);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Mma<float>::frag fragA_split(const float *S, int ld, int m0, int k0) {
    const int l = lane_id();
    const float *p = S + (m0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
    Mma<float>::frag f;
    f.lo = *(const float4v *)p;
    f.hi = *(const float4v *)(p + 16);
    return f;
}

// A fragment with split k slots from the transpose of a row-major S[k][m]:
// lane (q, i) gets S[k0 + 4q + e][m0 + i] and S[k0 + 16 + 4q + e][m0 + i].
__device__ __forceinline__ half8 fragAT_split(const _Float16 *S, int ld, int m0, int k0) {
    const half4 a = __builtin_bit_cast(half4, read_T4((const uint16_t *)(S + k0 * ld), ld, m0));
    const half4 b = __builtin_bit_cast(half4, read_T4((const uint16_t *)(S + (k0 + 16) * ld), ld, m0));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Mma<float>::frag fragAT_split(const float *S, int ld, int m0, int k0) {
    const int l = lane_id(), q = l >> 4, m = m0 + (l & 15);
    Mma<float>::frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.lo[e] = S[(k0 + 4 * q + e) * ld + m];
        f.hi[e] = S[(k0 + 16 + 4 * q + e) * ld + m];
    }
    return f;
}

// Store an accumulator tile transposed, dst[n][m] (m contiguous), with one
// 8-byte (f16) or 16-byte (fp32) LDS store per lane.
__device__ __forceinline__ void store_T(_Float16 *dst, int ld, const float4v &acc) {
    const int l = lane_id();
    half4 h;
    h[0] = (_Float16)acc[0];
    h[1] = (_Float16)acc[1];
    h[2] = (_Float16)acc[2];
    h[3] = (_Float16)acc[3];
    *(half4 *)(dst + (l & 15) * ld + 4 * (l >> 4)) = h;
}
__device__ __forceinline__ void store_T(float *dst, int ld, const float4v &acc) {
    const int l = lane_id();
    *(float4v *)(dst + (l & 15) * ld + 4 * (l >> 4)) = acc;
}

}  // namespace gdn
