// Branch-free access to one row of a matrix, in chunks of 4 elements, for the
// row-per-program kernels (softmax, RMSNorm, log-softmax, mean).
//
// The row is a buffer resource whose record count ends at the row's last
// byte, so reads past the row return zero and writes past it are dropped by
// the hardware; a read then replaces the positions past `cols` by the caller's
// fill value (the identity of its fold).  No access sits in a branch, so the
// compiler issues all of a wave's loads before waiting for any.  VEC: one 8-
// (bfloat16) or 16-byte (binary32) access per chunk (needs cols % 4 == 0 and
// an aligned row); otherwise one access per element.  Both give the same values.
#pragma once

#include "common.hpp"

namespace bi {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Buffer resource of `bytes` bytes at a wave-uniform address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
    const uint64_t v = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// Chunk c of a row of `cols` elements (bfloat16 if BF16, else binary32), as
// binary32 (times `scale` if SCALED), with `fill` past cols.  NT = 2 makes
// the loads non-temporal (for data read once that should not evict what is
// reused).
template <bool BF16, bool VEC, bool SCALED = false, int NT = 0>
__device__ __forceinline__ f32x4_t row_load(__amdgpu_buffer_rsrc_t r, int c, int cols, float fill,
                                            float scale = 1.0f) {
    f32x4_t x;
    if constexpr (VEC && BF16) {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, c * 8, 0, NT);
        x = f32x4_t{bf16lo_to_f32(w[0]), bf16hi_to_f32(w[0]), bf16lo_to_f32(w[1]), bf16hi_to_f32(w[1])};
    } else if constexpr (VEC) {
        x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, c * 16, 0, NT));
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) x[e] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (4 * c + e) * 2, 0, NT));
            else x[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (4 * c + e) * 4, 0, NT));
        }
    }
    if constexpr (VEC) {   // cols % 4 == 0: a chunk is all inside the row or all past it
        const bool ok = 4 * c < cols;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (SCALED) x[e] = ok ? x[e] * scale : fill;
            else                  x[e] = ok ? x[e] : fill;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (SCALED) x[e] = 4 * c + e < cols ? x[e] * scale : fill;
            else                  x[e] = 4 * c + e < cols ? x[e] : fill;
        }
    }
    return x;
}

// Store chunk c (elements past the row's end are dropped by the buffer).
// AUX = 2: non-temporal (outputs too large to stay in the caches).
template <bool VEC, int AUX = 0>
__device__ __forceinline__ void row_store(__amdgpu_buffer_rsrc_t r, int c, f32x4_t y, bool out_bf16) {
    if (out_bf16) {
        if constexpr (VEC) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])}, r,
                                                  c * 8, 0, AUX);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pack_bf16x2(y[e], 0.0f), r, (4 * c + e) * 2, 0, AUX);
        }
    } else {
        if constexpr (VEC) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, y), r, c * 16, 0, AUX);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[e]), r, (4 * c + e) * 4, 0, AUX);
        }
    }
}

}  // namespace bi
