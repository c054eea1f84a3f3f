// Device-side helpers shared by the HIP kernels of the batch-invariant path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bfloat16 bits -> binary32 (exact: bfloat16 is the upper half of binary32).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

// Two binary32 values -> two bfloat16 (a in the low half), round to nearest
// even.  gfx950's v_cvt_pk_bf16_f32; it agrees bit for bit with
// f32_to_bf16_rne on all 2^32 inputs (NaN quieting and subnormals included).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Two binary32 values -> two IEEE binary16 (a in the low half), round to
// nearest even (the language's conversion; overflow gives infinity).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// 16-bit element type of the matrix-core path: bfloat16 or binary16.
template <bool F16>
__device__ __forceinline__ uint32_t pack16x2(float a, float b) {
    if constexpr (F16) return pack_f16x2(a, b);
    else               return pack_bf16x2(a, b);
}
template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint16_t h) {
    if constexpr (F16) return f16_to_f32(h);
    else               return bf16_to_f32(h);
}

// Output element store in the requested dtype (0 = binary32, 1 = bfloat16).
template <int OUT_BF16>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float v) {
    if constexpr (OUT_BF16)
        ((uint16_t*)base)[idx] = f32_to_bf16_rne(v);
    else
        ((float*)base)[idx] = v;
}

}  // namespace bi
