// The persistent 16-bit GEMM with 128x128 tiles and no LDS reservation, so
// that two of its workgroups (66 KiB of LDS each) can share a compute unit.
// Benchmark library only: it exists to show that the bits do not depend on
// how many workgroups share a unit.
#include <hip/hip_runtime.h>

#include "gemm_bf16.hpp"

namespace bi {
static_assert(2 * G16Cfg<128, 128, false>::LDS <= 160 * 1024, "two workgroups fit one compute unit");

Gemm16Kern gemm16_kernel_128x128_shared(int kc, int out16) {
    static const Gemm16Kern t[2][2] = {
        {gemm_bf16_persistent<false, 0, true, false, 128, 128, false>,
         gemm_bf16_persistent<false, 1, true, false, 128, 128, false>},
        {gemm_bf16_persistent<true, 0, true, false, 128, 128, false>,
         gemm_bf16_persistent<true, 1, true, false, 128, 128, false>}};
    return t[kc][out16];
}
}  // namespace bi
