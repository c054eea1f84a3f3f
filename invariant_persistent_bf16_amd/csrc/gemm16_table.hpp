// Kernel table of the persistent 16-bit GEMM for one tile shape.  Each tile
// shape is instantiated in its own translation unit (gemm16_*.hip) so that
// the library's sources compile in parallel.  Every shape reserves more than
// half of a compute unit's 160 KiB of LDS, so that the persistent grid (at
// most one workgroup per compute unit) lands one workgroup on each unit.
#pragma once

#include "gemm_bf16.hpp"

// [f16][B K-contiguous][16-bit out][vector epilogue]
#define BI_GEMM16_TABLE(BMV, BNV)                                                                          \
    namespace bi {                                                                                         \
    static_assert(2 * G16Cfg<BMV, BNV>::LDS > 160 * 1024 && G16Cfg<BMV, BNV>::LDS <= 160 * 1024,          \
                  "exactly one workgroup per compute unit");                                               \
    Gemm16Kern gemm16_kernel_##BMV##x##BNV(int f16, int kc, int out16, int cvec) {                         \
        static const Gemm16Kern t[2][2][2][2] = {                                                          \
            {{{gemm_bf16_persistent<false, 0, false, false, BMV, BNV>,                                     \
               gemm_bf16_persistent<false, 0, true, false, BMV, BNV>},                                     \
              {gemm_bf16_persistent<false, 1, false, false, BMV, BNV>,                                     \
               gemm_bf16_persistent<false, 1, true, false, BMV, BNV>}},                                    \
             {{gemm_bf16_persistent<true, 0, false, false, BMV, BNV>,                                      \
               gemm_bf16_persistent<true, 0, true, false, BMV, BNV>},                                      \
              {gemm_bf16_persistent<true, 1, false, false, BMV, BNV>,                                      \
               gemm_bf16_persistent<true, 1, true, false, BMV, BNV>}}},                                    \
            {{{gemm_bf16_persistent<false, 0, false, true, BMV, BNV>,                                      \
               gemm_bf16_persistent<false, 0, true, true, BMV, BNV>},                                      \
              {gemm_bf16_persistent<false, 1, false, true, BMV, BNV>,                                      \
               gemm_bf16_persistent<false, 1, true, true, BMV, BNV>}},                                     \
             {{gemm_bf16_persistent<true, 0, false, true, BMV, BNV>,                                       \
               gemm_bf16_persistent<true, 0, true, true, BMV, BNV>},                                       \
              {gemm_bf16_persistent<true, 1, false, true, BMV, BNV>,                                       \
               gemm_bf16_persistent<true, 1, true, true, BMV, BNV>}}}};                                    \
        return t[f16][kc][out16][cvec];                                                                    \
    }                                                                                                      \
    }
