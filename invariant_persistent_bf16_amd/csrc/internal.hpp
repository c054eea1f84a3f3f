// Host-side descriptors shared by the public entry points and the
// benchmark-only variants (one library source tree, one set of kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// A (possibly batched) GEMM: slice s in [0, G1*G2) with s1 = s / G2,
// s2 = s % G2; operand X of slice s starts at X + s1*sX1 + s2*sX2.
struct GemmDesc {
    int64_t G1, G2, M, N, K;
    const void* A; int64_t sA1, sA2, sAm, sAk;
    const void* B; int64_t sB1, sB2, sBk, sBn;
    const void* bias; int64_t sBias2;
    int bias_rows;   // bias broadcast along columns (0, addmm) or rows (1, conv)
    void* C; int64_t sC1, sC2, sCm, sCn;
    int in_dtype, out_dtype;
};

int device_cu_count(int* cus);
int gemm_check(const GemmDesc& d);
int gemm_launch(const GemmDesc& d, hipStream_t st, int grid_override);

}  // namespace bi
