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
// Rows per block of the small-tile kernel that gemm_launch picks for a 16-bit
// product (0: the persistent 256x256 kernel).
int gemm_tile_rows(const GemmDesc& d, int cus);
// tile_rows: -1 lets the shape choose the kernel; 0 forces the persistent
// 256x256 kernel (on grid_override workgroups if > 0); 32, 64 or 128 force
// the small-tile kernel with blocks of that many rows.  Every choice gives the
// same bits.
// ev (optional): events that the runtime records at the start and the end
// of the GEMM kernel's own execution (hipExtLaunchKernelGGL), for timing.
struct LaunchEvents {
    hipEvent_t start, stop;
};
int gemm_launch(const GemmDesc& d, hipStream_t st, int grid_override, int tile_rows = -1,
                const LaunchEvents* ev = nullptr);
GemmDesc mm_desc(int64_t M, int64_t N, int64_t K, const void* A, int64_t sAm, int64_t sAk,
                 const void* B, int64_t sBk, int64_t sBn, const void* bias, void* C,
                 int64_t sCm, int64_t sCn, int in_dtype, int out_dtype);

}  // namespace bi
