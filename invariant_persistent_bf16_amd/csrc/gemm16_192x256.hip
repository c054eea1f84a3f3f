// Persistent 16-bit GEMM kernels with 192x256 tiles (see gemm_bf16.hpp).
#include <hip/hip_runtime.h>

#include "gemm16_table.hpp"

BI_GEMM16_TABLE(192, 256)
