// Persistent 16-bit GEMM kernels with 128x128 tiles (see gemm_bf16.hpp).
#include <hip/hip_runtime.h>

#include "gemm16_table.hpp"

BI_GEMM16_TABLE(128, 128)
