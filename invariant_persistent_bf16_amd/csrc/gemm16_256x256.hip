// Persistent 16-bit GEMM kernels with 256x256 tiles (see gemm_bf16.hpp).
#include <hip/hip_runtime.h>

#include "gemm16_table.hpp"

BI_GEMM16_TABLE(256, 256)
