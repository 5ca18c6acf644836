// Error text shared by the library's entry points: the last HIP error a call on
// this thread saw, as returned by gemm_last_hip_error().
#pragma once

#include <hip/hip_runtime.h>

#include "spgemm.h"

namespace spg {

// Records hipGetErrorString(e) for this thread and returns GEMM_ERR_HIP.
gemm_status hip_fail(hipError_t e);
const char* last_hip_error();

}  // namespace spg
