/*
 * spgelu.h -- C ABI of the standalone elementwise tanh-GELU for MI355X (gfx950).
 *
 *   y[i] = gelu(x[i]),   gelu(x) = 0.5 x (1 + tanh(0.7978845608 (x + 0.044715 x^3)))
 *
 * The operation is the loop fusion the XLA:GPU emitters page works through in
 * its "Loop emitter" example (a bf16 [6,512,4096] tensor through the tanh
 * approximation of GELU) and the GeLU kernel of the Triton lecture notes (one
 * program per 1024-element block, masked tail).  It is the unfused counterpart
 * of the GEMM's GEMM_EPI_GELU_TANH epilogue (spgemm.h) and uses the same
 * arithmetic: the element is widened to fp32, the function is evaluated in fp32
 * with the constants above, and the result is rounded to nearest-even into the
 * element type.
 *
 * Conventions:
 *   - x and y are device pointers to n contiguous elements of `dtype`
 *     (GEMM_F16, GEMM_BF16 or GEMM_F32), owned by the caller.  y == x (in place)
 *     is allowed; any other overlap is not (not checked).
 *   - Any n >= 0 and any element alignment are accepted.  When x and y are both
 *     16-byte aligned the kernel moves 16 bytes per lane per access; otherwise it
 *     falls back to element-wise accesses.  n == 0 is a no-op.
 *   - Asynchronous on `stream` (0 = null stream); never allocates or synchronizes.
 *   - Errors are status codes (gemm_status): INVALID_ARG for n < 0, a NULL pointer
 *     with n > 0, or an unknown dtype (all checked before any HIP call); HIP for a
 *     launch failure, with the text in gemm_last_hip_error().
 */
#ifndef SPGELU_H
#define SPGELU_H

#include "spgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

gemm_status gelu_run(const void* x, void* y, int64_t n, gemm_dtype dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPGELU_H */
