/*
 * batq_vendor.h — hipBLASLt's block-scaled MXFP4 GEMM on the path's operands,
 * for comparison only.
 *
 * Not part of the path and not in libbatq.so.  A separate library,
 * libbatq_vendor.so, links against hipBLASLt, so that the W4A4 GEMM
 * [BATQuant note (en.papernotes.org), Key Designs §4: Y = Q(XP) Q(P^-1 W^T)]
 * can be timed and checked beside the vendor library's own kernel for the same
 * product, on the same GPU, operands and output.
 *
 * Operands are those of batq_mxfp4_gemm (batq.h):
 *   xq  [M][K/2]  E2M1 codes, row-major, element 2i in the low nibble
 *   xs  [M][K/32] UE8M0 scales
 *   wq  [N][K/2]  E2M1 codes of the prepared weights, row-major
 *   ws  [N][K/32] UE8M0 scales
 *   y   [M][N]    bf16 output, row-major
 * hipBLASLt is column-major.  Y^T (N x M, leading dimension N) = op(A) op(B)
 * with A = the weight codes (a K x N column-major matrix, transposed) and
 * B = the activation codes (K x M column-major, not transposed).  Both are
 * scaled per 32 elements along K (HIPBLASLT_MATMUL_MATRIX_SCALE_VEC32_UE8M0).
 * The computation is fp32, with beta = 0.
 *
 * All pointers are device pointers.  Calls are asynchronous on `stream`.  The
 * library allocates no device memory: the caller passes the workspace.
 * Return values: 0 on success, otherwise
 *   -1  bad arguments: a size <= 0, K not a multiple of 32, max_algos
 *       outside [1, 64], algo outside [0, algos), a NULL pointer;
 *   -2  a hipBLASLt call failed: batq_vendor_last_status gives its status;
 *   -3  the heuristic offers no algorithm for this shape.
 */
#ifndef BATQ_VENDOR_H
#define BATQ_VENDOR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct batq_vendor_gemm batq_vendor_gemm;

/* Plans Y = X W^T for an M x N x K problem.  It asks hipBLASLt's heuristic
 * for up to max_algos algorithms that fit `workspace_bytes` of workspace.
 * On success *plan owns a hipBLASLt handle and descriptors until
 * batq_vendor_gemm_destroy.  On failure *plan is NULL. */
int batq_vendor_gemm_create(int64_t M, int64_t N, int64_t K, int32_t max_algos, size_t workspace_bytes,
                            batq_vendor_gemm** plan);

/* The number of algorithms the heuristic returned (>= 1), in its order of
 * preference.  Returns -1 for a NULL plan. */
int32_t batq_vendor_gemm_algos(const batq_vendor_gemm* plan);

/* Runs algorithm `algo` of the plan.  The workspace has the plan's
 * workspace_bytes.  A plan is not safe to run from two threads at once,
 * because the scale pointers are set on its descriptor for each call. */
int batq_vendor_gemm_run(batq_vendor_gemm* plan, int32_t algo, const uint8_t* xq, const uint8_t* xs,
                         const uint8_t* wq, const uint8_t* ws, uint16_t* y, void* workspace, hipStream_t stream);

/* Releases the plan.  Does nothing for NULL. */
void batq_vendor_gemm_destroy(batq_vendor_gemm* plan);

/* hipBLASLt's version number (hipblasLtGetVersion), or -1 if it cannot be read. */
int32_t batq_vendor_version(void);

/* The status of the last hipBLASLt call that failed in this library, or 0. */
int32_t batq_vendor_last_status(void);

#ifdef __cplusplus
}
#endif

#endif /* BATQ_VENDOR_H */
