/*
 * batq.h — C ABI of the BATQuant W4A4 deployment path on MI355X (gfx950).
 *
 * What the library computes (BATQuant pages; cited by page and section):
 *   A linear layer Y = X W^T is rewritten as Y = (X P)(P^-1 W^T).  P is block
 *   diagonal over the 32-channel MXFP4 blocks, each block P_i = B_i (x) A with one
 *   shared a x a factor A and a private b x b factor B_i, a * b = 32
 *   [en.papernotes.org BATQuant note, Key Designs §1-§2; nubint.ai review, 提案手法].
 *   The activation side is transformed online, clipped block-wise with
 *   sigmoid-mapped ratios on the block max/min, and quantised to MXFP4; the
 *   weight side P^-1 W^T is fused and quantised offline; the two quantised
 *   operands meet in a W4A4 GEMM [en.papernotes.org, Overall Architecture;
 *   Key Designs §3; A Worked Example].
 *
 * Conventions shared by every entry point:
 *   - Row-major everywhere.  Block i of row m is channels [32 i, 32 i + 32).
 *   - Vec convention of the block transform (the pages leave it open): row
 *     vector, y_b = x_b P_i with P_i[a r + c][a r' + c'] = B_i[r][r'] A[c][c'].
 *   - MXFP4 storage: codes [rows][K/2] bytes, element 2j in the low nibble of
 *     byte j; code = sign << 3 | magnitude index into {0,.5,1,1.5,2,3,4,6};
 *     scales [rows][K/32] bytes, UE8M0 (value 2^(byte-127)).
 *   - Scale exponent floor(log2 amax) - 2 clamped to [-127, 127] (OCP MX v1.0
 *     rule), elements rounded to nearest E2M1 with ties to the even code, |v| >= 6
 *     saturating to 6, sign kept (a negative value rounding to 0 is code 0x8).
 *   - Device pointers unless the name ends in _host.  Every device call is
 *     asynchronous on `stream` (0 = the null stream).  The library never
 *     allocates, frees or synchronises and keeps no pointer after returning.
 *     Its only mutable global state is the device array of the no-allocation
 *     decode entry point (calls of that entry point that overlap on one GPU
 *     race); every other call on distinct streams is thread-safe.
 *   - The caller owns every buffer and keeps it alive until the stream work
 *     completes.
 *   - Errors: every argument check runs on the host before any HIP call and
 *     returns a status without launching anything; a launch failure reported by
 *     hipGetLastError maps to BATQ_ERR_HIP.  Nothing is printed, nothing thrown.
 *   - Non-finite inputs are outside the defined domain (results unspecified,
 *     no fault).
 */
#ifndef BATQ_H
#define BATQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BATQ_ABI_VERSION 5

typedef enum {
  BATQ_OK = 0,
  BATQ_ERR_NULL = 1,        /* a required pointer is NULL                         */
  BATQ_ERR_SHAPE = 2,       /* negative size, K not a positive multiple of 32,
                               leading dimension smaller than K, a*b != 32        */
  BATQ_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks the stated
                               alignment                                          */
  BATQ_ERR_UNSUPPORTED = 4, /* a outside {1,2,4,8,16,32} or unknown output type   */
  BATQ_ERR_SINGULAR = 5,    /* a factor is singular or too ill-conditioned        */
  BATQ_ERR_HIP = 6,         /* the HIP runtime rejected a launch                  */
  BATQ_ERR_TOO_LARGE = 7    /* the problem needs more scratch than the
                               no-allocation entry point holds                    */
} batq_status;

typedef enum { BATQ_OUT_BF16 = 0, BATQ_OUT_F32 = 1 } batq_out_dtype;

/* BATQ_ABI_VERSION of the built library. */
int batq_abi_version(void);

/* Static English text of a status code ("unknown status" for other values). */
const char* batq_status_str(int status);

/* ---------------------------------------------------------------- host helpers
 * Host-only; no HIP call.
 */

/* Clip ratios r = sigmoid(logit), evaluated in double and rounded once to float:
 * the deployed form of the learnable block-wise clipping parameters, which a
 * sigmoid maps into (0, 1) [en.papernotes.org, Key Designs §3].
 * logits_host, ratios_host: n floats each (may alias).  n >= 0.
 * Errors: NULL (either pointer NULL with n > 0), SHAPE (n < 0). */
batq_status batq_clip_ratios(const float* logits_host, float* ratios_host, int64_t n);

/* Inverse-transposed GPK factors for the offline weight side.  Because
 * (B_i (x) A)^-T = B_i^-T (x) A^-T, the weight transform W P^-T is the same
 * block transform with factors A^-T and B_i^-T [en.papernotes.org, Key Designs
 * §1-§2: the inverse is absorbed into the weights].
 * A_host: [a][a] floats; B_host: [nblocks][b][b] floats.
 * AinvT_host: [a][a]; BinvT_host: [nblocks][b][b] (outputs, float, computed by
 * Gauss-Jordan elimination with partial pivoting in double, rounded once).
 * Errors: NULL; SHAPE (nblocks < 0, a*b != 32); UNSUPPORTED (a not a power of two
 * in 1..32); SINGULAR (a zero pivot or an estimated 1-norm condition number above
 * 1e6 for any factor; outputs then unspecified). */
batq_status batq_gpk_invert(int32_t a, int32_t b, int64_t nblocks, const float* A_host,
                            const float* B_host, float* AinvT_host, float* BinvT_host);

/* --------------------------------------------------------------- device calls */

/* Online activation path, one fused kernel: per row m and block i,
 *   y = x_b (B_i (x) A)                      (block transform, fp32 accumulation)
 *   z = min(max(y, r_lo[i] * min(y)), r_hi[i] * max(y))   (block-wise clipping)
 *   Xs[m][i] = e + 127, Xq codes = RNE_E2M1(z / 2^e)      (MXFP4 quantisation)
 * [en.papernotes.org, A Worked Example: transform block by block, clip, quantise;
 *  Key Designs §1-§3].
 * X_bf16: [M][ldx] bfloat16, row stride ldx elements (ldx >= K, ldx % 8 == 0,
 *         X 16-byte aligned).
 * A: [a][a] float; B: [K/32][b][b] float (the factors, row-major).
 * r_hi, r_lo: [K/32] float clip ratios (batq_clip_ratios), or both NULL for no
 *         clipping.  One NULL and one non-NULL is BATQ_ERR_NULL.
 * Xq: [M][K/2] bytes (16-byte aligned); Xs: [M][K/32] bytes.
 * M == 0 is a no-op.  Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, HIP. */
batq_status batq_act_transform_quant(const void* X_bf16, int64_t M, int64_t K, int64_t ldx,
                                     int32_t a, int32_t b, const float* A, const float* B,
                                     const float* r_hi, const float* r_lo,
                                     uint8_t* Xq, uint8_t* Xs, hipStream_t stream);

/* Offline weight side: W' = W P^-T block by block (the transpose of P^-1 W^T),
 * clipped with one ratio pair per (output row, block), MXFP4-quantised with the
 * same rules [en.papernotes.org, Overall Architecture; Key Designs §3: weights
 * receive analogous treatment].  Run once per layer; round-to-nearest, no GPTQ.
 * W_bf16: [N][ldw] bfloat16 (ldw >= K, ldw % 8 == 0, 16-byte aligned).
 * AinvT: [a][a]; BinvT: [K/32][b][b] float — the outputs of batq_gpk_invert.
 * wr_hi, wr_lo: [N][K/32] float ratios, or both NULL for no clipping.
 * Wq: [N][K/2] (16-byte aligned); Ws: [N][K/32].
 * N == 0 is a no-op.  Errors: as batq_act_transform_quant. */
batq_status batq_weight_prep(const void* W_bf16, int64_t N, int64_t K, int64_t ldw,
                             int32_t a, int32_t b, const float* AinvT, const float* BinvT,
                             const float* wr_hi, const float* wr_lo,
                             uint8_t* Wq, uint8_t* Ws, hipStream_t stream);

/* W4A4 GEMM on MXFP4 operands: Y[m][n] = sum_k deq(Xq)[m][k] * deq(Wq)[n][k] with
 * FP32 accumulation on the block-scaled MFMA units, written as float or as
 * bfloat16 (round to nearest even) [en.papernotes.org, Key Designs §1 and §4:
 * the product Q(XP) Q(P^-1 W^T); all linear layers use low-bit matmul].
 * Xq: [M][K/2], Xs: [M][K/32], Wq: [N][K/2], Ws: [N][K/32] (code rows 16-byte
 * aligned, which K % 32 == 0 gives for 16-byte aligned bases).
 * Y: [M][N] of the chosen type, 4-byte aligned.
 * M == 0 or N == 0 is a no-op.  Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, HIP. */
batq_status batq_mxfp4_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                            const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y,
                            batq_out_dtype out, hipStream_t stream);

/* ------------------------------------------------- packed-weight fast path
 * The weight side is fixed after the offline step, so it can also be stored
 * in the order the matrix cores consume it.  The packed GEMM computes exactly
 * the same sums, in the same order, as batq_mxfp4_gemm; it needs K % 256 == 0.
 */

/* Bytes of the packed form of an [N][K/2] + [N][K/32] MXFP4 weight:
 * ceil(N/32) * (K/256) * 4352.  Returns -1 for N < 0 or K not a positive
 * multiple of 256.  Host only. */
int64_t batq_weight_packed_bytes(int64_t N, int64_t K);

/* Offline: repack Wq/Ws (batq_weight_prep outputs) for batq_mxfp4_gemm_packed.
 * Layout, per group of 32 rows n32 and 256-k stage s (4352 bytes): four
 * sub-steps j of 64 lanes x 16 code bytes (lane l: MX block 8s + 4(l/32) + j of
 * row 32 n32 + l%32), then 64 lanes x 4 scale bytes (lane l: blocks
 * 8s + 4(l/32) + 0..3 of the same row).  Rows past N are zero codes with unit
 * scale.  Wp: batq_weight_packed_bytes(N, K) bytes, 16-byte aligned.
 * Wq 16-byte aligned.  N == 0 is a no-op.
 * Errors: NULL, SHAPE (K % 256 != 0), ALIGN, HIP. */
batq_status batq_weight_pack(const uint8_t* Wq, const uint8_t* Ws, int64_t N, int64_t K, uint8_t* Wp,
                             hipStream_t stream);

/* Y[M][N] = deq(Xq,Xs) deq(W)^T with W given packed by batq_weight_pack; same
 * result as batq_mxfp4_gemm on the unpacked operands [en.papernotes.org, Key
 * Designs §1 and §4].  Xq, Xs and Wp 16-byte aligned, Y 4-byte aligned.  M == 0 or N == 0 is a no-op.
 * Errors: NULL, SHAPE (K % 256 != 0), ALIGN, UNSUPPORTED (output type), HIP. */
batq_status batq_mxfp4_gemm_packed(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wp, int64_t M,
                                   int64_t N, int64_t K, void* Y, batq_out_dtype out, hipStream_t stream);

/* Host-only query: which kernel batq_mxfp4_gemm_packed (act_fp8 == 0) or
 * batq_mxfp8_gemm_packed (act_fp8 != 0) launches for this shape.  0: one
 * 128 x 256 tile per workgroup, one workgroup per CU; 1: the same tiles and
 * the same results bit for bit, two workgroups per CU with direct-to-LDS
 * activation loads (more than 256 tiles, K / 256 in {4, 8, 16, 48}, activation
 * codes under 2 GiB).  For profiling and reports; -1 on a bad shape. */
int32_t batq_packed_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t act_fp8);

/* Host-only query: which instance batq_act_transform_quant (and the other
 * entry points built on the same kernel: _mxfp8, batq_weight_prep,
 * batq_kv_cache_quant) launches for `rows` rows of K channels.  0: two
 * workgroups per CU, each compute wave also loading (grids of 512 or more
 * workgroups; with the skewed tile walk where every workgroup gets 16 or more
 * tiles of equal walks); 1: one workgroup per CU with a dedicated loader wave
 * (smaller grids).  Both give the same codes bit for bit.
 * For profiling and reports; -1 on a bad shape (rows < 0, K <= 0 or
 * K % 32 != 0). */
int32_t batq_transform_kernel(int64_t rows, int64_t K);

/* ------------------------------------------------ W4A8: MXFP8 activations
 * The pages also report a W4A8 setting: MXFP8 activations against the same
 * MXFP4 weights [nubint.ai review, Table 2], with E4M3 elements
 * [en.papernotes.org, Loss & Training].  The encoding is the OCP MX E4M3 format: one code byte per element (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest value
 * 448, S.1111.111 never produced), one UE8M0 scale per 32 elements with
 * exponent floor(log2 amax) - 8 clamped to [-127, 127], elements rounded to
 * nearest with ties to the even code, |v| > 448 saturating to 448, sign kept.
 */

/* Online activation path with MXFP8 output: the same block transform and
 * clipping as batq_act_transform_quant, then MXFP8 quantisation.
 * Xq8: [M][K] bytes (E4M3 codes, element k at byte k), 16-byte aligned;
 * Xs: [M][K/32]; every other argument, check and error as for
 * batq_act_transform_quant. */
batq_status batq_act_transform_quant_mxfp8(const void* X_bf16, int64_t M, int64_t K, int64_t ldx,
                                           int32_t a, int32_t b, const float* A, const float* B,
                                           const float* r_hi, const float* r_lo,
                                           uint8_t* Xq8, uint8_t* Xs, hipStream_t stream);

/* W4A8 GEMM: Y[m][n] = sum_k deq8(Xq8, Xs)[m][k] * deq4(W)[n][k] with W packed
 * by batq_weight_pack, FP32 accumulation on the block-scaled FP8 x FP4 MFMA
 * units, bfloat16 (round to nearest even) or float output.
 * Accuracy: on top of fp32 accumulation, these units sum each run of 8
 * consecutive k in a fixed-point window 13 bits below the run's largest
 * exponent sum, truncating smaller products toward zero; a run loses less than
 * 7 * 2^-12 of its largest |x w| (measured; the FP4 x FP4 path is not affected).
 * Xq8 [M][K] (16-byte aligned), Xs [M][K/32] (16-byte aligned), Wp 16-byte
 * aligned, Y [M][N] 4-byte aligned.  M == 0 or N == 0 is a no-op.
 * Errors: NULL, SHAPE (K % 256 != 0), ALIGN, UNSUPPORTED (output type), HIP. */
batq_status batq_mxfp8_gemm_packed(const uint8_t* Xq8, const uint8_t* Xs, const uint8_t* Wp, int64_t M,
                                   int64_t N, int64_t K, void* Y, batq_out_dtype out, hipStream_t stream);

/* ------------------------------------------------ KV-cache quantisation
 * The pages place transforms on the key and value cache paths, per head, and
 * report KV8 and KV4 settings (W4A8KV8, W4A8KV4) [en.papernotes.org, Overall
 * Architecture; nubint.ai review, Table 2].  Here a token's K (or V) row,
 * all heads side by side (HD = heads x head_dim channels, head_dim a multiple
 * of 32 so that no block straddles two heads), goes through the same block
 * transform, optional block-wise clipping and MX quantisation as activations,
 * and is written to its cache slot.
 */

/* KV_bf16: [T][ld] bfloat16 new rows (ld >= HD, ld % 8 == 0, 16-byte aligned);
 * A: [a][a], B: [HD/32][b][b] (one private factor per 32-channel block of each
 * head); r_hi, r_lo: [HD/32] clip ratios or both NULL.  slots: [T] int64 device
 * array (8-byte aligned), token t goes to cache row slots[t]; slots outside
 * [0, cache_rows) are skipped, slots must be distinct.  fmt: 4 (MXFP4 E2M1
 * codes, cache_q [cache_rows][HD/2]) or 8 (MXFP8 E4M3, cache_q
 * [cache_rows][HD]); cache_s [cache_rows][HD/32] scales; cache_q 16-byte
 * aligned.  Rows not named by a slot are left untouched.  T == 0 is a no-op.
 * Errors: NULL, SHAPE (HD not a positive multiple of 32, negative sizes),
 * ALIGN, UNSUPPORTED (factor size or fmt), HIP. */
batq_status batq_kv_cache_quant(const void* KV_bf16, int64_t T, int64_t HD, int64_t ld, int32_t a, int32_t b,
                                const float* A, const float* B, const float* r_hi, const float* r_lo,
                                const int64_t* slots, int64_t cache_rows, int32_t fmt, uint8_t* cache_q,
                                uint8_t* cache_s, hipStream_t stream);

/* ------------------------------------------------ fused decode step
 * For decode-sized batches the online transform and quantisation run inside
 * the GEMM's prologue instead of as a separate launch [en.papernotes.org, Key
 * Designs §1-§4 and A Worked Example: transform, clip, quantise, multiply;
 * the pages report the online transform's cost as the decode overhead].
 */
#define BATQ_DECODE_MAX_M 32
/* Largest K of the decode calls: 8191 K splits of two 256-k stages (the
 * kernel counts splits in 13 bits). */
#define BATQ_DECODE_MAX_K 4193792

/* Workspace bytes batq_w4a4_decode needs for (M, N, K): 16 KiB of arrival
 * counters, then fp32 partial tiles, one per 128-column chunk, K split and
 * token, where a K split covers two 256-k stages; 0 when K is at most 512 (one
 * split: Y is written directly, no workspace is touched).
 * -1 for M outside [0, 32], N outside [0, 524288] or K not a positive
 * multiple of 256 up to 4193792 (8191 K splits). */
int64_t batq_decode_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Y[M][N] = deq(Q(X P)) deq(Wp)^T with the activation path fused into the
 * GEMM, in one launch: the block transform, clip and MXFP4 quantisation of X
 * (bit-identical to batq_act_transform_quant) feed the block-scaled MFMA
 * against weights packed by batq_weight_pack, split over 128-column chunks and
 * K splits of two 256-k stages.  Each split's fp32 partial tile goes to the
 * workspace; the workgroup that finishes a chunk last adds the chunk's
 * partials in split order and writes Y, so results are deterministic and
 * within the fp32 accumulation bound of the unsplit product.
 * X_bf16: [M][ldx] bf16, 1 <= M <= 32 (M == 0 or N == 0 is a no-op), K a
 * multiple of 256 up to 4193792, N up to 524288, ldx >= K and a multiple of 8,
 * X 16-byte aligned.  A, B,
 * r_hi, r_lo: as for batq_act_transform_quant (ratios may both be NULL: no
 * clipping).  Wp: packed weights for (N, K), 16-byte aligned.  Y: [M][N] bf16
 * or float, 4-byte aligned.  Xq [M][K/2] (8-byte aligned) and Xs [M][K/32]:
 * optional, both NULL or both set; when set they also receive the quantised
 * activations.  workspace: device memory of at least
 * batq_decode_workspace_bytes(M, N, K) bytes, 256-byte aligned, owned by the
 * caller.  Its first 16 KiB (the arrival counters) must be zero before the
 * workspace's first use (allocate it zeroed); every call leaves them zero
 * again.  The rest may hold anything (the call writes what it reads).  Calls
 * that share a workspace must not overlap (use one stream).
 * Errors: SHAPE (also a workspace that is too small), NULL, ALIGN,
 * UNSUPPORTED (factor size or output type), HIP. */
batq_status batq_w4a4_decode(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, int32_t b,
                             const float* A, const float* B, const float* r_hi,
                             const float* r_lo, const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out,
                             uint8_t* Xq, uint8_t* Xs, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------------ fused decode, no allocation
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same computation, kernels and results (bit for bit) as
 * batq_w4a4_decode; the fp32 partial tiles go to a device array inside the
 * library instead of a caller workspace.
 */

/* Size of that array: BATQ_ERR_TOO_LARGE for any (M, N, K) whose
 * batq_decode_workspace_bytes exceeds it.  Host only. */
int64_t batq_decode_noalloc_scratch_bytes(void);

/* As batq_w4a4_decode, without the workspace arguments.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  The first
 * call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current; the device of the calling
 * thread must be the stream's device, as for any launch) and keeps its
 * address; each GPU holds its copy until the process ends.  The array starts
 * zeroed (its arrival counters must), and every call leaves the counters zero
 * and overwrites the partials it reads, so nothing needs clearing between
 * calls; calls that overlap on one GPU (other streams, other threads) race:
 * serialise them.  The array keeps the last call's partials.
 * Errors: as batq_w4a4_decode; TOO_LARGE (see above); HIP (also the address
 * lookup failing). */
batq_status batq_w4a4_decode_noalloc(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, int32_t b,
                                     const float* A, const float* B, const float* r_hi,
                                     const float* r_lo, const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out,
                                     uint8_t* Xq, uint8_t* Xs, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BATQ_H */
