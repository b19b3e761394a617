/*
 * batq_probe.h — measurement probes shipped in the same library as batq.h.
 *
 * Not part of the path: these kernels measure the ceilings that the path's
 * kernels are judged against (the matrix-instruction rate on this part, the
 * shader clock it sustains, and HBM read and copy bandwidth), so that a
 * roofline fraction can be set against both the published peak and what a
 * loop of the same instruction, or a plain stream, reaches on the same GPU.
 * Same conventions as batq.h: device pointers, asynchronous on `stream`, the
 * library allocates nothing, argument checks run before any HIP call.
 */
#ifndef BATQ_PROBE_H
#define BATQ_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "batq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The block-scaled 32x32x64 FP4 matrix instruction of the W4A4 GEMM in a
 * register-only loop: `workgroups` workgroups of 4 waves, each wave `iters`
 * rounds of 8 independent instructions (131072 flops each), unit scales.
 * random_data 0: every operand register holds E2M1 1.0; 1: hashed random bits
 * per lane and register (seeded by `seed`), which toggle between issues.
 * sink: one float per wave (4 * workgroups floats, the accumulator sum).
 * clocks: two 64-bit counts per wave (8 * workgroups), the shader-clock cycles
 * (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) the loop took.
 * Errors: SHAPE (workgroups outside [1, 2^20], iters <= 0), NULL, ALIGN, HIP. */
batq_status batq_probe_mfma_fp4(int64_t workgroups, int32_t iters, int32_t random_data, uint32_t seed, float* sink,
                                unsigned long long* clocks, hipStream_t stream);

/* Stream sizes must be positive multiples of this many bytes (256 threads x 8
 * loads x 16 bytes); a stream runs on up to 4096 workgroups, each reading a
 * contiguous range with non-temporal 16-byte loads. */
int64_t batq_probe_stream_granule(void);

/* Reads `bytes` of src (16-byte aligned) once with 16-byte loads, each
 * workgroup streaming a contiguous range; sink receives one xor word per
 * workgroup (room for 4096 uint32).  Errors: SHAPE (bytes not a multiple of the
 * granule), NULL, ALIGN, HIP. */
batq_status batq_probe_hbm_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Copies `bytes` from src to dst (both 16-byte aligned, not overlapping) with
 * 16-byte loads and stores, same split as batq_probe_hbm_read.
 * Errors: SHAPE, NULL, ALIGN, HIP. */
batq_status batq_probe_hbm_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* A read:write stream: reads `read_bytes` of src once and writes
 * read_bytes / ratio bytes to dst (each written 16-byte word the xor of
 * `ratio` read words), same split as batq_probe_hbm_read.  ratio 4 is the mix
 * of the activation transform (bf16 in, MXFP4 codes out).
 * Errors: SHAPE (read_bytes not a multiple of the granule), UNSUPPORTED (ratio
 * not 1, 2, 4 or 8), NULL, ALIGN, HIP. */
batq_status batq_probe_hbm_stream(const void* src, int64_t read_bytes, void* dst, int32_t ratio,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BATQ_PROBE_H */
