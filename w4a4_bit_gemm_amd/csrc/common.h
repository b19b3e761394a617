// Shared device helpers for the gfx950 kernels of the BATQuant W4A4 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace batq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits, round to nearest even, on gfx950's converter
// (v_cvt_pk_bf16_f32).  For every non-NaN input it gives the same bits as the
// integer rounding (u + 0x7FFF + ((u >> 16) & 1)) >> 16 (checked over all
// 2^32 patterns on the device); the bf16-output tests pin it against numpy.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two at once, one instruction: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

}  // namespace batq

// Host-side launchers (defined next to their kernels).
namespace batq {
struct TransformQuantArgs {
  const uint16_t* x;    // [rows][ldx] bf16
  int64_t ldx;
  int64_t rows;
  int64_t K;
  int a_log2;           // shared factor size a = 1 << a_log2, private size 32 / a
  const float* A;       // [a][a]
  const float* B;       // [K/32][b][b]
  const float* r_hi;    // clip ratios or nullptr (no clipping)
  const float* r_lo;
  int64_t r_ld;         // ratio index = row * r_ld + block (0: shared over rows)
  uint8_t* q;           // [rows][K/2] (E2M1) or [rows][K] (E4M3)
  uint8_t* s;           // [rows][K/32]
  int fp8 = 0;          // 1: MXFP8 (E4M3) codes instead of MXFP4 (E2M1)
  const int64_t* slot = nullptr;  // output row of each input row (KV cache), or nullptr: the row itself
  int64_t out_rows = 0;           // rows of q / s when slot is set; other slots are skipped
};
hipError_t launch_transform_quant(const TransformQuantArgs& args, hipStream_t stream);
// True where launch_transform_quant runs one workgroup per CU with a dedicated
// loader wave (grids of fewer than two workgroups per CU); otherwise it runs
// two per CU, each compute wave also loading.
bool transform_uses_one_per_cu(int64_t rows, int64_t K);

struct GemmArgs {
  const uint8_t* xq;
  const uint8_t* xs;
  const uint8_t* wq;
  const uint8_t* ws;
  int64_t M, N, K;
  void* y;
  int out_f32;
  int vec_store;  // Y 16-byte aligned and rows a whole number of 16-byte chunks
  int a_fp8 = 0;  // packed GEMM only: xq holds E4M3 codes [M][K] (W4A8) instead of E2M1 [M][K/2]
};
hipError_t launch_mxfp4_gemm(const GemmArgs& args, hipStream_t stream);

// Packed weight layout for the GEMM's B operand (see mxfp4_gemm.hip):
// per 32-row group and 256-k stage, 4 x 64 lanes x 16 code bytes followed by
// 64 lanes x 4 scale bytes.
constexpr int64_t kPackGroupBytes = 4 * 64 * 16 + 64 * 4;
inline int64_t packed_weight_bytes(int64_t N, int64_t K) { return ((N + 31) / 32) * (K / 256) * kPackGroupBytes; }
hipError_t launch_weight_pack(const uint8_t* wq, const uint8_t* ws, int64_t N, int64_t K, uint8_t* wp,
                              hipStream_t stream);
// Same GemmArgs; wq points at the packed buffer and ws is unused.
hipError_t launch_mxfp4_gemm_packed(const GemmArgs& args, hipStream_t stream);
// The two-workgroups-per-CU form of the same product (mxfp4_gemm_packed_dma.hip),
// for the shapes where packed_dma_applies() holds.
bool packed_dma_applies(const GemmArgs& args);
hipError_t launch_mxfp4_gemm_packed_dma(const GemmArgs& args, hipStream_t stream);
// Fused decode step (decode_fused.hip): transform + clip + MXFP4 quantisation
// of M <= 32 tokens inside the GEMM on packed weights, one launch split over
// (128-column chunk, K split of two 256-k stages); the last workgroup of each
// chunk adds its splits' partial tiles in split order.
struct DecodeArgs {
  const uint16_t* x;    // [M][ldx] bf16
  int64_t ldx;
  int64_t M, K, N;
  int a_log2;
  const float* A;       // [a][a]
  const float* B;       // [K/32][b][b]
  const float* r_hi;    // [K/32] or nullptr (no clipping)
  const float* r_lo;
  const uint8_t* wp;    // packed weights
  void* y;              // [M][N]
  int out_f32;
  uint8_t* xq;          // optional [M][K/2] codes and [M][K/32] scales, or nullptr
  uint8_t* xs;
  float* part;          // workspace: arrival counters, then fp32 partial tiles [N/128][splits][M][128]
};
int64_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_decode_fused(const DecodeArgs& args, hipStream_t stream);
// Arrival counters of the decode step's K splits: the first bytes of every
// workspace, one 32-bit counter per 128-column chunk (N up to 524288).
constexpr int64_t kDecodeCounterBytes = 16384;
constexpr int64_t kDecodeMaxN = kDecodeCounterBytes / 4 * 128;
// The no-allocation decode path's partial tiles: a device array of this many
// bytes (decode_fused.hip), whose address on the current device
// decode_scratch returns (looked up once per device).
constexpr int64_t kDecodeScratchBytes = 16ll << 20;
hipError_t decode_scratch(void** ptr);
}  // namespace batq
