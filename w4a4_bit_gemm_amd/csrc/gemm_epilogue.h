// Bf16 output epilogue shared by the packed GEMM kernels (gfx950): one wave's
// MT x NT accumulator tiles of 32 x 32 (rows m0 + 32 i + ..., columns
// n0 + 32 k + ...) leave as 16-byte row chunks of bf16, through the wave's
// own LDS band and without any workgroup barrier.
#pragma once
#include "common.h"

namespace batq {

// Bytes of one wave's staged band: 32 rows of its 32 NT columns in bf16.
template <int NT>
constexpr int epi_bf16_row_bytes() { return 2 * 32 * NT; }
template <int NT>
constexpr int epi_bf16_wave_bytes() { return 32 * epi_bf16_row_bytes<NT>(); }

// The accumulators are converted to bf16 before staging.  Lane (r, g) of a
// 32 x 32 accumulator holds one column (r) and rows 8 (q / 4) + 4 g + q % 4
// of its 16 registers q, so lanes r and r ^ 1 swap one value per pair of rows
// (DPP) and each writes a bf16 pair of two adjacent columns of one row: half
// the bytes and half the LDS writes of fp32 staging.  Dword d of staged row r
// sits at d ^ 16 (r & 1) (for NT = 2 a row is 32 dwords): the two rows a write
// instruction touches use disjoint banks, and the eight 16-byte chunks of a
// row that one read instruction's eight lanes fetch cover all 32.  A band's
// four read-backs go out together, then its stores; `full` (the whole tile
// inside Y with 16-byte aligned rows, uniform per workgroup) drops the
// per-chunk bounds checks.  Stores are non-temporal: nothing here reads Y
// again, and cached output lines would evict operand lines that other tiles
// still reuse.  Conversion is round to nearest even, as f32x2_to_bf16x2_rne.
template <int MT, int NT>
__device__ __forceinline__ void store_bf16_tile(const GemmArgs& p, f32x16 (&acc)[MT][NT], int64_t m0, int64_t n0,
                                                int lane, uint8_t* stage, bool full) {
  static_assert(NT == 2, "the row swizzle assumes 32-dword rows");
  constexpr int kRow = epi_bf16_row_bytes<NT>();
  constexpr int kIt = 32 * kRow / 1024;  // 16-byte chunks per lane and band
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) asm volatile("" : "+a"(acc[i][k]));
  // The epilogue's inputs pass through an empty asm so that none of its
  // address arithmetic is hoisted above the stage loop.
  int lane_e = lane;
  int64_t m0e = m0, n0e = n0;
  asm volatile("" : "+v"(lane_e), "+s"(m0e), "+s"(n0e));
  const int r32 = lane_e & 31, ge = lane_e >> 5;
  const bool odd = (r32 & 1) != 0;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int a = 0; a < 16; a += 2) {
        // registers a, a + 1: rows 8 (a / 4) + 4 g + a % 4 and the next one
        const float v0 = acc[i][k][a], v1 = acc[i][k][a + 1];
        const float send = odd ? v0 : v1;
        const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
        const uint32_t w = odd ? f32x2_to_bf16x2_rne(recv, v1) : f32x2_to_bf16x2_rne(v0, recv);
        const int row = 8 * (a >> 2) + 4 * ge + (a & 3) + (odd ? 1 : 0);
        const int dw = (16 * k + (r32 >> 1)) ^ ((row & 1) << 4);
        *reinterpret_cast<uint32_t*>(stage + row * kRow + 4 * dw) = w;
      }
    u32x4 v[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int rr = 8 * it + (lane_e >> 3);
      v[it] = *reinterpret_cast<const u32x4*>(stage + rr * kRow + 16 * ((lane_e & 7) ^ ((rr & 1) << 2)));
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int64_t row = m0e + 32 * i + 8 * it + (lane_e >> 3);
      const int64_t col = n0e + 8 * (lane_e & 7);
      uint16_t* dst = reinterpret_cast<uint16_t*>(p.y) + row * p.N + col;
      if (full) {
        __builtin_nontemporal_store(v[it], reinterpret_cast<u32x4*>(dst));
      } else if (row < p.M && col < p.N) {
        if (col + 8 <= p.N && p.vec_store) {
          __builtin_nontemporal_store(v[it], reinterpret_cast<u32x4*>(dst));
        } else {
          const uint32_t hb[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
          for (int e = 0; e < 8; ++e)
            if (col + e < p.N) dst[e] = (uint16_t)(hb[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

}  // namespace batq
