// W4A4 GEMM with the weight operand in a packed, MFMA-lane-ordered layout.
//
// Same product and accumulation order as the canonical GEMM [BATQuant note
// (en.papernotes.org), Key Designs §1 and §4], for weights that were packed
// once, offline, after batq_weight_prep.  Packing matters because on gfx950
// the canonical kernel is bound by LDS traffic: every operand byte is written
// to and read back from LDS.  With the weights in lane order, each wave loads
// its weight fragments with fully coalesced 1 KB instructions straight into
// registers, and only the activation tile (shared by the four waves) goes
// through LDS, which cuts LDS bytes per MFMA roughly in half.
//
// Packed layout, per group of 32 weight rows (n32) and per 256-k stage (s),
// 4352 bytes:
//   codes: 4 sub-steps j x 64 lanes x 16 bytes.  Lane l = (r, g), r = l % 32,
//          g = l / 32, holds MX block 8 s + 4 g + j of row 32 n32 + r.
//   scales: 64 lanes x 4 bytes: lane l holds the scale bytes of blocks
//          8 s + 4 g + 0..3 of row 32 n32 + r (byte j = block 8 s + 4 g + j).
// Rows past N are zero codes with unit scales.
//
// Kernel: workgroup tile 128 (M) x 256 (N); wave w owns all 128 rows and
// columns 64 w .. 64 w + 63 (4 x 2 MFMA tiles of 32 x 32).  Activation codes
// travel global -> registers -> a two-slot LDS ring (16 KB per stage, loaded
// three stages ahead); weights go straight to registers (three sets, two
// stages ahead).  Activation scales: a row's scales are 8 bytes per stage and
// 128 rows apart, so when K / 256 is a multiple of 4 they are fetched four
// stages at a time (one 16-byte load per thread instead of four 4-byte loads
// that each touch 32 cache lines) into a two-group LDS ring.
#include "gemm_epilogue.h"

namespace batq {

namespace {

constexpr int kMT = 4;         // 32-row A tiles per wave
constexpr int kNT = 2;         // 32-column B tiles per wave
constexpr int kBM = 32 * kMT;  // 128
constexpr int kBN = 4 * 32 * kNT;  // 256, four waves along N
constexpr int kRowBytes = 128;
constexpr int kAStage = kBM * kRowBytes;        // 16 KB
constexpr int kAScale = kBM * 8;                // 1 KB
constexpr int kEpiStride = 32 * kNT + 8;        // floats
constexpr int kEpiWave = 32 * kEpiStride * 4;   // bytes (also holds a bf16 band)
static_assert(kEpiWave >= epi_bf16_wave_bytes<kNT>(), "a wave's bf16 band fits its fp32 band");
constexpr int kGroupM = 8;                      // row tiles per band of the tile order

__device__ __forceinline__ i32x8 op(uint4 v) {
  i32x8 r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

template <int J>
__device__ __forceinline__ f32x16 mfma_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(a), op(b), acc, 4, 4, J, (int)sa, J, (int)sb);
}

// E4M3 activations x E2M1 weights (the W4A8 setting).  The E4M3 operand of a
// lane (row r, half g) is 32 bytes: k = 16 g .. 16 g + 15 of the 64-k step in
// bytes 0..15 and k = 32 + 16 g .. 32 + 16 g + 15 in bytes 16..31, while the
// E2M1 operand keeps 32 consecutive k per lane half; each lane's scale byte
// covers the 32-k block of its half (all checked on the device).
template <int J>
__device__ __forceinline__ f32x16 mfma_fp8_fp4(uint4 alo, uint4 ahi, uint4 b, uint32_t sa, uint32_t sb,
                                               f32x16 acc) {
  const i32x8 a = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, op(b), acc, 0, 4, J, (int)sa, J, (int)sb);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------------------ packing

__global__ __launch_bounds__(256) void weight_pack_kernel(const uint8_t* __restrict__ wq,
                                                          const uint8_t* __restrict__ ws, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ wp) {
  const int64_t nst = K / 256;
  const int64_t groups = ((N + 31) / 32) * nst;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // one (n32, s) per wave
  if (item >= groups) return;
  const int lane = threadIdx.x & 63;
  const int64_t n32 = item / nst;
  const int64_t s = item % nst;
  const int64_t row = 32 * n32 + (lane & 31);
  const int g = lane >> 5;
  uint8_t* dst = wp + item * kPackGroupBytes;
  uint32_t sc = 0x7F7F7F7Fu;
  uint4 c[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if (row < N) {
    const uint8_t* qr = wq + row * (K / 2) + 16 * (8 * s + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const uint4*>(qr + 16 * j);
    const uint8_t* sr = ws + row * (K / 32) + 8 * s + 4 * g;
    sc = (uint32_t)sr[0] | (uint32_t)sr[1] << 8 | (uint32_t)sr[2] << 16 | (uint32_t)sr[3] << 24;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(dst + j * 1024 + 16 * lane) = c[j];
  *reinterpret_cast<uint32_t*>(dst + 4096 + 4 * lane) = sc;
}

// -------------------------------------------------------------------- GEMM

// Register sets are plain named variables (declared by the macros below): an
// aggregate (array or vector type) either reaches the early alloca passes
// with loop-variable indices and lands in scratch, or forces whole-aggregate
// live ranges that the allocator cannot split.  kNT == 2 is assumed.
static_assert(kNT == 2, "weight register sets below hold two 32-column tiles");

// Stage index laundered through an empty asm: the address arithmetic that
// depends on it cannot be hoisted out of its pipeline step, so fully unrolled
// kernels do not keep every stage's addresses live at once.
__device__ __forceinline__ int64_t opaque_stage(int64_t s) {
  asm volatile("" : "+s"(s));
  return s;
}

__device__ __forceinline__ const uint8_t* b_src(const uint8_t* wp, int64_t n32, int64_t nst, int64_t s) {
  return wp + (n32 * nst + s) * kPackGroupBytes;
}
__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

#define BATQ_DECL_B(n) \
  uint4 n##_00, n##_01, n##_02, n##_03, n##_10, n##_11, n##_12, n##_13; \
  uint32_t n##_s0, n##_s1;
// weight stage ST of this wave's two 32-row groups -> set n
#define BATQ_LOAD_B(n, ST)                                                                     \
  {                                                                                            \
    const int64_t off_ = opaque_stage(ST) * kPackGroupBytes;                                   \
    const uint8_t* s0_ = b_base0 + off_;                                                       \
    const uint8_t* s1_ = b_base1 + off_;                                                       \
    n##_00 = ld16(s0_); n##_01 = ld16(s0_ + 1024); n##_02 = ld16(s0_ + 2048); n##_03 = ld16(s0_ + 3072); \
    n##_s0 = ld4(s0_ + 4096 - 12 * lane);                                                      \
    n##_10 = ld16(s1_); n##_11 = ld16(s1_ + 1024); n##_12 = ld16(s1_ + 2048); n##_13 = ld16(s1_ + 3072); \
    n##_s1 = ld4(s1_ + 4096 - 12 * lane);                                                      \
  }
// The two column groups' halves of BATQ_LOAD_B, issued separately (below).
#define BATQ_LOAD_B0(n, ST)                                                                    \
  {                                                                                            \
    const uint8_t* s0_ = b_base0 + opaque_stage(ST) * kPackGroupBytes;                         \
    n##_00 = ld16(s0_); n##_01 = ld16(s0_ + 1024); n##_02 = ld16(s0_ + 2048); n##_03 = ld16(s0_ + 3072); \
    n##_s0 = ld4(s0_ + 4096 - 12 * lane);                                                      \
  }
#define BATQ_LOAD_B1(n, ST)                                                                    \
  {                                                                                            \
    const uint8_t* s1_ = b_base1 + opaque_stage(ST) * kPackGroupBytes;                         \
    n##_10 = ld16(s1_); n##_11 = ld16(s1_ + 1024); n##_12 = ld16(s1_ + 2048); n##_13 = ld16(s1_ + 3072); \
    n##_s1 = ld4(s1_ + 4096 - 12 * lane);                                                      \
  }
// A step's loads for later stages go out between the MFMAs of its stage, each
// right after one MFMA (the scheduling groups pin that order): the weights
// after sub-steps 0 and 1, the activations after sub-step 2.  Issued in front
// of the stage, as before, they held the one wave per SIMD behind the queue of
// vector loads with nothing else to cover it: spread out, the results are
// bit-identical and the GEMM is faster (alternating A/B in one process):
// 2048 x 4096 x 12288 by 5.7 % (E2M1) and 9.9 % (E4M3), 512 x 4096 x 4096 by
// 10.7 %, 1024 x 4096 x 5120 (runtime stage loop) by 16 %.  The loads are
// plain loads, so the compiler's wait counts follow them wherever they sit.
// BATQ_ILk: k (MFMA, load) pairs, then the sub-step's other MFMAs.
#define BATQ_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 1, J); __builtin_amdgcn_sched_group_barrier(0x020, 1, J);
#define BATQ_IL4(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 4, J);
#define BATQ_IL5(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 3, J);
#define BATQ_IL8(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J) BATQ_MV(J)
#define BATQ_DECL_A(n) uint4 n##_0, n##_1, n##_2, n##_3, n##_4, n##_5, n##_6, n##_7; uint32_t n##_s;
// activation stage ST -> set n: thread owns code chunks id = tid + 256 i
// (E2M1: row id / 8, chunk id % 8, i < 4; E4M3: row id / 16, chunk id % 16,
// i < 8) and scale dword (row tid / 2, half tid % 2)
#define BATQ_LOAD_A(n, ST)                                                                     \
  {                                                                                            \
    const int64_t st_ = opaque_stage(ST);                                                      \
    const int64_t off_ = st_ * kARow;                                                          \
    n##_0 = ld16(a_base0 + off_);                                                              \
    n##_1 = ld16(a_base1 + off_);                                                              \
    n##_2 = ld16(a_base2 + off_);                                                              \
    n##_3 = ld16(a_base3 + off_);                                                              \
    if constexpr (A8) {                                                                        \
      n##_4 = ld16(a_base4 + off_);                                                            \
      n##_5 = ld16(a_base5 + off_);                                                            \
      n##_6 = ld16(a_base6 + off_);                                                            \
      n##_7 = ld16(a_base7 + off_);                                                            \
    }                                                                                          \
    if (!GS) n##_s = ld4(a_sbase + 8 * st_);                                                   \
  }
#define BATQ_STORE_A(n, SLOT)                                                                  \
  {                                                                                            \
    if constexpr (A8) {                                                                        \
      a_dst8(SLOT, tid)[0] = n##_0;                                                            \
      a_dst8(SLOT, tid + 256)[0] = n##_1;                                                      \
      a_dst8(SLOT, tid + 512)[0] = n##_2;                                                      \
      a_dst8(SLOT, tid + 768)[0] = n##_3;                                                      \
      a_dst8(SLOT, tid + 1024)[0] = n##_4;                                                     \
      a_dst8(SLOT, tid + 1280)[0] = n##_5;                                                     \
      a_dst8(SLOT, tid + 1536)[0] = n##_6;                                                     \
      a_dst8(SLOT, tid + 1792)[0] = n##_7;                                                     \
    } else {                                                                                   \
      a_dst(SLOT, tid)[0] = n##_0;                                                             \
      a_dst(SLOT, tid + 256)[0] = n##_1;                                                       \
      a_dst(SLOT, tid + 512)[0] = n##_2;                                                       \
      a_dst(SLOT, tid + 768)[0] = n##_3;                                                       \
    }                                                                                          \
    if (!GS) *reinterpret_cast<uint32_t*>((SLOT) + kAStg + 4 * tid) = n##_s;                   \
  }
// Grouped activation scales (GS): group G = stages 4G .. 4G+3.  Thread
// (row tid / 2, half h = tid % 2) loads the 16 bytes of stages 4G + 2h and
// 4G + 2h + 1 of its row; they are stored stage-major (1 KB per stage, 8 bytes
// per row) so that the MMA's scale reads match the per-stage layout.
#define BATQ_LOAD_AS(G) asg = ld16(a_gbase + 32 * opaque_stage(__builtin_amdgcn_readfirstlane((int)(G))));
#define BATQ_STORE_AS(G)                                                                       \
  {                                                                                            \
    uint8_t* sg_ = (((G) & 1) ? sgrp1 : sgrp0) + 2048 * (tid & 1) + 8 * (tid >> 1);            \
    *reinterpret_cast<uint2*>(sg_) = make_uint2(asg.x, asg.y);                                 \
    *reinterpret_cast<uint2*>(sg_ + 1024) = make_uint2(asg.z, asg.w);                          \
  }

// Stage-invariant per-thread source pointers (row clamped: rows past the edge
// read a valid row and are never stored).
__device__ __forceinline__ const uint8_t* a_row_base(const GemmArgs& p, int64_t m0, int id) {
  int64_t gr = m0 + (id >> 3);
  gr = gr < p.M ? gr : p.M - 1;
  return p.xq + gr * (p.K >> 1) + 16 * (id & 7);
}
__device__ __forceinline__ const uint8_t* a_scale_base(const GemmArgs& p, int64_t m0, int tid, int bytes) {
  int64_t gr = m0 + (tid >> 1);
  gr = gr < p.M ? gr : p.M - 1;
  return p.xs + gr * (p.K >> 5) + bytes * (tid & 1);
}
__device__ __forceinline__ uint4* a_dst(uint8_t* slot, int id) {
  const int row = id >> 3;
  return reinterpret_cast<uint4*>(slot + row * kRowBytes + 16 * ((id & 7) ^ swz(row)));
}
// E4M3 activations: 256-byte rows (one stage), 16-byte chunk c of row r at
// position c ^ (r % 16): the MMA's reads of one chunk over 16 consecutive
// rows hit 16 different bank groups.
constexpr int kRowBytes8 = 256;
__device__ __forceinline__ const uint8_t* a_row_base8(const GemmArgs& p, int64_t m0, int id) {
  int64_t gr = m0 + (id >> 4);
  gr = gr < p.M ? gr : p.M - 1;
  return p.xq + gr * p.K + 16 * (id & 15);
}
__device__ __forceinline__ uint4* a_dst8(uint8_t* slot, int id) {
  const int row = id >> 4;
  return reinterpret_cast<uint4*>(slot + row * kRowBytes8 + 16 * ((id & 15) ^ (row & 15)));
}
__device__ __forceinline__ uint4 lds_frag8(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(base + row * kRowBytes8 + 16 * (chunk ^ (row & 15)));
}

__device__ __forceinline__ uint4 lds_frag(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(base + row * kRowBytes + 16 * (chunk ^ swz(row)));
}

template <int J>
__device__ __forceinline__ void mma_sub(f32x16 (&acc)[kMT][kNT], const uint4 (&fa)[kMT], uint4 b0, uint4 b1,
                                        uint32_t bs0, uint32_t bs1, const uint32_t (&sa)[kMT]) {
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    acc[i][0] = mfma_fp4<J>(fa[i], b0, sa[i], bs0, acc[i][0]);
    acc[i][1] = mfma_fp4<J>(fa[i], b1, sa[i], bs1, acc[i][1]);
  }
}

__device__ __forceinline__ void read_a(const uint8_t* As, int j, uint4 (&fa)[kMT], int r32, int g) {
#pragma unroll
  for (int i = 0; i < kMT; ++i) fa[i] = lds_frag(As, 32 * i + r32, 4 * g + j);
}

// E4M3 fragments of sub-step J into the named registers P##l0..3 / P##h0..3:
// half g of MX blocks J and 4 + J of the stage (16-byte chunks 2 J + g and
// 8 + 2 J + g of the row).  Named scalars, not arrays: arrays of vectors here
// end up in scratch.
#define BATQ_RD8(SLOT, J, P)                                                                   \
  P##l0 = lds_frag8(SLOT, r32, 2 * (J) + g);                                                   \
  P##h0 = lds_frag8(SLOT, r32, 8 + 2 * (J) + g);                                               \
  P##l1 = lds_frag8(SLOT, 32 + r32, 2 * (J) + g);                                              \
  P##h1 = lds_frag8(SLOT, 32 + r32, 8 + 2 * (J) + g);                                          \
  P##l2 = lds_frag8(SLOT, 64 + r32, 2 * (J) + g);                                              \
  P##h2 = lds_frag8(SLOT, 64 + r32, 8 + 2 * (J) + g);                                          \
  P##l3 = lds_frag8(SLOT, 96 + r32, 2 * (J) + g);                                              \
  P##h3 = lds_frag8(SLOT, 96 + r32, 8 + 2 * (J) + g);
#define BATQ_MM8(J, P, B0, B1, BS0, BS1)                                                       \
  acc[0][0] = mfma_fp8_fp4<J>(P##l0, P##h0, B0, sa_[0], BS0, acc[0][0]);                       \
  acc[0][1] = mfma_fp8_fp4<J>(P##l0, P##h0, B1, sa_[0], BS1, acc[0][1]);                       \
  acc[1][0] = mfma_fp8_fp4<J>(P##l1, P##h1, B0, sa_[1], BS0, acc[1][0]);                       \
  acc[1][1] = mfma_fp8_fp4<J>(P##l1, P##h1, B1, sa_[1], BS1, acc[1][1]);                       \
  acc[2][0] = mfma_fp8_fp4<J>(P##l2, P##h2, B0, sa_[2], BS0, acc[2][0]);                       \
  acc[2][1] = mfma_fp8_fp4<J>(P##l2, P##h2, B1, sa_[2], BS1, acc[2][1]);                       \
  acc[3][0] = mfma_fp8_fp4<J>(P##l3, P##h3, B0, sa_[3], BS0, acc[3][0]);                       \
  acc[3][1] = mfma_fp8_fp4<J>(P##l3, P##h3, B1, sa_[3], BS1, acc[3][1]);

// Stage S from an LDS slot and a weight register set into the accumulators,
// with the LDS reads of sub-step j+1 issued ahead of the MFMAs of sub-step j,
// and the loads of later stages (weights S + kBDist into set BPF, activations
// S + 3 into set ANEXT) between the MFMAs.
#define BATQ_MMA_STAGE(SLOT, n, SCALES, S, BPF, ANEXT)                                        \
  {                                                                                            \
    uint32_t sa_[kMT];                                                                         \
    _Pragma("unroll") for (int i = 0; i < kMT; ++i)                                            \
      sa_[i] = ld4((SCALES) + (32 * i + r32) * 8 + 4 * g);                                     \
    const bool ld_b_ = NST == 0 || (S) + kBDist < NST;                                         \
    const bool ld_a_ = NST == 0 || (S) + 3 < NST;                                              \
    if constexpr (A8) {                                                                        \
      uint4 x0l0, x0h0, x0l1, x0h1, x0l2, x0h2, x0l3, x0h3;                                    \
      uint4 x1l0, x1h0, x1l1, x1h1, x1l2, x1h2, x1l3, x1h3;                                    \
      BATQ_RD8(SLOT, 0, x0)                                                                    \
      BATQ_RD8(SLOT, 1, x1)                                                                    \
      sched_fence();                                                                           \
      BATQ_MM8(0, x0, n##_00, n##_10, n##_s0, n##_s1)                                          \
      if (ld_b_) { BATQ_LOAD_B0(BPF, BATQ_CL((S) + kBDist)) BATQ_IL5(0) }                       \
      sched_fence();                                                                           \
      BATQ_RD8(SLOT, 2, x0)                                                                    \
      sched_fence();                                                                           \
      BATQ_MM8(1, x1, n##_01, n##_11, n##_s0, n##_s1)                                          \
      if (ld_b_) { BATQ_LOAD_B1(BPF, BATQ_CL((S) + kBDist)) BATQ_IL5(1) }                       \
      sched_fence();                                                                           \
      BATQ_RD8(SLOT, 3, x1)                                                                    \
      sched_fence();                                                                           \
      BATQ_MM8(2, x0, n##_02, n##_12, n##_s0, n##_s1)                                          \
      if (ld_a_) { BATQ_LOAD_A(ANEXT, BATQ_CL((S) + 3)) BATQ_IL8(2) }                           \
      sched_fence();                                                                           \
      BATQ_MM8(3, x1, n##_03, n##_13, n##_s0, n##_s1)                                          \
    } else {                                                                                   \
      uint4 fa0_[kMT], fa1_[kMT];                                                              \
      read_a(SLOT, 0, fa0_, r32, g);                                                           \
      read_a(SLOT, 1, fa1_, r32, g);                                                           \
      sched_fence();                                                                           \
      mma_sub<0>(acc, fa0_, n##_00, n##_10, n##_s0, n##_s1, sa_);                              \
      if (ld_b_) { BATQ_LOAD_B0(BPF, BATQ_CL((S) + kBDist)) BATQ_IL5(0) }                       \
      sched_fence();                                                                           \
      read_a(SLOT, 2, fa0_, r32, g);                                                           \
      sched_fence();                                                                           \
      mma_sub<1>(acc, fa1_, n##_01, n##_11, n##_s0, n##_s1, sa_);                              \
      if (ld_b_) { BATQ_LOAD_B1(BPF, BATQ_CL((S) + kBDist)) BATQ_IL5(1) }                       \
      sched_fence();                                                                           \
      read_a(SLOT, 3, fa1_, r32, g);                                                           \
      sched_fence();                                                                           \
      mma_sub<2>(acc, fa0_, n##_02, n##_12, n##_s0, n##_s1, sa_);                              \
      if (ld_a_) { BATQ_LOAD_A(ANEXT, BATQ_CL((S) + 3)) BATQ_IL4(2) }                           \
      sched_fence();                                                                           \
      mma_sub<3>(acc, fa1_, n##_03, n##_13, n##_s0, n##_s1, sa_);                              \
    }                                                                                          \
  }

// NST > 0: stage count fixed at compile time, loop fully unrolled (exact
// compiler wait counts).  NST == 0: runtime stage count.
// A8: E4M3 activations (W4A8) instead of E2M1.
template <int NST, bool GS, bool A8>
__global__ __launch_bounds__(256) void mxfp4_gemm_packed_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  constexpr int kARow = A8 ? kRowBytes8 : kRowBytes;  // activation bytes per row and stage
  constexpr int kAStg = kBM * kARow;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[GS ? kAStg : kAStg + kAScale];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[GS ? kAStg : kAStg + kAScale];
  __shared__ __attribute__((aligned(1024))) uint8_t sgrp0[GS ? 4096 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sgrp1[GS ? 4096 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t epi_buf[4 * kEpiWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  // XCD-aware order: consecutive workgroups go to the 8 XCDs in turn, so XCD x
  // receives the contiguous range [x total / 8, (x + 1) total / 8) of t ...
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  // ... walked in bands of kGroupM row tiles, so that an XCD's concurrent
  // workgroups share a small activation panel that stays in its L2.
  const int gsz = kGroupM * tiles_n;
  const int first_tm = (t / gsz) * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_tm);
  const int tm = first_tm + (t % gsz) % gm;
  const int tn = (t % gsz) / gm;
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t n0 = (int64_t)tn * kBN + 64 * wave;  // this wave's first column
  const int64_t n32_0 = n0 / 32;
  const int64_t nst = NST > 0 ? NST : p.K / 256;
  const int64_t last = nst - 1;
  const int64_t n32_max = (p.N + 31) / 32;
  // Each of the wave's two 32-column groups is clamped on its own to the last
  // group: a clamped group is computed (so every wave reaches every barrier)
  // but its columns lie past N and are never stored.
  const int64_t n32_g0 = n32_0 < n32_max ? n32_0 : n32_max - 1;
  const int64_t n32_g1 = n32_0 + 1 < n32_max ? n32_0 + 1 : n32_max - 1;

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int k = 0; k < kNT; ++k) acc[i][k] = f32x16{};

  // Pipeline (all loads are plain loads into registers, so the compiler's
  // in-order wait counts stay exact): at step s, stage s is read from LDS slot
  // s % 2; activation stage s+1 moves registers -> the other slot; activation
  // stage s+3 and weight stage s+2 are requested.  Stage indices of the
  // prefetches are clamped to the last stage (a clamped load re-reads an
  // L2-resident stage and is never used), keeping every step branch-free.
#define BATQ_CL(x) ((x) < last ? (x) : last)
  const uint8_t* const a_base0 = A8 ? a_row_base8(p, m0, tid) : a_row_base(p, m0, tid);
  const uint8_t* const a_base1 = A8 ? a_row_base8(p, m0, tid + 256) : a_row_base(p, m0, tid + 256);
  const uint8_t* const a_base2 = A8 ? a_row_base8(p, m0, tid + 512) : a_row_base(p, m0, tid + 512);
  const uint8_t* const a_base3 = A8 ? a_row_base8(p, m0, tid + 768) : a_row_base(p, m0, tid + 768);
  const uint8_t* const a_base4 = A8 ? a_row_base8(p, m0, tid + 1024) : nullptr;
  const uint8_t* const a_base5 = A8 ? a_row_base8(p, m0, tid + 1280) : nullptr;
  const uint8_t* const a_base6 = A8 ? a_row_base8(p, m0, tid + 1536) : nullptr;
  const uint8_t* const a_base7 = A8 ? a_row_base8(p, m0, tid + 1792) : nullptr;
  const uint8_t* const a_sbase = a_scale_base(p, m0, tid, 4);   // per-stage scales
  const uint8_t* const a_gbase = a_scale_base(p, m0, tid, 16);  // grouped scales
  const int64_t ngrp = nst >> 2;
  const uint8_t* const b_base0 = b_src(p.wq, n32_g0, nst, 0) + 16 * lane;
  const uint8_t* const b_base1 = b_src(p.wq, n32_g1, nst, 0) + 16 * lane;
  BATQ_DECL_A(a0)
  BATQ_DECL_A(a1)
  uint4 asg;
  BATQ_DECL_B(b0)
  BATQ_DECL_B(b1)
  BATQ_DECL_B(b2)
  // Weights are prefetched kBDist stages ahead: two for E2M1 (three register
  // sets), one for E4M3, whose MFMAs take twice as long per stage and whose
  // activation fragments need the registers (two sets).
  constexpr int kBDist = A8 ? 1 : 2;
  BATQ_LOAD_A(a0, 0)
  BATQ_LOAD_B(b0, 0)
  if (NST == 0 || NST > 1) {
    BATQ_LOAD_A(a1, BATQ_CL(1))
    if (kBDist == 2) BATQ_LOAD_B(b1, BATQ_CL(1))
  }
  if (GS) BATQ_LOAD_AS(0)
  BATQ_STORE_A(a0, slot0)
  if (GS) {
    BATQ_STORE_AS(0)
    if (NST == 0 || NST > 4) BATQ_LOAD_AS(ngrp > 1 ? 1 : 0)
  }
  if (NST == 0 || NST > 2) BATQ_LOAD_A(a0, BATQ_CL(2))
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();

  // With a compile-time stage count the tail prefetches are simply omitted
  // (the conditions fold away); a runtime count keeps them, clamped.
// J: the step's phase modulo 12 (compile time); S: the step (may be runtime).
#define BATQ_STEP(S, J, CUR, NEXT, ANEXT, BCUR, BPF)                                            \
  {                                                                                            \
    if (NST == 0 || (S) + 1 < NST) BATQ_STORE_A(ANEXT, NEXT)   /* act stage s+1 -> LDS */       \
    if (GS && (J) % 4 == 0 && (NST == 0 || (S) + 4 < NST)) {   /* scale groups */              \
      if (NST > 0 || (S) + 4 < nst) BATQ_STORE_AS(((S) >> 2) + 1)                              \
      if (NST == 0 || (S) + 8 < NST)                                                           \
        BATQ_LOAD_AS(((S) >> 2) + 2 < ngrp ? ((S) >> 2) + 2 : ngrp - 1)                        \
    }                                                                                          \
    sched_fence();                                                                             \
    const uint8_t* scales_ = GS ? ((((S) >> 2) & 1) ? sgrp1 : sgrp0) + 1024 * ((J) % 4)        \
                                : (CUR) + kAStg;                                               \
    BATQ_MMA_STAGE(CUR, BCUR, scales_, S, BPF, ANEXT)                                          \
    __builtin_amdgcn_s_waitcnt(0xC07F);          /* lgkmcnt(0): s+1 written, s read */         \
    block_barrier();                                                                           \
  }
  // Slots alternate with period 2 and weight sets with period 3.
#define BATQ_STEP6(S)                                                                          \
  switch ((S) % 6) {                                                                           \
    case 0: BATQ_STEP(S, S, slot0, slot1, a1, b0, b2) break;                                   \
    case 1: BATQ_STEP(S, S, slot1, slot0, a0, b1, b0) break;                                   \
    case 2: BATQ_STEP(S, S, slot0, slot1, a1, b2, b1) break;                                   \
    case 3: BATQ_STEP(S, S, slot1, slot0, a0, b0, b2) break;                                   \
    case 4: BATQ_STEP(S, S, slot0, slot1, a1, b1, b0) break;                                   \
    default: BATQ_STEP(S, S, slot1, slot0, a0, b2, b1) break;                                  \
  }
  // E4M3: weight sets alternate with period 2.
#define BATQ_STEP4(S)                                                                          \
  switch ((S) % 2) {                                                                           \
    case 0: BATQ_STEP(S, S, slot0, slot1, a1, b0, b1) break;                                   \
    default: BATQ_STEP(S, S, slot1, slot0, a0, b1, b0) break;                                  \
  }
  if (NST > 0) {
    if constexpr (A8) {
#pragma unroll
      for (int s = 0; s < NST; ++s) BATQ_STEP4(s)
    } else {
#pragma unroll
      for (int s = 0; s < NST; ++s) BATQ_STEP6(s)
    }
  } else if constexpr (A8) {
    // Period 4 = lcm(2 slots, 2 weight sets, 4 stages per scale group).
    for (int64_t s = 0; s < nst; s += 4) {
      BATQ_STEP(s, 0, slot0, slot1, a1, b0, b1)
      if (s + 1 < nst) BATQ_STEP(s + 1, 1, slot1, slot0, a0, b1, b0)
      if (s + 2 < nst) BATQ_STEP(s + 2, 2, slot0, slot1, a1, b0, b1)
      if (s + 3 < nst) BATQ_STEP(s + 3, 3, slot1, slot0, a0, b1, b0)
    }
  } else {
    // Period 12 = lcm(2 slots, 3 weight sets, 4 stages per scale group).
    for (int64_t s = 0; s < nst; s += 12) {
      BATQ_STEP(s, 0, slot0, slot1, a1, b0, b2)
      if (s + 1 < nst) BATQ_STEP(s + 1, 1, slot1, slot0, a0, b1, b0)
      if (s + 2 < nst) BATQ_STEP(s + 2, 2, slot0, slot1, a1, b2, b1)
      if (s + 3 < nst) BATQ_STEP(s + 3, 3, slot1, slot0, a0, b0, b2)
      if (s + 4 < nst) BATQ_STEP(s + 4, 4, slot0, slot1, a1, b1, b0)
      if (s + 5 < nst) BATQ_STEP(s + 5, 5, slot1, slot0, a0, b2, b1)
      if (s + 6 < nst) BATQ_STEP(s + 6, 6, slot0, slot1, a1, b0, b2)
      if (s + 7 < nst) BATQ_STEP(s + 7, 7, slot1, slot0, a0, b1, b0)
      if (s + 8 < nst) BATQ_STEP(s + 8, 8, slot0, slot1, a1, b2, b1)
      if (s + 9 < nst) BATQ_STEP(s + 9, 9, slot1, slot0, a0, b0, b2)
      if (s + 10 < nst) BATQ_STEP(s + 10, 10, slot0, slot1, a1, b1, b0)
      if (s + 11 < nst) BATQ_STEP(s + 11, 11, slot1, slot0, a0, b2, b1)
    }
  }
#undef BATQ_STEP4
#undef BATQ_STEP6
#undef BATQ_STEP
#undef BATQ_CL

  // Bf16 output: converted before staging, in the wave's own band (the
  // epilogue of the two-per-CU kernels).  Here, with one workgroup per CU and
  // a private fp32 band already, it measured equal (2048 x 4096 x 12288:
  // 46.5 against 46.4 us; the whole epilogue is 3.3 us of it).
  if (!p.out_f32) {
    // tile and wave are uniform; the helper takes them in scalar registers
    const int64_t m0u = (int64_t)__builtin_amdgcn_readfirstlane(tm) * kBM;
    const int64_t c0u = (int64_t)__builtin_amdgcn_readfirstlane(tn) * kBN;
    store_bf16_tile(p, acc, m0u, c0u + 64 * __builtin_amdgcn_readfirstlane(wave), lane, epi_buf + wave * kEpiWave,
                    m0u + kBM <= p.M && c0u + kBN <= p.N && p.vec_store);
    return;
  }
  // Fp32 output through LDS: one 32-row band per pass, 16-byte row chunks out.
  float* epi = reinterpret_cast<float*>(epi_buf + wave * kEpiWave);
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
#pragma unroll
    for (int k = 0; k < kNT; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rs = 8 * (r >> 2) + 4 * g + (r & 3);
        epi[rs * kEpiStride + 32 * k + r32] = acc[i][k][r];
      }
#pragma unroll
    for (int it = 0; it < 32 * 4 * kNT / 64; ++it) {
      const int id = it * 64 + lane;
      const int rs = id / (4 * kNT);
      const int cc = id % (4 * kNT);
      const float* src = epi + rs * kEpiStride + 8 * cc;
      const float4 lo = reinterpret_cast<const float4*>(src)[0];
      const float4 hi = reinterpret_cast<const float4*>(src)[1];
      const int64_t row = m0 + 32 * i + rs;
      const int64_t col = n0 + 8 * cc;
      if (row >= p.M || col >= p.N) continue;
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      // Output stores are non-temporal: Y is not read again here, and cached
      // output lines would evict operand lines that other tiles still reuse.
      if (p.out_f32) {
        float* dst = reinterpret_cast<float*>(p.y) + row * p.N + col;
        if (col + 8 <= p.N && p.vec_store) {
          __builtin_nontemporal_store(f32x4{lo.x, lo.y, lo.z, lo.w}, reinterpret_cast<f32x4*>(dst));
          __builtin_nontemporal_store(f32x4{hi.x, hi.y, hi.z, hi.w}, reinterpret_cast<f32x4*>(dst) + 1);
        } else {
          for (int e = 0; e < 8; ++e)
            if (col + e < p.N) dst[e] = v[e];
        }
      } else {
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.y) + row * p.N + col;
        uint32_t hb[4];  // bf16 pairs
#pragma unroll
        for (int e = 0; e < 4; ++e) hb[e] = f32x2_to_bf16x2_rne(v[2 * e], v[2 * e + 1]);
        if (col + 8 <= p.N && p.vec_store) {
          __builtin_nontemporal_store(u32x4{hb[0], hb[1], hb[2], hb[3]}, reinterpret_cast<u32x4*>(dst));
        } else {
          for (int e = 0; e < 8; ++e)
            if (col + e < p.N) dst[e] = (uint16_t)(hb[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

template <int NST, bool GS, bool A8>
hipError_t launch_packed_t(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = (int)((args.M + kBM - 1) / kBM);
  const int tiles_n = (int)((args.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((mxfp4_gemm_packed_kernel<NST, GS, A8>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, args,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

template <int NST, bool GS>
hipError_t launch_packed(const GemmArgs& args, hipStream_t stream) {
  return args.a_fp8 ? launch_packed_t<NST, GS, true>(args, stream) : launch_packed_t<NST, GS, false>(args, stream);
}

}  // namespace

hipError_t launch_weight_pack(const uint8_t* wq, const uint8_t* ws, int64_t N, int64_t K, uint8_t* wp,
                              hipStream_t stream) {
  const int64_t groups = ((N + 31) / 32) * (K / 256);
  hipLaunchKernelGGL(weight_pack_kernel, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, stream, wq, ws, N, K, wp);
  return hipGetLastError();
}

hipError_t launch_mxfp4_gemm_packed(const GemmArgs& args, hipStream_t stream) {
  if (packed_dma_applies(args)) return launch_mxfp4_gemm_packed_dma(args, stream);
  switch (args.K / 256) {
    case 1: return launch_packed<1, false>(args, stream);
    case 2: return launch_packed<2, false>(args, stream);
    case 4: return launch_packed<4, true>(args, stream);
    case 8: return launch_packed<8, true>(args, stream);
    case 16: return launch_packed<16, true>(args, stream);
    case 48: return launch_packed<48, true>(args, stream);
    default:
      return (args.K / 256) % 4 == 0 ? launch_packed<0, true>(args, stream) : launch_packed<0, false>(args, stream);
  }
}

}  // namespace batq
