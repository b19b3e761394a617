// W4A4 GEMM on packed weights, two workgroups per CU: Y = deq(Xq, Xs) deq(W)^T
// with FP32 accumulation [BATQuant note (en.papernotes.org), Key Designs §1 and
// §4: the product Q(XP) Q(P^-1 W^T) on block-scaled MXFP4 operands].
//
// Same tile (128 x 256), same operands and the same MFMA sequence per output
// as the kernel in mxfp4_gemm_packed.hip, so the results are bit-identical;
// what changes is how the data gets to the matrix cores.  With more than one
// tile per CU, two resident workgroups cover each other's barrier waits and
// LDS reads, which is worth 13-18 % on gfx950.  Two fit only if a workgroup
// needs at most 256 registers per lane (128 accumulators + 128 others) and
// 64 KB of LDS, so:
//   activation codes  global -> LDS by 16-byte direct-to-LDS buffer loads (no
//                     staging registers), two stages ahead, three-slot ring;
//                     a row's 16-byte chunk c sits at position c ^ swz(row);
//   activation scales the same way, four stages (32 bytes of a row) per load,
//                     two-group ring;
//   weights           packed, lane-ordered records straight into registers,
//                     one stage ahead (two register sets), the loads spread
//                     between the MFMAs of the stage before;
//   fragments         each sub-step's four activation fragments are read just
//                     before its eight MFMAs (the other workgroup hides them).
// Each wave waits only for its own loads (exact vmcnt), then one workgroup
// barrier per stage publishes every wave's loads and frees the slot that the
// next loads overwrite.  A bf16 output tile leaves through each wave's own
// 4 KB of LDS, converted before staging and without a workgroup barrier; an
// fp32 one through the ring (its own kernel instance).
// A second kernel does the same for E4M3 activations (the W4A8 setting), with
// 256-byte rows and a two-slot ring (see w4a8_gemm_packed_dma_kernel).
//
// Needs a compile-time stage count K / 256 that is a multiple of 4, and
// activations small enough for 32-bit buffer offsets (packed_dma_applies
// checks both on the host).
#include "gemm_epilogue.h"

namespace batq {

namespace {

constexpr int kMT = 4;                          // 32-row A tiles per wave
constexpr int kNT = 2;                          // 32-column B tiles per wave
constexpr int kBM = 32 * kMT;                   // 128 rows per tile
constexpr int kBN = 4 * 32 * kNT;               // 256 columns, four waves along N
constexpr int kRowBytes = 128;                  // activation code bytes per row and stage
constexpr int kSlotBytes = kBM * kRowBytes;     // one stage of the tile's activations
constexpr int kSGroupBytes = kBM * 32;          // scales of four stages
constexpr int kEpiStride = 32 * kNT + 8;        // floats per staged output row
constexpr int kEpiWave = 32 * kEpiStride * 4;   // bytes of one wave's staged 32-row band
constexpr int kQPerWave = kSlotBytes / 1024 / 4;  // code DMA instructions per wave and stage (4)
constexpr int kGroupM = 8;                      // row tiles per band of the tile order
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ i32x8 op(uint4 v) {
  i32x8 r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}
template <int J>
__device__ __forceinline__ f32x16 mfma_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(a), op(b), acc, 4, 4, J, (int)sa, J, (int)sb);
}
// A sub-step reads one 16-byte chunk of 32 consecutive rows per instruction;
// this placement of chunk c of row r (c ^ swz(r)) measured fastest.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// Younger loads a step may leave in flight: a stage's code loads, plus the
// scale-group load when one was issued after the weights.  n is a
// compile-time constant once the stage loop is unrolled.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case kQPerWave: wait_vmcnt<kQPerWave>(); break;
    case kQPerWave + 1: wait_vmcnt<kQPerWave + 1>(); break;
    default: wait_vmcnt<0>(); break;
  }
}
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
// Buffer loads of the packed weights: the lane part of the offset in one
// register, the record offset in a scalar (no per-stage 64-bit address
// arithmetic; 3-4 % faster than plain global loads on config-2 and config-5
// shapes).
__device__ __forceinline__ uint4 bl16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint32_t bl4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0);
}
// Stage offsets pass through an empty asm so that the per-stage address
// arithmetic stays in its pipeline step.
__device__ __forceinline__ int64_t opaque_stage(int64_t s) {
  asm volatile("" : "+s"(s));
  return s;
}

#define DMA_DECL_B(n) \
  uint4 n##_00, n##_01, n##_02, n##_03, n##_10, n##_11, n##_12, n##_13; \
  uint32_t n##_s0, n##_s1;
// Weight record of stage ST for both 32-column groups: four 1 KB code
// sub-steps and the 256-byte scale block, 16 (4) bytes per lane.
#define DMA_LOAD_B(n, ST)                                                                      \
  {                                                                                            \
    const int o_ = (int)(opaque_stage(ST) * kPackGroupBytes);                                  \
    n##_00 = bl16(wrs0, lane16, o_); n##_01 = bl16(wrs0, lane16, o_ + 1024);                   \
    n##_02 = bl16(wrs0, lane16, o_ + 2048); n##_03 = bl16(wrs0, lane16, o_ + 3072);            \
    n##_s0 = bl4(wrs0, lane4, o_ + 4096);                                                      \
    n##_10 = bl16(wrs1, lane16, o_); n##_11 = bl16(wrs1, lane16, o_ + 1024);                   \
    n##_12 = bl16(wrs1, lane16, o_ + 2048); n##_13 = bl16(wrs1, lane16, o_ + 3072);            \
    n##_s1 = bl4(wrs1, lane4, o_ + 4096);                                                      \
  }
// The loads a step issues for later stages go out between its MFMAs, each
// right after one MFMA of a sub-step (the scheduling groups below pin that
// order), rather than in front of the first MFMA.  There they held each
// wave's in-order issue back behind the queue of vector loads at every stage
// start.  Spread out, the results are bit-identical and the GEMM is faster on
// the 16384 x 4096 x 4096 and 2048 x 12288 x 4096 shapes (alternating A/B in
// one process): 4.6 and 6.6 % with E2M1 activations, 3.3 and 3.1 % with
// E4M3.  The issue order within a step is unchanged, so its vmcnt waits are
// too.  DMA_ILk: k (MFMA, load) pairs, then the sub-step's other MFMAs.
#define DMA_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 1, J); __builtin_amdgcn_sched_group_barrier(0x020, 1, J);
#define DMA_IL2(J) DMA_MV(J) DMA_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 6, J);
#define DMA_IL3(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 5, J);
#define DMA_IL4(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 4, J);
#define DMA_IL5(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) DMA_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 3, J);
// One 16-byte (DMA_W) or 4-byte (DMA_WS) part of a weight record.
#define DMA_W(R, WRS, ST, OFF) R = bl16(WRS, lane16, (int)(opaque_stage(ST) * kPackGroupBytes) + (OFF));
#define DMA_WS(R, WRS, ST) R = bl4(WRS, lane4, (int)(opaque_stage(ST) * kPackGroupBytes) + 4096);
// One descriptor per 32-column group, based at its first record (a group's
// NST records stay under 2 GiB: checked on the host), and the lane offsets of
// a record's code (16 l) and scale (4 l) bytes.
#define DECL_WEIGHTS                                                                           \
  const __amdgpu_buffer_rsrc_t wrs0 = __builtin_amdgcn_make_buffer_rsrc(                       \
      (void*)(p.wq + n32_g0 * NST * kPackGroupBytes), (short)0, NST * (int)kPackGroupBytes, 0x00020000); \
  const __amdgpu_buffer_rsrc_t wrs1 = __builtin_amdgcn_make_buffer_rsrc(                       \
      (void*)(p.wq + n32_g1 * NST * kPackGroupBytes), (short)0, NST * (int)kPackGroupBytes, 0x00020000); \
  const uint32_t lane16 = 16u * (uint32_t)lane, lane4 = 4u * (uint32_t)lane;

// Tile t of a tm x tn grid: consecutive workgroups go to the 8 XCDs in turn,
// so XCD x receives a contiguous range of t, walked in bands of kGroupM row
// tiles that share an activation panel in that XCD's L2.
__device__ __forceinline__ void tile_coords(int t, int tm, int tn, int& m, int& n) {
  const int total = tm * tn;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int gsz = kGroupM * tn;
  const int first = (t / gsz) * kGroupM;
  const int gm = min(kGroupM, tm - first);
  m = first + (t % gsz) % gm;
  n = (t % gsz) / gm;
}

// Output tile from the accumulators, through LDS: each wave stages its
// 32-row bands at `stage` (kEpiWave bytes, in memory the ring also uses: the
// caller is done with it once every wave reaches the barrier below).
__device__ __forceinline__ void store_tile_at(const GemmArgs& p, f32x16 (&acc)[kMT][kNT], int64_t m0, int64_t c0,
                                              int wave, int lane, uint8_t* stage) {
  // The accumulators are final here: an empty asm that reads them keeps the
  // last stages' MFMAs from sinking into the epilogue, which would keep their
  // operands live across it.
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int k = 0; k < kNT; ++k) asm volatile("" : "+a"(acc[i][k]));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();                     // every wave is done with the ring

  // Epilogue through LDS: one 32-row band per pass, 16-byte row chunks out;
  // waves 0, 1 stage in slot0 and waves 2, 3 in slot1.  Its inputs pass
  // through an empty asm so that none of its address arithmetic is hoisted
  // above the stage loop.
  int lane_e = lane, wave_e = wave;
  int64_t m0e = m0, c0e = c0;
  asm volatile("" : "+v"(lane_e), "+s"(wave_e), "+s"(m0e), "+s"(c0e));
  const int r32e = lane_e & 31, ge = lane_e >> 5;
  float* epi = reinterpret_cast<float*>(stage);
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    sched_fence();
#pragma unroll
    for (int k = 0; k < kNT; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rs = 8 * (r >> 2) + 4 * ge + (r & 3);
        epi[rs * kEpiStride + 32 * k + r32e] = acc[i][k][r];
      }
#pragma unroll
    for (int it = 0; it < 32 * 4 * kNT / 64; ++it) {
      const int id = it * 64 + lane_e;
      const int rs = id / (4 * kNT);
      const int cc = id % (4 * kNT);
      // Lanes 4-7 of every 8 read their upper half first: eight lanes'
      // 16-byte reads then cover all 32 banks once instead of half of them
      // twice.
      const float* src = epi + rs * kEpiStride + 8 * cc;
      const int sw = (cc >> 2) & 1;
      const float4 first = *reinterpret_cast<const float4*>(src + 4 * sw);
      const float4 second = *reinterpret_cast<const float4*>(src + 4 - 4 * sw);
      const float4 lo = sw ? second : first;
      const float4 hi = sw ? first : second;
      const int64_t row = m0e + 32 * i + rs;
      const int64_t col = c0e + 64 * wave_e + 8 * cc;
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

__device__ __forceinline__ void store_tile(const GemmArgs& p, f32x16 (&acc)[kMT][kNT], int64_t m0, int64_t c0,
                                           int wave, int lane, uint8_t* slot0, uint8_t* slot1) {
  store_tile_at(p, acc, m0, c0, wave, lane, (wave < 2 ? slot0 : slot1) + (wave & 1) * kEpiWave);
}

constexpr int kStageWave = epi_bf16_wave_bytes<kNT>();  // one wave's bf16 band (4 KB)

// F32OUT: fp32 output through the ring slots (one epilogue per instance: with
// both in one kernel the accumulators stayed live into each and spilled).
template <int NST, bool F32OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mxfp4_gemm_packed_dma_kernel(
    GemmArgs p, int tiles_m, int tiles_n) {
  static_assert(NST % 4 == 0, "scale groups span four stages");
  // Separate arrays, so that the compiler sees which LDS reads each DMA can
  // alias.  stg holds each wave's bf16 output band (fp32 output stages one
  // wave's band in each of slot0..slot2 and stg).
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sg0[kSGroupBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sg1[kSGroupBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stg[4 * kStageWave];
  static_assert(kEpiWave <= kSlotBytes && kEpiWave <= 4 * kStageWave, "an fp32 band fits a slot and stg");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t c0 = (int64_t)tn * kBN;
  const int64_t n0 = c0 + 64 * wave;  // this wave's first column
  const int64_t n32_max = (p.N + 31) / 32;
  // Each of the wave's two 32-column groups is clamped on its own: a clamped
  // group is computed (so every wave reaches every barrier) but its columns
  // lie past N and are never stored.
  const int64_t n32_g0 = n0 / 32 < n32_max ? n0 / 32 : n32_max - 1;
  const int64_t n32_g1 = n0 / 32 + 1 < n32_max ? n0 / 32 + 1 : n32_max - 1;
  DECL_WEIGHTS

  // Activation codes: instruction q of this wave fills LDS bytes
  // [1024 (kQPerWave wave + q), +1024) = rows 8 (kQPerWave wave + q) + l / 8;
  // lane l fetches the row's chunk (l % 8) ^ swz(row) for position l % 8.
  // Rows past M read row M - 1 and are never stored.
  const uint32_t krow = (uint32_t)(p.K >> 1);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.xq, (short)0, (int)(p.M * (int64_t)krow), 0x00020000);
  uint32_t qoff[kQPerWave];
#pragma unroll
  for (int q = 0; q < kQPerWave; ++q) {
    const int row = 8 * (kQPerWave * wave + q) + (lane >> 3);
    const int64_t gr = m0 + row < p.M ? m0 + row : p.M - 1;
    qoff[q] = (uint32_t)gr * krow + 16u * (uint32_t)((lane & 7) ^ swz(row));
  }
  // Activation scales, four stages (32 bytes of a row) per group: wave w
  // covers rows 32 w + l % 32, 16-byte half l / 32 (stages 2 h, 2 h + 1), so
  // LDS holds [wave][half][32 rows][16 bytes].  Rows 16 bytes apart (rather
  // than 32) put a stage's 64 scale words of a sub-tile on twice as many banks.
  const uint32_t srow = (uint32_t)(p.K >> 5);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.xs, (short)0, (int)(p.M * (int64_t)srow), 0x00020000);
  uint32_t soff;
  {
    const int row = 32 * wave + (lane & 31);
    const int64_t gr = m0 + row < p.M ? m0 + row : p.M - 1;
    soff = (uint32_t)gr * srow + 16u * (uint32_t)(lane >> 5);
  }
#define DMA_A(SLOT, ST)                                                                         \
  _Pragma("unroll") for (int q = 0; q < kQPerWave; ++q)                                         \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void*)((SLOT) + 1024 * (kQPerWave * wave + q)), 16, \
                                             (int)qoff[q], (int)((ST) * kRowBytes), 0, 0);
#define DMA_S(SG, G) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)((SG) + 1024 * wave), 16, (int)soff, (int)((G) * 32), 0, 0);

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int k = 0; k < kNT; ++k) acc[i][k] = f32x16{};
  DMA_DECL_B(b0)
  DMA_DECL_B(b1)
  // Issue order per wave: scale group 0, codes of stage 0, weights of stage
  // 0, codes of stage 1; then each step S issues weights S + 1, the scale
  // group that starts at S + 2 (if any) and codes S + 2.
  DMA_S(sg0, 0)
  DMA_A(slot0, 0)
  DMA_LOAD_B(b0, 0)
  DMA_A(slot1, 1)

  // One sub-step j: the four activation fragments (rows 32 i + r32, chunk
  // 4 g + j) from LDS, then 4 x 2 MFMAs, weight-stationary: the four of
  // column group 0, then those of group 1 in reverse row order, so that one
  // operand stays the same from each MFMA to the next (fewer operand bits
  // toggle; 1 % faster on config 2 and 5 shapes).  Every accumulator still
  // takes its sub-steps in order, so the results are unchanged.
#define DMA_RD(SLOT, FO, I) *reinterpret_cast<const uint4*>((SLOT) + (FO) + 4096 * (I))
#define DMA_SUB(SLOT, FO, J, n)                                                                \
  uint4 fa_[kMT];                                                                              \
  _Pragma("unroll") for (int i = 0; i < kMT; ++i) fa_[i] = DMA_RD(SLOT, FO, i);                \
  _Pragma("unroll") for (int i = 0; i < kMT; ++i)                                              \
    acc[i][0] = mfma_fp4<J>(fa_[i], n##_0##J, sa_[i], n##_s0, acc[i][0]);                     \
  _Pragma("unroll") for (int i = kMT - 1; i >= 0; --i)                                         \
    acc[i][1] = mfma_fp4<J>(fa_[i], n##_1##J, sa_[i], n##_s1, acc[i][1]);
  // The lane parts of a stage's LDS addresses are recomputed per stage (behind
  // an empty asm) so that they are not held for every stage at once.
#define DMA_OFFSETS(SG, SQI)                                                                   \
  uint32_t so_ = r32 * 16 + 4 * g;                                                             \
  uint32_t fo0_ = r32 * kRowBytes + 16 * ((4 * g) ^ swz(r32));                                  \
  uint32_t fo1_ = r32 * kRowBytes + 16 * ((4 * g + 1) ^ swz(r32));                              \
  uint32_t fo2_ = r32 * kRowBytes + 16 * ((4 * g + 2) ^ swz(r32));                              \
  uint32_t fo3_ = r32 * kRowBytes + 16 * ((4 * g + 3) ^ swz(r32));                              \
  asm volatile("" : "+v"(so_), "+v"(fo0_), "+v"(fo1_), "+v"(fo2_), "+v"(fo3_));                \
  uint32_t sa_[kMT];                                                                           \
  _Pragma("unroll") for (int i = 0; i < kMT; ++i) sa_[i] = ld4((SG) + so_ + 1024 * i + 512 * ((SQI) >> 1) + 8 * ((SQI) & 1));
  // Step S: wait for stage S (weights issued one step ago, codes two, scale
  // group at least two), barrier, compute stage S while issuing the loads of
  // stages S + 1 (weights over sub-steps 0-2) and S + 2 (scale group, codes).
#define DMA_STEP(S, CUR, NXT2, SG, SGN, BCUR, BNXT1)                                           \
  {                                                                                            \
    wait_vm(((S) + 1 < NST) ? (kQPerWave + (((S) + 1) % 4 == 0 ? 1 : 0)) : 0);                 \
    block_barrier();                                                                           \
    sched_fence();                                                                             \
    DMA_OFFSETS(SG, (S) % 4)                                                                   \
    {                                                                                          \
      DMA_SUB(CUR, fo0_, 0, BCUR)                                                              \
      if ((S) + 1 < NST) {                                                                     \
        DMA_W(BNXT1##_00, wrs0, (S) + 1, 0) DMA_W(BNXT1##_01, wrs0, (S) + 1, 1024)              \
        DMA_W(BNXT1##_02, wrs0, (S) + 1, 2048) DMA_W(BNXT1##_03, wrs0, (S) + 1, 3072)           \
        DMA_IL4(0)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      DMA_SUB(CUR, fo1_, 1, BCUR)                                                              \
      if ((S) + 1 < NST) {                                                                     \
        DMA_WS(BNXT1##_s0, wrs0, (S) + 1) DMA_W(BNXT1##_10, wrs1, (S) + 1, 0)                   \
        DMA_W(BNXT1##_11, wrs1, (S) + 1, 1024) DMA_W(BNXT1##_12, wrs1, (S) + 1, 2048)           \
        DMA_IL4(1)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      DMA_SUB(CUR, fo2_, 2, BCUR)                                                              \
      if ((S) + 1 < NST) {                                                                     \
        DMA_W(BNXT1##_13, wrs1, (S) + 1, 3072) DMA_WS(BNXT1##_s1, wrs1, (S) + 1)                \
        if ((S) + 2 < NST && ((S) + 2) % 4 == 0) {                                             \
          DMA_S(SGN, ((S) + 2) / 4)                                                            \
          DMA_IL3(2)                                                                           \
        } else {                                                                               \
          DMA_IL2(2)                                                                           \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      DMA_SUB(CUR, fo3_, 3, BCUR)                                                              \
      if ((S) + 2 < NST) {                                                                     \
        DMA_A(NXT2, (S) + 2)                                                                   \
        DMA_IL4(3)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
  }
  // Code slots cycle with period 3 (stage s in slot s % 3), weight sets with
  // period 2, scale groups with period 8 (stage s reads group s / 4 from
  // sg[(s / 4) % 2]; SGN is where the group starting at s + 2 goes): 24.
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    switch (s % 24) {
      case 0: DMA_STEP(s, slot0, slot2, sg0, sg0, b0, b1) break;
      case 1: DMA_STEP(s, slot1, slot0, sg0, sg0, b1, b0) break;
      case 2: DMA_STEP(s, slot2, slot1, sg0, sg1, b0, b1) break;
      case 3: DMA_STEP(s, slot0, slot2, sg0, sg1, b1, b0) break;
      case 4: DMA_STEP(s, slot1, slot0, sg1, sg1, b0, b1) break;
      case 5: DMA_STEP(s, slot2, slot1, sg1, sg1, b1, b0) break;
      case 6: DMA_STEP(s, slot0, slot2, sg1, sg0, b0, b1) break;
      case 7: DMA_STEP(s, slot1, slot0, sg1, sg0, b1, b0) break;
      case 8: DMA_STEP(s, slot2, slot1, sg0, sg0, b0, b1) break;
      case 9: DMA_STEP(s, slot0, slot2, sg0, sg0, b1, b0) break;
      case 10: DMA_STEP(s, slot1, slot0, sg0, sg1, b0, b1) break;
      case 11: DMA_STEP(s, slot2, slot1, sg0, sg1, b1, b0) break;
      case 12: DMA_STEP(s, slot0, slot2, sg1, sg1, b0, b1) break;
      case 13: DMA_STEP(s, slot1, slot0, sg1, sg1, b1, b0) break;
      case 14: DMA_STEP(s, slot2, slot1, sg1, sg0, b0, b1) break;
      case 15: DMA_STEP(s, slot0, slot2, sg1, sg0, b1, b0) break;
      case 16: DMA_STEP(s, slot1, slot0, sg0, sg0, b0, b1) break;
      case 17: DMA_STEP(s, slot2, slot1, sg0, sg0, b1, b0) break;
      case 18: DMA_STEP(s, slot0, slot2, sg0, sg1, b0, b1) break;
      case 19: DMA_STEP(s, slot1, slot0, sg0, sg1, b1, b0) break;
      case 20: DMA_STEP(s, slot2, slot1, sg1, sg1, b0, b1) break;
      case 21: DMA_STEP(s, slot0, slot2, sg1, sg1, b1, b0) break;
      case 22: DMA_STEP(s, slot1, slot0, sg1, sg0, b0, b1) break;
      default: DMA_STEP(s, slot2, slot1, sg1, sg0, b1, b0) break;
    }
  }
#undef DMA_STEP
#undef DMA_OFFSETS
#undef DMA_SUB
#undef DMA_RD
#undef DMA_S
#undef DMA_A

  if constexpr (F32OUT)
    store_tile_at(p, acc, m0, c0, wave, lane, wave == 0 ? slot0 : wave == 1 ? slot1 : wave == 2 ? slot2 : stg);
  else
    store_bf16_tile(p, acc, m0, c0 + 64 * wave, lane, stg + wave * kStageWave,
                    m0 + kBM <= p.M && c0 + kBN <= p.N && p.vec_store);
}

// E4M3 activations x packed E2M1 weights (the W4A8 setting): the same tile,
// weights and scales, bit-identical to the E4M3 path of the packed kernel.
// An activation row is 256 bytes per stage (32 KB per stage of the tile), so
// the code ring has two slots (codes one stage ahead) to stay within 72 KB of
// LDS per workgroup.  The row layout is that kernel's: 16-byte chunk c of row
// r at position c ^ (r % 16).  The E4M3 operand of lane (r, g) in sub-step j
// is chunks 2 j + g and 8 + 2 j + g of its row (see mfma_fp8_fp4).
constexpr int kRowBytes8 = 256;
constexpr int kSlotBytes8 = kBM * kRowBytes8;        // 32 KB
constexpr int kQPerWave8 = kSlotBytes8 / 1024 / 4;   // 8 code DMA instructions per wave and stage
static_assert(2 * kEpiWave <= kSlotBytes8, "two waves' epilogue bands fit one slot");

template <int J>
__device__ __forceinline__ f32x16 mfma_fp8_fp4(uint4 alo, uint4 ahi, uint4 b, uint32_t sa, uint32_t sb,
                                               f32x16 acc) {
  const i32x8 a = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, op(b), acc, 0, 4, J, (int)sa, J, (int)sb);
}

template <int NST, bool F32OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void w4a8_gemm_packed_dma_kernel(
    GemmArgs p, int tiles_m, int tiles_n) {
  static_assert(NST % 4 == 0, "scale groups span four stages");
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kSlotBytes8];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kSlotBytes8];
  __shared__ __attribute__((aligned(1024))) uint8_t sg0[kSGroupBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sg1[kSGroupBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t c0 = (int64_t)tn * kBN;
  const int64_t n0 = c0 + 64 * wave;
  const int64_t n32_max = (p.N + 31) / 32;
  const int64_t n32_g0 = n0 / 32 < n32_max ? n0 / 32 : n32_max - 1;
  const int64_t n32_g1 = n0 / 32 + 1 < n32_max ? n0 / 32 + 1 : n32_max - 1;
  DECL_WEIGHTS

  // Codes: instruction q of this wave fills LDS bytes [1024 (8 wave + q),
  // +1024) = rows 4 (8 wave + q) + l / 16; lane l fetches the row's chunk
  // (l % 16) ^ (row % 16) for position l % 16.  The swizzle repeats every
  // four instructions, so four lane offsets serve all eight: instructions
  // 4..7 (rows 16 further on) use a second descriptor based 16 rows later.
  // The whole row offset is in the vector offset, which the range check
  // covers, so rows past M read zeros without touching memory; they are
  // never stored.
  const uint32_t krow = (uint32_t)p.K;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.xq, (short)0, (int)(p.M * (int64_t)krow), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs16 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.xq + 16 * (int64_t)krow), (short)0, p.M > 16 ? (int)((p.M - 16) * (int64_t)krow) : 0, 0x00020000);
  uint32_t qoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * (kQPerWave8 * wave + q) + (lane >> 4);
    qoff[q] = (uint32_t)(m0 + row) * krow + 16u * (uint32_t)((lane & 15) ^ (row & 15));
  }
  const uint32_t srow = (uint32_t)(p.K >> 5);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.xs, (short)0, (int)(p.M * (int64_t)srow), 0x00020000);
  uint32_t soff;
  {
    const int row = 32 * wave + (lane & 31);
    const int64_t gr = m0 + row < p.M ? m0 + row : p.M - 1;
    soff = (uint32_t)gr * srow + 16u * (uint32_t)(lane >> 5);
  }
#define DMA_A8(SLOT, ST)                                                                        \
  {                                                                                            \
    const uint32_t st_ = (uint32_t)opaque_stage((ST) * kRowBytes8);                            \
    _Pragma("unroll") for (int q = 0; q < kQPerWave8; ++q)                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds((q >> 2) ? xrs16 : xrs,                         \
                                               (lds_void*)((SLOT) + 1024 * (kQPerWave8 * wave + q)), 16, \
                                               (int)qoff[q & 3], (int)st_, 0, 0);               \
  }
#define DMA_S8(SG, G) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)((SG) + 1024 * wave), 16, (int)soff, (int)((G) * 32), 0, 0);

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int k = 0; k < kNT; ++k) acc[i][k] = f32x16{};
  DMA_DECL_B(b0)
  DMA_DECL_B(b1)
  // Issue order per wave: scale group 0, codes and weights of stage 0; then
  // step S issues the weights, the scale group starting at S + 1 (if any)
  // and the codes of stage S + 1.  So each step waits for everything.
  DMA_S8(sg0, 0)
  DMA_A8(slot0, 0)
  DMA_LOAD_B(b0, 0)

  // Sub-step j: rows 32 i + r32, chunks 2 j + g and 8 + 2 j + g.  The lane
  // offsets are recomputed per sub-step behind an empty asm, so that they are
  // not all held across the stage loop.
#define RD8(SLOT, I, FO) *reinterpret_cast<const uint4*>((SLOT) + 8192 * (I) + (FO))
#define SUB8(SLOT, J, n)                                                                       \
  uint32_t flo_ = r32 * kRowBytes8 + 16 * ((2 * (J) + g) ^ (r32 & 15));                        \
  uint32_t fhi_ = r32 * kRowBytes8 + 16 * ((8 + 2 * (J) + g) ^ (r32 & 15));                    \
  asm volatile("" : "+v"(flo_), "+v"(fhi_));                                                   \
  uint4 lo_[kMT], hi_[kMT];                                                                    \
  _Pragma("unroll") for (int i = 0; i < kMT; ++i) {                                            \
    lo_[i] = RD8(SLOT, i, flo_);                                                               \
    hi_[i] = RD8(SLOT, i, fhi_);                                                               \
  }                                                                                            \
  _Pragma("unroll") for (int i = 0; i < kMT; ++i) {                                            \
    acc[i][0] = mfma_fp8_fp4<J>(lo_[i], hi_[i], n##_0##J, sa_[i], n##_s0, acc[i][0]);         \
    acc[i][1] = mfma_fp8_fp4<J>(lo_[i], hi_[i], n##_1##J, sa_[i], n##_s1, acc[i][1]);         \
  }
  // Half H of a stage's code loads (four of the eight).
#define DMA_A8H(SLOT, ST, H)                                                                   \
  {                                                                                            \
    const uint32_t st_ = (uint32_t)opaque_stage((ST) * kRowBytes8);                            \
    _Pragma("unroll") for (int q = 4 * (H); q < 4 * (H) + 4; ++q)                              \
      __builtin_amdgcn_raw_ptr_buffer_load_lds((q >> 2) ? xrs16 : xrs,                         \
                                               (lds_void*)((SLOT) + 1024 * (kQPerWave8 * wave + q)), 16, \
                                               (int)qoff[q & 3], (int)st_, 0, 0);               \
  }
  // As in the E2M1 kernel, the loads for stage S + 1 (weights, scale group,
  // codes, in that order) go out between stage S's MFMAs, each right after
  // one of them, rather than in front of the first.
#define STEP8(S, CUR, NXT, SG, SGN, BCUR, BNXT)                                                \
  {                                                                                            \
    wait_vmcnt<0>();                                                                           \
    block_barrier();                                                                           \
    sched_fence();                                                                             \
    uint32_t so_ = r32 * 16 + 4 * g;                                                           \
    asm volatile("" : "+v"(so_));                                                              \
    uint32_t sa_[kMT];                                                                         \
    _Pragma("unroll") for (int i = 0; i < kMT; ++i) sa_[i] = ld4((SG) + so_ + 1024 * i + 512 * (((S) % 4) >> 1) + 8 * (((S) % 4) & 1)); \
    {                                                                                          \
      SUB8(CUR, 0, BCUR)                                                                       \
      if ((S) + 1 < NST) {                                                                     \
        DMA_W(BNXT##_00, wrs0, (S) + 1, 0) DMA_W(BNXT##_01, wrs0, (S) + 1, 1024)                \
        DMA_W(BNXT##_02, wrs0, (S) + 1, 2048) DMA_W(BNXT##_03, wrs0, (S) + 1, 3072)             \
        DMA_WS(BNXT##_s0, wrs0, (S) + 1)                                                       \
        DMA_IL5(0)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      SUB8(CUR, 1, BCUR)                                                                       \
      if ((S) + 1 < NST) {                                                                     \
        DMA_W(BNXT##_10, wrs1, (S) + 1, 0) DMA_W(BNXT##_11, wrs1, (S) + 1, 1024)                \
        DMA_W(BNXT##_12, wrs1, (S) + 1, 2048) DMA_W(BNXT##_13, wrs1, (S) + 1, 3072)             \
        DMA_WS(BNXT##_s1, wrs1, (S) + 1)                                                       \
        DMA_IL5(1)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      SUB8(CUR, 2, BCUR)                                                                       \
      if ((S) + 1 < NST) {                                                                     \
        if (((S) + 1) % 4 == 0) {                                                              \
          DMA_S8(SGN, ((S) + 1) / 4)                                                           \
          DMA_A8H(NXT, (S) + 1, 0)                                                             \
          DMA_IL5(2)                                                                           \
        } else {                                                                               \
          DMA_A8H(NXT, (S) + 1, 0)                                                             \
          DMA_IL4(2)                                                                           \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
    {                                                                                          \
      SUB8(CUR, 3, BCUR)                                                                       \
      if ((S) + 1 < NST) {                                                                     \
        DMA_A8H(NXT, (S) + 1, 1)                                                               \
        DMA_IL4(3)                                                                             \
      }                                                                                        \
    }                                                                                          \
    sched_fence();                                                                             \
  }
  // Stage s: codes in slot s % 2, weights in set s % 2, scales of group s / 4
  // in sg[(s / 4) % 2]; SGN is where the group starting at s + 1 goes.
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    switch (s % 8) {
      case 0: STEP8(s, slot0, slot1, sg0, sg0, b0, b1) break;
      case 1: STEP8(s, slot1, slot0, sg0, sg0, b1, b0) break;
      case 2: STEP8(s, slot0, slot1, sg0, sg0, b0, b1) break;
      case 3: STEP8(s, slot1, slot0, sg0, sg1, b1, b0) break;
      case 4: STEP8(s, slot0, slot1, sg1, sg1, b0, b1) break;
      case 5: STEP8(s, slot1, slot0, sg1, sg1, b1, b0) break;
      case 6: STEP8(s, slot0, slot1, sg1, sg1, b0, b1) break;
      default: STEP8(s, slot1, slot0, sg1, sg0, b1, b0) break;
    }
  }
#undef STEP8
#undef DMA_A8H
#undef SUB8
#undef RD8
#undef DMA_S8
#undef DMA_A8

  // Stage NST - 1 (NST even) reads slot1; every wave has passed the barrier
  // after which nothing reads or fills slot0 again, so each wave stages its
  // bf16 band there without a workgroup barrier.
  static_assert(NST % 2 == 0 && 4 * kStageWave <= kSlotBytes8, "bf16 bands fit the free slot");
  if constexpr (F32OUT)
    store_tile(p, acc, m0, c0, wave, lane, slot0, slot1);
  else
    store_bf16_tile(p, acc, m0, c0 + 64 * wave, lane, slot0 + wave * kStageWave,
                    m0 + kBM <= p.M && c0 + kBN <= p.N && p.vec_store);
}

template <int NST, bool A8>
hipError_t launch_t(const GemmArgs& args, int tiles_m, int tiles_n, hipStream_t stream) {
  if constexpr (A8) {
    if (args.out_f32)
      hipLaunchKernelGGL((w4a8_gemm_packed_dma_kernel<NST, true>), dim3(tiles_m * tiles_n), dim3(256), 0, stream,
                         args, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((w4a8_gemm_packed_dma_kernel<NST, false>), dim3(tiles_m * tiles_n), dim3(256), 0, stream,
                         args, tiles_m, tiles_n);
  } else if (args.out_f32)
    hipLaunchKernelGGL((mxfp4_gemm_packed_dma_kernel<NST, true>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, args,
                       tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((mxfp4_gemm_packed_dma_kernel<NST, false>), dim3(tiles_m * tiles_n), dim3(256), 0, stream,
                       args, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

// Worth it once there is more than one tile per CU (256 CUs); needs a stage
// count that is compiled here and activations small enough for the 32-bit
// offsets of a buffer descriptor.
bool packed_dma_applies(const GemmArgs& a) {
  const int64_t nst = a.K / 256;
  if (nst != 4 && nst != 8 && nst != 16 && nst != 48) return false;
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  const int64_t act_bytes = a.a_fp8 ? a.M * a.K : a.M * (a.K >> 1);
  return tiles > 256 && tiles < (int64_t)1 << 31 && act_bytes < (int64_t)1 << 31;
}

hipError_t launch_mxfp4_gemm_packed_dma(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = (int)((args.M + kBM - 1) / kBM);
  const int tiles_n = (int)((args.N + kBN - 1) / kBN);
  if (args.a_fp8) {
    switch (args.K / 256) {
      case 4: return launch_t<4, true>(args, tiles_m, tiles_n, stream);
      case 8: return launch_t<8, true>(args, tiles_m, tiles_n, stream);
      case 16: return launch_t<16, true>(args, tiles_m, tiles_n, stream);
      case 48: return launch_t<48, true>(args, tiles_m, tiles_n, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (args.K / 256) {
    case 4: return launch_t<4, false>(args, tiles_m, tiles_n, stream);
    case 8: return launch_t<8, false>(args, tiles_m, tiles_n, stream);
    case 16: return launch_t<16, false>(args, tiles_m, tiles_n, stream);
    case 48: return launch_t<48, false>(args, tiles_m, tiles_n, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace batq
