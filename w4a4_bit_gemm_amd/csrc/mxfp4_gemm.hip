// W4A4 GEMM on MXFP4 operands with the gfx950 block-scaled matrix cores.
//
// Y[m][n] = sum_k deq(Xq)[m][k] * deq(Wq)[n][k], FP32 accumulation
// [BATQuant note (en.papernotes.org), Key Designs §1: Q(XP) Q(P^-1 W^T);
//  Key Designs §4: all linear layers use low-bit matrix multiplication].
//
// Instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1.  Lane l
// supplies 32 consecutive k of row (l % 32) — exactly one MX block, 16 bytes —
// and that block's UE8M0 scale byte, picked out of a 32-bit register by OPSEL.
// The k order inside one instruction is free as long as both operands agree, so
// within every 256-k step lane half g covers blocks 4g..4g+3, one per
// instruction: a lane consumes 64 contiguous code bytes and one aligned 4-byte
// group of scales per row and step, in the canonical [rows][K/2], [rows][K/32]
// layouts.
//
// Main kernel (K % 256 == 0): workgroup tile BM x BN, 4 waves each owning
// (32 MT) x (32 NT) of the output.  Per 256-k stage, both operand tiles go
// global -> registers -> LDS: two register sets keep two stages in flight from
// memory while a third is read out of one of two LDS slots by the matrix cores
// (one barrier per stage).  Rows sit 128 bytes apart in LDS with their 16-byte
// chunks XOR-swizzled by row pair: eight consecutive threads load one whole
// 128-byte row segment, and the MFMA-side ds_read_b128s stay free of bank
// conflicts.  Workgroups are numbered so
// that each of the 8 XCDs (each with its own L2) owns a contiguous band of N
// tiles across all M tiles.  The epilogue goes through LDS to write 16-byte
// row-contiguous chunks.  A simpler direct-load kernel covers other K.
#include "common.h"

namespace batq {

namespace {

// ------------------------------------------------------------- shared helpers

__device__ __forceinline__ i32x8 op(uint4 v) {
  i32x8 r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

template <int J>
__device__ __forceinline__ f32x16 mfma_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(a), op(b), acc, 4, 4, J, (int)sa, J, (int)sb);
}

__device__ __forceinline__ void store_out8(const GemmArgs& p, int64_t row, int64_t col, const float* v) {
  if (row >= p.M) return;
  if (p.out_f32) {
    float* dst = reinterpret_cast<float*>(p.y) + row * p.N + col;
    if (col + 8 <= p.N && p.vec_store) {
      reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int e = 0; e < 8; ++e)
        if (col + e < p.N) dst[e] = v[e];
    }
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.y) + row * p.N + col;
    uint32_t h[4];  // bf16 pairs
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = f32x2_to_bf16x2_rne(v[2 * e], v[2 * e + 1]);
    if (col + 8 <= p.N && p.vec_store) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
    } else {
      for (int e = 0; e < 8; ++e)
        if (col + e < p.N) dst[e] = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// ------------------------------------------------- main kernel (K % 256 == 0)

constexpr int kStageK = 256;       // k per pipeline stage
constexpr int kRowBytes = 128;     // code bytes per row per stage
constexpr int kEpiPad = 8;         // fp32 row padding in the epilogue buffer

template <int MT, int NT>
struct Tile {
  static constexpr int kWaves = 4;  // 2 x 2 waves
  static constexpr int BM = 64 * MT;
  static constexpr int BN = 64 * NT;
  static constexpr int kA = BM * kRowBytes;
  static constexpr int kB = BN * kRowBytes;
  static constexpr int kAs = BM * 8;
  static constexpr int kBs = BN * 8;
  static constexpr int kStage = kA + kB + kAs + kBs;
  static constexpr int kEpiStride = 32 * NT + kEpiPad;  // floats
  static constexpr int kEpiWave = 32 * kEpiStride * 4;  // bytes per wave per pass
  };

// LDS slot of a 16-byte chunk: chunk ^ swz(row).  gfx950's LDS has 64 banks of
// 4 bytes and serves a ds_read_b128 16 lanes at a time; the MFMA fragment
// reads put 16 consecutive rows at the same logical chunk in one pass.  With
// 128-byte rows, row parity picks the bank half, so (row >> 1) & 7 gives those
// 16 rows 16 distinct (half, slot) bank groups.  The 16 threads of a
// ds_write_b128 pass cover two adjacent rows (one per half): also conflict-free.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Workgroup barrier without the implicit wait for all outstanding memory
// operations that __syncthreads() carries (that wait would also drain the
// prefetches of later stages).  The memory clobber keeps the compiler from
// moving LDS accesses across it; callers wait for the loads they need first.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
using u32vec = uint32_t __attribute__((ext_vector_type(N)));

// One stage of operands held in registers between its global load and its
// LDS write: each thread owns fixed 16-byte chunks of the A and B code tiles
// and fixed dwords of the scale tiles.  The storage is clang vector types, not
// arrays, so it always lives in VGPRs (arrays in a struct reach the early
// alloca-promotion pass with loop-variable indices and end up in memory).
template <int MT, int NT>
struct StageRegs {
  using T = Tile<MT, NT>;
  static constexpr int kThreads = 64 * T::kWaves;
  static constexpr int kAq = T::BM * 8 / kThreads;   // 16-byte chunks per thread
  static constexpr int kBq = T::BN * 8 / kThreads;
  static constexpr int kAs = T::BM * 2 / kThreads;   // scale dwords per thread
  static constexpr int kBs = T::BN * 2 / kThreads;
  static_assert(T::BM * 8 % kThreads == 0 && T::BN * 8 % kThreads == 0, "code tile split");
  static_assert(T::BM * 2 % kThreads == 0 && T::BN * 2 % kThreads == 0, "scale tile split");
  static_assert(kAs == 2 && kBs == 1, "scale staging below assumes 2 + 1 dwords");
  u32vec<4 * kAq> a;
  u32vec<4 * kBq> b;
  u32vec<2> as;
  uint32_t bs;

  // Chunk id = tid + kThreads * i; 8 consecutive threads cover one 128-byte row
  // segment (coalesced); the chunk's LDS slot is XOR-swizzled by row.
  __device__ __forceinline__ void load(const GemmArgs& p, int64_t m0, int64_t n0, int64_t s, int tid) {
    const int64_t qld = p.K >> 1;
    const int64_t sld = p.K >> 5;
    const int64_t kbyte0 = s * kRowBytes;
    const int64_t kb0 = s * 8;
#pragma unroll
    for (int i = 0; i < kAq; ++i) {
      const int id = tid + kThreads * i;
      int64_t gr = m0 + (id >> 3);
      gr = gr < p.M ? gr : p.M - 1;  // rows past the edge read a valid row, never stored
      const uint4 v = *reinterpret_cast<const uint4*>(p.xq + gr * qld + kbyte0 + 16 * (id & 7));
      a[4 * i] = v.x; a[4 * i + 1] = v.y; a[4 * i + 2] = v.z; a[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < kBq; ++i) {
      const int id = tid + kThreads * i;
      int64_t gr = n0 + (id >> 3);
      gr = gr < p.N ? gr : p.N - 1;
      const uint4 v = *reinterpret_cast<const uint4*>(p.wq + gr * qld + kbyte0 + 16 * (id & 7));
      b[4 * i] = v.x; b[4 * i + 1] = v.y; b[4 * i + 2] = v.z; b[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + kThreads * i;
      int64_t gr = m0 + (id >> 1);
      gr = gr < p.M ? gr : p.M - 1;
      as[i] = *reinterpret_cast<const uint32_t*>(p.xs + gr * sld + kb0 + 4 * (id & 1));
    }
    {
      int64_t gr = n0 + (tid >> 1);
      gr = gr < p.N ? gr : p.N - 1;
      bs = *reinterpret_cast<const uint32_t*>(p.ws + gr * sld + kb0 + 4 * (tid & 1));
    }
  }

  __device__ __forceinline__ void store(uint8_t* slot, int tid) const {
#pragma unroll
    for (int i = 0; i < kAq; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3;
      *reinterpret_cast<uint4*>(slot + row * kRowBytes + 16 * ((id & 7) ^ swz(row))) =
          make_uint4(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]);
    }
#pragma unroll
    for (int i = 0; i < kBq; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3;
      *reinterpret_cast<uint4*>(slot + T::kA + row * kRowBytes + 16 * ((id & 7) ^ swz(row))) =
          make_uint4(b[4 * i], b[4 * i + 1], b[4 * i + 2], b[4 * i + 3]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint32_t*>(slot + T::kA + T::kB + 4 * (tid + kThreads * i)) = as[i];
    *reinterpret_cast<uint32_t*>(slot + T::kA + T::kB + T::kAs + 4 * tid) = bs;
  }
};

__device__ __forceinline__ uint4 lds_frag(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(base + row * kRowBytes + 16 * (chunk ^ swz(row)));
}

template <int MT, int NT>
__device__ __forceinline__ void read_frags(const uint8_t* As, const uint8_t* Bs, int j, uint4 (&fa)[MT],
                                           uint4 (&fb)[NT], int wm, int wn, int r32, int g) {
#pragma unroll
  for (int i = 0; i < MT; ++i) fa[i] = lds_frag(As, wm * 32 * MT + 32 * i + r32, 4 * g + j);
#pragma unroll
  for (int i = 0; i < NT; ++i) fb[i] = lds_frag(Bs, wn * 32 * NT + 32 * i + r32, 4 * g + j);
}

template <int J, int MT, int NT>
__device__ __forceinline__ void mfma_block(f32x16 (&acc)[MT][NT], const uint4 (&fa)[MT], const uint4 (&fb)[NT],
                                           const uint32_t (&sa)[MT], const uint32_t (&sb)[NT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[i][k] = mfma_fp4<J>(fa[i], fb[k], sa[i], sb[k], acc[i][k]);
}

// Keep the instruction scheduler from moving anything across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// One pipeline step.  Inside the 256-k stage the four 64-k sub-steps are
// software-pipelined: the LDS fragments of sub-step j+1 are requested before
// the MFMAs of sub-step j, so LDS reads overlap matrix-core work even though
// the four waves run in lock-step.  The optional register -> LDS store of the
// next stage and the prefetch of a later stage sit between MFMA groups.
template <int MT, int NT, bool kStore, bool kLoad>
__device__ __forceinline__ void gemm_step(const GemmArgs& p, const uint8_t* cur, uint8_t* next,
                                          StageRegs<MT, NT>& rnext, f32x16 (&acc)[MT][NT], int64_t pf, int64_t m0,
                                          int64_t n0, int tid, int wm, int wn, int r32, int g) {
  using T = Tile<MT, NT>;
  const uint8_t* As = cur;
  const uint8_t* Bs = cur + T::kA;
  const uint8_t* Asc = cur + T::kA + T::kB;
  const uint8_t* Bsc = Asc + T::kAs;
  uint32_t sa[MT], sb[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
    sa[i] = *reinterpret_cast<const uint32_t*>(Asc + (wm * 32 * MT + 32 * i + r32) * 8 + 4 * g);
#pragma unroll
  for (int i = 0; i < NT; ++i)
    sb[i] = *reinterpret_cast<const uint32_t*>(Bsc + (wn * 32 * NT + 32 * i + r32) * 8 + 4 * g);
  uint4 fa0[MT], fb0[NT], fa1[MT], fb1[NT];
  read_frags<MT, NT>(As, Bs, 0, fa0, fb0, wm, wn, r32, g);
  read_frags<MT, NT>(As, Bs, 1, fa1, fb1, wm, wn, r32, g);
  sched_fence();
  mfma_block<0>(acc, fa0, fb0, sa, sb);
  sched_fence();
  if (kStore) rnext.store(next, tid);  // stage s+1: registers -> LDS
  read_frags<MT, NT>(As, Bs, 2, fa0, fb0, wm, wn, r32, g);
  sched_fence();
  mfma_block<1>(acc, fa1, fb1, sa, sb);
  sched_fence();
  if (kLoad) rnext.load(p, m0, n0, pf, tid);  // prefetch a later stage
  read_frags<MT, NT>(As, Bs, 3, fa1, fb1, wm, wn, r32, g);
  sched_fence();
  mfma_block<2>(acc, fa0, fb0, sa, sb);
  sched_fence();
  mfma_block<3>(acc, fa1, fb1, sa, sb);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): stage s+1 written, stage s read
  block_barrier();
}

template <int MT, int NT>
__global__ __launch_bounds__(256) void mxfp4_gemm_lds_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  using T = Tile<MT, NT>;
  using R = StageRegs<MT, NT>;
  static_assert(T::kWaves * T::kEpiWave <= T::kStage, "epilogue fits in one LDS slot");
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[T::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[T::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // XCD-aware tile order: consecutive workgroup ids go round-robin to the 8
  // XCDs, so give XCD x the contiguous tile range [x * per, (x + 1) * per).
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int64_t m0 = (int64_t)tm * T::BM;
  const int64_t n0 = (int64_t)tn * T::BN;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[i][k] = f32x16{};

  const int64_t nstages = p.K / kStageK;
  // Pipeline: stage s is read from LDS slot s % 2 while stage s + 1 moves from
  // registers into the other slot and stage s + 2 (and s + 3) is in flight from
  // memory into registers.  Register set s % 2 carries stages s, s + 2, ...
  // Every load below is unconditional, with its stage index clamped to the last
  // stage: the compiler then sees the same pending loads on every path into
  // the loop and keeps its vmcnt waits exact (a clamped prefetch re-reads an
  // L2-resident stage and is never stored).
  const int64_t last = nstages - 1;
  R r0, r1;
  r0.load(p, m0, n0, 0, tid);
  r1.load(p, m0, n0, 1 < last ? 1 : last, tid);
  r0.store(slot0, tid);
  r0.load(p, m0, n0, 2 < last ? 2 : last, tid);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS writes done
  block_barrier();

  // Steady state: store stage s+1, prefetch stage s+3, compute stage s.
  int64_t s = 0;
  for (; s + 2 < nstages; s += 2) {
    gemm_step<MT, NT, true, true>(p, slot0, slot1, r1, acc, s + 3 < last ? s + 3 : last, m0, n0, tid, wm, wn,
                                  r32, g);
    gemm_step<MT, NT, true, true>(p, slot1, slot0, r0, acc, s + 4 < last ? s + 4 : last, m0, n0, tid, wm, wn,
                                  r32, g);
  }
  // Tail: one or two steps left (s is even).  Each step ends with a barrier, so
  // every wave is done with both slots before slot 0 holds the epilogue.
  if (s + 1 < nstages) {
    gemm_step<MT, NT, true, false>(p, slot0, slot1, r1, acc, 0, m0, n0, tid, wm, wn, r32, g);
    gemm_step<MT, NT, false, false>(p, slot1, slot0, r0, acc, 0, m0, n0, tid, wm, wn, r32, g);
  } else {
    gemm_step<MT, NT, false, false>(p, slot0, slot1, r1, acc, 0, m0, n0, tid, wm, wn, r32, g);
  }

  // Epilogue through LDS: one 32-row band of the wave's tile per pass.
  float* epi = reinterpret_cast<float*>(slot0 + wave * T::kEpiWave);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rs = 8 * (r >> 2) + 4 * g + (r & 3);
        epi[rs * T::kEpiStride + 32 * k + r32] = acc[i][k][r];
      }
    constexpr int kChunks = 32 * 4 * NT;  // 8-float chunks in the band
#pragma unroll
    for (int it = 0; it < kChunks / 64; ++it) {
      const int id = it * 64 + lane;
      const int rs = id / (4 * NT);
      const int cc = id % (4 * NT);
      const float* src = epi + rs * T::kEpiStride + 8 * cc;
      float v[8];
      const float4 lo = reinterpret_cast<const float4*>(src)[0];
      const float4 hi = reinterpret_cast<const float4*>(src)[1];
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      const int64_t row = m0 + wm * 32 * MT + 32 * i + rs;
      const int64_t col = n0 + wn * 32 * NT + 8 * cc;
      if (col < p.N) store_out8(p, row, col, v);
    }
  }
}

// --------------------------------- direct-to-LDS kernel (K = 256 * NST, NST fixed)
//
// Same tile, fragment layout and in-stage software pipeline as above, but the
// operand tiles go global -> LDS with gfx950's 16-byte direct-to-LDS loads:
// no VGPR staging and no ds_write instructions (which measured as the
// kernel's bottleneck).  A ring of three LDS slots keeps stages s+1 and s+2 in
// flight while stage s is consumed.  The stage loop is fully unrolled for a
// compile-time stage count: in straight-line code the compiler can tell the
// slots apart and keeps its wait counts exact, whereas a loop back-edge makes
// it wait for every outstanding direct-to-LDS load before the first LDS read.

typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int MT, int NT>
struct StageDma {
  using T = Tile<MT, NT>;
  // direct-to-LDS instructions per wave per stage; one instruction moves
  // 64 lanes x 16 bytes = 8 rows x 128 bytes of codes, or 64 x 4 bytes =
  // 32 rows x 8 bytes of scales
  static constexpr int kAq = T::BM / 8 / T::kWaves;
  static constexpr int kBq = T::BN / 8 / T::kWaves;
  static constexpr int kAsq = T::BM / 32 / T::kWaves;
  static constexpr int kBsq = T::BN / 32 / T::kWaves;
  static constexpr int kPerStage = kAq + kBq + kAsq + kBsq;
  static_assert(T::BM % (32 * T::kWaves) == 0 && T::BN % (32 * T::kWaves) == 0, "tile split");

  // Part 0: A codes of the first half of the rows, 1: the second half, 2: B
  // codes, 3: both scale blocks; all four in that order make issue().
  __device__ static __forceinline__ void issue(const GemmArgs& p, uint8_t* slot, int64_t m0, int64_t n0,
                                               int64_t s, int wave, int lane) {
    issue_part(p, slot, m0, n0, s, wave, lane, 0);
    issue_part(p, slot, m0, n0, s, wave, lane, 1);
    issue_part(p, slot, m0, n0, s, wave, lane, 2);
    issue_part(p, slot, m0, n0, s, wave, lane, 3);
  }
  __device__ static __forceinline__ void issue_part(const GemmArgs& p, uint8_t* slot, int64_t m0, int64_t n0,
                                                    int64_t s, int wave, int lane, int part) {
    const int64_t qld = p.K >> 1;
    const int64_t sld = p.K >> 5;
    const int64_t kbyte0 = s * kRowBytes;
    const int64_t kb0 = s * 8;
    const int rsub = lane >> 3;
    const int slotpos = lane & 7;
#pragma unroll
    for (int i = 0; i < kAq; ++i) {
      if ((part == 0) != (i < kAq / 2) || part > 1) continue;
      const int q = wave + T::kWaves * i;
      const int row = 8 * q + rsub;
      int64_t gr = m0 + row;
      gr = gr < p.M ? gr : p.M - 1;  // rows past the edge read a valid row, never stored
      // lane lands at slot position `slotpos` of `row`; fetch the chunk that belongs there
      __builtin_amdgcn_global_load_lds(p.xq + gr * qld + kbyte0 + 16 * (slotpos ^ swz(row)),
                                       (lds_void*)(slot + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kBq; ++i) {
      if (part != 2) continue;
      const int q = wave + T::kWaves * i;
      const int row = 8 * q + rsub;
      int64_t gr = n0 + row;
      gr = gr < p.N ? gr : p.N - 1;
      __builtin_amdgcn_global_load_lds(p.wq + gr * qld + kbyte0 + 16 * (slotpos ^ swz(row)),
                                       (lds_void*)(slot + T::kA + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAsq; ++i) {
      if (part != 3) continue;
      const int q = wave + T::kWaves * i;
      int64_t gr = m0 + 32 * q + (lane >> 1);
      gr = gr < p.M ? gr : p.M - 1;
      __builtin_amdgcn_global_load_lds(p.xs + gr * sld + kb0 + 4 * (lane & 1),
                                       (lds_void*)(slot + T::kA + T::kB + q * 256), 4, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kBsq; ++i) {
      if (part != 3) continue;
      const int q = wave + T::kWaves * i;
      int64_t gr = n0 + 32 * q + (lane >> 1);
      gr = gr < p.N ? gr : p.N - 1;
      __builtin_amdgcn_global_load_lds(p.ws + gr * sld + kb0 + 4 * (lane & 1),
                                       (lds_void*)(slot + T::kA + T::kB + T::kAs + q * 256), 4, 0, 0);
    }
  }
};

// Stage s from LDS slot `cur` into the matrix cores, LDS fragments of sub-step
// j+1 requested before the MFMAs of sub-step j, and the direct-to-LDS loads of
// stage s + 2 between the MFMAs.
// load_part(j) issues part j of the stage that is two ahead (or nothing,
// returning false).  The scheduling groups place each of its loads right after
// one MFMA of block j: issued in front of the first MFMA instead, the stage's
// loads held each wave's in-order issue behind the queue of vector loads.
// Bit-identical; alternating A/B in one process: 2048 x 12288 x 4096 -6.8 %,
// 2048 x 4096 x 12288 -7.5 %, 16384 x 4096 x 4096 -1.3 %.
#define UN_MV(J) __builtin_amdgcn_sched_group_barrier(0x008, 1, J); __builtin_amdgcn_sched_group_barrier(0x020, 1, J);
template <int MT, int NT, typename L>
__device__ __forceinline__ void mma_stage(const uint8_t* cur, f32x16 (&acc)[MT][NT], int wm, int wn, int r32,
                                          int g, L&& load_part) {
  using T = Tile<MT, NT>;
  const uint8_t* As = cur;
  const uint8_t* Bs = cur + T::kA;
  const uint8_t* Asc = cur + T::kA + T::kB;
  const uint8_t* Bsc = Asc + T::kAs;
  uint32_t sa[MT], sb[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
    sa[i] = *reinterpret_cast<const uint32_t*>(Asc + (wm * 32 * MT + 32 * i + r32) * 8 + 4 * g);
#pragma unroll
  for (int i = 0; i < NT; ++i)
    sb[i] = *reinterpret_cast<const uint32_t*>(Bsc + (wn * 32 * NT + 32 * i + r32) * 8 + 4 * g);
  uint4 fa0[MT], fb0[NT], fa1[MT], fb1[NT];
  read_frags<MT, NT>(As, Bs, 0, fa0, fb0, wm, wn, r32, g);
  read_frags<MT, NT>(As, Bs, 1, fa1, fb1, wm, wn, r32, g);
  sched_fence();
  mfma_block<0>(acc, fa0, fb0, sa, sb);
  if (load_part(0)) { UN_MV(0) UN_MV(0) UN_MV(0) UN_MV(0) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0); }
  sched_fence();
  read_frags<MT, NT>(As, Bs, 2, fa0, fb0, wm, wn, r32, g);
  sched_fence();
  mfma_block<1>(acc, fa1, fb1, sa, sb);
  if (load_part(1)) { UN_MV(1) UN_MV(1) UN_MV(1) UN_MV(1) __builtin_amdgcn_sched_group_barrier(0x008, 4, 1); }
  sched_fence();
  read_frags<MT, NT>(As, Bs, 3, fa1, fb1, wm, wn, r32, g);
  sched_fence();
  mfma_block<2>(acc, fa0, fb0, sa, sb);
  if (load_part(2)) { UN_MV(2) UN_MV(2) UN_MV(2) UN_MV(2) __builtin_amdgcn_sched_group_barrier(0x008, 4, 2); }
  sched_fence();
  mfma_block<3>(acc, fa1, fb1, sa, sb);
  if (load_part(3)) { UN_MV(3) UN_MV(3) UN_MV(3) __builtin_amdgcn_sched_group_barrier(0x008, 5, 3); }
}
#undef UN_MV

template <int MT, int NT>
__device__ __forceinline__ void epilogue(const GemmArgs& p, uint8_t* buf, const f32x16 (&acc)[MT][NT], int64_t m0,
                                         int64_t n0, int wave, int lane, int wm, int wn, int r32, int g) {
  using T = Tile<MT, NT>;
  float* epi = reinterpret_cast<float*>(buf + wave * T::kEpiWave);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rs = 8 * (r >> 2) + 4 * g + (r & 3);
        epi[rs * T::kEpiStride + 32 * k + r32] = acc[i][k][r];
      }
    constexpr int kChunks = 32 * 4 * NT;  // 8-float chunks in the band
#pragma unroll
    for (int it = 0; it < kChunks / 64; ++it) {
      const int id = it * 64 + lane;
      const int rs = id / (4 * NT);
      const int cc = id % (4 * NT);
      const float* src = epi + rs * T::kEpiStride + 8 * cc;
      float v[8];
      const float4 lo = reinterpret_cast<const float4*>(src)[0];
      const float4 hi = reinterpret_cast<const float4*>(src)[1];
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      const int64_t row = m0 + wm * 32 * MT + 32 * i + rs;
      const int64_t col = n0 + wn * 32 * NT + 8 * cc;
      if (col < p.N) store_out8(p, row, col, v);
    }
  }
}

template <int MT, int NT, int NST>
__global__ __launch_bounds__(256) void mxfp4_gemm_dma_kernel(GemmArgs p, int tiles_m, int tiles_n) {
  using T = Tile<MT, NT>;
  using D = StageDma<MT, NT>;
  static_assert(T::kWaves * T::kEpiWave <= T::kStage, "epilogue fits in one LDS slot");
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[T::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[T::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[T::kStage];
  uint8_t* const slots[3] = {slot0, slot1, slot2};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);  // XCD-aware order
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int64_t m0 = (int64_t)tm * T::BM;
  const int64_t n0 = (int64_t)tn * T::BN;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[i][k] = f32x16{};

  D::issue(p, slot0, m0, n0, 0, wave, lane);
  if (NST > 1) D::issue(p, slot1, m0, n0, 1, wave, lane);
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    if (s + 1 < NST)
      wait_vmcnt<D::kPerStage>();  // this wave's loads of stage s landed; s+1 may fly
    else
      wait_vmcnt<0>();
    block_barrier();  // stage s complete for all waves; all waves are past stage s-1
    sched_fence();
    mma_stage<MT, NT>(slots[s % 3], acc, wm, wn, r32, g, [&](int part) {
      if (s + 2 >= NST) return false;
      D::issue_part(p, slots[(s + 2) % 3], m0, n0, s + 2, wave, lane, part);
      return true;
    });
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();  // every wave is done with the ring before slot 0 holds the epilogue
  epilogue<MT, NT>(p, slot0, acc, m0, n0, wave, lane, wm, wn, r32, g);
}

// ------------------------------------------------- fallback kernel (any K % 32)

struct Frag {
  uint4 codes[4];
  uint32_t scales;
};

__device__ __forceinline__ void load_frag(Frag& f, const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                          int64_t row, int64_t kb_first, int64_t nb) {
  const uint8_t* qr = q + row * (nb * 16);
  const uint8_t* sr = s + row * nb;
  uint32_t sc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t kb = kb_first + j;
    if (kb < nb) {
      f.codes[j] = *reinterpret_cast<const uint4*>(qr + kb * 16);
      sc |= (uint32_t)sr[kb] << (8 * j);
    } else {
      f.codes[j] = make_uint4(0, 0, 0, 0);  // zero codes with unit scale add nothing
      sc |= 127u << (8 * j);
    }
  }
  f.scales = sc;
}

__global__ __launch_bounds__(256) void mxfp4_gemm_direct_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int64_t nb = p.K >> 5;
  const int64_t m_base = (int64_t)blockIdx.y * 128 + 64 * (wave >> 1);
  const int64_t n_base = (int64_t)blockIdx.x * 128 + 64 * (wave & 1);

  int64_t arow[2], brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t m = m_base + 32 * t + r32;
    const int64_t n = n_base + 32 * t + r32;
    arow[t] = m < p.M ? m : p.M - 1;
    brow[t] = n < p.N ? n : p.N - 1;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k) acc[i][k] = f32x16{};

  for (int64_t kb0 = 0; kb0 < nb; kb0 += 8) {
    Frag fa[2], fb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      load_frag(fa[t], p.xq, p.xs, arow[t], kb0 + 4 * g, nb);
      load_frag(fb[t], p.wq, p.ws, brow[t], kb0 + 4 * g, nb);
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        acc[tm][tn] = mfma_fp4<0>(fa[tm].codes[0], fb[tn].codes[0], fa[tm].scales, fb[tn].scales, acc[tm][tn]);
        acc[tm][tn] = mfma_fp4<1>(fa[tm].codes[1], fb[tn].codes[1], fa[tm].scales, fb[tn].scales, acc[tm][tn]);
        acc[tm][tn] = mfma_fp4<2>(fa[tm].codes[2], fb[tn].codes[2], fa[tm].scales, fb[tn].scales, acc[tm][tn]);
        acc[tm][tn] = mfma_fp4<3>(fa[tm].codes[3], fb[tn].codes[3], fa[tm].scales, fb[tn].scales, acc[tm][tn]);
      }
  }
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int64_t col = n_base + 32 * tn + r32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m_base + 32 * tm + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < p.M) {
          const float v = acc[tm][tn][r];
          if (p.out_f32)
            reinterpret_cast<float*>(p.y)[row * p.N + col] = v;
          else
            reinterpret_cast<uint16_t*>(p.y)[row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
}

template <int MT, int NT>
hipError_t launch_lds(const GemmArgs& args, hipStream_t stream) {
  using T = Tile<MT, NT>;
  const int tiles_m = (int)((args.M + T::BM - 1) / T::BM);
  const int tiles_n = (int)((args.N + T::BN - 1) / T::BN);
  hipLaunchKernelGGL((mxfp4_gemm_lds_kernel<MT, NT>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, args,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

template <int MT, int NT, int NST>
hipError_t launch_dma(const GemmArgs& args, hipStream_t stream) {
  using T = Tile<MT, NT>;
  const int tiles_m = (int)((args.M + T::BM - 1) / T::BM);
  const int tiles_n = (int)((args.N + T::BN - 1) / T::BN);
  hipLaunchKernelGGL((mxfp4_gemm_dma_kernel<MT, NT, NST>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, args,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_mxfp4_gemm(const GemmArgs& args, hipStream_t stream) {
  const bool scales_aligned = ((uintptr_t)args.xs % 4 == 0) && ((uintptr_t)args.ws % 4 == 0);
  if (args.K % kStageK == 0 && scales_aligned) {
    switch (args.K / kStageK) {  // stage counts with a fully unrolled direct-to-LDS kernel
      case 1: return launch_dma<4, 2, 1>(args, stream);
      case 2: return launch_dma<4, 2, 2>(args, stream);
      case 3: return launch_dma<4, 2, 3>(args, stream);
      case 4: return launch_dma<4, 2, 4>(args, stream);
      case 8: return launch_dma<4, 2, 8>(args, stream);
      case 16: return launch_dma<4, 2, 16>(args, stream);
      case 48: return launch_dma<4, 2, 48>(args, stream);
      default: break;
    }
    return launch_lds<4, 2>(args, stream);
  }
  dim3 grid((unsigned)((args.N + 127) / 128), (unsigned)((args.M + 127) / 128));
  hipLaunchKernelGGL(mxfp4_gemm_direct_kernel, grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace batq
