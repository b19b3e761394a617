// Fused block transform + block-wise clipping + MXFP4 quantisation (gfx950).
//
// Computes, for every row and 32-channel block i [BATQuant note
// (en.papernotes.org), A Worked Example: transform block by block, clip,
// quantise; Key Designs §1-§3]:
//   y   = x_b (B_i (x) A)                       row-vector convention
//   z   = min(max(y, r_lo * min y), r_hi * max y)
//   e   = floor(log2 max|z|) - 2 (clamped),     codes = RNE_E2M1(z / 2^e)
//
// Design.  The block transform is a dense 32x32 contraction per block, so it
// runs on the matrix cores instead of the vector ALUs, which would otherwise
// bound the kernel (12+ FMAs per element for the Kronecker-factored form
// against a budget of ~18 vector ops per element at 70% of HBM bandwidth, with
// packed FP32 math unavailable).  Each wave owns one block i, builds the
// explicit P_i = kron(B_i, A) once in registers as an exact three-way bf16
// split (hi + mid + lo, ~26 significant bits of the exact fp32xfp32 product),
// and then streams tokens 32 at a time through
//     Y^T[32 ch x 32 tok] = P_i^T[32 x 32] * X^T[32 x 32 tok]
// with v_mfma_f32_32x32x16_bf16: the bf16 activations are the B operand as
// loaded (8 contiguous channels per lane, no conversion), the split parts of
// P_i^T are the A operand, accumulated lo -> mid -> hi in fp32.  Each output
// lane then holds 16 of a token's 32 channels and its partner lane (lane ^ 32)
// the other 16, so the block min/max, clip, scale and E2M1 conversion are
// lane-local plus one cross-half exchange.  E2M1 rounding uses the hardware
// converter v_cvt_scalef32_pk_fp4_f32 (round to nearest even, saturating,
// sign-preserving) on z * 2^-e, which is exact.
//
// The same kernel also produces MXFP8 (E4M3) codes for the W4A8 setting
// [nubint.ai review, Table 2; en.papernotes.org, Loss & Training: E4M3
// elements]: e = floor(log2 max|z|) - 8 (the largest E4M3
// exponent), one byte per element.  Its converter v_cvt_scalef32_pk_fp8_f32
// rounds to nearest even with subnormals but does not saturate (it returns the
// NaN code above 448), so z is clamped to +-448 * 2^e first, which leaves the
// round-to-nearest decision unchanged.
#include "block_quant.h"

namespace batq {

namespace {

constexpr int kBlocksPerWG = 8;  // one 32-channel block per compute wave; 8 blocks = 128 code bytes per row
constexpr int kStorerWaves = 4;  // waves 0-3 also write the staged codes and scales
// The wave that issues the global -> LDS tile loads: the last compute wave, or
// (DL) a ninth wave that does nothing else.
template <bool DL>
constexpr int kLoaderWave = DL ? kBlocksPerWG : kBlocksPerWG - 1;
template <bool DL>
constexpr int kThreads = 64 * (kBlocksPerWG + (DL ? 1 : 0));
// Cache policy of the X loads: non-temporal (bit 1 of the buffer instructions'
// cache-policy field), since every X byte is read once.  Measured: faster for
// the activation and E2M1 cache paths, slower for E4M3 cache writes, which
// keep the default policy.
constexpr int kStreamLoad = 2;
constexpr int kTT = 32;                        // tokens per tile (one MFMA group)
static_assert(kLoaderWave<false> >= kStorerWaves, "the loader issues no stores");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Two 16-byte LDS reads that complete inside the same asm block.  Written
// as asm because the compiler cannot tell these reads from the slots that
// direct-to-LDS loads are still filling, and would otherwise wait for every
// load in flight; the loader's exact wait and the barrier before the reads
// already order them after the tile's own loads.
__device__ __forceinline__ void lds_read2_b128(const uint8_t* p0, const uint8_t* p1, uint4& v0, uint4& v1) {
  const uint32_t a0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p0;
  const uint32_t a1 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p1;
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1)
      : "v"(a0), "v"(a1)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Persistent workgroup: one column of 8 blocks (256 channels) and the token
// tiles ty = y, y + gy, ... (32 tokens each), with
// two workgroups resident per CU.  Every wave w computes block blk0 + w: it
// builds its P_i split once, then per tile runs the MFMA transform, clip,
// scale and codes into one of two LDS staging buffers.  Waves also have a
// second role, chosen so that no wave's memory-counter waits ever cover
// another kind of traffic:
//   loader (wave 7)   keeps kRing - 1 tiles in flight: 16-byte direct-to-LDS
//                     loads, one instruction = two whole 512-byte row segments;
//                     row r keeps its 16-byte chunk c at position c ^ (r & 15),
//                     so the MFMA operand reads (16 consecutive rows, same
//                     chunk) hit 16 different bank groups.  It issues no
//                     stores, so its wait for a tile is an exact count;
//   storers (0-3)     after computing tile i, wave w writes rows 8 w .. 8 w + 7
//                     of tile i - 1's staged codes as 16-byte row-contiguous
//                     chunks (whole 128-byte lines per row) and its scales as
//                     8-byte row pieces.  They never wait for their stores.
// One workgroup barrier per tile, X_i: tile i is in its slot, tile i - 1 is
// staged (and may be stored), tile i - 2's staging has been stored (its
// buffer takes tile i).  With a single staging buffer it took two (measured
// 4-6 % slower).
template <bool F8>
struct TQSmem {
  static constexpr int kXRow = 512;        // bytes per staged bf16 row (256 channels)
  static constexpr int kX = kTT * kXRow;   // one tile slot
  // LDS tile slots (kRing - 1 tiles in flight): E4M3 staging is twice as
  // large, and two workgroups per CU must still fit (4 x 16 + 2 x 8.5 KB would not).
  static constexpr int kRing = F8 ? 3 : 4;
  // staged code row: 128 (E2M1) or 256 (E4M3) bytes + 16 pad, conflict-free writes
  static constexpr int kQRow = F8 ? 272 : 144;
};

// PER_ROW: one ratio pair per (row, block), read per tile (the weight side);
// otherwise one pair per block, read once (activations), which keeps every
// memory wait out of the activations' tile loop.  F8: MXFP8 (E4M3) codes, one
// byte per element (the W4A8 setting); otherwise MXFP4 (E2M1), two per byte.
// STREAM: non-temporal code and scale stores, for outputs that the next
// kernel does not read (cache rows written through the slot mapping).
// Tile walk.  Default (t1 == 0): workgroup x gy + y takes column group x and
// tile rows y, y + gy, ...  Skewed (t1 > 0; the grid is exactly two
// workgroups per CU): workgroups are dispatched in id order, one per CU
// first, and the first one on a CU runs ahead of the second (measured: it
// ends ~6 us earlier on 16-tile workgroups).  So the first half of the ids
// takes t1 consecutive tile rows each and the second half t2 = 2 t - t1,
// with gy / 2 workgroups per column in each half; ids that share a tile row
// stay congruent mod 8 (same XCD) as in the default walk.
// The lane's factor entries, as load_p_factors gives them, with fewer loads
// when a >= 8: each run of 8 consecutive k = 16 ks + 8 h + t then lies in one
// row of B_i and in 8 consecutive rows of A, and for a <= 16 the lane's two
// runs read the same rows of A.  At a = 8 that is 10 loads instead of 32.
// These are the workgroup's first loads after the loader's tile requests, so
// fewer of them wait less behind that traffic.
__device__ __forceinline__ PFactors load_factor_runs(const float* __restrict__ A, const float* __restrict__ Bi, int la,
                                                     int j, int h) {
  if (la < 3) return load_p_factors(A, Bi, la, j, h);
  const int a = 1 << la, amask = a - 1, bdim = 32 >> la;
  PFactors f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const float bv = Bi[((16 * ks + 8 * h) >> la) * bdim + (j >> la)];
#pragma unroll
    for (int t = 0; t < 8; ++t) f.bv[ks][t] = bv;
  }
  const int r0 = (8 * h) & amask, ja = j & amask;
#pragma unroll
  for (int t = 0; t < 8; ++t) f.av[0][t] = A[(r0 + t) * a + ja];
  if (la <= 4) {
#pragma unroll
    for (int t = 0; t < 8; ++t) f.av[1][t] = f.av[0][t];
  } else {
    const int r1 = (16 + 8 * h) & amask;
#pragma unroll
    for (int t = 0; t < 8; ++t) f.av[1][t] = A[(r1 + t) * a + ja];
  }
  return f;
}

template <bool PER_ROW, bool F8, bool STREAM, bool DL>
__device__ __forceinline__ void transform_quant_tiles(const TransformQuantArgs& p, int64_t gy, int t1) {
  using T = TQSmem<F8>;
  constexpr int kXPolicy = (F8 && STREAM) ? 0 : kStreamLoad;
  constexpr int kRing = T::kRing;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kRing * T::kX];
  __shared__ __attribute__((aligned(16))) uint8_t qs[2 * kTT * T::kQRow];  // two staging buffers
  __shared__ __attribute__((aligned(16))) uint8_t ss[2 * kTT * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nb = p.K >> 5;
  // Workgroup id = x gy + y: with gy a multiple of 8, every column group x of
  // tile row y lands on the same XCD (ids go to the XCDs in turn), so the
  // 8-byte scale pieces of a row's 128-byte scale line merge in one L2.
  const int64_t tiles = (p.rows + kTT - 1) / kTT;
  int64_t blk0, ty0, tstep, ntile;  // uniform per workgroup
  if (t1 == 0) {
    blk0 = ((int64_t)blockIdx.x / gy) * kBlocksPerWG;
    ty0 = (int64_t)blockIdx.x % gy;
    tstep = gy;
    ntile = ty0 < tiles ? (tiles - ty0 + tstep - 1) / tstep : 0;
  } else {
    const int64_t pairs = gy / 2;                    // workgroups per column in each half
    const int64_t half = (int64_t)gridDim.x / 2;
    const int64_t set = (int64_t)blockIdx.x / half;  // 0: dispatched first
    const int64_t r = (int64_t)blockIdx.x % half;
    const int64_t k = r % pairs;
    const int64_t t2 = 2 * (tiles / gy) - t1;
    blk0 = (r / pairs) * kBlocksPerWG;
    ty0 = set == 0 ? k * t1 : pairs * t1 + k * t2;
    tstep = 1;
    ntile = set == 0 ? t1 : t2;
  }
  const int64_t nblk = (nb - blk0) < kBlocksPerWG ? (nb - blk0) : kBlocksPerWG;  // valid blocks here

  // ---------------------------------------------------------- compute waves
  const int64_t blk = blk0 + wave;
  const bool blk_ok = blk < nb && wave < kBlocksPerWG;  // other waves only keep the barriers
  const int j = lane & 31;  // output channel (A-operand row) / token slot (B column)
  const int h = lane >> 5;  // which 8-channel half of each 16-channel k step

  const bool loader = wave == kLoaderWave<DL>;
  // Loader: tile i (< ntile) -> its slot, kTT / 2 load instructions per tile.
  // Addressing: per-lane byte offsets within a 16-row half tile, against a
  // buffer descriptor based at that half's first row whose size ends at the
  // last byte of X.  The whole row offset is in the vector offset, which the
  // hardware range check covers, so rows past the end read zeros (never
  // stored) without touching memory.  Instruction q covers rows 2q and
  // 2q + 1: lane l fetches row 2q + l / 32, logical 16-byte chunk
  // c = (l % 32) ^ (row % 16) (chunks past K read a valid column, unused).
  // The swizzle repeats every 8 instructions, so the same 8 offsets serve
  // both halves, rows 16..31 through the second descriptor.
  const uint32_t ld2 = (uint32_t)(p.ldx * 2);  // row stride in bytes
  uint32_t voff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 2 * q + (lane >> 5);
    const int c = (lane & 31) ^ (row & 15);
    const int64_t col = blk0 * 32 + 8 * c;
    voff[q] = (uint32_t)row * ld2 + (col < p.K ? (uint32_t)(col * 2) : 0u);
  }
  const uint8_t* const xb = reinterpret_cast<const uint8_t*>(p.x);
  auto load_tile = [&](int64_t i, int slot) {
    const int64_t tok0 = (ty0 + i * tstep) * kTT;
    uint8_t* dst = xs + slot * T::kX;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t row0 = tok0 + 16 * half;
      // bytes from the half tile's first row to the end of X (none: every load reads zeros)
      const int64_t left = row0 < p.rows ? (p.rows - row0) * (int64_t)ld2 : 0;
      const int nrec = left < 0x7FFFFFFF ? (int)left : 0x7FFFFFFF;
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(xb + row0 * (int64_t)ld2), (short)0, nrec, 0x00020000);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (8 * half + q) * 1024), 16, (int)voff[q],
                                                 0, 0, kXPolicy);
    }
  };
  // The first tiles are requested before anything else, so that their latency
  // overlaps the factor and ratio loads below (loads issued after them only
  // make the loader's later waits stricter).
  if (loader) {
    for (int i = 0; i < kRing - 1; ++i)
      if (i < ntile) load_tile(i, i);
  }

  // P_i^T as MFMA A operand, exact three-way bf16 split (not needed by a
  // loader that computes no block).
  PSplit ps{};
  if (!(DL && loader))
    ps = split_p(load_factor_runs(p.A, p.B + (blk_ok ? blk : 0) * (32 >> p.a_log2) * (32 >> p.a_log2), p.a_log2, j, h));
  // Ratios shared by every token (activations) are read once here.
  const bool clip = p.r_hi != nullptr;
  const bool per_row = PER_ROW && clip;
  float rh_blk = 1.0f, rl_blk = 1.0f;
  if (clip && !per_row && blk_ok) {
    rh_blk = p.r_hi[blk];
    rl_blk = p.r_lo[blk];
  }

  static_assert(kRing == 3 || kRing == 4, "the loader's wait distinguishes up to 2 younger tiles");
  const int64_t qld = F8 ? p.K : (p.K >> 1);

  // Output row of token tok: tok itself, or its cache slot (a slot outside
  // [0, out_rows) is skipped).
  auto out_row = [&](int64_t tok) -> int64_t {
    if (p.slot == nullptr) return tok;
    const int64_t r = p.slot[tok];
    return r >= 0 && r < p.out_rows ? r : -1;
  };
  // Storer wave w: rows 8 w .. 8 w + 7 of tile ti's codes and scales from
  // staging buffer sb; 16 (E2M1) or 32 (E4M3) code bytes per block and row.
  auto store_rows = [&](int64_t ti, int sb) {
    constexpr int kChunks = F8 ? 16 : 8;  // 16-byte chunks per staged row
    const int64_t tok0 = (ty0 + ti * tstep) * kTT;
    const uint8_t* qsb = qs + sb * kTT * T::kQRow;
#pragma unroll
    for (int k = 0; k < kChunks / 8; ++k) {
      const int id = lane + 64 * k;
      const int row = 8 * wave + id / kChunks;
      const int c = id % kChunks;
      const int64_t tok = tok0 + row;
      if (tok < p.rows && c / (kChunks / 8) < nblk) {
        const int64_t orow = out_row(tok);
        if (orow >= 0) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(qsb + row * T::kQRow + 16 * c);
          u32x4* dst = reinterpret_cast<u32x4*>(p.q + orow * qld + blk0 * (2 * kChunks) + 16 * c);
          if constexpr (STREAM) __builtin_nontemporal_store(v, dst);
          else *dst = v;
        }
      }
    }
    if (lane < 8) {
      const int row = 8 * wave + lane;
      const int64_t tok = tok0 + row;
      const int64_t orow = tok < p.rows ? out_row(tok) : -1;
      if (orow >= 0) {
        uint8_t* dst = p.s + orow * nb + blk0;
        const uint8_t* src = ss + sb * kTT * 8 + row * 8;
        if (nblk == 8 && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
          const unsigned long long v = *reinterpret_cast<const unsigned long long*>(src);
          if constexpr (STREAM) __builtin_nontemporal_store(v, reinterpret_cast<unsigned long long*>(dst));
          else *reinterpret_cast<unsigned long long*>(dst) = v;
        } else {
          for (int c = 0; c < nblk; ++c) dst[c] = src[c];
        }
      }
    }
  };

  for (int64_t i = 0; i < ntile; ++i) {
    if (loader) {
      // tile i has landed once at most the younger tiles' loads are pending
      const int64_t younger = ntile - 1 - i;
      if (younger >= 2 && kRing == 4) {
        wait_vmcnt<2 * (kTT / 2)>();
      } else if (younger >= 1) {
        wait_vmcnt<kTT / 2>();
      } else {
        wait_vmcnt<0>();
      }
    }
    block_barrier();  // X_i
    if (loader && i + kRing - 1 < ntile) load_tile(i + kRing - 1, (int)((i + kRing - 1) % kRing));
    const int sb = (int)(i & 1);
    if (blk_ok) {
      const int64_t tok0 = (ty0 + i * tstep) * kTT;
      const uint8_t* xt = xs + (int)(i % kRing) * T::kX;
      const int row = j;
      const uint8_t* xr = xt + row * T::kXRow;
      uint4 x0, x1;
      lds_read2_b128(xr + 16 * ((4 * wave + h) ^ (row & 15)), xr + 16 * ((4 * wave + 2 + h) ^ (row & 15)), x0, x1);
      const f32x16 acc = transform_block(ps, x0, x1);
      // acc[r] = y[token tok0 + row][channel 8 (r/4) + 4 h + r%4 of block blk]
      float rh = rh_blk, rl = rl_blk;
      if (per_row) {
        int64_t tok = tok0 + row;
        tok = tok < p.rows ? tok : p.rows - 1;
        const int64_t ri = tok * p.r_ld + blk;
        rh = p.r_hi[ri];
        rl = p.r_lo[ri];
      }
      uint8_t* qsb = qs + sb * kTT * T::kQRow;
      int sbyte;
      if constexpr (F8) {
        *reinterpret_cast<uint4*>(qsb + row * T::kQRow + 32 * wave + 16 * h) = quant_block_e4m3(acc, rh, rl, h, sbyte);
      } else {
        *reinterpret_cast<uint2*>(qsb + row * T::kQRow + 16 * wave + 8 * h) = quant_block_e2m1(acc, rh, rl, h, sbyte);
      }
      if (h == 0) ss[sb * kTT * 8 + row * 8 + wave] = (uint8_t)sbyte;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    if (wave < kStorerWaves && i > 0) store_rows(i - 1, sb ^ 1);
  }
  if (ntile > 0) {
    block_barrier();  // the last tile is staged
    if (wave < kStorerWaves) store_rows(ntile - 1, (int)((ntile - 1) & 1));
  }
}

// Two instances per mode: DL = false, the loader is also a compute wave and
// two workgroups share a CU (the skewed walk); DL = true, a ninth wave only
// loads, one workgroup per CU (every other grid).
template <bool PER_ROW, bool F8>
__global__ __launch_bounds__(kThreads<false>) __attribute__((amdgpu_waves_per_eu(4))) void transform_quant_kernel(
    TransformQuantArgs p, int64_t gy, int t1) {
  transform_quant_tiles<PER_ROW, F8, false, false>(p, gy, t1);
}
template <bool PER_ROW, bool F8>
__global__ __launch_bounds__(kThreads<true>) __attribute__((amdgpu_waves_per_eu(5))) void transform_quant_dl_kernel(
    TransformQuantArgs p, int64_t gy, int t1) {
  transform_quant_tiles<PER_ROW, F8, false, true>(p, gy, t1);
}

// Cache rows are not read by the next kernel, so they are streamed past L2.
template <bool F8>
__global__ __launch_bounds__(kThreads<false>) __attribute__((amdgpu_waves_per_eu(4))) void kv_cache_quant_kernel(
    TransformQuantArgs p, int64_t gy, int t1) {
  transform_quant_tiles<false, F8, true, false>(p, gy, t1);
}
template <bool F8>
__global__ __launch_bounds__(kThreads<true>) __attribute__((amdgpu_waves_per_eu(5))) void kv_cache_quant_dl_kernel(
    TransformQuantArgs p, int64_t gy, int t1) {
  transform_quant_tiles<false, F8, true, true>(p, gy, t1);
}

// Grid height for a target of about `target` workgroups.  With fewer than 4
// tiles each a workgroup's ring never fills (2048 x 4096: 10.1 us with 256
// workgroups of 4 tiles, 11.1 us with 512 of 2), so fewer, longer workgroups
// are used as long as there remains one per CU (smaller grids measured
// slower).  gy is kept a multiple of 8 where it can be (see the workgroup
// order in the kernel).
int64_t grid_rows(int64_t gx, int64_t tiles, int64_t target) {
  int64_t gy = target / gx;
  if (gy >= 8) gy -= gy % 8;
  if (gy < 1) gy = 1;
  int64_t cap = tiles / 4;
  if (cap >= 8) cap -= cap % 8;
  const int64_t one_per_cu = (256 + gx - 1) / gx;
  if (cap < one_per_cu) cap = one_per_cu;
  if (gy > cap) gy = cap;
  if (gy > tiles) gy = tiles;
  return gy;
}

template <bool DL>
void launch_instance(const TransformQuantArgs& args, dim3 grid, int64_t gy, int t1, hipStream_t stream) {
  const bool per_row = args.r_hi != nullptr && args.r_ld != 0;
  const dim3 block(kThreads<DL>);
  if (args.slot != nullptr && !per_row) {
    if (args.fp8)
      hipLaunchKernelGGL((DL ? kv_cache_quant_dl_kernel<true> : kv_cache_quant_kernel<true>), grid, block, 0, stream,
                         args, gy, t1);
    else
      hipLaunchKernelGGL((DL ? kv_cache_quant_dl_kernel<false> : kv_cache_quant_kernel<false>), grid, block, 0, stream,
                         args, gy, t1);
  } else if (args.fp8) {
    if (per_row)
      hipLaunchKernelGGL((DL ? transform_quant_dl_kernel<true, true> : transform_quant_kernel<true, true>), grid, block,
                         0, stream, args, gy, t1);
    else
      hipLaunchKernelGGL((DL ? transform_quant_dl_kernel<false, true> : transform_quant_kernel<false, true>), grid,
                         block, 0, stream, args, gy, t1);
  } else {
    if (per_row)
      hipLaunchKernelGGL((DL ? transform_quant_dl_kernel<true, false> : transform_quant_kernel<true, false>), grid,
                         block, 0, stream, args, gy, t1);
    else
      hipLaunchKernelGGL((DL ? transform_quant_dl_kernel<false, false> : transform_quant_kernel<false, false>), grid,
                         block, 0, stream, args, gy, t1);
  }
}


// Two workgroups fit per CU (70 KB of LDS each).  Where a grid of two per CU
// gives every workgroup 16 or more tiles of equal walks, it runs with the
// skewed walk (see transform_quant_tiles): 17 tiles against 15 at 16 per
// workgroup, 4.8 % less time on 16384 x 4096 (alternating A/B).
bool skewed_walk(int64_t gx, int64_t gy, int64_t tiles) {
  return gx * gy == 512 && gy % 16 == 0 && tiles % gy == 0 && tiles / gy >= 16;
}

}  // namespace

bool transform_uses_one_per_cu(int64_t rows, int64_t K) {
  const int64_t gx = ((K >> 5) + kBlocksPerWG - 1) / kBlocksPerWG;
  const int64_t tiles = (rows + kTT - 1) / kTT;
  return gx * grid_rows(gx, tiles, 512) < 512;
}

hipError_t launch_transform_quant(const TransformQuantArgs& args, hipStream_t stream) {
  const int64_t nb = args.K >> 5;
  const int64_t gx = (nb + kBlocksPerWG - 1) / kBlocksPerWG;
  const int64_t tiles = (args.rows + kTT - 1) / kTT;
  const int64_t gy2 = grid_rows(gx, tiles, 512);
  if (gx * gy2 >= 512) {
    const int t1 = skewed_walk(gx, gy2, tiles) ? (int)(tiles / gy2 + tiles / gy2 / 16) : 0;
    launch_instance<false>(args, dim3((unsigned)(gx * gy2)), gy2, t1, stream);
    return hipGetLastError();
  }
  // Grids of fewer than two workgroups per CU: one workgroup per CU with a
  // dedicated loader wave, so that no compute wave waits behind a queue of
  // tile loads (with one workgroup per CU nothing else covers that wait).
  // Same codes bit for bit; alternating A/B in one process: 2048 x 4096
  // 9.1 -> 7.8 us (E4M3 9.9 -> 8.9 us), 2048 x 12288 17.7 -> 16.3 us.  Where
  // two workgroups per CU fill the grid it was equal or slower (16384 x 4096
  // equal, E4M3 5 % slower; 16384 x 1024 KV-cache writes 9-15 % slower).
  const int64_t gy1 = grid_rows(gx, tiles, 256);
  launch_instance<true>(args, dim3((unsigned)(gx * gy1)), gy1, 0, stream);
  return hipGetLastError();
}

}  // namespace batq
