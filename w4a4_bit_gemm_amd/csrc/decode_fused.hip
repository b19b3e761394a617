// Fused decode step: block transform + clip + MXFP4 quantisation of a small
// activation batch (M <= 32 tokens) inside the W4A4 GEMM on packed weights
// [BATQuant note (en.papernotes.org), Key Designs §1-§4: Y = Q(XP) Q(P^-1 W^T);
// A Worked Example: transform block by block, clip, quantise, multiply].
//
// At decode sizes a separate transform launch is pure latency, and a GEMM
// tiled over M cannot keep enough weight bytes in flight.  So one launch
// splits the work over (128-column chunk c, K split sp of up to kSplitStages
// 256-k stages), one workgroup of 8 waves each:
//   1. wave w requests the activation-side inputs of block w of each stage of
//      the split (factor entries, the tokens' channels, ratios), then its
//      weight record: 32-column group w % 4 of stage w / 4.  A wave's loads
//      complete in issue order, so the transform waits only for the
//      activation side while the weight bytes stream in behind it;
//   2. wave w transforms and quantises its blocks for all tokens with the
//      same per-block arithmetic as the transform kernel (block_quant.h): the
//      codes are identical bit for bit.  They are staged in LDS in the MFMA
//      operand order;
//   3. wave w multiplies its stage's codes with its weight record on the
//      block-scaled MFMA; the two waves of a column group add their
//      accumulators in stage order through LDS;
//   4. with one split the result is Y.  Otherwise each workgroup writes its
//      fp32 partial tile with device-scope stores (they go to the coherence
//      point, past this XCD's L2), waits until they are acknowledged, and
//      counts itself on its chunk's counter with one device-scope atomic.
//      The workgroup that arrives last reads the chunk's partials with
//      device-scope loads, adds them in split order and writes Y, then
//      returns the counter to zero.  No workgroup ever waits for another;
//      no cache-wide write-back or invalidation is needed; the sum is
//      deterministic.
#include <mutex>

#include "block_quant.h"

namespace batq {

namespace {

// Scratch of the no-allocation entry point (batq_w4a4_decode_noalloc): the
// fp32 partial tiles go to this device array instead of a caller workspace.
// Each GPU holds its own copy until the process ends.  On the host the name is
// only a stand-in, never an address: host code uses the pointer that
// hipGetSymbolAddress returns for the current device (decode_scratch below).
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

constexpr int kQRow = 144;        // staged code row: 8 blocks x 16 bytes + 16 pad (conflict-free reads)
constexpr int kSplitStages = 2;   // 256-k stages per K split
constexpr int kChunkCols = 128;   // columns per workgroup: four 32-column groups
constexpr int kDecWaves = 8;      // one block of each stage per wave; one (group, stage) product per wave
constexpr int kGroups = kChunkCols / 32;
static_assert(kGroups * kSplitStages == kDecWaves, "one (column group, stage) product per wave");

template <int J>
__device__ __forceinline__ f32x16 mfma_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x16 acc) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, J, (int)sa, J, (int)sb);
}
__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
// Weight records are read once per step: non-temporal loads keep them from
// displacing the partial tiles that the reduction reads next.
__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld4_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Factor entries behind lane (j, h)'s part of P_i^T for a compile-time shared
// size 2^LA: P_i[k][j] = Bi[k >> LA][j >> LA] * A[k % a][j % a]; entries that
// coincide are loaded once (10 loads at a = 8 instead of 32).
template <int LA>
__device__ __forceinline__ PFactors load_p_factors_la(const float* __restrict__ A, const float* __restrict__ Bi,
                                                      int j, int h) {
  constexpr int a = 1 << LA;
  constexpr int bdim = 32 >> LA;
  PFactors f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int k = 16 * ks + 8 * h + t;
      f.bv[ks][t] = Bi[(k >> LA) * bdim + (j >> LA)];
      f.av[ks][t] = A[(k & (a - 1)) * a + (j & (a - 1))];
    }
  return f;
}

// Inputs of one activation block for the wave's 32 token slots: factor
// entries, the lane's 16 channels of token j (zero for j >= M), the ratios.
struct ActIn {
  PFactors f;
  uint4 x0, x1;
  float rh, rl;
};
// Every load is unconditional (rows past M read row M - 1 and are zeroed
// after), so that no branch separates the loads: the compiler's wait for
// them then counts exactly the loads issued later, the weights' included.
template <int LA>
__device__ __forceinline__ ActIn load_act(const DecodeArgs& p, int64_t blk, int j, int h) {
  constexpr int bdim = 32 >> LA;
  ActIn in;
  in.f = load_p_factors_la<LA>(p.A, p.B + blk * bdim * bdim, j, h);
  const int64_t row = j < p.M ? j : p.M - 1;
  const uint16_t* xr = p.x + row * p.ldx + blk * 32 + 8 * h;
  in.x0 = *reinterpret_cast<const uint4*>(xr);
  in.x1 = *reinterpret_cast<const uint4*>(xr + 16);
  in.rh = p.r_hi ? p.r_hi[blk] : 1.0f;
  in.rl = p.r_lo ? p.r_lo[blk] : 1.0f;
  return in;
}
__device__ __forceinline__ uint4 zero_unless(bool keep, uint4 v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// Output element of a 32-row x 32-column MFMA tile: lane (r32, g), register r
// holds row 8 (r / 4) + 4 g + r % 4 of column r32.
__device__ __forceinline__ int tile_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Bytes of the per-chunk arrival counters at the start of the workspace: a
// fixed region, so that calls of any shape find their counters where earlier
// calls left them at zero (never under an earlier call's partials).
__host__ __device__ constexpr int64_t counter_bytes(int64_t) { return kDecodeCounterBytes; }

// The arguments the first loads depend on come first, as scalars (no
// aggregate): they are preloaded into SGPRs at wave launch, so that the
// activation-side loads go out without waiting for a kernel-argument load
// (0.2 us of a ~8 us step).  shape = M | nsplit << 6 | nchunk << 19.
template <int LA>
__global__ __launch_bounds__(64 * kDecWaves) void decode_fused_kernel(const uint16_t* __restrict__ x,
                                                                       const float* __restrict__ A,
                                                                       const float* __restrict__ B, const float* r_hi,
                                                                       const float* r_lo, int64_t ldx, uint32_t shape,
                                                                       int K, DecodeArgs p) {
  const int nchunk = (int)(shape >> 19);
  const int nsplit = (int)((shape >> 6) & 0x1FFF);
  p.x = x;
  p.A = A;
  p.B = B;
  p.r_hi = r_hi;
  p.r_lo = r_lo;
  p.ldx = ldx;
  p.M = (int64_t)(shape & 63);
  p.K = K;
  __shared__ __attribute__((aligned(16))) uint8_t qs[kSplitStages][32 * kQRow];
  __shared__ __attribute__((aligned(16))) uint8_t ss[kSplitStages][32 * 8];
  __shared__ __attribute__((aligned(16))) float red[kDecWaves - kGroups][16 * 64];
  __shared__ int last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x % nchunk;
  const int sp = blockIdx.x / nchunk;
  const int64_t nst = p.K / 256;
  const int64_t s0 = (int64_t)sp * kSplitStages;
  const int nstage = (int)(nst - s0 < kSplitStages ? nst - s0 : kSplitStages);  // stages of this split
  const int j = lane & 31;
  const int h = lane >> 5;

  // 1. activation side of block `wave` of every stage, then the weights.
  ActIn in[kSplitStages];
#pragma unroll
  for (int t = 0; t < kSplitStages; ++t) {  // a stage past the split's end reloads its last one (unused)
    const int64_t blk = (s0 + (t < nstage ? t : nstage - 1)) * 8 + wave;
    in[t] = load_act<LA>(p, blk, j, h);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int gsel = wave % kGroups;  // 32-column group within the chunk
  const int tsel = wave / kGroups;  // stage of the split whose product this wave forms
  const int64_t n32_max = (p.N + 31) / 32;
  const int64_t gq = (int64_t)c * kGroups + gsel;
  const int64_t g32 = gq < n32_max ? gq : n32_max - 1;  // a clamped group is computed, never stored
  uint4 b[4];
  {
    const int tl = tsel < nstage ? tsel : nstage - 1;  // past the split's end: a valid record, unused
    const uint8_t* r = p.wp + (g32 * nst + s0 + tl) * kPackGroupBytes + 16 * lane;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) b[jj] = ld16_stream(r + 1024 * jj);
  }
  const uint32_t bsc = ld4_stream(p.wp + (g32 * nst + s0 + (tsel < nstage ? tsel : nstage - 1)) * kPackGroupBytes +
                                  4096 + 4 * lane);
  __builtin_amdgcn_sched_barrier(0);

  // 2. transform and quantise; codes staged in LDS in the MFMA operand order.
#pragma unroll
  for (int t = 0; t < kSplitStages; ++t) {
    if (t >= nstage) break;
    const int64_t blk = (s0 + t) * 8 + wave;
    const PSplit ps = split_p(in[t].f);
    const f32x16 acc = transform_block(ps, zero_unless(j < p.M, in[t].x0), zero_unless(j < p.M, in[t].x1));
    int sbyte;
    const uint2 code = quant_block_e2m1(acc, in[t].rh, in[t].rl, h, sbyte);
    *reinterpret_cast<uint2*>(&qs[t][j * kQRow + 16 * wave + 8 * h]) = code;
    if (h == 0) ss[t][j * 8 + wave] = (uint8_t)sbyte;
    if (p.xq != nullptr && c == 0 && j < p.M) {  // optional copy of the quantised activations
      *reinterpret_cast<uint2*>(p.xq + (int64_t)j * (p.K >> 1) + blk * 16 + 8 * h) = code;
      if (h == 0) p.xs[(int64_t)j * (p.K >> 5) + blk] = (uint8_t)sbyte;
    }
  }
  __syncthreads();

  // 3. MMA of stage tsel against column group gsel: lane (r32, g) of sub-step
  // jj carries block 4 g + jj of token r32 (the packed record holds the
  // matching blocks of its rows).
  const int r32 = lane & 31;
  const int g = lane >> 5;
  f32x16 acc = {};
  if (tsel < nstage) {
    const uint8_t* qrow = &qs[tsel][r32 * kQRow + 64 * g];
    const uint32_t sa = ld4(&ss[tsel][r32 * 8 + 4 * g]);
    acc = mfma_fp4<0>(ld16(qrow), b[0], sa, bsc, acc);
    acc = mfma_fp4<1>(ld16(qrow + 16), b[1], sa, bsc, acc);
    acc = mfma_fp4<2>(ld16(qrow + 32), b[2], sa, bsc, acc);
    acc = mfma_fp4<3>(ld16(qrow + 48), b[3], sa, bsc, acc);
  }
  // The waves of stage 1 hand their accumulators to the wave of stage 0 of
  // their column group, which adds them in stage order.
  if (wave >= kGroups) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave - kGroups][r * 64 + lane] = acc[r];
  }
  __syncthreads();
  const int64_t M = p.M;
  const int64_t col = (int64_t)c * kChunkCols + 32 * gsel + r32;
  if (wave < kGroups) {
    if (nstage > 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += red[wave][r * 64 + lane];
    }
    if (nsplit == 1) {  // 4. the whole K: this tile is Y
      if (col < p.N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = tile_row(r, g);
          if (row < M) {
            if (p.out_f32)
              reinterpret_cast<float*>(p.y)[row * p.N + col] = acc[r];
            else
              reinterpret_cast<uint16_t*>(p.y)[row * p.N + col] = (uint16_t)f32_to_bf16_rne(acc[r]);
          }
        }
      }
    } else {  // 4. the split's partial tile [M][kChunkCols], past this XCD's L2
      float* part = p.part + counter_bytes(nchunk) / 4 + ((int64_t)c * nsplit + sp) * M * kChunkCols;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tile_row(r, g);
        if (row < M)
          __hip_atomic_store(part + row * kChunkCols + 32 * gsel + r32, acc[r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (nsplit == 1) return;
  // Every store of this workgroup is acknowledged before it counts itself.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* cnt = reinterpret_cast<unsigned*>(p.part) + c;
  if (tid == 0) {
    const unsigned arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = arrived == (unsigned)(nsplit - 1);
  }
  __syncthreads();
  if (!last) return;
  // The last workgroup of chunk c: Y = the splits' partials added in split
  // order, one (row, 4-column quad) per thread per pass.  The partials are
  // read with device-scope buffer loads (cache-policy bit sc1: never served
  // from a stale line of this XCD's L2), all of a thread's splits in flight
  // at once.
  const float* pc = p.part + counter_bytes(nchunk) / 4 + (int64_t)c * nsplit * M * kChunkCols;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)pc, (short)0, (int)(nsplit * M * kChunkCols * 4), 0x00020000);
  constexpr int kQuads = kChunkCols / 4;
  constexpr int kSc1 = 1 << 4;  // buffer cache-policy bit: device scope
  constexpr int kBatch = 8;
  for (int64_t item = tid; item < M * kQuads; item += 64 * kDecWaves) {
    const int64_t row = item / kQuads;
    const int q = (int)(item % kQuads);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int s0b = 0; s0b < nsplit; s0b += kBatch) {
      f32x4 v[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int sidx = s0b + t < nsplit ? s0b + t : nsplit - 1;  // in range; the extra ones are not added
        v[t] = __builtin_amdgcn_raw_buffer_load_b128(prs, (int)((((int64_t)sidx * M + row) * kChunkCols + 4 * q) * 4),
                                                     0, kSc1);
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t)
        if (s0b + t < nsplit) sum += v[t];
    }
    const int64_t col0 = (int64_t)c * kChunkCols + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t cc = col0 + e;
      if (cc >= p.N) break;
      if (p.out_f32)
        reinterpret_cast<float*>(p.y)[row * p.N + cc] = sum[e];
      else
        reinterpret_cast<uint16_t*>(p.y)[row * p.N + cc] = (uint16_t)f32_to_bf16_rne(sum[e]);
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
}

template <int LA>
hipError_t launch_t(const DecodeArgs& a, int nchunk, int nsplit, hipStream_t stream) {
  const uint32_t shape = (uint32_t)a.M | ((uint32_t)nsplit << 6) | ((uint32_t)nchunk << 19);
  hipLaunchKernelGGL((decode_fused_kernel<LA>), dim3(nchunk * nsplit), dim3(64 * kDecWaves), 0, stream, a.x, a.A, a.B,
                     a.r_hi, a.r_lo, a.ldx, shape, (int)a.K, a);
  return hipGetLastError();
}

}  // namespace

int64_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t nchunk = (N + kChunkCols - 1) / kChunkCols, nst = K / 256;
  const int64_t nsplit = (nst + kSplitStages - 1) / kSplitStages;
  return nsplit > 1 ? counter_bytes(nchunk) + nchunk * nsplit * M * kChunkCols * 4 : 0;
}

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_fused(const DecodeArgs& args, hipStream_t stream) {
  const int64_t nchunk = (args.N + kChunkCols - 1) / kChunkCols, nst = args.K / 256;
  const int nsplit = (int)((nst + kSplitStages - 1) / kSplitStages);
  switch (args.a_log2) {
    case 0: return launch_t<0>(args, (int)nchunk, nsplit, stream);
    case 1: return launch_t<1>(args, (int)nchunk, nsplit, stream);
    case 2: return launch_t<2>(args, (int)nchunk, nsplit, stream);
    case 3: return launch_t<3>(args, (int)nchunk, nsplit, stream);
    case 4: return launch_t<4>(args, (int)nchunk, nsplit, stream);
    default: return launch_t<5>(args, (int)nchunk, nsplit, stream);
  }
}

}  // namespace batq
