// Fused decode step: block transform + clip + MXFP4 quantisation of a small
// activation batch (M <= 32 tokens) inside the W4A4 GEMM on packed weights
// [BATQuant note (en.papernotes.org), Key Designs §1-§4: Y = Q(XP) Q(P^-1 W^T);
// A Worked Example: transform block by block, clip, quantise, multiply].
//
// At decode sizes a separate transform launch is pure latency, and a GEMM
// tiled over M cannot keep enough weight bytes in flight.  So the work is
// split over (256-column chunk c, K split sp of SPW 256-k stages):
//
// decode_partial_kernel, one workgroup per (c, sp):
//   1. every wave requests its weight records (its 64 columns, SPW stages)
//      before the transform, so that HBM latency overlaps it.  A wave's loads
//      complete in issue order, so with one stage per workgroup the wave's
//      activation-side loads (factor entries, token rows, ratios) go out just
//      before the weights: the transform then waits only for them.  With
//      more stages their registers would not fit, and they follow the weights;
//   2. the workgroup transforms and quantises the split's activation blocks
//      for all tokens with the same per-block arithmetic as the transform
//      kernel (block_quant.h): the codes are identical bit for bit.  They are
//      staged in LDS in the MFMA operand order;
//   3. each wave multiplies them with its weights on the block-scaled MFMA,
//      stage by stage in one accumulator, and stores the fp32 partial tile.
// decode_reduce_kernel then sums the splits of every output in split order
// (deterministic) and writes Y.  The launch boundary orders the two, so no
// workgroup ever waits for or synchronises with another.
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

constexpr int kQRow = 144;  // staged code row: 8 blocks x 16 bytes + 16 pad (conflict-free reads)

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

// Inputs of one activation block for the wave's 32 token slots: factor
// entries, the lane's 16 channels of token j (zero for j >= M), the ratios.
struct ActIn {
  PFactors f;
  uint4 x0, x1;
  float rh, rl;
};
__device__ __forceinline__ ActIn load_act(const DecodeArgs& p, int64_t blk, int j, int h) {
  const int bdim = 32 >> p.a_log2;
  ActIn in;
  in.f = load_p_factors(p.A, p.B + blk * bdim * bdim, p.a_log2, j, h);
  in.x0 = in.x1 = make_uint4(0, 0, 0, 0);
  if (j < p.M) {
    const uint16_t* xr = p.x + (int64_t)j * p.ldx + blk * 32 + 8 * h;
    in.x0 = *reinterpret_cast<const uint4*>(xr);
    in.x1 = *reinterpret_cast<const uint4*>(xr + 16);
  }
  in.rh = p.r_hi ? p.r_hi[blk] : 1.0f;
  in.rl = p.r_lo ? p.r_lo[blk] : 1.0f;
  return in;
}

template <int SPW>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs p, int nchunk, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint8_t qs[SPW][32 * kQRow];
  __shared__ __attribute__((aligned(16))) uint8_t ss[SPW][32 * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x % nchunk;
  const int sp = blockIdx.x / nchunk;
  const int64_t nst = p.K / 256;
  const int64_t s0 = (int64_t)sp * SPW;

  // Wave w quantises blocks w and w + 4 of every stage of the split for
  // tokens 0..31 (rows >= M are zero and never stored).
  const int j = lane & 31;
  const int h = lane >> 5;
  ActIn pre[2];
  if constexpr (SPW == 1) {
    if (s0 < nst) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) pre[bb] = load_act(p, s0 * 8 + wave + 4 * bb, j, h);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 1. weight records of this wave's two 32-column groups for the split's
  // stages (stages past K are never requested).
  const int64_t n0 = (int64_t)c * 256 + 64 * wave;
  const int64_t n32_max = (p.N + 31) / 32;
  const int64_t g0 = n0 / 32 < n32_max ? n0 / 32 : n32_max - 1;  // clamped groups are computed, never stored
  const int64_t g1 = n0 / 32 + 1 < n32_max ? n0 / 32 + 1 : n32_max - 1;
  uint4 b0[SPW][4], b1[SPW][4];
  uint32_t bs0[SPW], bs1[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    if (s0 + t < nst) {
      const uint8_t* r0 = p.wp + (g0 * nst + s0 + t) * kPackGroupBytes + 16 * lane;
      const uint8_t* r1 = p.wp + (g1 * nst + s0 + t) * kPackGroupBytes + 16 * lane;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        b0[t][jj] = ld16_stream(r0 + 1024 * jj);
        b1[t][jj] = ld16_stream(r1 + 1024 * jj);
      }
      bs0[t] = ld4_stream(r0 + 4096 - 12 * lane);
      bs1[t] = ld4_stream(r1 + 4096 - 12 * lane);
    }
  }

  if constexpr (SPW == 1) __builtin_amdgcn_sched_barrier(0);

  // 2. activation blocks, staged in LDS in the MFMA operand order.
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    if (s0 + t >= nst) break;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int lb = wave + 4 * bb;  // block within the stage
      const int64_t blk = (s0 + t) * 8 + lb;
      const ActIn in = SPW == 1 ? pre[bb] : load_act(p, blk, j, h);
      const f32x16 acc = transform_block(split_p(in.f), in.x0, in.x1);
      int sbyte;
      const uint2 code = quant_block_e2m1(acc, in.rh, in.rl, h, sbyte);
      *reinterpret_cast<uint2*>(&qs[t][j * kQRow + 16 * lb + 8 * h]) = code;
      if (h == 0) ss[t][j * 8 + lb] = (uint8_t)sbyte;
      if (p.xq != nullptr && c == 0 && j < p.M) {  // optional copy of the quantised activations
        *reinterpret_cast<uint2*>(p.xq + (int64_t)j * (p.K >> 1) + blk * 16 + 8 * h) = code;
        if (h == 0) p.xs[(int64_t)j * (p.K >> 5) + blk] = (uint8_t)sbyte;
      }
    }
  }
  __syncthreads();

  // 3. MMA: lane (r32, g) of sub-step jj carries block 4 g + jj of token r32
  // (the packed weight record holds the matching blocks of its rows).
  const int r32 = lane & 31;
  const int g = lane >> 5;
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    if (s0 + t >= nst) break;
    const uint8_t* qrow = &qs[t][r32 * kQRow + 64 * g];
    const uint32_t sa = ld4(&ss[t][r32 * 8 + 4 * g]);
    const uint4 a0 = ld16(qrow), a1 = ld16(qrow + 16), a2 = ld16(qrow + 32), a3 = ld16(qrow + 48);
    acc0 = mfma_fp4<0>(a0, b0[t][0], sa, bs0[t], acc0);
    acc1 = mfma_fp4<0>(a0, b1[t][0], sa, bs1[t], acc1);
    acc0 = mfma_fp4<1>(a1, b0[t][1], sa, bs0[t], acc0);
    acc1 = mfma_fp4<1>(a1, b1[t][1], sa, bs1[t], acc1);
    acc0 = mfma_fp4<2>(a2, b0[t][2], sa, bs0[t], acc0);
    acc1 = mfma_fp4<2>(a2, b1[t][2], sa, bs1[t], acc1);
    acc0 = mfma_fp4<3>(a3, b0[t][3], sa, bs0[t], acc0);
    acc1 = mfma_fp4<3>(a3, b1[t][3], sa, bs1[t], acc1);
  }

  // 4. partial tile [M][256] of (c, sp); lane (r32, g), register r holds row
  // 8 (r / 4) + 4 g + r % 4 of columns 64 wave + r32 and 64 wave + 32 + r32.
  const int64_t M = p.M;
  float* part = p.part + ((int64_t)c * nsplit + sp) * M * 256;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * g + (r & 3);
    if (row < M) {
      part[row * 256 + 64 * wave + r32] = acc0[r];
      part[row * 256 + 64 * wave + 32 + r32] = acc1[r];
    }
  }
}

// Y[row][4 q .. 4 q + 3 of chunk c] = sum of the splits' partials, in split
// order; one (row, 4-column quad) per thread, all splits loaded together.
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs p, int nchunk, int nsplit) {
  const int64_t M = p.M;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over nchunk x M x 64
  if (item >= (int64_t)nchunk * M * 64) return;
  const int64_t c = item / (M * 64);
  const int64_t row = (item / 64) % M;
  const int q = (int)(item % 64);
  const float* pc = p.part + c * nsplit * M * 256 + row * 256 + 4 * q;
  constexpr int kBatch = 16;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
      v[t] = s0 + t < nsplit ? *reinterpret_cast<const float4*>(pc + (int64_t)(s0 + t) * M * 256)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      sum.x += v[t].x;
      sum.y += v[t].y;
      sum.z += v[t].z;
      sum.w += v[t].w;
    }
  }
  const float out[4] = {sum.x, sum.y, sum.z, sum.w};
  const int64_t col0 = c * 256 + 4 * q;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t col = col0 + e;
    if (col >= p.N) break;
    if (p.out_f32)
      reinterpret_cast<float*>(p.y)[row * p.N + col] = out[e];
    else
      reinterpret_cast<uint16_t*>(p.y)[row * p.N + col] = (uint16_t)f32_to_bf16_rne(out[e]);
  }
}

// Stages per workgroup: one (the most workgroups, and each wave's activation
// loads go out ahead of its weights) unless the fp32 partials would rival the
// weights in bytes, i.e. above 16 tokens on grids of more than one workgroup
// per CU: then two.  Measured on 1-32 tokens with K, N in {4096, 12288}: one
// stage is 10-40 % faster up to 16 tokens; at 32 tokens two are 5-7 % faster
// once there are more than 256 workgroups, and equal or slower below.
int stages_per_wg(int64_t M, int64_t nchunk, int64_t nst) {
  return (M <= 16 || nchunk * nst <= 256) ? 1 : 2;
}

template <int SPW>
hipError_t launch_t(const DecodeArgs& a, int nchunk, int nsplit, hipStream_t stream) {
  hipLaunchKernelGGL(decode_partial_kernel<SPW>, dim3(nchunk * nsplit), dim3(256), 0, stream, a, nchunk, nsplit);
  const int64_t items = (int64_t)nchunk * a.M * 64;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a, nchunk,
                     nsplit);
  return hipGetLastError();
}

}  // namespace

int64_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t nchunk = (N + 255) / 256, nst = K / 256;
  const int spw = stages_per_wg(M, nchunk, nst);
  return nchunk * ((nst + spw - 1) / spw) * M * 256 * 4;
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
  const int64_t nchunk = (args.N + 255) / 256, nst = args.K / 256;
  const int spw = stages_per_wg(args.M, nchunk, nst);
  const int nsplit = (int)((nst + spw - 1) / spw);
  return spw == 2 ? launch_t<2>(args, (int)nchunk, nsplit, stream) : launch_t<1>(args, (int)nchunk, nsplit, stream);
}

}  // namespace batq
