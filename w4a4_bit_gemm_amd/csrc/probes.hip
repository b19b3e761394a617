// Measurement probes: the ceilings the path's kernels are set against.
//
// Not part of the path.  Each probe isolates one resource of the chip:
//   batq_probe_mfma_fp4  the block-scaled 32x32x64 FP4 matrix instruction the
//                        GEMM issues, in a register-only loop (no memory
//                        traffic), with constant or random operand bits, and
//                        the shader clock the waves ran at (s_memtime cycles
//                        against the 100 MHz s_memrealtime counter);
//   batq_probe_hbm_read  a streaming read of a buffer far larger than the
//                        Infinity Cache;
//   batq_probe_hbm_copy  a streaming copy (read + write) of such a buffer;
//   batq_probe_hbm_stream a read:write stream in a fixed ratio.
// The streams read with non-temporal loads, the policy of every one-time read
// in the path's kernels: on this part it lifts a plain read stream from about
// 6.2 to 7.1 TB/s.  Each workgroup streams one contiguous range; up to 4096
// workgroups (two rounds of resident ones) let the dispatcher even out the
// tail, which a read:write stream measurably needs.
// Declared in include/batq_probe.h.
#include "batq.h"
#include "batq_probe.h"
#include "common.h"

namespace batq {
namespace {

constexpr int kChains = 8;  // independent accumulators per wave: the matrix pipe never waits on a result

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Each wave: `iters` rounds of kChains MFMAs on register operands.  Random
// data: every lane and register gets its own hashed bits (consecutive MFMAs
// of a round take different operand registers, so the bits toggle between
// issues);
// constant data: every operand register holds 0x22222222 (E2M1 1.0
// everywhere).  Scales are 1.  The accumulators are reduced to one float per
// wave so that nothing is dead.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void probe_mfma_fp4_kernel(int iters, int random_data, uint32_t seed, float* sink,
                                                             unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  i32x8 a[2], b[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = hash32(seed ^ hash32((uint32_t)(lane * 64 + r * 8 + e) + 0x9E3779B9u * (uint32_t)(wave_id & 7)));
      const uint32_t h2 = hash32(h + 0x632BE5ABu);
      a[r][e] = e < 4 ? (int)(random_data ? h : 0x22222222u) : 0;
      b[r][e] = e < 4 ? (int)(random_data ? h2 : 0x22222222u) : 0;
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c & 1], b[(c >> 1) & 1], acc[c], 4, 4, 0, 127, 0,
                                                                127);
  }
  // the results are final before the clocks are read again
#pragma unroll
  for (int c = 0; c < kChains; ++c) asm volatile("" : "+v"(acc[c]));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (lane == 0) {
    sink[wave_id] = s;
    clocks[2 * wave_id] = t1 - t0;
    clocks[2 * wave_id + 1] = r1 - r0;
  }
}

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread per round

__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup g streams the contiguous range [g * per, (g + 1) * per) of 16-byte
// words (per is a multiple of kStreamThreads * kUnroll), xor-reduces it and
// writes one word.
__global__ __launch_bounds__(kStreamThreads) void probe_read_kernel(const uint4* __restrict__ src, int64_t per,
                                                                    uint32_t* sink) {
  const uint4* p = src + (int64_t)blockIdx.x * per + threadIdx.x;
  uint4 x = make_uint4(0, 0, 0, 0);
  for (int64_t i = 0; i < per; i += kStreamThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld_stream(p + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      x.x ^= v[u].x;
      x.y ^= v[u].y;
      x.z ^= v[u].z;
      x.w ^= v[u].w;
    }
  }
  const uint32_t r = x.x ^ x.y ^ x.z ^ x.w;
  __shared__ uint32_t red[kStreamThreads];
  red[threadIdx.x] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kStreamThreads; ++i) t ^= red[i];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(kStreamThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst, int64_t per) {
  const int64_t base = (int64_t)blockIdx.x * per + threadIdx.x;
  for (int64_t i = 0; i < per; i += kStreamThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld_stream(src + base + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[base + i + u * kStreamThreads] = v[u];
  }
}

// Reads `per` 16-byte words per workgroup and writes per / R, each written
// word the xor of R read words (a read:write mix like the transform's, whose
// bf16 rows are about four times its codes).
template <int R>
__global__ __launch_bounds__(kStreamThreads) void probe_stream_kernel(const uint4* __restrict__ src,
                                                                      uint4* __restrict__ dst, int64_t per) {
  static_assert(kUnroll % R == 0, "whole written words per round");
  const int64_t rbase = (int64_t)blockIdx.x * per + threadIdx.x;
  const int64_t wbase = (int64_t)blockIdx.x * (per / R) + threadIdx.x;
  for (int64_t i = 0; i < per; i += kStreamThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld_stream(src + rbase + i + u * kStreamThreads);
#pragma unroll
    for (int o = 0; o < kUnroll / R; ++o) {
      uint4 x = v[o * R];
#pragma unroll
      for (int r = 1; r < R; ++r) {
        x.x ^= v[o * R + r].x;
        x.y ^= v[o * R + r].y;
        x.z ^= v[o * R + r].z;
        x.w ^= v[o * R + r].w;
      }
      dst[wbase + i / R + o * kStreamThreads] = x;
    }
  }
}

// Workgroups and 16-byte words per workgroup for a stream of `bytes`: up to
// 4096 workgroups, each range a whole number of rounds of kStreamThreads x
// kUnroll words.
bool stream_split(int64_t bytes, int64_t& groups, int64_t& per) {
  const int64_t round = (int64_t)kStreamThreads * kUnroll;
  if (bytes <= 0 || bytes % (16 * round) != 0) return false;
  const int64_t units = bytes / (16 * round);
  groups = 4096;
  while (groups > 1 && units % groups != 0) groups /= 2;
  per = bytes / 16 / groups;
  return true;
}

}  // namespace
}  // namespace batq

extern "C" {

int64_t batq_probe_stream_granule(void) { return 256LL * 8 * 16; }

batq_status batq_probe_mfma_fp4(int64_t workgroups, int32_t iters, int32_t random_data, uint32_t seed, float* sink,
                                unsigned long long* clocks, hipStream_t stream) {
  if (workgroups <= 0 || workgroups > (1 << 20) || iters <= 0) return BATQ_ERR_SHAPE;
  if (sink == nullptr || clocks == nullptr) return BATQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(clocks) % 8 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return BATQ_ERR_ALIGN;
  hipLaunchKernelGGL(batq::probe_mfma_fp4_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters,
                     random_data, seed, sink, clocks);
  return hipGetLastError() == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

batq_status batq_probe_hbm_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  int64_t groups, per;
  if (!batq::stream_split(bytes, groups, per)) return BATQ_ERR_SHAPE;
  if (src == nullptr || sink == nullptr) return BATQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return BATQ_ERR_ALIGN;
  hipLaunchKernelGGL(batq::probe_read_kernel, dim3((unsigned)groups), dim3(batq::kStreamThreads), 0, stream,
                     static_cast<const uint4*>(src), per, sink);
  return hipGetLastError() == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

batq_status batq_probe_hbm_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  int64_t groups, per;
  if (!batq::stream_split(bytes, groups, per)) return BATQ_ERR_SHAPE;
  if (src == nullptr || dst == nullptr) return BATQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return BATQ_ERR_ALIGN;
  hipLaunchKernelGGL(batq::probe_copy_kernel, dim3((unsigned)groups), dim3(batq::kStreamThreads), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), per);
  return hipGetLastError() == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

batq_status batq_probe_hbm_stream(const void* src, int64_t read_bytes, void* dst, int32_t ratio,
                                  hipStream_t stream) {
  int64_t groups, per;
  if (!batq::stream_split(read_bytes, groups, per)) return BATQ_ERR_SHAPE;
  if (ratio != 1 && ratio != 2 && ratio != 4 && ratio != 8) return BATQ_ERR_UNSUPPORTED;
  if (src == nullptr || dst == nullptr) return BATQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return BATQ_ERR_ALIGN;
  const auto* s = static_cast<const uint4*>(src);
  auto* d = static_cast<uint4*>(dst);
  const dim3 g((unsigned)groups), b(batq::kStreamThreads);
  switch (ratio) {
    case 1: hipLaunchKernelGGL(batq::probe_stream_kernel<1>, g, b, 0, stream, s, d, per); break;
    case 2: hipLaunchKernelGGL(batq::probe_stream_kernel<2>, g, b, 0, stream, s, d, per); break;
    case 4: hipLaunchKernelGGL(batq::probe_stream_kernel<4>, g, b, 0, stream, s, d, per); break;
    default: hipLaunchKernelGGL(batq::probe_stream_kernel<8>, g, b, 0, stream, s, d, per); break;
  }
  return hipGetLastError() == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

}  // extern "C"
