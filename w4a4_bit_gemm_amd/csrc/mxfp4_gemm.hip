// W4A4 GEMM on MXFP4 operands with the gfx950 block-scaled matrix cores.
//
// Y[m][n] = sum_k deq(Xq)[m][k] * deq(Wq)[n][k], FP32 accumulation
// [BATQuant note (en.papernotes.org), Key Designs §1: Q(XP) Q(P^-1 W^T);
//  Key Designs §4: all linear layers use low-bit matrix multiplication].
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1: lane l supplies
// 32 consecutive k of row (l % 32) — exactly one MX block, 16 bytes — plus that
// block's UE8M0 scale byte, selected out of a 32-bit register by OPSEL.  Since
// the k order inside one instruction is free as long as both operands agree,
// lane half g covers blocks 4g..4g+3 of every 8-block (256-k) step, one block
// per instruction: a lane reads 64 contiguous code bytes and one 4-byte group
// of scales per row and step.
#include "common.h"

namespace batq {

namespace {

constexpr int kTileM = 128;
constexpr int kTileN = 128;

struct Frag {
  uint4 codes[4];  // 4 blocks x 16 bytes
  uint32_t scales; // byte j = scale of block j
};

__device__ __forceinline__ void load_frag(Frag& f, const uint8_t* __restrict__ q,
                                          const uint8_t* __restrict__ s, int64_t row, int64_t kb_first,
                                          int64_t nb) {
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
      f.codes[j] = make_uint4(0, 0, 0, 0);  // zero codes, unit scale
      sc |= 127u << (8 * j);
    }
  }
  f.scales = sc;
}

__device__ __forceinline__ i32x8 op(uint4 v) {
  i32x8 r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

template <int J>
__device__ __forceinline__ f32x16 mfma_blk(const Frag& a, const Frag& b, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(a.codes[J]), op(b.codes[J]), acc, 4, 4, J,
                                                         (int)a.scales, J, (int)b.scales);
}

__global__ __launch_bounds__(256) void mxfp4_gemm_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int64_t nb = p.K >> 5;
  const int64_t m_base = (int64_t)blockIdx.y * kTileM + 64 * (wave >> 1);
  const int64_t n_base = (int64_t)blockIdx.x * kTileN + 64 * (wave & 1);

  int64_t arow[2], brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t m = m_base + 32 * t + r32;
    const int64_t n = n_base + 32 * t + r32;
    arow[t] = m < p.M ? m : p.M - 1;  // out-of-range rows read a valid row, never stored
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
        acc[tm][tn] = mfma_blk<0>(fa[tm], fb[tn], acc[tm][tn]);
        acc[tm][tn] = mfma_blk<1>(fa[tm], fb[tn], acc[tm][tn]);
        acc[tm][tn] = mfma_blk<2>(fa[tm], fb[tn], acc[tm][tn]);
        acc[tm][tn] = mfma_blk<3>(fa[tm], fb[tn], acc[tm][tn]);
      }
  }

  // acc[tm][tn][r] = Y[m_base + 32 tm + 8 (r/4) + 4 g + r%4][n_base + 32 tn + r32]
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
          if (p.out_f32) {
            reinterpret_cast<float*>(p.y)[row * p.N + col] = v;
          } else {
            reinterpret_cast<uint16_t*>(p.y)[row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
          }
        }
      }
    }
}

}  // namespace

hipError_t launch_mxfp4_gemm(const GemmArgs& args, hipStream_t stream) {
  dim3 grid((unsigned)((args.N + kTileN - 1) / kTileN), (unsigned)((args.M + kTileM - 1) / kTileM));
  hipLaunchKernelGGL(mxfp4_gemm_kernel, grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace batq
