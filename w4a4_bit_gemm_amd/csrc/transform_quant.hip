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
#include "common.h"

namespace batq {

namespace {

constexpr int kWavesPerWG = 8;  // one 32-channel block per wave; 8 blocks = 128 code bytes per row

// Exact product pa * pb split into three bf16 parts, hi + mid + lo, whose sum
// differs from the product by at most ~2^-27 of it.
__device__ __forceinline__ void split3(float pa, float pb, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  float r0 = pa * pb;
  float e0 = __builtin_fmaf(pa, pb, -r0);  // exact rounding error of the product
  hi = f32_to_bf16_rne(r0);
  float rem = (r0 - bf16_to_f32(hi)) + e0;  // r0 - hi is exact
  mid = f32_to_bf16_rne(rem);
  float rem2 = rem - bf16_to_f32(mid);     // exact
  lo = f32_to_bf16_rne(rem2);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 load_row8(const uint16_t* __restrict__ p) {
  return *reinterpret_cast<const uint4*>(p);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile of one workgroup: TT tokens x 8 consecutive blocks (256 channels).
//  1. The bf16 tile (TT x 512 bytes) moves global -> LDS with 16-byte
//     direct-to-LDS loads, one instruction = two whole 512-byte row segments.
//     Row r keeps its 16-byte chunk c at position c ^ (r & 15), so the MFMA
//     operand reads below (16 consecutive rows, same chunk) hit 16 different
//     bank groups.
//  2. While those loads fly, each wave (one block) builds its P_i split.
//  3. Per 32-token group: MFMA transform, clip, scale, E2M1 codes; codes and
//     scale bytes go to LDS staging buffers.
//  4. Codes leave in 16-byte row-contiguous chunks (whole 128-byte lines per
//     row of the tile); scale bytes in 8-byte row pieces.
template <int TT>
struct TQTile {
  static constexpr int kXRow = 512;        // bytes per staged bf16 row (256 channels)
  static constexpr int kX = TT * kXRow;
  static constexpr int kQRow = 144;        // 128 code bytes + 16 pad: conflict-free 8-byte writes
  static constexpr int kQ = TT * kQRow;
  static constexpr int kS = TT * 8;
};

template <int TT>
__global__ __launch_bounds__(512) void transform_quant_kernel(TransformQuantArgs p) {
  using T = TQTile<TT>;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[T::kX];
  __shared__ __attribute__((aligned(16))) uint8_t qs[T::kQ];
  __shared__ __attribute__((aligned(16))) uint8_t ss[T::kS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t nb = p.K >> 5;
  const int64_t blk0 = (int64_t)blockIdx.x * kWavesPerWG;
  const int64_t blk = blk0 + wave;
  const bool blk_ok = blk < nb;  // waves past the last block still load and sync
  const int64_t tok0 = (int64_t)blockIdx.y * TT;

  // 1. global -> LDS: TT / 2 instructions of 1 KB, TT / 16 per wave
#pragma unroll
  for (int i = 0; i < TT / 16; ++i) {
    const int q = wave + kWavesPerWG * i;
    const int row = 2 * q + (lane >> 5);
    const int pc = lane & 31;              // position in the staged row
    const int c = pc ^ (row & 15);         // logical 16-byte chunk stored there
    int64_t gr = tok0 + row;
    gr = gr < p.rows ? gr : p.rows - 1;    // rows past the end re-read the last row
    int64_t col = blk0 * 32 + 8 * c;       // first channel of the chunk
    col = col < p.K ? col : 0;             // chunks past K read a valid column, unused
    __builtin_amdgcn_global_load_lds(p.x + gr * p.ldx + col, (lds_void*)(xs + q * 1024), 16, 0, 0);
  }

  const int j = lane & 31;  // output channel (A-operand row) / token slot (B column)
  const int h = lane >> 5;  // which 8-channel half of each 16-channel k step

  // 2. P_i^T as MFMA A operand: lane holds P_i[16 ks + 8 h + t][j], t = 0..7,
  //    as an exact three-way bf16 split.
  const int la = p.a_log2;
  const int a = 1 << la;
  const int amask = a - 1;
  const int bdim = 32 >> la;
  uint4 phi[2], pmid[2], plo[2];
  {
    const float* __restrict__ Bi = p.B + (blk_ok ? blk : 0) * bdim * bdim;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t hw[8], mw[8], lw[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int k = 16 * ks + 8 * h + t;
        const float bv = Bi[(k >> la) * bdim + (j >> la)];
        const float av = p.A[(k & amask) * a + (j & amask)];
        split3(bv, av, hw[t], mw[t], lw[t]);
      }
      phi[ks] = make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16);
      pmid[ks] = make_uint4(mw[0] | mw[1] << 16, mw[2] | mw[3] << 16, mw[4] | mw[5] << 16, mw[6] | mw[7] << 16);
      plo[ks] = make_uint4(lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads landed
  block_barrier();                      // ... and every other wave's

  // 3. per 32-token group
  if (blk_ok) {
#pragma unroll
    for (int gi = 0; gi < TT / 32; ++gi) {
      const int row = 32 * gi + j;
      const uint8_t* xr = xs + row * T::kXRow;
      const uint4 x0 = *reinterpret_cast<const uint4*>(xr + 16 * ((4 * wave + h) ^ (row & 15)));
      const uint4 x1 = *reinterpret_cast<const uint4*>(xr + 16 * ((4 * wave + 2 + h) ^ (row & 15)));
      f32x16 acc = {};
      const bf16x8 bx0 = as_bf16x8(x0), bx1 = as_bf16x8(x1);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(plo[0]), bx0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(plo[1]), bx1, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pmid[0]), bx0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pmid[1]), bx1, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(phi[0]), bx0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(phi[1]), bx1, acc, 0, 0, 0);
      // acc[r] = y[token tok0 + row][channel 8 (r/4) + 4 h + r%4 of block blk]

      float mx = acc[0], mn = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        mx = fmaxf(mx, acc[r]);
        mn = fminf(mn, acc[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mn = fminf(mn, __shfl_xor(mn, 32));

      int64_t tok = tok0 + row;
      tok = tok < p.rows ? tok : p.rows - 1;
      float rh = 1.0f, rl = 1.0f;
      if (p.r_hi != nullptr) {
        const int64_t ri = tok * p.r_ld + blk;
        rh = p.r_hi[ri];
        rl = p.r_lo[ri];
      }
      const float u = __fmul_rn(rh, mx);
      const float l = fminf(__fmul_rn(rl, mn), u);  // l > u clamps everything to u
      const float zmax = __builtin_amdgcn_fmed3f(mx, l, u);
      const float zmin = __builtin_amdgcn_fmed3f(mn, l, u);
      const float amax = fmaxf(fabsf(zmax), fabsf(zmin));
      // scale byte = e + 127 = max(biased exponent of amax - 2, 0)
      const int sbyte = max((int)(__float_as_uint(amax) >> 23) - 2, 0);
      const float inv = __uint_as_float((uint32_t)(254 - sbyte) << 23);  // 2^-e, exact

      uint32_t wA = 0, wB = 0;
#define BATQ_CVT(word, r, sel)                                                        \
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(                                    \
      word, __builtin_amdgcn_fmed3f(acc[r], l, u) * inv,                              \
      __builtin_amdgcn_fmed3f(acc[r + 1], l, u) * inv, 1.0f, sel)
      BATQ_CVT(wA, 0, 0);
      BATQ_CVT(wA, 2, 1);
      BATQ_CVT(wA, 4, 2);
      BATQ_CVT(wA, 6, 3);
      BATQ_CVT(wB, 8, 0);
      BATQ_CVT(wB, 10, 1);
      BATQ_CVT(wB, 12, 2);
      BATQ_CVT(wB, 14, 3);
#undef BATQ_CVT
      // Lane half h holds code bytes {4q + 2h, 4q + 2h + 1}, q = 0..3, with
      // q = 0,1 in wA and q = 2,3 in wB.  Swap so that half 0 holds bytes 0..7
      // and half 1 bytes 8..15 of the token's 16-byte code segment.
      const uint32_t send = h ? wA : wB;
      const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
      const uint32_t keep = h ? wB : wA;
      const uint32_t first = h ? recv : keep;
      const uint32_t second = h ? keep : recv;
      const uint32_t out_lo = (first & 0xFFFFu) | (second << 16);
      const uint32_t out_hi = (first >> 16) | (second & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(qs + row * T::kQRow + 16 * wave + 8 * h) = make_uint2(out_lo, out_hi);
      if (h == 0) ss[row * 8 + wave] = (uint8_t)sbyte;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staged codes and scales written
  block_barrier();

  // 4. codes: TT rows x up to 128 bytes in 16-byte chunks
  const int64_t qld = p.K >> 1;
  const int64_t nblk = (nb - blk0) < kWavesPerWG ? (nb - blk0) : kWavesPerWG;  // valid blocks in tile
#pragma unroll
  for (int i = 0; i < (TT * 8 + 511) / 512; ++i) {
    const int id = tid + 512 * i;
    if (id >= TT * 8) break;
    const int row = id >> 3;
    const int c = id & 7;
    const int64_t tok = tok0 + row;
    if (tok < p.rows && c < nblk)
      *reinterpret_cast<uint4*>(p.q + tok * qld + blk0 * 16 + 16 * c) =
          *reinterpret_cast<const uint4*>(qs + row * T::kQRow + 16 * c);
  }
  //    scales: one thread per row
  if (tid < TT) {
    const int64_t tok = tok0 + tid;
    if (tok < p.rows) {
      uint8_t* dst = p.s + tok * nb + blk0;
      const uint8_t* src = ss + tid * 8;
      if (nblk == 8 && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
      } else {
        for (int c = 0; c < nblk; ++c) dst[c] = src[c];
      }
    }
  }
}

}  // namespace

hipError_t launch_transform_quant(const TransformQuantArgs& args, hipStream_t stream) {
  const int64_t nb = args.K >> 5;
  const unsigned gx = (unsigned)((nb + kWavesPerWG - 1) / kWavesPerWG);
  // Tokens per workgroup: 64 (three resident workgroups per CU, 42 KB of LDS
  // each), 128 for layers too small to give every CU two workgroups of 64,
  // 32 for a handful of tokens.
  int tt = 64;
  if ((int64_t)gx * ((args.rows + 63) / 64) < 512) tt = 128;
  if (args.rows <= 32) tt = 32;
  dim3 grid(gx, (unsigned)((args.rows + tt - 1) / tt));
  switch (tt) {
    case 128: hipLaunchKernelGGL(transform_quant_kernel<128>, grid, dim3(512), 0, stream, args); break;
    case 64: hipLaunchKernelGGL(transform_quant_kernel<64>, grid, dim3(512), 0, stream, args); break;
    default: hipLaunchKernelGGL(transform_quant_kernel<32>, grid, dim3(512), 0, stream, args); break;
  }
  return hipGetLastError();
}

}  // namespace batq
