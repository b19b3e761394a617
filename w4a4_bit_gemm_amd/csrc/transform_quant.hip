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

constexpr int kWavesPerBlock = 4;  // one 32-channel block per wave

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

__global__ __launch_bounds__(256) void transform_quant_kernel(TransformQuantArgs p, int tokens_per_wg) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nb = p.K >> 5;
  const int64_t blk = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (blk >= nb) return;  // whole wave leaves; the kernel has no barriers

  const int j = lane & 31;  // output channel (A-operand row) / token slot (B column)
  const int h = lane >> 5;  // which 8-channel half of each 16-channel k step
  const int la = p.a_log2;
  const int a = 1 << la;
  const int amask = a - 1;
  const int bdim = 32 >> la;

  // P_i^T as MFMA A operand: lane holds P_i[16 ks + 8 h + t][j], t = 0..7.
  uint4 phi[2], pmid[2], plo[2];
  {
    const float* __restrict__ Bi = p.B + blk * bdim * bdim;
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

  const int64_t tok0 = (int64_t)blockIdx.y * tokens_per_wg;
  int64_t tok_end = tok0 + tokens_per_wg;
  if (tok_end > p.rows) tok_end = p.rows;
  const int64_t qld = p.K >> 1;

  // First tile's operands; invalid token slots read a valid row (tok0) and
  // store nothing.
  int64_t t_cur = tok0 + j;
  const uint16_t* xr = p.x + (t_cur < tok_end ? t_cur : tok0) * p.ldx + blk * 32 + 8 * h;
  uint4 x0 = load_row8(xr);
  uint4 x1 = load_row8(xr + 16);

  for (int64_t base = tok0; base < tok_end; base += 32) {
    // prefetch the next 32 tokens
    const int64_t t_nxt = base + 32 + j;
    const uint16_t* xn = p.x + (t_nxt < tok_end ? t_nxt : tok0) * p.ldx + blk * 32 + 8 * h;
    uint4 n0 = x0, n1 = x1;
    if (base + 32 < tok_end) {
      n0 = load_row8(xn);
      n1 = load_row8(xn + 16);
    }

    f32x16 acc = {};
    const bf16x8 bx0 = as_bf16x8(x0), bx1 = as_bf16x8(x1);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(plo[0]), bx0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(plo[1]), bx1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pmid[0]), bx0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pmid[1]), bx1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(phi[0]), bx0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(phi[1]), bx1, acc, 0, 0, 0);
    // acc[r] = y[token base + j][channel 8 (r/4) + 4 h + r%4]

    float mx = acc[0], mn = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      mx = fmaxf(mx, acc[r]);
      mn = fminf(mn, acc[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mn = fminf(mn, __shfl_xor(mn, 32));

    const int64_t tok = base + j;
    const bool valid = tok < tok_end;
    const int64_t tok_c = valid ? tok : tok0;
    float rh = 1.0f, rl = 1.0f;
    if (p.r_hi != nullptr) {
      const int64_t ri = tok_c * p.r_ld + blk;
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
    // q = 0,1 in wA and q = 2,3 in wB.  Swap so that half 0 stores bytes 0..7
    // and half 1 bytes 8..15 of the token's 16-byte code row segment.
    const uint32_t send = h ? wA : wB;
    const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
    const uint32_t keep = h ? wB : wA;
    const uint32_t first = h ? recv : keep;
    const uint32_t second = h ? keep : recv;
    const uint32_t out_lo = (first & 0xFFFFu) | (second << 16);
    const uint32_t out_hi = (first >> 16) | (second & 0xFFFF0000u);
    if (valid) {
      *reinterpret_cast<uint2*>(p.q + tok * qld + blk * 16 + 8 * h) = make_uint2(out_lo, out_hi);
      if (h == 0) p.s[tok * nb + blk] = (uint8_t)sbyte;
    }
    x0 = n0;
    x1 = n1;
  }
}

}  // namespace

hipError_t launch_transform_quant(const TransformQuantArgs& args, hipStream_t stream) {
  const int64_t nb = args.K >> 5;
  // Enough token chunks to give every CU several workgroups; each wave's
  // P_i set-up is amortised over its chunk.
  int tokens_per_wg = 128;
  if (args.rows <= 256) tokens_per_wg = 32;
  dim3 grid((unsigned)((nb + kWavesPerBlock - 1) / kWavesPerBlock),
            (unsigned)((args.rows + tokens_per_wg - 1) / tokens_per_wg));
  hipLaunchKernelGGL(transform_quant_kernel, grid, dim3(64 * kWavesPerBlock), 0, stream, args,
                     tokens_per_wg);
  return hipGetLastError();
}

}  // namespace batq
