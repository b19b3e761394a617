// Per-block arithmetic of the online activation path, shared by every kernel
// that quantises activations (the fused transform kernel and the fused decode
// GEMM), so that they produce the same codes bit for bit.
//
// For one 32-channel block i and 32 tokens held by one wave [BATQuant note
// (en.papernotes.org), A Worked Example and Key Designs §1-§3]:
//   y = x_b (B_i (x) A)                    row-vector convention
//   z = min(max(y, r_lo min y), r_hi max y)
//   e = floor(log2 max|z|) - emax,         codes = RNE(z / 2^e)
// The transform is a 32 x 32 contraction on the bf16 matrix cores with P_i
// split exactly into three bf16 parts; lane (j, h) of the result holds token j
// and channels 8 (r / 4) + 4 h + r % 4, r = 0..15, so that the block min/max,
// clip, scale and rounding are lane-local plus one exchange between the two
// lane halves.
#pragma once
#include "common.h"

namespace batq {

typedef short v2i16 __attribute__((ext_vector_type(2)));

// Exact products pa0 * pb0 and pa1 * pb1, each split into three bf16 parts
// hi + mid + lo whose sum differs from the product by at most ~2^-27 of it;
// returned as packed pairs (product 0 in the low half).
__device__ __forceinline__ void split3x2(float pa0, float pb0, float pa1, float pb1, uint32_t& hi, uint32_t& mid,
                                         uint32_t& lo) {
  const float r0 = pa0 * pb0, r1 = pa1 * pb1;
  const float e0 = __builtin_fmaf(pa0, pb0, -r0);  // exact rounding errors of the products
  const float e1 = __builtin_fmaf(pa1, pb1, -r1);
  hi = f32x2_to_bf16x2_rne(r0, r1);
  const float q0 = (r0 - __uint_as_float(hi << 16)) + e0;  // r - hi is exact
  const float q1 = (r1 - __uint_as_float(hi & 0xFFFF0000u)) + e1;
  mid = f32x2_to_bf16x2_rne(q0, q1);
  const float s0 = q0 - __uint_as_float(mid << 16);  // exact
  const float s1 = q1 - __uint_as_float(mid & 0xFFFF0000u);
  lo = f32x2_to_bf16x2_rne(s0, s1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// P_i^T as the MFMA A operand: lane (j, h) holds P_i[16 ks + 8 h + t][j],
// t = 0..7, in parts[ks], as an exact three-way bf16 split.  A: [a][a],
// Bi: [b][b] with a = 1 << la, b = 32 / a.
struct PSplit {
  uint4 hi[2], mid[2], lo[2];
};
// The factor entries behind the lane's part of P_i^T:
// P_i[k][j] = Bi[k / a][j / a] * A[k % a][j % a].  Loading is separate from
// the split arithmetic so that a kernel can request these loads ahead of
// bulk loads of its own (a wave's loads complete in issue order).
struct PFactors {
  float bv[2][8], av[2][8];
};
__device__ __forceinline__ PFactors load_p_factors(const float* __restrict__ A, const float* __restrict__ Bi, int la,
                                                   int j, int h) {
  const int a = 1 << la;
  const int amask = a - 1;
  const int bdim = 32 >> la;
  PFactors f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int k = 16 * ks + 8 * h + t;
      f.bv[ks][t] = Bi[(k >> la) * bdim + (j >> la)];
      f.av[ks][t] = A[(k & amask) * a + (j & amask)];
    }
  return f;
}
__device__ __forceinline__ PSplit split_p(const PFactors& f) {
  PSplit ps;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t hw[4], mw[4], lw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      split3x2(f.bv[ks][2 * t], f.av[ks][2 * t], f.bv[ks][2 * t + 1], f.av[ks][2 * t + 1], hw[t], mw[t], lw[t]);
    ps.hi[ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    ps.mid[ks] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
    ps.lo[ks] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  return ps;
}
// y for one block and 32 tokens: x0 / x1 are the lane's 8 bf16 channels
// 8 h .. 8 h + 7 and 16 + 8 h .. 16 + 8 h + 7 of token j; the parts are
// accumulated lo -> mid -> hi in fp32.
__device__ __forceinline__ f32x16 transform_block(const PSplit& ps, uint4 x0, uint4 x1) {
  f32x16 acc = {};
  const bf16x8 bx0 = as_bf16x8(x0), bx1 = as_bf16x8(x1);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.lo[0]), bx0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.lo[1]), bx1, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.mid[0]), bx0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.mid[1]), bx1, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.hi[0]), bx0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ps.hi[1]), bx1, acc, 0, 0, 0);
  return acc;
}

// Block bounds: u, l (clip) and the scale byte max(biased exponent of
// max|z| - emax, 0), for emax 2 (E2M1) or 8 (E4M3).  rh = rl = 1 is no clip.
__device__ __forceinline__ void block_bounds(const f32x16& acc, float rh, float rl, int emax, float& u, float& l,
                                             int& sbyte) {
  float mx = acc[0], mn = acc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    mx = fmaxf(mx, acc[r]);
    mn = fminf(mn, acc[r]);
  }
  {
    // lanes l and l ^ 32 hold the two halves of a token's 32 channels
    const auto smx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    const auto smn = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    mx = fmaxf(__uint_as_float(smx[0]), __uint_as_float(smx[1]));
    mn = fminf(__uint_as_float(smn[0]), __uint_as_float(smn[1]));
  }
  u = __fmul_rn(rh, mx);
  l = fminf(__fmul_rn(rl, mn), u);  // l > u clamps everything to u
  const float zmax = __builtin_amdgcn_fmed3f(mx, l, u);
  const float zmin = __builtin_amdgcn_fmed3f(mn, l, u);
  const float amax = fmaxf(fabsf(zmax), fabsf(zmin));
  sbyte = max((int)(__float_as_uint(amax) >> 23) - emax, 0);
}

// E2M1 codes of one block: returns the lane's half of the token's 16-byte code
// segment (half h: bytes 8 h .. 8 h + 7, element 2 k in the low nibble of byte
// k) and the scale byte.  Call from every lane of the wave (the exceptional
// scale is detected per wave).
__device__ __forceinline__ uint2 quant_block_e2m1(const f32x16& acc, float rh, float rl, int h, int& sbyte) {
  float u, l;
  block_bounds(acc, rh, rl, 2, u, l, sbyte);
  // The converter divides by its scale operand, so 2^e goes in directly
  // (z / 2^e is exact).  2^-127 (scale byte 0, a block below 2^-125) is not a
  // normal float: such waves take the explicit multiply by 2^-e.
  uint32_t wA = 0, wB = 0;
#define BATQ_CVT(word, r, sel, M, S)                                                  \
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(                                    \
      word, __builtin_amdgcn_fmed3f(acc[r], l, u) M, __builtin_amdgcn_fmed3f(acc[r + 1], l, u) M, S, sel)
#define BATQ_CVT_ALL(M, S)                                                            \
  BATQ_CVT(wA, 0, 0, M, S);                                                           \
  BATQ_CVT(wA, 2, 1, M, S);                                                           \
  BATQ_CVT(wA, 4, 2, M, S);                                                           \
  BATQ_CVT(wA, 6, 3, M, S);                                                           \
  BATQ_CVT(wB, 8, 0, M, S);                                                           \
  BATQ_CVT(wB, 10, 1, M, S);                                                          \
  BATQ_CVT(wB, 12, 2, M, S);                                                          \
  BATQ_CVT(wB, 14, 3, M, S);
  if (__builtin_amdgcn_ballot_w64(sbyte == 0) == 0) {
    const float scale = __uint_as_float((uint32_t)sbyte << 23);  // 2^e
    BATQ_CVT_ALL(, scale)
  } else {
    const float inv = __uint_as_float((uint32_t)(254 - sbyte) << 23);  // 2^-e, exact
    BATQ_CVT_ALL(*inv, 1.0f)
  }
#undef BATQ_CVT_ALL
#undef BATQ_CVT
  // Lane half h holds code bytes {4q + 2h, 4q + 2h + 1}, q = 0..3, with q = 0,1
  // in wA and q = 2,3 in wB.  Swap so that half 0 holds bytes 0..7 and half 1
  // bytes 8..15 of the token's 16-byte code segment.
  const uint32_t send = h ? wA : wB;
  const auto sw = __builtin_amdgcn_permlane32_swap(send, send, false, false);
  const uint32_t recv = h ? sw[0] : sw[1];  // the partner lane's word
  const uint32_t keep = h ? wB : wA;
  const uint32_t first = h ? recv : keep;
  const uint32_t second = h ? keep : recv;
  return make_uint2((first & 0xFFFFu) | (second << 16), (first >> 16) | (second & 0xFFFF0000u));
}

// E4M3 codes of one block: returns the lane's half of the token's 32 code
// bytes (half h: bytes 16 h .. 16 h + 15) and the scale byte.  Call from every
// lane of the wave.
__device__ __forceinline__ uint4 quant_block_e4m3(const f32x16& acc, float rh, float rl, int h, int& sbyte) {
  float u, l;
  block_bounds(acc, rh, rl, 8, u, l, sbyte);
  // The converter does not saturate (beyond 448 it returns NaN), so the clip
  // bounds are narrowed to +-448 * 2^e, which clamps every value the way
  // rounding with saturation would.
  uint32_t wq[4];
  if (__builtin_amdgcn_ballot_w64(sbyte == 0) == 0) {
    const float scale = __uint_as_float((uint32_t)sbyte << 23);  // 2^e
    const float sat = 448.0f * scale;                             // exact
    const float u8 = fminf(u, sat);
    const float l8 = fminf(fmaxf(l, -sat), u8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v2i16 r = {0, 0};
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(acc[4 * q], l8, u8),
                                                   __builtin_amdgcn_fmed3f(acc[4 * q + 1], l8, u8), scale, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(acc[4 * q + 2], l8, u8),
                                                   __builtin_amdgcn_fmed3f(acc[4 * q + 3], l8, u8), scale, true);
      wq[q] = __builtin_bit_cast(uint32_t, r);
    }
  } else {
    const float inv = __uint_as_float((uint32_t)(254 - sbyte) << 23);  // 2^-e, exact
#define BATQ_V8(r) __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(acc[r], l, u) * inv, -448.0f, 448.0f)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v2i16 r = {0, 0};
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, BATQ_V8(4 * q), BATQ_V8(4 * q + 1), 1.0f, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, BATQ_V8(4 * q + 2), BATQ_V8(4 * q + 3), 1.0f, true);
      wq[q] = __builtin_bit_cast(uint32_t, r);
    }
#undef BATQ_V8
  }
  // wq[q] holds channels 8q + 4h .. 8q + 4h + 3.  Half 0 keeps channels 0..15
  // (its q0, q1 and the partner's), half 1 channels 16..31.
  const uint32_t s0 = h ? wq[0] : wq[2];
  const uint32_t s1 = h ? wq[1] : wq[3];
  const auto r0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
  const uint32_t p0 = h ? r0[0] : r0[1];
  const uint32_t p1 = h ? r1[0] : r1[1];
  return h ? make_uint4(p0, wq[2], p1, wq[3]) : make_uint4(wq[0], p0, wq[1], p1);
}

}  // namespace batq
