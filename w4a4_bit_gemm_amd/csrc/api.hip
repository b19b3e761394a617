// C ABI of the BATQuant W4A4 path: argument checks, host helpers, launches.
// Every check runs before any HIP call; see include/batq.h for the contract.
#include <math.h>
#include <string.h>

#include "batq.h"
#include "common.h"

namespace {

bool is_pow2_factor(int32_t a) { return a == 1 || a == 2 || a == 4 || a == 8 || a == 16 || a == 32; }

int log2_exact(int32_t a) {
  int l = 0;
  while ((1 << l) < a) ++l;
  return l;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Gauss-Jordan inverse with partial pivoting in double.  Writes inv^T.
// Returns false for a zero pivot or a 1-norm condition estimate above 1e6.
bool invert_transpose(int n, const float* m, float* out_T) {
  double aug[32][64];
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < n; ++j) aug[i][j] = (double)m[i * n + j];
    for (int j = 0; j < n; ++j) aug[i][n + j] = (i == j) ? 1.0 : 0.0;
  }
  double norm_m = 0.0;
  for (int j = 0; j < n; ++j) {
    double c = 0.0;
    for (int i = 0; i < n; ++i) c += fabs((double)m[i * n + j]);
    if (c > norm_m) norm_m = c;
  }
  for (int col = 0; col < n; ++col) {
    int piv = col;
    for (int r = col + 1; r < n; ++r)
      if (fabs(aug[r][col]) > fabs(aug[piv][col])) piv = r;
    if (aug[piv][col] == 0.0) return false;
    if (piv != col)
      for (int j = 0; j < 2 * n; ++j) {
        double t = aug[col][j];
        aug[col][j] = aug[piv][j];
        aug[piv][j] = t;
      }
    const double d = aug[col][col];
    for (int j = 0; j < 2 * n; ++j) aug[col][j] /= d;
    for (int r = 0; r < n; ++r) {
      if (r == col || aug[r][col] == 0.0) continue;
      const double f = aug[r][col];
      for (int j = 0; j < 2 * n; ++j) aug[r][j] -= f * aug[col][j];
    }
  }
  double norm_inv = 0.0;
  for (int j = 0; j < n; ++j) {
    double c = 0.0;
    for (int i = 0; i < n; ++i) c += fabs(aug[i][n + j]);
    if (c > norm_inv) norm_inv = c;
  }
  if (!(norm_m * norm_inv <= 1e6)) return false;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) out_T[j * n + i] = (float)aug[i][n + j];
  return true;
}

batq_status check_transform_args(const void* x, int64_t rows, int64_t K, int64_t ld, int32_t a, int32_t b,
                                 const float* A, const float* B, const float* r_hi, const float* r_lo,
                                 const uint8_t* q, const uint8_t* s) {
  if (rows < 0 || K < 0 || ld < 0) return BATQ_ERR_SHAPE;
  if (K == 0 || K % 32 != 0 || ld < K) return BATQ_ERR_SHAPE;
  if ((int64_t)a * (int64_t)b != 32) return BATQ_ERR_SHAPE;
  if (!is_pow2_factor(a)) return BATQ_ERR_UNSUPPORTED;
  if (x == nullptr || A == nullptr || B == nullptr || q == nullptr || s == nullptr) return BATQ_ERR_NULL;
  if ((r_hi == nullptr) != (r_lo == nullptr)) return BATQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || ld % 8 != 0) return BATQ_ERR_ALIGN;
  if (!aligned(A, 4) || !aligned(B, 4) || (r_hi && (!aligned(r_hi, 4) || !aligned(r_lo, 4))))
    return BATQ_ERR_ALIGN;
  return BATQ_OK;
}

batq_status run_transform(const void* x, int64_t rows, int64_t K, int64_t ld, int32_t a, const float* A,
                          const float* B, const float* r_hi, const float* r_lo, int64_t r_ld, uint8_t* q,
                          uint8_t* s, hipStream_t stream, int fp8 = 0, const int64_t* slot = nullptr,
                          int64_t out_rows = 0) {
  if (rows == 0) return BATQ_OK;
  batq::TransformQuantArgs args;
  args.x = static_cast<const uint16_t*>(x);
  args.ldx = ld;
  args.rows = rows;
  args.K = K;
  args.a_log2 = log2_exact(a);
  args.A = A;
  args.B = B;
  args.r_hi = r_hi;
  args.r_lo = r_lo;
  args.r_ld = r_ld;
  args.q = q;
  args.s = s;
  args.fp8 = fp8;
  args.slot = slot;
  args.out_rows = out_rows;
  return batq::launch_transform_quant(args, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

}  // namespace

extern "C" {

int batq_abi_version(void) { return BATQ_ABI_VERSION; }

const char* batq_status_str(int status) {
  switch (status) {
    case BATQ_OK: return "ok";
    case BATQ_ERR_NULL: return "a required pointer is NULL";
    case BATQ_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 32, ld >= K, a*b == 32)";
    case BATQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case BATQ_ERR_UNSUPPORTED: return "unsupported factor size or output type";
    case BATQ_ERR_SINGULAR: return "singular or ill-conditioned transform factor";
    case BATQ_ERR_HIP: return "HIP launch failed";
    case BATQ_ERR_TOO_LARGE: return "the problem needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

batq_status batq_clip_ratios(const float* logits_host, float* ratios_host, int64_t n) {
  if (n < 0) return BATQ_ERR_SHAPE;
  if (n > 0 && (logits_host == nullptr || ratios_host == nullptr)) return BATQ_ERR_NULL;
  for (int64_t i = 0; i < n; ++i) ratios_host[i] = (float)(1.0 / (1.0 + exp(-(double)logits_host[i])));
  return BATQ_OK;
}

batq_status batq_gpk_invert(int32_t a, int32_t b, int64_t nblocks, const float* A_host, const float* B_host,
                            float* AinvT_host, float* BinvT_host) {
  if (nblocks < 0 || (int64_t)a * (int64_t)b != 32) return BATQ_ERR_SHAPE;
  if (!is_pow2_factor(a)) return BATQ_ERR_UNSUPPORTED;
  if (A_host == nullptr || AinvT_host == nullptr) return BATQ_ERR_NULL;
  if (nblocks > 0 && (B_host == nullptr || BinvT_host == nullptr)) return BATQ_ERR_NULL;
  if (!invert_transpose(a, A_host, AinvT_host)) return BATQ_ERR_SINGULAR;
  for (int64_t i = 0; i < nblocks; ++i)
    if (!invert_transpose(b, B_host + i * b * b, BinvT_host + i * b * b)) return BATQ_ERR_SINGULAR;
  return BATQ_OK;
}

batq_status batq_act_transform_quant(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a,
                                     int32_t b, const float* A, const float* B, const float* r_hi,
                                     const float* r_lo, uint8_t* Xq, uint8_t* Xs, hipStream_t stream) {
  const batq_status st = check_transform_args(X_bf16, M, K, ldx, a, b, A, B, r_hi, r_lo, Xq, Xs);
  if (st != BATQ_OK) return st;
  return run_transform(X_bf16, M, K, ldx, a, A, B, r_hi, r_lo, 0, Xq, Xs, stream);
}

batq_status batq_weight_prep(const void* W_bf16, int64_t N, int64_t K, int64_t ldw, int32_t a, int32_t b,
                             const float* AinvT, const float* BinvT, const float* wr_hi, const float* wr_lo,
                             uint8_t* Wq, uint8_t* Ws, hipStream_t stream) {
  const batq_status st = check_transform_args(W_bf16, N, K, ldw, a, b, AinvT, BinvT, wr_hi, wr_lo, Wq, Ws);
  if (st != BATQ_OK) return st;
  return run_transform(W_bf16, N, K, ldw, a, AinvT, BinvT, wr_hi, wr_lo, K / 32, Wq, Ws, stream);
}

batq_status batq_mxfp4_gemm(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                            int64_t M, int64_t N, int64_t K, void* Y, batq_out_dtype out, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return BATQ_ERR_SHAPE;
  if (K == 0 || K % 32 != 0) return BATQ_ERR_SHAPE;
  if (out != BATQ_OUT_BF16 && out != BATQ_OUT_F32) return BATQ_ERR_UNSUPPORTED;
  if (Xq == nullptr || Xs == nullptr || Wq == nullptr || Ws == nullptr || Y == nullptr) return BATQ_ERR_NULL;
  if (!aligned(Xq, 16) || !aligned(Wq, 16) || !aligned(Y, 4)) return BATQ_ERR_ALIGN;
  if (M == 0 || N == 0) return BATQ_OK;
  batq::GemmArgs args;
  args.xq = Xq;
  args.xs = Xs;
  args.wq = Wq;
  args.ws = Ws;
  args.M = M;
  args.N = N;
  args.K = K;
  args.y = Y;
  args.out_f32 = (out == BATQ_OUT_F32);
  args.vec_store = aligned(Y, 16) && (N % (args.out_f32 ? 4 : 8) == 0);
  return batq::launch_mxfp4_gemm(args, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

int64_t batq_weight_packed_bytes(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % 256 != 0) return -1;
  return batq::packed_weight_bytes(N, K);
}

batq_status batq_weight_pack(const uint8_t* Wq, const uint8_t* Ws, int64_t N, int64_t K, uint8_t* Wp,
                             hipStream_t stream) {
  if (N < 0 || K <= 0 || K % 256 != 0) return BATQ_ERR_SHAPE;
  if (Wq == nullptr || Ws == nullptr || Wp == nullptr) return BATQ_ERR_NULL;
  if (!aligned(Wq, 16) || !aligned(Wp, 16)) return BATQ_ERR_ALIGN;
  if (N == 0) return BATQ_OK;
  return batq::launch_weight_pack(Wq, Ws, N, K, Wp, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

batq_status batq_mxfp4_gemm_packed(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wp, int64_t M,
                                   int64_t N, int64_t K, void* Y, batq_out_dtype out, hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 256 != 0) return BATQ_ERR_SHAPE;
  if (out != BATQ_OUT_BF16 && out != BATQ_OUT_F32) return BATQ_ERR_UNSUPPORTED;
  if (Xq == nullptr || Xs == nullptr || Wp == nullptr || Y == nullptr) return BATQ_ERR_NULL;
  if (!aligned(Xq, 16) || !aligned(Xs, 16) || !aligned(Wp, 16) || !aligned(Y, 4)) return BATQ_ERR_ALIGN;
  if (M == 0 || N == 0) return BATQ_OK;
  batq::GemmArgs args;
  args.xq = Xq;
  args.xs = Xs;
  args.wq = Wp;
  args.ws = nullptr;
  args.M = M;
  args.N = N;
  args.K = K;
  args.y = Y;
  args.out_f32 = (out == BATQ_OUT_F32);
  args.vec_store = aligned(Y, 16) && (N % (args.out_f32 ? 4 : 8) == 0);
  return batq::launch_mxfp4_gemm_packed(args, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

batq_status batq_act_transform_quant_mxfp8(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a,
                                           int32_t b, const float* A, const float* B, const float* r_hi,
                                           const float* r_lo, uint8_t* Xq8, uint8_t* Xs, hipStream_t stream) {
  const batq_status st = check_transform_args(X_bf16, M, K, ldx, a, b, A, B, r_hi, r_lo, Xq8, Xs);
  if (st != BATQ_OK) return st;
  return run_transform(X_bf16, M, K, ldx, a, A, B, r_hi, r_lo, 0, Xq8, Xs, stream, 1);
}

batq_status batq_mxfp8_gemm_packed(const uint8_t* Xq8, const uint8_t* Xs, const uint8_t* Wp, int64_t M, int64_t N,
                                   int64_t K, void* Y, batq_out_dtype out, hipStream_t stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 256 != 0) return BATQ_ERR_SHAPE;
  if (out != BATQ_OUT_BF16 && out != BATQ_OUT_F32) return BATQ_ERR_UNSUPPORTED;
  if (Xq8 == nullptr || Xs == nullptr || Wp == nullptr || Y == nullptr) return BATQ_ERR_NULL;
  if (!aligned(Xq8, 16) || !aligned(Xs, 16) || !aligned(Wp, 16) || !aligned(Y, 4)) return BATQ_ERR_ALIGN;
  if (M == 0 || N == 0) return BATQ_OK;
  batq::GemmArgs args;
  args.xq = Xq8;
  args.xs = Xs;
  args.wq = Wp;
  args.ws = nullptr;
  args.M = M;
  args.N = N;
  args.K = K;
  args.y = Y;
  args.out_f32 = (out == BATQ_OUT_F32);
  args.vec_store = aligned(Y, 16) && (N % (args.out_f32 ? 4 : 8) == 0);
  args.a_fp8 = 1;
  return batq::launch_mxfp4_gemm_packed(args, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}


int32_t batq_transform_kernel(int64_t rows, int64_t K) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
  return batq::transform_uses_one_per_cu(rows, K) ? 1 : 0;
}

int32_t batq_packed_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t act_fp8) {
  if (M < 0 || N < 0 || K <= 0 || K % 256 != 0) return -1;
  batq::GemmArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  a.a_fp8 = act_fp8 != 0;
  return batq::packed_dma_applies(a) ? 1 : 0;
}

int64_t batq_decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || M > BATQ_DECODE_MAX_M || N < 0 || N > batq::kDecodeMaxN || K <= 0 || K % 256 != 0 ||
      K > BATQ_DECODE_MAX_K)
    return -1;
  return batq::decode_workspace_bytes(M, N, K);
}

namespace {

// Checks shared by both decode entry points (everything but the workspace).
batq_status check_decode_args(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, int32_t b,
                              const float* A, const float* B, const float* r_hi,
                              const float* r_lo, const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out,
                              uint8_t* Xq, uint8_t* Xs) {
  if (M < 0 || M > BATQ_DECODE_MAX_M || N < 0 || N > batq::kDecodeMaxN || K <= 0 || K % 256 != 0 ||
      K > BATQ_DECODE_MAX_K || ldx < K)
    return BATQ_ERR_SHAPE;
  if ((int64_t)a * (int64_t)b != 32) return BATQ_ERR_SHAPE;
  if (!is_pow2_factor(a)) return BATQ_ERR_UNSUPPORTED;
  if (out != BATQ_OUT_BF16 && out != BATQ_OUT_F32) return BATQ_ERR_UNSUPPORTED;
  if (X_bf16 == nullptr || A == nullptr || B == nullptr || Wp == nullptr || Y == nullptr) return BATQ_ERR_NULL;
  if ((r_hi == nullptr) != (r_lo == nullptr) || (Xq == nullptr) != (Xs == nullptr)) return BATQ_ERR_NULL;
  if (!aligned(X_bf16, 16) || ldx % 8 != 0 || !aligned(Wp, 16) || !aligned(Y, 4))
    return BATQ_ERR_ALIGN;
  if (!aligned(A, 4) || !aligned(B, 4) || (r_hi && (!aligned(r_hi, 4) || !aligned(r_lo, 4))) ||
      (Xq && !aligned(Xq, 8)))
    return BATQ_ERR_ALIGN;
  return BATQ_OK;
}

batq_status run_decode(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, const float* A,
                       const float* B, const float* r_hi, const float* r_lo,
                       const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out, uint8_t* Xq, uint8_t* Xs,
                       void* part, hipStream_t stream) {
  batq::DecodeArgs args;
  args.x = static_cast<const uint16_t*>(X_bf16);
  args.ldx = ldx;
  args.M = M;
  args.K = K;
  args.N = N;
  args.a_log2 = log2_exact(a);
  args.A = A;
  args.B = B;
  args.r_hi = r_hi;
  args.r_lo = r_lo;
  args.wp = Wp;
  args.y = Y;
  args.out_f32 = out == BATQ_OUT_F32;
  args.xq = Xq;
  args.xs = Xs;
  args.part = static_cast<float*>(part);
  return batq::launch_decode_fused(args, stream) == hipSuccess ? BATQ_OK : BATQ_ERR_HIP;
}

}  // namespace

batq_status batq_w4a4_decode(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, int32_t b,
                             const float* A, const float* B, const float* r_hi,
                             const float* r_lo, const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out,
                             uint8_t* Xq, uint8_t* Xs, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  const batq_status st =
      check_decode_args(X_bf16, M, K, ldx, a, b, A, B, r_hi, r_lo, Wp, N, Y, out, Xq, Xs);
  if (st != BATQ_OK) return st;
  if (workspace == nullptr) return BATQ_ERR_NULL;
  if (!aligned(workspace, 256)) return BATQ_ERR_ALIGN;
  if (workspace_bytes < batq::decode_workspace_bytes(M, N, K)) return BATQ_ERR_SHAPE;
  if (M == 0 || N == 0) return BATQ_OK;
  return run_decode(X_bf16, M, K, ldx, a, A, B, r_hi, r_lo, Wp, N, Y, out, Xq, Xs, workspace, stream);
}

int64_t batq_decode_noalloc_scratch_bytes(void) { return batq::kDecodeScratchBytes; }

batq_status batq_w4a4_decode_noalloc(const void* X_bf16, int64_t M, int64_t K, int64_t ldx, int32_t a, int32_t b,
                                     const float* A, const float* B, const float* r_hi,
                                     const float* r_lo, const uint8_t* Wp, int64_t N, void* Y, batq_out_dtype out,
                                     uint8_t* Xq, uint8_t* Xs, hipStream_t stream) {
  const batq_status st =
      check_decode_args(X_bf16, M, K, ldx, a, b, A, B, r_hi, r_lo, Wp, N, Y, out, Xq, Xs);
  if (st != BATQ_OK) return st;
  if (batq::decode_workspace_bytes(M, N, K) > batq::kDecodeScratchBytes) return BATQ_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return BATQ_OK;
  void* part = nullptr;
  if (batq::decode_scratch(&part) != hipSuccess || part == nullptr) return BATQ_ERR_HIP;
  return run_decode(X_bf16, M, K, ldx, a, A, B, r_hi, r_lo, Wp, N, Y, out, Xq, Xs, part, stream);
}

batq_status batq_kv_cache_quant(const void* KV_bf16, int64_t T, int64_t HD, int64_t ld, int32_t a, int32_t b,
                                const float* A, const float* B, const float* r_hi, const float* r_lo,
                                const int64_t* slots, int64_t cache_rows, int32_t fmt, uint8_t* cache_q,
                                uint8_t* cache_s, hipStream_t stream) {
  if (cache_rows < 0) return BATQ_ERR_SHAPE;
  if (fmt != 4 && fmt != 8) return BATQ_ERR_UNSUPPORTED;
  const batq_status st = check_transform_args(KV_bf16, T, HD, ld, a, b, A, B, r_hi, r_lo, cache_q, cache_s);
  if (st != BATQ_OK) return st;
  if (T > 0 && slots == nullptr) return BATQ_ERR_NULL;
  if (!aligned(slots, 8)) return BATQ_ERR_ALIGN;
  return run_transform(KV_bf16, T, HD, ld, a, A, B, r_hi, r_lo, 0, cache_q, cache_s, stream, fmt == 8 ? 1 : 0, slots,
                       cache_rows);
}

}  // extern "C"
