"""Vectorised fp64 oracle of the BATQuant deployment path (test infrastructure only).

What the path computes, and where the pages say so:

* A linear layer Y = X W^T is rewritten as Y = (X P)(P^-1 W^T) with an invertible
  P; the activation side X P is computed online and the weight side P^-1 W^T is
  fused offline; with quantisation Q both sides are quantised, Q(XP) Q(P^-1 W^T)
  [BATQuant note (en.papernotes.org), Key Designs §1, the arg-min objective;
  Overall Architecture; A Worked Example].
* P is block diagonal; each block acts only on the 32 channels of one MXFP
  quantisation block and carries no translation term [same page, Key Designs §1].
* Each block is P_i = B_i (x) A (Kronecker product) with one shared 8x8 A and a
  private 4x4 B_i per block; the shared size is swept over {1, 2, 4, 8, 16, 32}
  with the private size 32/|A| [nubint.ai review, 提案手法; en.papernotes.org,
  Key Designs §2].
* Block-wise learnable clipping: two ratios per quantisation block, mapped into
  (0, 1) by a sigmoid, act on the block maximum and minimum; weights get the
  analogous treatment [en.papernotes.org, Key Designs §3].
* MXFP4: E2M1 elements whose positive values are 0.5, 1, 1.5, 2, 3, 4, 6 (plus
  zero and negatives), one UE8M0 (power-of-two) scale per 32 elements
  [en.papernotes.org, Background & Motivation; 10100.com BRQ article, section 1].
* Order on the online path: transform block by block, clip, quantise, multiply by
  the processed weights [en.papernotes.org, A Worked Example].

Readings where the pages are silent or damaged (each is also listed in the design
notes of the repository):

* Vec convention (the pages say the equations giving it are damaged): row-vector,
  y_b = x_b P_i with x_b the 32 channels of block i in channel order, and
  P_i[a*r + c, a*r' + c'] = B_i[r, r'] * A[c, c'] (numpy.kron(B_i, A)).
* Clip: bounds u = sigmoid(alpha_i) * max(y_b), l = sigmoid(beta_i) * min(y_b);
  values are clamped, z = min(max(y, l), u) (max with l first), and the scale is
  derived from the clamped block.  Ratios are sigmoid evaluated in fp64 and
  rounded once to fp32; that fp32 value is the deployed parameter.
* Scale: the pages fix only a power-of-two scale per 32 elements.  The exponent
  follows the OCP Microscaling v1.0 conversion: e = floor(log2(amax)) - 2 (2 is
  the largest exponent of E2M1), clamped to [-127, 127]; an all-zero block gets
  e = -127.  The stored byte is e + 127.
* Element rounding: nearest E2M1 value, ties to the even code, magnitudes >= 6
  saturate to 6; the sign bit is kept, so a negative value that rounds to zero is
  code 0x8.  Codes are packed two per byte, even element in the low nibble.
* Decision precision: the transform is exact here (fp64 on bf16 inputs, error far
  below an fp32 ulp); its result is held in fp32, the precision the GPU kernel
  takes its clip/scale/rounding decisions in, and the clip bounds are fp32
  products.  Everything after that is exact in fp32.
* Weight side: W' = W P^-T block by block (the transpose of P^-1 W^T), then the
  same clip (one ratio pair per (output row, block); no clip when absent) and the
  same quantiser.  Plain round-to-nearest (RTN) replaces GPTQ, which needs
  calibration data.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# MXFP4 element and scale format
# ---------------------------------------------------------------------------

#: E2M1 magnitudes of codes 0..7 (code bit 3 is the sign).  The seven positive
#: values are printed on the pages [en.papernotes.org, Background & Motivation].
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_MAX_EXP = 2  # 6 = 1.5 * 2**2
BLOCK = 32  # MX block size and transform block size


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    """Code (0..15) -> value in fp64: (-1)^bit3 * grid[bits 0..2]."""
    code = np.asarray(code).astype(np.int64)
    mag = np.asarray(E2M1_GRID, dtype=np.float64)[code & 7]
    return np.where(code & 8, -mag, mag)


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """Round fp64 values (already divided by the block scale) to E2M1 codes.

    Nearest grid value; on a tie the value with the even code wins; magnitudes
    beyond 6 take 6.  The magnitude code is the number of grid midpoints the
    magnitude has passed, where a tie counts as passed exactly when the upper
    neighbour's code is even (midpoints 0.75, 1.75, 3.5) and as not passed when
    the lower neighbour's code is even (0.25, 1.25, 2.5, 5).
    """
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    mag = ((m > 0.25).astype(np.int64) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
           + (m > 2.5) + (m >= 3.5) + (m > 5.0))
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def shared_exponent(amax: np.ndarray, emax: int = E2M1_MAX_EXP) -> np.ndarray:
    """OCP MX scale exponent of a block: floor(log2 amax) - emax (emax: the
    largest exponent of the element format, 2 for E2M1, 8 for E4M3), clamped
    to [-127, 127]; amax == 0 gives -127.  floor(log2) is read exactly from the
    binary exponent (frexp), never from a rounded logarithm."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)  # amax = mant * 2**ex with mant in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - emax
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127)


# ---------------------------------------------------------------------------
# MXFP8 (E4M3) elements, for the W4A8 setting of the pages
# ---------------------------------------------------------------------------
# The pages report a W4A8 configuration (MXFP8 activations with MXFP4 weights)
# [nubint.ai review, Table 2] and name E4M3 as its element format
# [en.papernotes.org, Loss & Training].  The bit-level definition is the OCP
# MX v1.0 E4M3 format: sign, 4 exponent bits (bias 7), 3 mantissa bits,
# subnormals at exponent field 0, no infinities, S.1111.111 is NaN, largest
# finite value 448 = 1.75 * 2**8.

E4M3_MAX_EXP = 8
E4M3_MAX = 448.0


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Code (0..255) -> value in fp64 (NaN for S.1111.111)."""
    c = np.asarray(code).astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


#: The 127 finite non-negative E4M3 values, in code order (codes 0..126).
E4M3_GRID = e4m3_decode(np.arange(127))


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Round fp64 values (already divided by the block scale) to E4M3 codes:
    the nearest finite grid value, ties to the even code, magnitudes from 448
    upward saturate to 448; the sign bit is kept (so -0 is code 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    m = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(E4M3_GRID, m, side="left")  # first grid value >= m
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = m - E4M3_GRID[lo]
    d_hi = E4M3_GRID[hi] - m
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(E4M3_GRID[hi] == m, hi, np.where(take_hi, hi, lo))
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


#: Element formats of the MX quantiser: largest exponent and the names of the
#: rounding and decoding functions (looked up at call time).
_FORMATS = {
    "e2m1": (E2M1_MAX_EXP, "e2m1_round", "e2m1_decode"),
    "e4m3": (E4M3_MAX_EXP, "e4m3_round", "e4m3_decode"),
}


def element_format(fmt: str):
    """(largest exponent, rounding function, decoding function) of ``fmt``."""
    emax, rnd, dec = _FORMATS[fmt]
    g = globals()
    return emax, g[rnd], g[dec]


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, K] codes -> [rows, K/2] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize(codes: np.ndarray, scale_bytes: np.ndarray, fmt: str = "e2m1") -> np.ndarray:
    """MX codes -> fp64: element value times 2^(byte - 127) of its 32-block."""
    rows, K = codes.shape
    vals = element_format(fmt)[2](codes).reshape(rows, K // BLOCK, BLOCK)
    sc = np.ldexp(1.0, np.asarray(scale_bytes, dtype=np.int64) - 127)
    return (vals * sc[..., None]).reshape(rows, K)


# ---------------------------------------------------------------------------
# Transform parameters
# ---------------------------------------------------------------------------


def clip_ratio(logits: np.ndarray) -> np.ndarray:
    """sigmoid(logit) evaluated in fp64 and rounded once to fp32."""
    x = np.asarray(logits, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def block_matrices(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Explicit per-block matrices P_i = kron(B_i, A), fp64, shape [nb, 32, 32]."""
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    return np.stack([np.kron(B64[i], A64) for i in range(B64.shape[0])])


def inverse_transpose_blocks(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """P_i^-T for every block, from the explicit 32x32 matrix (numpy.linalg.inv)."""
    P = block_matrices(A, B)
    return np.stack([np.linalg.inv(P[i]).T for i in range(P.shape[0])])


def param_count_gpk(K: int, a: int) -> int:
    """Shared A (a x a) plus one private B_i ((32/a) x (32/a)) per block."""
    b = BLOCK // a
    return a * a + (K // BLOCK) * b * b


def param_count_naive_kron(K: int, a: int) -> int:
    """Both Kronecker factors stored for every block."""
    b = BLOCK // a
    return (K // BLOCK) * (a * a + b * b)


def param_count_full_blocks(K: int) -> int:
    """A full 32x32 matrix per block."""
    return (K // BLOCK) * BLOCK * BLOCK


def param_count_flatquant(K: int) -> int:
    """A global Kronecker factorisation with two sqrt(K) x sqrt(K) factors.  The
    pages print 8,192 at K = 4096 for FlatQuant; 2 * 64^2 is our inference of
    how that number arises."""
    s = int(round(math.sqrt(K)))
    return 2 * s * s


# ---------------------------------------------------------------------------
# Transform, clip and quantisation
# ---------------------------------------------------------------------------


def transform(X: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Y[:, block i] = X[:, block i] @ P_i in fp64 (row-vector convention)."""
    X64 = np.asarray(X, dtype=np.float64)
    rows, K = X64.shape
    nb = K // BLOCK
    Xb = X64.reshape(rows, nb, BLOCK).transpose(1, 0, 2)  # [nb, rows, 32]
    Y = np.matmul(Xb, P)  # [nb, rows, 32]
    return np.ascontiguousarray(Y.transpose(1, 0, 2)).reshape(rows, K)


def transform_abs_sum(X: np.ndarray, P: np.ndarray) -> np.ndarray:
    """S[:, j] = sum_k |x_k| |P_i[k, j]|: the scale of every fp32 rounding error
    any evaluation of the transform can make."""
    return transform(np.abs(np.asarray(X, dtype=np.float64)), np.abs(P))


def _broadcast_ratio(r: Optional[np.ndarray], rows: int, nb: int) -> np.ndarray:
    if r is None:
        return np.ones((rows, nb), dtype=np.float32)
    r = np.asarray(r, dtype=np.float32)
    return np.broadcast_to(r, (rows, nb)) if r.ndim == 1 else r


def clip_and_quantize(Y32: np.ndarray, r_hi: Optional[np.ndarray], r_lo: Optional[np.ndarray],
                      fmt: str = "e2m1"):
    """Clip every 32-block of fp32 values and quantise it to MXFP4 (``fmt``
    "e2m1") or MXFP8 ("e4m3").

    Returns (codes uint8 [rows, K], scale bytes uint8 [rows, K/32], z fp32).
    r_hi, r_lo: fp32 ratios, shape [K/32] (shared over rows) or [rows, K/32];
    None means no clipping (ratio 1, which leaves every value unchanged).
    """
    Y32 = np.asarray(Y32, dtype=np.float32)
    rows, K = Y32.shape
    nb = K // BLOCK
    yb = Y32.reshape(rows, nb, BLOCK)
    rh = _broadcast_ratio(r_hi, rows, nb)
    rl = _broadcast_ratio(r_lo, rows, nb)
    hi = yb.max(axis=2)
    lo = yb.min(axis=2)
    u = (rh * hi).astype(np.float32)  # fp32 products, round to nearest
    l = (rl * lo).astype(np.float32)
    z = np.minimum(np.maximum(yb, l[..., None]), u[..., None])
    amax = np.abs(z).max(axis=2)
    emax, rnd, _ = element_format(fmt)
    e = shared_exponent(amax, emax)
    v = np.ldexp(z.astype(np.float64), -e[..., None])  # exact
    codes = rnd(v).reshape(rows, K)
    scales = (e + 127).astype(np.uint8)
    return codes, scales, z.reshape(rows, K)


# ---------------------------------------------------------------------------
# Decision intervals: which outputs an fp32 evaluation of the transform may flip
# ---------------------------------------------------------------------------

#: Worst number of fp32 roundings one transformed value sees in the GPU kernel:
#: a + b <= 33 for the factored product, plus 2 for the fp32 rounding of the
#: inverted factors on the weight side, plus one spare.
ROUNDINGS = 36
_U32 = 2.0 ** -24


def gamma(n: int, u: float = _U32) -> float:
    """Higham's gamma_n = n u / (1 - n u)."""
    return n * u / (1.0 - n * u)


@dataclass
class Decisions:
    codes: np.ndarray  # uint8 [rows, K]
    scales: np.ndarray  # uint8 [rows, nb]
    block_free: np.ndarray  # bool [rows, nb]: scale may legitimately differ
    elem_free: np.ndarray  # bool [rows, K]: code may legitimately differ
    zero_sign_free: np.ndarray  # bool [rows, K]: exact zero, codes 0x0 / 0x8 both valid
    y64: np.ndarray  # fp64 transformed values
    z32: np.ndarray  # fp32 clipped values (oracle's)

    @property
    def n_exempt(self) -> int:
        blk = np.repeat(self.block_free, BLOCK, axis=1)
        return int(np.count_nonzero(self.elem_free | blk))


def _interval_abs(lo: np.ndarray, hi: np.ndarray):
    a_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    a_hi = np.maximum(np.abs(lo), np.abs(hi))
    return a_lo, a_hi


def decisions(Y64: np.ndarray, S: np.ndarray, r_hi, r_lo, exact: bool = False, fmt: str = "e2m1") -> Decisions:
    """Quantise the fp64 transform result and mark every decision that an fp32
    evaluation of it may take the other way.

    The GPU kernel's fp32 transform value of element j lies within
    beta_j = gamma_ROUNDINGS * S_j of the exact value (Higham's bound for sums of
    products, S_j = sum |x||P|).  Every later step is monotone in its inputs
    (max/min, the clip, |.|, the exponent, the division by 2^e, the rounding), so
    running them on the interval ends bounds every value the kernel can reach:
    a block whose scale exponent differs between the ends is free (scale and all
    its codes), an element whose code differs between the ends is free.  Every
    other decision is fixed by the exact result and must match bit for bit.
    ``exact=True`` asserts the kernel's arithmetic is exact for these inputs (for
    example A and B_i identities on bf16 data) and marks nothing free.
    """
    Y64 = np.asarray(Y64, dtype=np.float64)
    rows, K = Y64.shape
    nb = K // BLOCK
    Y32 = Y64.astype(np.float32)
    codes, scales, z32 = clip_and_quantize(Y32, r_hi, r_lo, fmt)
    emax, rnd, _ = element_format(fmt)
    zero_sign_free = (np.asarray(S) == 0.0)
    if exact:
        f = np.zeros((rows, K), dtype=bool)
        return Decisions(codes, scales, np.zeros((rows, nb), bool), f, zero_sign_free, Y64, z32)

    beta = (gamma(ROUNDINGS) + 2.0 ** -45) * np.asarray(S, dtype=np.float64)
    rh = _broadcast_ratio(r_hi, rows, nb).astype(np.float64)
    rl = _broadcast_ratio(r_lo, rows, nb).astype(np.float64)
    y_lo = (Y64 - beta).reshape(rows, nb, BLOCK)
    y_hi = (Y64 + beta).reshape(rows, nb, BLOCK)
    hi_lo, hi_hi = y_lo.max(axis=2), y_hi.max(axis=2)
    lo_lo, lo_hi = y_lo.min(axis=2), y_hi.min(axis=2)
    w = 2.0 ** -22  # covers rounding the extremum to fp32 and the fp32 product
    u_lo, u_hi = rh * hi_lo, rh * hi_hi
    u_lo, u_hi = u_lo - w * np.abs(u_lo), u_hi + w * np.abs(u_hi)
    l_lo, l_hi = rl * lo_lo, rl * lo_hi
    l_lo, l_hi = l_lo - w * np.abs(l_lo), l_hi + w * np.abs(l_hi)
    z_lo = np.minimum(np.maximum(y_lo, l_lo[..., None]), u_lo[..., None])
    z_hi = np.minimum(np.maximum(y_hi, l_hi[..., None]), u_hi[..., None])
    a_lo, a_hi = _interval_abs(z_lo, z_hi)
    e_lo = shared_exponent(a_lo.max(axis=2), emax)
    e_hi = shared_exponent(a_hi.max(axis=2), emax)
    block_free = e_lo != e_hi
    e = e_hi
    c_lo = rnd(np.ldexp(z_lo, -e[..., None]))
    c_hi = rnd(np.ldexp(z_hi, -e[..., None]))
    elem_free = (c_lo != c_hi).reshape(rows, K) & ~zero_sign_free
    return Decisions(codes, scales, block_free, elem_free, zero_sign_free, Y64, z32)


# ---------------------------------------------------------------------------
# The two sides of the layer
# ---------------------------------------------------------------------------


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def act_transform_quant(X_bits: np.ndarray, A: np.ndarray, B: np.ndarray,
                        alpha: Optional[np.ndarray], beta: Optional[np.ndarray],
                        exact: bool = False, fmt: str = "e2m1") -> Decisions:
    """Online activation path: y_b = x_b P_i, clip with sigmoid(alpha_i) * max and
    sigmoid(beta_i) * min (no clipping when the logits are None), MX quantise:
    MXFP4 (``fmt`` "e2m1", the W4A4 path) or MXFP8 ("e4m3", the W4A8 setting)
    [en.papernotes.org, A Worked Example; Key Designs §1-§3]."""
    if (alpha is None) != (beta is None):
        raise ValueError("alpha and beta must both be given or both be None")
    X = bf16_values(X_bits)
    P = block_matrices(A, B)
    Y = transform(X, P)
    S = transform_abs_sum(X, P)
    rh = None if alpha is None else clip_ratio(alpha)
    rl = None if beta is None else clip_ratio(beta)
    return decisions(Y, S, rh, rl, exact=exact, fmt=fmt)


def kv_cache_rows(slots: np.ndarray, cache_rows: int) -> np.ndarray:
    """Placement of new K/V rows in a cache: input row t lands in cache row
    slots[t]; a slot outside [0, cache_rows) places nothing.  Returns the input
    row of every cache row (-1: not written)."""
    src = np.full(cache_rows, -1, dtype=np.int64)
    for t, r in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= r < cache_rows:
            src[r] = t
    return src


def kv_cache_quant(KV_bits: np.ndarray, A: np.ndarray, B: np.ndarray, alpha: Optional[np.ndarray],
                   beta: Optional[np.ndarray], fmt: str = "e2m1", exact: bool = False) -> Decisions:
    """K or V rows (all heads of a token side by side, head_dim a multiple of 32)
    through the per-block transform, clipping and MX quantisation of the
    activation path, MXFP4 (KV4) or MXFP8 E4M3 (KV8) [en.papernotes.org,
    Overall Architecture: transforms on the key and value cache paths, per
    head; nubint.ai review, Table 2: KV8, KV4].  The decisions are per input
    row; kv_cache_rows gives their cache rows."""
    return act_transform_quant(KV_bits, A, B, alpha, beta, exact=exact, fmt=fmt)


def weight_prep(W_bits: np.ndarray, A: np.ndarray, B: np.ndarray,
                walpha: Optional[np.ndarray], wbeta: Optional[np.ndarray],
                exact: bool = False) -> Decisions:
    """Offline weight side: W' = W P^-T per block (that is (P^-1 W^T)^T), clip
    with per-(row, block) ratios (none when the logits are None), MXFP4 quantise
    [en.papernotes.org, Overall Architecture; Key Designs §1, §3]."""
    W = bf16_values(W_bits)
    PinvT = inverse_transpose_blocks(A, B)
    Y = transform(W, PinvT)
    S = transform_abs_sum(W, PinvT)
    rh = None if walpha is None else clip_ratio(walpha)
    rl = None if wbeta is None else clip_ratio(wbeta)
    return decisions(Y, S, rh, rl, exact=exact)


def gemm(xq_codes: np.ndarray, xs: np.ndarray, wq_codes: np.ndarray, ws: np.ndarray,
         x_fmt: str = "e2m1") -> np.ndarray:
    """Y = deq(Xq) deq(Wq)^T in fp64 [en.papernotes.org, Key Designs §1: the
    product Q(XP) Q(P^-1 W^T)]; the activation codes are MXFP4 or, for W4A8,
    MXFP8 (``x_fmt`` "e4m3"); weights are MXFP4."""
    return dequantize(xq_codes, xs, x_fmt) @ dequantize(wq_codes, ws).T


def gemm_abs(xq_codes, xs, wq_codes, ws, x_fmt: str = "e2m1") -> np.ndarray:
    """sum_k |x_k w_k| for every output: the scale of fp32 accumulation error."""
    return np.abs(dequantize(xq_codes, xs, x_fmt)) @ np.abs(dequantize(wq_codes, ws)).T


def gemm_rows_cols(xq_codes, xs, wq_codes, ws, rows, cols, x_fmt: str = "e2m1"):
    """Sampled outputs Y[rows][:, cols] and their abs-sums, one by one."""
    Xd = dequantize(xq_codes[rows], xs[rows], x_fmt)
    Wd = dequantize(wq_codes[cols], ws[cols])
    return Xd @ Wd.T, np.abs(Xd) @ np.abs(Wd).T


def unquantized_layer(X_bits, W_bits) -> np.ndarray:
    """Y = X W^T in fp64 on the bf16 inputs (no transform, no quantisation)."""
    return bf16_values(X_bits) @ bf16_values(W_bits).T
