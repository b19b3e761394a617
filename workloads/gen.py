"""Seeded generators for the five linear-layer workloads.

Shapes follow the Qwen3-8B layers the BATQuant pages evaluate on (hidden 4096,
MLP intermediate 12288; calibration sequences of 2048 tokens; batch 64 x prefill
256 = 16384 tokens for the end-to-end speed point) [BATQuant note
(en.papernotes.org), Loss & Training; Key Findings].  The outlier recipe for the
down-projection input uses the "top 0.1 % by magnitude" notion of an outlier from
the BRQ article [10100.com BRQ article, section 4, Figure 6 caption].  No model,
dataset or trained transform is available, so every tensor is synthetic.

Recipe (all draws in float64, then rounded once to float32, then to bfloat16 with
round-to-nearest-even on the bit pattern):

* seeds: ``numpy.random.default_rng(1000*cfg + t)`` with tensor ids
  t = 0:X, 1:W, 2:A, 3:B, 4:alpha, 5:beta, 6:weight alpha, 7:weight beta,
  8:outlier picks, 9:second SwiGLU operand.  The shared-factor sweep draws its
  factors from ``default_rng(1000*cfg + 100*a + t)``.
* A = I_a + 0.05 N(0,1), B_i = I_b + 0.05 N(0,1) (float32 parameters).
* clip logits alpha, beta ~ N(3, 0.5) per block; weight logits ~ N(3, 0.5) per
  (output row, block) (float32 parameters).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

SWEEP_A = (1, 2, 4, 8, 16, 32)


@dataclass(frozen=True)
class ConfigSpec:
    cfg: int
    name: str
    M: int
    K: int
    N: int
    x_kind: str  # "normal" | "t3" | "swiglu"
    outliers: str  # description, see _apply_outliers


CONFIGS: Dict[int, ConfigSpec] = {
    1: ConfigSpec(1, "tiny", 64, 256, 256, "normal", "channels 7,200 x40"),
    2: ConfigSpec(2, "upgate_prefill", 2048, 4096, 12288, "t3", "8 random channels x50"),
    3: ConfigSpec(3, "down_prefill", 2048, 12288, 4096, "swiglu", "0.1% entries x100"),
    4: ConfigSpec(4, "decode", 16, 4096, 4096, "t3", "8 random channels x50"),
    5: ConfigSpec(5, "large_prefill", 16384, 4096, 4096, "t3", "8 random channels x50"),
}


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest) -> bfloat16 bits (round to nearest even)."""
    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f32.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    cfg: int
    M: int
    K: int
    N: int
    a: int
    b: int
    X_bits: np.ndarray  # uint16 [M, K] bf16 activations
    W_bits: Optional[np.ndarray]  # uint16 [N, K] bf16 weights
    A: np.ndarray  # float32 [a, a]   shared factor
    B: np.ndarray  # float32 [nb, b, b] private factors
    alpha: np.ndarray  # float32 [nb] upper clip logits
    beta: np.ndarray  # float32 [nb] lower clip logits
    walpha: Optional[np.ndarray]  # float32 [N, nb]
    wbeta: Optional[np.ndarray]  # float32 [N, nb]
    meta: dict = field(default_factory=dict)

    @property
    def nb(self) -> int:
        return self.K // 32


def _rng(cfg: int, t: int, a: Optional[int] = None) -> np.random.Generator:
    if a is None:
        return np.random.default_rng(1000 * cfg + t)
    return np.random.default_rng(1000 * cfg + 100 * a + t)


def _draw_x(spec: ConfigSpec, M: int, K: int) -> np.ndarray:
    r0 = _rng(spec.cfg, 0)
    if spec.x_kind == "normal":
        x = r0.standard_normal((M, K))
    elif spec.x_kind == "t3":
        x = r0.standard_t(3, size=(M, K))
    elif spec.x_kind == "swiglu":
        g = r0.standard_normal((M, K))
        u = _rng(spec.cfg, 9).standard_normal((M, K))
        x = g / (1.0 + np.exp(-g)) * u
    else:  # pragma: no cover
        raise ValueError(spec.x_kind)
    r8 = _rng(spec.cfg, 8)
    if spec.cfg == 1:
        x[:, [7, 200]] *= 40.0
    elif spec.x_kind == "t3":
        ch = r8.choice(K, size=8, replace=False)
        x[:, ch] *= 50.0
    elif spec.x_kind == "swiglu":
        n = int(round(0.001 * M * K))
        idx = r8.choice(M * K, size=n, replace=False)
        x.reshape(-1)[idx] *= 100.0
    return x


def make_factors(cfg: int, K: int, a: int, sweep: bool = False):
    """Near-identity GPK factors A (a x a) and B_i (b x b), float32."""
    b = 32 // a
    nb = K // 32
    key = a if sweep else None
    A = np.eye(a) + 0.05 * _rng(cfg, 2, key).standard_normal((a, a))
    B = np.eye(b)[None, :, :] + 0.05 * _rng(cfg, 3, key).standard_normal((nb, b, b))
    return A.astype(np.float32), B.astype(np.float32)


def _sylvester(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_factors(K: int, a: int = 8):
    """Block-Hadamard factors, float32: A = H_a / sqrt(a) and every B_i =
    H_b / sqrt(b) (b = 32 / a), so that P_i = B_i (x) A = H_32 / sqrt(32)
    (Sylvester ordering), the block rotation of the BRQ article (10100.com)."""
    b = 32 // a
    A = (_sylvester(a) / np.sqrt(a)).astype(np.float32)
    B = np.tile((_sylvester(b) / np.sqrt(b)).astype(np.float32), (K // 32, 1, 1))
    return A, B


def make_workload(cfg: int, a: int = 8, M: Optional[int] = None, with_weights: bool = True) -> Workload:
    """Build config ``cfg`` (1..5).  ``M`` overrides the token count (rows are
    drawn for the full config and the first M kept, so a smaller M is a prefix of
    the full activation); ``a`` selects the shared-factor size (b = 32 / a)."""
    spec = CONFIGS[cfg]
    if a not in SWEEP_A:
        raise ValueError(f"shared factor size must be one of {SWEEP_A}")
    K, N = spec.K, spec.N
    Mfull = spec.M
    x = _draw_x(spec, Mfull, K)
    Mx = Mfull if M is None else M
    if Mx > Mfull:
        raise ValueError("M larger than the config's token count")
    X_bits = f64_to_bf16_bits(x[:Mx])
    del x
    nb = K // 32
    A, B = make_factors(cfg, K, a, sweep=(cfg == 5))
    alpha = _rng(cfg, 4).normal(3.0, 0.5, nb).astype(np.float32)
    beta = _rng(cfg, 5).normal(3.0, 0.5, nb).astype(np.float32)
    W_bits = walpha = wbeta = None
    if with_weights:
        W_bits = f64_to_bf16_bits(_rng(cfg, 1).normal(0.0, 0.02, (N, K)))
        walpha = _rng(cfg, 6).normal(3.0, 0.5, (N, nb)).astype(np.float32)
        wbeta = _rng(cfg, 7).normal(3.0, 0.5, (N, nb)).astype(np.float32)
    return Workload(spec.name, cfg, Mx, K, N, a, 32 // a, X_bits, W_bits, A, B,
                    alpha, beta, walpha, wbeta, meta={"x_kind": spec.x_kind, "outliers": spec.outliers})


def make_custom(M: int, K: int, N: int, a: int = 8, seed: int = 0, x_kind: str = "t3",
                outlier_scale: float = 50.0, n_outlier_channels: int = 2) -> Workload:
    """Small seeded workload of any shape (ragged sizes, edge cases)."""
    if K % 32 or a not in SWEEP_A:
        raise ValueError("K must be a multiple of 32 and a one of the sweep sizes")
    rng = np.random.default_rng(seed)
    if x_kind == "t3":
        x = rng.standard_t(3, size=(M, K))
    else:
        x = rng.standard_normal((M, K))
    if n_outlier_channels and M > 0:
        ch = rng.choice(K, size=min(n_outlier_channels, K), replace=False)
        x[:, ch] *= outlier_scale
    b = 32 // a
    nb = K // 32
    A = (np.eye(a) + 0.05 * rng.standard_normal((a, a))).astype(np.float32)
    B = (np.eye(b)[None] + 0.05 * rng.standard_normal((nb, b, b))).astype(np.float32)
    alpha = rng.normal(3.0, 0.5, nb).astype(np.float32)
    beta = rng.normal(3.0, 0.5, nb).astype(np.float32)
    W = rng.normal(0.0, 0.02, (N, K))
    walpha = rng.normal(3.0, 0.5, (N, nb)).astype(np.float32)
    wbeta = rng.normal(3.0, 0.5, (N, nb)).astype(np.float32)
    return Workload(f"custom_{M}x{K}x{N}_a{a}_s{seed}", 0, M, K, N, a, b, f64_to_bf16_bits(x),
                    f64_to_bf16_bits(W), A, B, alpha, beta, walpha, wbeta, meta={"x_kind": x_kind})


# ------------------------------------------------------------ large operands
#
# Operands larger than 2 GiB are built from a seeded base of R0 rows: row r of
# the large operand is base row r % R0, its columns rotated by `unit` times
# (r // R0) % `period` positions (whole MX blocks), so that every group of R0
# rows differs from the others and a row read from the wrong group gives
# different values.  The device side applies the same rotation per group
# (large_group_shift); the host side rebuilds any sampled row (large_rows).


def large_group_shift(group: int, unit: int, period: int) -> int:
    """Column rotation of row group `group` (rows group*R0 .. group*R0 + R0 - 1)."""
    return unit * (group % period)


def large_rows(base: np.ndarray, rows: np.ndarray, unit: int, period: int) -> np.ndarray:
    """Rows `rows` of the large operand built from `base` (see above)."""
    R0 = base.shape[0]
    out = np.empty((len(rows), base.shape[1]), dtype=base.dtype)
    for i, r in enumerate(np.asarray(rows, dtype=np.int64)):
        out[i] = np.roll(base[r % R0], large_group_shift(int(r // R0), unit, period))
    return out
