"""Comparison helpers for the GPU parity tests (HIP path vs oracle)."""
from __future__ import annotations

import numpy as np

from oracle import batquant as ob

U32 = 2.0 ** -24


def rank(codes: np.ndarray) -> np.ndarray:
    """Position of an E2M1 code on the signed value line (-6 ... -0, +0 ... 6)."""
    c = codes.astype(np.int64)
    mag = c & 7
    return np.where(c & 8, -mag - 1, mag)


def compare_quant(packed_gpu: np.ndarray, scales_gpu: np.ndarray, dec: ob.Decisions, *, max_frac: float = 1e-5,
                  label: str = "") -> dict:
    """Scales bit-exact outside free blocks; codes bit-exact outside the free set
    (free elements and the codes of free blocks), exact zeros may carry either
    sign; every mismatch at a free element is to an adjacent code; mismatches
    are fewer than ``max_frac`` of the elements on large inputs."""
    codes_gpu = ob.unpack_codes(packed_gpu)
    assert codes_gpu.shape == dec.codes.shape, label
    assert scales_gpu.shape == dec.scales.shape, label
    rows, K = dec.codes.shape
    blk_free_el = np.repeat(dec.block_free, 32, axis=1)
    bad_scale = (scales_gpu != dec.scales) & ~dec.block_free
    assert not bad_scale.any(), f"{label}: {int(bad_scale.sum())} scale mismatches outside free blocks, " \
                                f"first at {np.argwhere(bad_scale)[0].tolist()}"
    mism = codes_gpu != dec.codes
    zero_ok = dec.zero_sign_free & ((codes_gpu & 7) == 0) & ((dec.codes & 7) == 0)
    mism &= ~zero_ok
    hard = mism & ~dec.elem_free & ~blk_free_el
    if hard.any():
        m, k = np.argwhere(hard)[0]
        raise AssertionError(f"{label}: {int(hard.sum())} code mismatches outside the free set; first at row {m} "
                             f"col {k}: gpu {codes_gpu[m, k]} oracle {dec.codes[m, k]} y64 {dec.y64[m, k]!r} "
                             f"scale {dec.scales[m, k // 32]}")
    soft = mism & dec.elem_free & ~blk_free_el
    if soft.any():
        assert np.all(np.abs(rank(codes_gpu[soft]) - rank(dec.codes[soft])) <= 1), label
    n_mism = int(mism.sum())
    n = rows * K
    if n >= 100_000:
        assert n_mism < max_frac * n, f"{label}: {n_mism} mismatches of {n}"
    return {"elements": n, "mismatches": n_mism, "free": dec.n_exempt,
            "free_blocks": int(dec.block_free.sum())}


def gemm_bound(abs_sum: np.ndarray, K: int) -> np.ndarray:
    """Worst-case fp32 accumulation error of a K-term dot product whose products
    are exact: gamma_K * sum |x w| (Higham), with gamma_K = K u / (1 - K u)."""
    return (K * U32 / (1.0 - K * U32)) * abs_sum


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) -> float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
