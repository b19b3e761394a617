"""Planted mistakes in the oracle (CPU only).

Each case replaces one oracle function with a plausible wrong version of it:
a dropped term, a transposed operand, a swapped index or factor, a wrong sign or
constant. It then checks that at least one of the oracle's pins in
test_oracle.py fails. A mutation that every pin accepted would mean the pins do
not constrain that part of the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import batquant as ob
from tests import test_oracle as T


def _orig(name):
    return getattr(ob, name)


def _kron_swapped(A, B):
    A64, B64 = np.asarray(A, np.float64), np.asarray(B, np.float64)
    return np.stack([np.kron(A64, B64[i]) for i in range(B64.shape[0])])


def _kron_dropped_offdiag_a(A, B):
    A64, B64 = np.asarray(A, np.float64), np.asarray(B, np.float64)
    return np.stack([np.kron(B64[i], np.diag(np.diag(A64))) for i in range(B64.shape[0])])


def _transform_transposed(X, P):
    return _orig_transform(X, np.swapaxes(P, -1, -2))


def _transform_dropped_term(X, P):
    P2 = np.array(P, dtype=np.float64, copy=True)
    P2[:, 31, :] = 0.0  # the last channel of every block no longer contributes
    return _orig_transform(X, P2)


def _clip_order_swapped(Y32, r_hi, r_lo, fmt="e2m1"):
    Y32 = np.asarray(Y32, dtype=np.float32)
    rows, K = Y32.shape
    nb = K // 32
    yb = Y32.reshape(rows, nb, 32)
    rh = ob._broadcast_ratio(r_hi, rows, nb)
    rl = ob._broadcast_ratio(r_lo, rows, nb)
    u = (rh * yb.max(axis=2)).astype(np.float32)
    l = (rl * yb.min(axis=2)).astype(np.float32)
    z = np.maximum(np.minimum(yb, u[..., None]), l[..., None])  # min first: wrong
    emax, rnd, _ = ob.element_format(fmt)
    e = ob.shared_exponent(np.abs(z).max(axis=2), emax)
    codes = rnd(np.ldexp(z.astype(np.float64), -e[..., None])).reshape(rows, K)
    return codes, (e + 127).astype(np.uint8), z.reshape(rows, K)


def _clip_ratios_swapped(Y32, r_hi, r_lo, fmt="e2m1"):
    return _orig_clip(Y32, r_lo, r_hi, fmt)


def _round_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    mag = ((m >= 0.25).astype(np.int64) + (m >= 0.75) + (m >= 1.25) + (m >= 1.75)
           + (m >= 2.5) + (m >= 3.5) + (m >= 5.0))
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def _round_no_saturation_step(v):
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    mag = ((m > 0.25).astype(np.int64) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
           + (m > 2.5) + (m >= 3.5))  # the 4 -> 6 step is missing
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def _round_unsigned_zero(v):
    codes = _orig_round(v)
    return np.where((codes & 7) == 0, 0, codes).astype(np.uint8)


def _exponent_off_by_one(amax, emax=2):
    return np.clip(_orig_exp(amax, emax) + 1, -127, 127)


def _exponent_via_log2(amax, emax=2):
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(amax.astype(np.float32))).astype(np.int64) - emax
    return np.clip(np.where(amax == 0, -127, e), -127, 127)


def _pack_high_nibble_first(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def _dequantize_scale_dropped(codes, scale_bytes, fmt="e2m1"):
    return ob.element_format(fmt)[2](codes)


def _dequantize_scale_sign(codes, scale_bytes, fmt="e2m1"):
    rows, K = codes.shape
    vals = ob.element_format(fmt)[2](codes).reshape(rows, K // 32, 32)
    sc = np.ldexp(1.0, 127 - np.asarray(scale_bytes, dtype=np.int64))  # wrong sign of the exponent
    return (vals * sc[..., None]).reshape(rows, K)


def _inverse_not_transposed(A, B):
    P = ob.block_matrices(A, B)
    return np.stack([np.linalg.inv(P[i]) for i in range(P.shape[0])])


def _sigmoid_wrong_sign(logits):
    x = np.asarray(logits, dtype=np.float64)
    return (1.0 / (1.0 + np.exp(x))).astype(np.float32)


def _e4m3_ties_up(v):
    v = np.asarray(v, dtype=np.float64)
    m = np.minimum(np.abs(v), ob.E4M3_MAX)
    g = ob.E4M3_GRID
    code = np.clip(np.searchsorted(g, m, side="right") - 1, 0, 126)
    nxt = np.clip(code + 1, 0, 126)
    code = np.where(m - g[code] >= g[nxt] - m, nxt, code)  # ties upward: wrong
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _e4m3_no_subnormals(v):
    codes = _orig_e4m3(v)
    return np.where((codes & 0x78) == 0, codes & 0x80, codes).astype(np.uint8)  # flush to zero


_orig_e4m3 = _orig("e4m3_round")
_orig_transform = _orig("transform")
_orig_clip = _orig("clip_and_quantize")
_orig_round = _orig("e2m1_round")
_orig_exp = _orig("shared_exponent")

KRON = [lambda: T.test_kron_block_matrix_equals_explicit_loops_and_factored_form(8),
        lambda: T.test_kron_block_matrix_equals_explicit_loops_and_factored_form(4)]
ROUND = [T.test_e2m1_round_equals_brute_force_nearest, T.test_e2m1_round_properties,
         T.test_e2m1_ties_go_to_even_code_not_away_from_zero, T.test_negative_values_rounding_to_zero_keep_sign,
         T.test_worked_examples]
SCALE = [T.test_shared_exponent_closed_form_at_powers_of_two, T.test_shared_exponent_puts_amax_in_4_to_8,
         T.test_worked_examples]
CLIP = [T.test_clip_bounds_are_ratio_times_block_max_and_min, T.test_clip_single_sign_block_order]
GEMM = [T.test_dequantize_uses_block_scale, T.test_gemm_fp64_equals_exact_rationals_on_tiny,
        T.test_end_to_end_approximates_unquantised_layer]

CASES = {
    "kron factors swapped": ("block_matrices", _kron_swapped, KRON),
    "off-diagonal of A dropped": ("block_matrices", _kron_dropped_offdiag_a, KRON),
    "transform transposed (column-vector convention)": ("transform", _transform_transposed, KRON),
    "one channel's term dropped from the transform": ("transform", _transform_dropped_term, KRON),
    "clamp order swapped": ("clip_and_quantize", _clip_order_swapped, CLIP),
    "clip ratios swapped": ("clip_and_quantize", _clip_ratios_swapped, CLIP),
    "ties rounded away from zero": ("e2m1_round", _round_ties_away, ROUND),
    "saturation step missing": ("e2m1_round", _round_no_saturation_step, ROUND),
    "sign of rounded zero dropped": ("e2m1_round", _round_unsigned_zero, ROUND),
    "scale exponent off by one": ("shared_exponent", _exponent_off_by_one, SCALE),
    "floor(log2) from a rounded logarithm": ("shared_exponent", _exponent_via_log2, SCALE),
    "nibble order swapped": ("pack_codes", _pack_high_nibble_first, [T.test_pack_low_nibble_is_even_element]),
    "block scale dropped in dequantisation": ("dequantize", _dequantize_scale_dropped, GEMM),
    "scale exponent sign flipped in dequantisation": ("dequantize", _dequantize_scale_sign, GEMM),
    "weight side uses P^-1 instead of P^-T": ("inverse_transpose_blocks", _inverse_not_transposed,
                                              [T.test_kron_inverse_identity,
                                               T.test_linear_layer_equivalence_without_quantisation]),
    "sigmoid sign flipped": ("clip_ratio", _sigmoid_wrong_sign, [T.test_clip_ratio_matches_library_sigmoid]),
    "E4M3 ties rounded upward": ("e4m3_round", _e4m3_ties_up,
                                 [T.test_e4m3_round_equals_brute_force_nearest, T.test_mxfp8_scale_rule_and_worked_block]),
    "E4M3 subnormals flushed": ("e4m3_round", _e4m3_no_subnormals, [T.test_e4m3_round_equals_brute_force_nearest]),
    "E4M3 largest exponent taken as 7": ("shared_exponent",
                                         lambda amax, emax=2: _orig_exp(amax, 7 if emax == 8 else emax),
                                         [T.test_mxfp8_scale_rule_and_worked_block]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    fn_name, mutant, pins = CASES[name]
    monkeypatch.setattr(ob, fn_name, mutant)
    failed = []
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(getattr(pin, "__name__", "pin"))
    assert failed, f"no pin caught the planted mistake: {name}"
