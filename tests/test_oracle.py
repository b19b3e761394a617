"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages print, a closed form, an
invariant, a textbook algorithm (brute force, Walsh-Hadamard) or a library
routine, chosen so that a plausible slip (transposed Kronecker factor, column
instead of row convention, dropped clip, log2-based exponent, ties away from
zero, lost sign of zero, wrong nibble order) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special

from oracle import batquant as ob
from oracle import scalar as osc
from tests.conftest import golden_path
from workloads import gen

# ---------------------------------------------------------------- E2M1 format


def _read_grid():
    with open(golden_path("e2m1_grid.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    return [float(t) for t in rows[0].split()]


def test_e2m1_positive_values_match_pages():
    printed = _read_grid()
    assert printed == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    pos = sorted(set(ob.e2m1_decode(np.arange(16))) - {0.0})
    assert [v for v in pos if v > 0] == printed
    assert [v for v in pos if v < 0] == [-v for v in reversed(printed)]


def test_e2m1_decode_codes_and_signed_zero():
    vals = ob.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == [0.0] + _read_grid()
    assert list(vals[8:]) == [-0.0] + [-v for v in _read_grid()]
    assert np.signbit(vals[8]) and not np.signbit(vals[0])


def _sweep_values():
    grid = np.arange(-8 * 4096, 8 * 4096 + 1, dtype=np.float64) / 4096.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    extra = []
    for m in np.concatenate([mids, -mids]):
        f = np.float32(m)
        extra += [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    extra += [-0.0, 0.0, 6.0, -6.0, 7.999, -7.999]
    return np.concatenate([grid, np.array(extra, dtype=np.float64)])


def test_e2m1_round_equals_brute_force_nearest():
    """Vectorised rounding (midpoint counting) equals an exhaustive nearest-value
    search with ties to the even code, on every multiple of 2^-12 in [-8, 8] and
    on each midpoint and its fp32 neighbours."""
    v = _sweep_values()
    got = ob.e2m1_round(v)
    signed = np.array([(c, ob.e2m1_decode(c)) for c in range(16)], dtype=object)
    for x, c in zip(v, got):
        # brute force over all 16 codes; prefer the even magnitude code on ties
        best = None
        for code, val in signed:
            if math.copysign(1.0, val) != math.copysign(1.0, x) and val != 0.0:
                continue
            if (code & 8) != (8 if math.copysign(1.0, x) < 0 else 0):
                continue
            d = abs(abs(x) - abs(val))
            key = (d, (code & 7) % 2)
            if best is None or key < best[0]:
                best = (key, code)
        assert c == best[1], (x, c, best)
        assert osc.round_e2m1(float(x)) == c


def test_e2m1_round_properties():
    v = _sweep_values()
    v = v[np.argsort(v, kind="stable")]
    codes = ob.e2m1_round(v)
    deq = ob.e2m1_decode(codes)
    # monotone non-decreasing in value
    assert np.all(np.diff(deq) >= 0)
    # within half the local grid step for |v| <= 6; saturates beyond
    grid = np.array(ob.E2M1_GRID)
    for x, d in zip(v, deq):
        ax = abs(x)
        if ax <= 6.0:
            hi = grid[np.searchsorted(grid, ax)] if ax < 6 else 6.0
            lo = grid[max(np.searchsorted(grid, ax, side="right") - 1, 0)]
            assert abs(abs(d) - ax) <= (hi - lo) / 2 + 1e-15
        else:
            assert abs(d) == 6.0
    # every grid value is a fixed point
    for c in range(16):
        assert ob.e2m1_round(ob.e2m1_decode(c)) == c


def test_e2m1_ties_go_to_even_code_not_away_from_zero():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]  # even codes: 0, 1.0, 1.0, 2, 2, 4, 4
    assert list(ob.e2m1_round(np.array(mids))) == want
    assert list(ob.e2m1_round(-np.array(mids))) == [w | 8 for w in want]


def test_negative_values_rounding_to_zero_keep_sign():
    assert ob.e2m1_round(np.array([-0.1]))[0] == 8
    assert ob.e2m1_round(np.array([-0.0]))[0] == 8
    assert ob.e2m1_round(np.array([0.1]))[0] == 0


# ----------------------------------------------------------------- scale rule


def test_shared_exponent_closed_form_at_powers_of_two():
    for k in range(-120, 126):
        p = np.float32(2.0 ** k)
        below = np.nextafter(p, np.float32(0))
        assert ob.shared_exponent(np.array([p]))[0] == max(k - 2, -127)
        assert ob.shared_exponent(np.array([below]))[0] == max(k - 3, -127)
        assert osc.scale_exponent(float(p)) == max(k - 2, -127)
        assert osc.scale_exponent(float(below)) == max(k - 3, -127)
    assert ob.shared_exponent(np.array([0.0]))[0] == -127


def test_shared_exponent_puts_amax_in_4_to_8():
    rng = np.random.default_rng(7)
    amax = np.exp(rng.uniform(-60, 60, 20000)).astype(np.float32).astype(np.float64)
    e = ob.shared_exponent(amax)
    v = np.ldexp(amax, -e)
    assert np.all((v >= 4.0) & (v < 8.0))


def test_log2_shortcut_is_caught():
    """The pin above catches a floor(np.log2(.)) exponent: just below a power of
    two, the float32 log2 rounds up to the integer."""
    below = np.nextafter(np.float32(8.0), np.float32(0))
    naive = int(np.floor(np.log2(below))) - 2
    assert naive != ob.shared_exponent(np.array([below]))[0]


def _read_worked():
    sec, amax_rows, block = None, [], {}
    with open(golden_path("mx_worked_examples.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            if ln.startswith("["):
                sec = ln
                continue
            if sec == "[amax]":
                a, s, c = ln.split()
                amax_rows.append((np.float32(a), int(s), int(c)))
            else:
                key, *vals = ln.split()
                block[key] = vals
    return amax_rows, block


def test_worked_examples():
    amax_rows, block = _read_worked()
    for amax, sbyte, code in amax_rows:
        y = np.zeros((1, 32), dtype=np.float32)
        y[0, 3] = amax
        codes, scales, _ = ob.clip_and_quantize(y, None, None)
        assert scales[0, 0] == sbyte, amax
        assert codes[0, 3] == code, amax
        assert np.all(codes[0, np.arange(32) != 3] == 0)
    y = np.zeros((1, 32), dtype=np.float32)
    vals = np.array([float(t) for t in block["values"]], dtype=np.float32)
    y[0, : len(vals)] = vals
    codes, scales, _ = ob.clip_and_quantize(y, None, None)
    assert scales[0, 0] == int(block["scale"][0])
    assert list(codes[0, : len(vals)]) == [int(t) for t in block["codes"]]
    # scalar form agrees
    c2, s2 = osc.quantize_block([float(v) for v in y[0]], 1.0, 1.0)
    assert c2 == list(codes[0]) and s2 == scales[0, 0]


def test_zero_block():
    codes, scales, _ = ob.clip_and_quantize(np.zeros((2, 64), np.float32), None, None)
    assert np.all(scales == 0) and np.all(codes == 0)


def test_pack_low_nibble_is_even_element():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    packed = ob.pack_codes(codes)
    assert list(packed[0]) == [0x21, 0x43, 0x0F]
    assert np.array_equal(ob.unpack_codes(packed), codes)


def test_dequantize_uses_block_scale():
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 7  # 6
    codes[0, 33] = 0xA  # -1
    deq = ob.dequantize(codes, np.array([[127 + 3, 127 - 2]], np.uint8))
    assert deq[0, 0] == 48.0 and deq[0, 33] == -0.25 and np.count_nonzero(deq) == 2


# --------------------------------------------------------------- clip ratios


def test_clip_ratio_matches_library_sigmoid():
    x = np.random.default_rng(3).normal(3, 2, 5000).astype(np.float32)
    r = ob.clip_ratio(x)
    assert r.dtype == np.float32
    assert np.array_equal(r, scipy.special.expit(x.astype(np.float64)).astype(np.float32))
    assert ob.clip_ratio(np.array([0.0]))[0] == np.float32(0.5)
    assert ob.clip_ratio(np.array([40.0]))[0] == np.float32(1.0)
    assert all(osc.sigmoid_f32(float(v)) == float(w) for v, w in zip(x[:200], r[:200]))


# ----------------------------------------------------------- clip semantics


def test_clip_bounds_are_ratio_times_block_max_and_min():
    """Values are clamped to [r_lo*min, r_hi*max] of their own block and the scale
    follows the clamped block."""
    y = np.zeros((1, 32), np.float32)
    y[0, :4] = [10.0, -4.0, 1.0, -1.0]
    r_hi = np.array([0.5], np.float32)
    r_lo = np.array([0.25], np.float32)
    codes, scales, z = ob.clip_and_quantize(y, r_hi, r_lo)
    assert z[0, 0] == 5.0 and z[0, 1] == -1.0 and z[0, 2] == 1.0 and z[0, 3] == -1.0
    # amax 5 -> e = 0; 5 is a tie -> 4 (code 6)
    assert scales[0, 0] == 127 and codes[0, 0] == 6
    # without the clip the scale would follow 10
    _, s0, _ = ob.clip_and_quantize(y, None, None)
    assert s0[0, 0] == 128


def test_clip_single_sign_block_order():
    """All-positive block with r_lo*min > r_hi*max: the fixed order
    min(max(y, l), u) maps every element to u."""
    y = np.full((1, 32), 2.0, np.float32)
    y[0, 0] = 2.5
    r_hi = np.array([0.5], np.float32)  # u = 1.25
    r_lo = np.array([0.9], np.float32)  # l = 1.8
    _, _, z = ob.clip_and_quantize(y, r_hi, r_lo)
    assert np.all(z == np.float32(1.25))
    c2, s2 = osc.quantize_block([float(v) for v in y[0]], 0.5, float(np.float32(0.9)))
    codes, scales, _ = ob.clip_and_quantize(y, r_hi, r_lo)
    assert c2 == list(codes[0]) and s2 == scales[0, 0]


# ---------------------------------------------------------------- transform


@pytest.mark.parametrize("a", gen.SWEEP_A)
def test_kron_block_matrix_equals_explicit_loops_and_factored_form(a):
    b = 32 // a
    rng = np.random.default_rng(a)
    A = rng.standard_normal((a, a))
    B = rng.standard_normal((3, b, b))
    P = ob.block_matrices(A, B)
    for i in range(3):
        assert np.array_equal(P[i], np.array(osc.block_matrix(A.tolist(), B[i].tolist())))
        assert np.array_equal(P[i], np.kron(B[i], A))
    X = rng.standard_normal((5, 96))
    Y = ob.transform(X, P)
    # factored "two small matmuls" on the b x a tile: Y_b = B_i^T X_b A
    for i in range(3):
        Xb = X[:, 32 * i: 32 * i + 32].reshape(5, b, a)
        Yf = np.einsum("rs,mrc,cd->msd", B[i], Xb, A).reshape(5, 32)
        assert np.allclose(Y[:, 32 * i: 32 * i + 32], Yf, rtol=1e-12, atol=1e-12)
    if a not in (1, 32) and a != b:
        # a transposed convention (column vector, P_i x) is a different map
        wrong = np.einsum("kj,mj->mk", P[0], X[:, :32])
        assert not np.allclose(wrong, Y[:, :32])


def test_kron_inverse_identity():
    rng = np.random.default_rng(11)
    A = np.eye(8) + 0.05 * rng.standard_normal((8, 8))
    B = np.eye(4)[None] + 0.05 * rng.standard_normal((4, 4, 4))
    PinvT = ob.inverse_transpose_blocks(A, B)
    for i in range(4):
        fac = np.kron(np.linalg.inv(B[i]), np.linalg.inv(A)).T
        assert np.allclose(PinvT[i], fac, rtol=1e-12, atol=1e-12)
        assert np.allclose(scipy.linalg.inv(np.kron(B[i], A)).T, PinvT[i], rtol=1e-12, atol=1e-13)


def test_linear_layer_equivalence_without_quantisation():
    """(X P)(P^-1 W^T) = X W^T, block by block (each 32-channel partial product
    is preserved), with random invertible non-orthogonal factors."""
    wl = gen.make_custom(16, 128, 24, a=4, seed=5)
    X = ob.bf16_values(wl.X_bits)
    W = ob.bf16_values(wl.W_bits)
    P = ob.block_matrices(wl.A, wl.B)
    PinvT = ob.inverse_transpose_blocks(wl.A, wl.B)
    Xp = ob.transform(X, P)
    Wp = ob.transform(W, PinvT)
    ref = X @ W.T
    assert np.allclose(Xp @ Wp.T, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
    for i in range(4):
        s = slice(32 * i, 32 * i + 32)
        assert np.allclose(Xp[:, s] @ Wp[:, s].T, X[:, s] @ W[:, s].T, rtol=1e-10, atol=1e-12)


def test_locality_no_output_depends_on_another_block():
    wl = gen.make_custom(8, 256, 8, a=8, seed=9)
    d0 = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    X2 = wl.X_bits.copy()
    X2[:, 96:128] = gen.f64_to_bf16_bits(np.random.default_rng(1).standard_normal((8, 32)) * 30)
    d1 = ob.act_transform_quant(X2, wl.A, wl.B, wl.alpha, wl.beta)
    other = np.ones(256, bool)
    other[96:128] = False
    assert np.array_equal(d0.codes[:, other], d1.codes[:, other])
    assert np.array_equal(np.delete(d0.scales, 3, axis=1), np.delete(d1.scales, 3, axis=1))
    assert np.array_equal(d0.y64[:, other], d1.y64[:, other])
    assert not np.array_equal(d0.codes[:, ~other], d1.codes[:, ~other])


def _fwht(x):
    """Iterative fast Walsh-Hadamard transform (natural/Sylvester order)."""
    x = np.array(x, dtype=np.float64)
    h = 1
    n = x.shape[-1]
    while h < n:
        y = x.reshape(x.shape[:-1] + (n // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        x = y.reshape(x.shape)
        h *= 2
    return x


def test_block_hadamard_special_case_is_orthogonal_fwht():
    """A = H8/sqrt(8), B_i = H4/2 gives P_i = H32/sqrt(32) (Sylvester), the
    block rotation of the BRQ article (10100.com, section 5): energy preserving,
    equal to a fast Walsh-Hadamard transform of each block."""
    H8 = scipy.linalg.hadamard(8) / math.sqrt(8)
    H4 = scipy.linalg.hadamard(4) / 2.0
    P = ob.block_matrices(H8, np.stack([H4, H4]))
    assert np.allclose(P[0], scipy.linalg.hadamard(32) / math.sqrt(32), atol=1e-15)
    X = np.random.default_rng(2).standard_normal((6, 64))
    Y = ob.transform(X, P)
    assert np.allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)
    assert np.allclose(np.linalg.norm(Y[:, :32], axis=1), np.linalg.norm(X[:, :32], axis=1), rtol=1e-13)
    ref = np.concatenate([_fwht(X[:, :32]), _fwht(X[:, 32:])], axis=1) / math.sqrt(32)
    assert np.allclose(Y, ref, atol=1e-13)


def test_extreme_shared_sizes():
    rng = np.random.default_rng(4)
    B1 = rng.standard_normal((2, 32, 32))
    P = ob.block_matrices(np.ones((1, 1)), B1)
    assert np.array_equal(P, B1)  # a = 1: one full private matrix per block
    A32 = rng.standard_normal((32, 32))
    Bs = rng.standard_normal((2, 1, 1))
    P = ob.block_matrices(A32, Bs)
    assert np.allclose(P[1], Bs[1, 0, 0] * A32)  # a = 32: scalar times shared


# ------------------------------------------------------------ param counts


def test_parameter_counts_match_pages():
    with open(golden_path("param_counts.txt")) as f:
        kv = dict(ln.split() for ln in f if ln.strip() and not ln.startswith("#"))
    K = int(kv["hidden"])
    assert ob.param_count_full_blocks(K) == int(kv["full_blocks"])
    assert ob.param_count_naive_kron(K, 8) == int(kv["naive_kronecker"])
    assert ob.param_count_gpk(K, 8) == int(kv["gpk"])
    assert ob.param_count_flatquant(K) == int(kv["flatquant"])
    lo = 100 * (1 - ob.param_count_gpk(K, 8) / ob.param_count_flatquant(K))
    hi = 100 * (1 - ob.param_count_gpk(K, 8) / ob.param_count_naive_kron(K, 8))
    assert math.floor(lo) == int(kv["reduction_low_percent"])
    assert math.floor(hi) == int(kv["reduction_high_percent"])
    # the shared-size sweep of the pages: private size is 32/|A|
    for a in gen.SWEEP_A:
        assert ob.param_count_gpk(K, a) == a * a + 128 * (32 // a) ** 2


# --------------------------------------------------- scalar vs vectorised


def test_scalar_and_vectorised_oracle_agree_on_tiny():
    wl = gen.make_workload(1)
    d = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    c, s = osc.act_transform_quant(wl.X_bits.tolist(), wl.A.tolist(), wl.B.tolist(),
                                   wl.alpha.tolist(), wl.beta.tolist())
    assert np.array_equal(d.codes, np.array(c, np.uint8))
    assert np.array_equal(d.scales, np.array(s, np.uint8))


def test_scalar_and_vectorised_weight_prep_agree():
    wl = gen.make_workload(1)
    rows = slice(0, 48)
    d = ob.weight_prep(wl.W_bits[rows], wl.A, wl.B, wl.walpha[rows], wl.wbeta[rows])
    c, s = osc.weight_prep(wl.W_bits[rows].tolist(), wl.A.tolist(), wl.B.tolist(),
                           wl.walpha[rows].tolist(), wl.wbeta[rows].tolist())
    assert np.array_equal(d.codes, np.array(c, np.uint8))
    assert np.array_equal(d.scales, np.array(s, np.uint8))
    dn = ob.weight_prep(wl.W_bits[rows], wl.A, wl.B, None, None)
    c, s = osc.weight_prep(wl.W_bits[rows].tolist(), wl.A.tolist(), wl.B.tolist())
    assert np.array_equal(dn.codes, np.array(c, np.uint8))


# -------------------------------------------------------------------- GEMM


def test_gemm_fp64_equals_exact_rationals_on_tiny():
    wl = gen.make_workload(1)
    x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    w = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)
    Y = ob.gemm(x.codes, x.scales, w.codes, w.scales)
    rows, cols = slice(0, 12), slice(0, 10)
    exact = osc.gemm_exact(x.codes[rows].tolist(), x.scales[rows].tolist(),
                           w.codes[cols].tolist(), w.scales[cols].tolist())
    assert np.array_equal(Y[rows, cols], np.array([[float(v) for v in r] for r in exact]))


def test_end_to_end_approximates_unquantised_layer():
    """Q(XP) Q(P^-1 W^T) stays close to X W^T (a loose sanity bound: 4-bit
    operands), and both quantised sides are needed to match the oracle chain."""
    wl = gen.make_workload(1)
    x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    w = ob.weight_prep(wl.W_bits, wl.A, wl.B, None, None)
    Y = ob.gemm(x.codes, x.scales, w.codes, w.scales)
    ref = ob.unquantized_layer(wl.X_bits, wl.W_bits)
    rel = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    assert rel < 0.35


# --------------------------------------------------------- decision intervals


def test_identity_factors_are_exact_and_free_of_exemptions():
    wl = gen.make_workload(1)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (8, 1, 1))
    logit = np.full(8, 40.0, np.float32)  # ratio 1.0: the plain OCP MX quantiser
    d = ob.act_transform_quant(wl.X_bits, A, B, logit, logit, exact=True)
    X = ob.bf16_values(wl.X_bits).astype(np.float32)
    codes, scales, _ = ob.clip_and_quantize(X, None, None)
    assert np.array_equal(d.codes, codes) and np.array_equal(d.scales, scales)
    assert d.n_exempt == 0


def test_fp32_evaluation_only_flips_exempt_decisions():
    """Evaluate the transform the way a GPU kernel may (fp32, factored, any
    order): every decision the interval analysis calls fixed must be identical."""
    for cfg in (1, 4):
        wl = gen.make_workload(cfg, with_weights=False)
        d = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
        X = ob.bf16_values(wl.X_bits).astype(np.float32)
        rows, K = X.shape
        nb = K // 32
        Xb = X.reshape(rows, nb, 4, 8)
        T = np.einsum("mirc,cd->mird", Xb, wl.A.astype(np.float32), dtype=np.float32)
        Y32 = np.einsum("irs,mird->misd", wl.B.astype(np.float32), T, dtype=np.float32).reshape(rows, K)
        codes, scales, _ = ob.clip_and_quantize(Y32, ob.clip_ratio(wl.alpha), ob.clip_ratio(wl.beta))
        fixed_blk = ~d.block_free
        assert np.array_equal(scales[fixed_blk], d.scales[fixed_blk])
        fixed = ~(d.elem_free | np.repeat(d.block_free, 32, axis=1) | d.zero_sign_free)
        assert np.array_equal(codes[fixed], d.codes[fixed])


def _window_case(y, S):
    """Decisions of one 32-element block with hand-chosen exact values and
    absolute sums (no clipping)."""
    Y = np.zeros((1, 32))
    A = np.zeros((1, 32))
    Y[0, :len(y)] = y
    A[0, :len(S)] = S
    return ob.decisions(Y, A, None, None)


def test_free_window_width_is_gamma36_of_the_abs_sum():
    """An element is free exactly when its exact value lies within
    beta = gamma_36 * S of a rounding boundary (S = sum |x||P|, the scale of
    every fp32 error the transform can make), and the window grows with S,
    not with |y|: checked on both sides of the boundary 0.75 at 0.9 beta and
    1.1 beta, for two values of S.  A block's scale is free exactly when its
    max lies within beta (plus the 2^-22 relative slack of the fp32 clip
    bound) of a power of two."""
    beta1 = ob.gamma(ob.ROUNDINGS) + 2.0 ** -45
    assert ob.ROUNDINGS == 36 and abs(ob.gamma(36) / (36 * 2.0 ** -24) - 1) < 1e-5
    for S in (1.0, 10.0):
        beta = beta1 * S
        for side in (+1, -1):
            near = _window_case([6.0, 0.75 + side * 0.9 * beta], [6.0, S])
            far = _window_case([6.0, 0.75 + side * 1.1 * beta], [6.0, S])
            assert near.elem_free[0, 1] and not far.elem_free[0, 1], (S, side)
            assert not near.block_free.any() and not far.block_free.any()
    # same |y|, ten times the abs sum: 1.1 beta(S=1) is inside the wider window
    assert _window_case([6.0, 0.75 + 1.1 * beta1], [6.0, 10.0]).elem_free[0, 1]
    # the scale window around the power of two 4 (e flips from -1 to 0)
    S = 4.0
    beta = beta1 * S
    for d, free in ((0.9, True), (1.2, False), (-0.9, True), (-1.1, False)):
        dec = _window_case([4.0 + d * beta, 1.0], [S, 1.0])
        assert bool(dec.block_free[0, 0]) == free, d


def test_transform_abs_sum_is_the_sum_of_absolute_products():
    """S = |x| |P| by hand on a block with cancellation (y = 0, S = 2) and the
    bf16 oracle path carries it: an exact zero keeps both signs, nothing else
    is free."""
    P = np.eye(32)[None].copy()
    P[0, 0, 0], P[0, 1, 0] = 1.0, 1.0  # y_0 = x_0 + x_1
    X = np.zeros((1, 32))
    X[0, 0], X[0, 1], X[0, 2] = 1.0, -1.0, 3.0
    S = ob.transform_abs_sum(X, P)
    assert S[0, 0] == 2.0 and S[0, 1] == 1.0 and S[0, 2] == 3.0
    assert ob.transform(X, P)[0, 0] == 0.0


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_exempt_window_stays_narrow(cfg):
    """On the configs' inputs: the stated exempt set (elements within 1e-6
    relative of a rounding boundary) is fewer than 1e-5 of the elements, as
    the parity rule requires; the rigorous free set (gamma_36 S, a few 1e-6
    of S; counted with every code of a free block) stays under 1.5e-5 plus
    one block (a bound blown up by a slip, such as a wrong gamma or S not in
    absolute values, fails here); no value is an exact zero."""
    from tests import parity

    M = {1: None, 2: 512, 3: 256, 4: None, 5: 512}[cfg]
    wl = gen.make_workload(cfg, M=M, with_weights=False)
    d = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    n = d.codes.size
    n_lit = int(parity.literal_window(d).sum())
    assert n_lit < 1e-5 * n or n_lit == 0, (n_lit, n)
    assert d.n_exempt <= 1.5e-5 * n + 32, (d.n_exempt, n)
    assert int(d.elem_free.sum()) <= 1.5e-5 * n + 1, (int(d.elem_free.sum()), n)
    assert not np.any(d.zero_sign_free)


def test_literal_window_marks_values_near_boundaries():
    """The stated window, by hand: 0.75 (1 + 5e-7) is inside, 0.75 (1 + 2e-6)
    outside; 2.5 (1 - 9e-7) inside; a grid value (2) is far from any
    boundary; with a block max of 12 (scale 2^1) the window applies to the
    scaled value, so 2 (0.75) (1 + 5e-7) is inside."""
    from tests import parity

    dec = _window_case([6.0, 0.75 * (1 + 5e-7), 0.75 * (1 + 2e-6), 2.5 * (1 - 9e-7), 2.0], [6.0, 1, 1, 1, 1])
    assert parity.literal_window(dec)[0, 1:5].tolist() == [True, False, True, False]
    dec = _window_case([12.0, 1.5 * (1 + 5e-7), 1.5 * (1 + 3e-6)], [12.0, 1, 1])
    assert dec.scales[0, 0] == 128
    assert parity.literal_window(dec)[0, 1:3].tolist() == [True, False]


def test_no_clip_is_the_plain_quantiser_and_tiny_blocks_use_the_lowest_scale():
    """No logits means no clipping: with identity factors the result is the
    plain OCP MX quantiser of x.  Blocks whose maximum lies just above the
    smallest normal float take scale byte 0 (e = -127) and nonzero codes,
    which the closed form fixes: x / 2^-127 for x = k 2^-126 is 2k."""
    K = 64
    x = np.zeros((2, K))
    x[:, :32] = np.array([1.0, 1.5, 2.0, 3.5] * 8) * 2.0 ** -126
    x[1, :32] *= -1
    x[:, 32:] = 0.7
    bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1))
    dec = ob.act_transform_quant(bits, A, B, None, None, exact=True)
    assert dec.scales[:, 0].tolist() == [0, 0]
    # 2k for k = 1, 1.5, 2, 3.5 -> 2, 3, 4, 7 (nearest E2M1: 2, 3, 4, 6) -> codes 4, 5, 6, 7
    assert dec.codes[0, :4].tolist() == [4, 5, 6, 7]
    assert dec.codes[1, :4].tolist() == [12, 13, 14, 15]
    # 0.7: e = floor(log2 0.7) - 2 = -3, 0.7 * 8 = 5.6 -> 6 (code 7)
    assert dec.scales[0, 1] == 124 and dec.codes[0, 32] == 7
    with pytest.raises(ValueError):
        ob.act_transform_quant(bits, A, B, None, np.zeros(2, np.float32))


def test_hadamard_factor_recipe_is_the_block_rotation():
    """The workload recipe's block-Hadamard factors give P_i = H_32 / sqrt(32)
    (checked against scipy's Sylvester construction) for every (a, b)."""
    for a in gen.SWEEP_A:
        A, B = gen.hadamard_factors(64, a)
        P = ob.block_matrices(A, B)
        assert P.shape == (2, 32, 32)
        assert np.allclose(P[1], scipy.linalg.hadamard(32) / math.sqrt(32), atol=1e-6)


# ------------------------------------------------ MXFP8 (E4M3), W4A8 setting


def _e4m3_grid_by_construction():
    """All finite non-negative E4M3 values, built from the format's fields (not
    from the oracle): subnormals m 2^-9, normals (8 + m) 2^(E - 10); the top
    mantissa of the top exponent is NaN."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for E in range(1, 16):
        for m in range(8):
            if E == 15 and m == 7:
                continue
            vals.append((8 + m) * 2.0 ** (E - 10))
    return np.array(vals)


def test_e4m3_decode_matches_the_format_definition():
    g = _e4m3_grid_by_construction()
    assert len(g) == 127 and np.all(np.diff(g) > 0)
    assert np.array_equal(ob.e4m3_decode(np.arange(127)), g)
    assert np.array_equal(ob.e4m3_decode(np.arange(128, 255)), -g)
    # landmarks of the OCP E4M3 format
    assert ob.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert ob.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert ob.e4m3_decode(np.array([0x38]))[0] == 1.0
    assert ob.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert np.isnan(ob.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_e4m3_round_equals_brute_force_nearest():
    """Nearest of the 127 grid values by exhaustive argmin, ties to the even
    code, saturation at 448, on random values and on every midpoint +-1 ulp."""
    g = _e4m3_grid_by_construction()
    rng = np.random.default_rng(8)
    mids = (g[1:] + g[:-1]) / 2
    v = np.concatenate([rng.uniform(0, 520, 4000), np.exp(rng.uniform(-12, 6.5, 4000)),
                        mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), g, [0.0, 448.0, 460.0, 1e6]])
    d = np.abs(g[None, :] - np.minimum(v, 448.0)[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near values take the even code
    want = np.where(cand.sum(axis=1) > 1, np.argmax(cand & (np.arange(127) % 2 == 0), axis=1), np.argmax(cand, axis=1))
    assert np.array_equal(ob.e4m3_round(v), want.astype(np.uint8))
    assert np.array_equal(ob.e4m3_round(-v), (want | 0x80).astype(np.uint8))
    assert ob.e4m3_round(np.array([-0.0]))[0] == 0x80


def test_mxfp8_scale_rule_and_worked_block():
    """E4M3's largest exponent is 8, so the scale puts amax / 2^e in [256, 512);
    a block with amax 1 gets e = -8 and 1.0 -> 256 = code 0x78; a value 0.3 in
    that block -> 76.8, whose binade [64, 128) has spacing 8 -> nearest 80
    (= 1.25 * 2^6: exponent field 13, mantissa 2, code 0x6A)."""
    rng = np.random.default_rng(9)
    amax = np.exp(rng.uniform(-40, 40, 1000))
    e = ob.shared_exponent(amax, ob.E4M3_MAX_EXP)
    r = amax / np.ldexp(1.0, e)
    assert np.all((r >= 256) & (r < 512))
    y = np.zeros((1, 32), np.float32)
    y[0, 0], y[0, 1] = 1.0, 0.3
    codes, scales, _ = ob.clip_and_quantize(y, None, None, "e4m3")
    assert scales[0, 0] == 127 - 8
    assert codes[0, 0] == 0x78 and ob.e4m3_decode(np.array([0x78]))[0] == 256.0
    assert codes[0, 1] == 0x6A and ob.e4m3_decode(np.array([0x6A]))[0] == 80.0


def test_mxfp8_quantisation_error_is_half_an_ulp():
    """Normal-range elements of an MXFP8 block come back within 2^-4 of their
    value (3 mantissa bits), except the block maxima in [448, 512) that saturate;
    MXFP8 is much finer than MXFP4 on the same block."""
    rng = np.random.default_rng(10)
    y = rng.standard_normal((64, 256)).astype(np.float32)
    c8, s8, z8 = ob.clip_and_quantize(y, None, None, "e4m3")
    d8 = ob.dequantize(c8, s8, "e4m3")
    z = z8.astype(np.float64)
    scale = np.repeat(np.ldexp(1.0, s8.astype(np.int64) - 127), 32, axis=1)
    v = np.abs(z) / scale
    normal = (v >= 2.0 ** -6) & (v <= 448.0)
    assert np.all(np.abs(d8 - z)[normal] <= 2.0 ** -4 * np.abs(z)[normal])
    sat = v > 448.0  # a block maximum in [448, 512) saturates to 448
    assert sat.any() and np.all(np.abs(d8)[sat] == 448.0 * scale[sat])
    c4, s4, _ = ob.clip_and_quantize(y, None, None, "e2m1")
    assert np.abs(ob.dequantize(c4, s4) - z).mean() > 3 * np.abs(d8 - z).mean()


def test_kv_cache_rows_places_valid_slots_only():
    """Cache placement: every in-range slot receives its token, out-of-range
    slots place nothing, untouched rows stay unwritten (brute force by hand)."""
    src = ob.kv_cache_rows(np.array([5, 0, -1, 9, 3, 10]), 10)
    assert src.tolist() == [1, -1, -1, 4, -1, 0, -1, -1, -1, 3]
    assert (ob.kv_cache_rows(np.array([], dtype=np.int64), 4) == -1).all()


def test_large_operand_rows_match_a_per_group_rotation():
    """gen.large_rows (the host side of the >2 GiB parity tests) equals the
    device-side construction those tests use, here run with torch on the CPU:
    each group of base-size rows rotated by whole blocks, distinct per group."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    R0, K = 64, 128
    base = rng.integers(0, 16, size=(R0, K), dtype=np.uint8)
    rows = 5 * R0 + 17
    src = torch.from_numpy(base)
    full = torch.empty((rows, K), dtype=src.dtype)
    for g in range((rows + R0 - 1) // R0):
        n = min(R0, rows - g * R0)
        full[g * R0:g * R0 + n] = torch.roll(src[:n], gen.large_group_shift(g, 32, K // 32), dims=1)
    pick = np.array([0, 1, R0 - 1, R0, 2 * R0 + 5, rows - 1])
    assert np.array_equal(full.numpy()[pick], gen.large_rows(base, pick, 32, K // 32))
    # the packed-byte form rotates by 16 bytes per 32 codes
    packed = torch.from_numpy(ob.pack_codes(base))
    g = 3
    assert np.array_equal(torch.roll(packed, gen.large_group_shift(g, 16, K // 32), dims=1).numpy(),
                          ob.pack_codes(gen.large_rows(base, np.arange(g * R0, (g + 1) * R0), 32, K // 32)))
    # rows of different groups differ; the rotation repeats after K / 32 groups
    assert not np.array_equal(full.numpy()[5], full.numpy()[R0 + 5])
    assert gen.large_group_shift(K // 32, 32, K // 32) == 0


def test_compare_quant_signed_zero_and_the_stated_window():
    """The parity rule on a synthetic block (scale 2^0, no clip): a +0 / -0
    mismatch passes where the fp32 error can flip the value's sign, and fails
    where it cannot; a free mismatch 3e-6 relative from a boundary still fails
    the stated 1e-6 window."""
    from tests import parity

    y = np.ones((1, 32))
    S = np.ones((1, 32))
    y[0, 0], S[0, 0] = 6.0, 6.0                   # block max: shared exponent 0
    y[0, 1], S[0, 1] = -2.3e-9, 0.5               # |y| far below gamma_36 S: sign free
    y[0, 2], S[0, 2] = -0.1, 0.1                  # rounds to -0, sign fixed
    y[0, 3], S[0, 3] = 0.75 * (1 + 3e-6), 5.0     # free, 3e-6 above the 0.75 boundary
    dec = ob.decisions(y, S, None, None)
    assert dec.scales[0, 0] == 127
    assert dec.codes[0, 1:4].tolist() == [8, 8, 2]
    assert dec.elem_free[0, 1] and not dec.elem_free[0, 2] and dec.elem_free[0, 3]
    assert not dec.zero_sign_free[0, 1]

    def run(k, code):
        c = dec.codes.copy()
        c[0, k] = code
        return parity.compare_quant(ob.pack_codes(c), dec.scales.copy(), dec, label="synthetic", max_frac=1.0)

    st = run(1, 0)
    assert (st["mismatches"], st["signed_zero"], st["mismatches_outside_literal"]) == (1, 1, 0)
    with pytest.raises(AssertionError, match="outside the free set"):
        run(2, 0)
    with pytest.raises(AssertionError, match="outside the stated 1e-6 window"):
        run(3, 1)
    parity.RESULTS[:] = [r for r in parity.RESULTS if r["label"] != "synthetic"]  # not a run's comparison
