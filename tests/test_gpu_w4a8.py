"""GPU parity of the W4A8 setting (MXFP8 activations, MXFP4 weights): the HIP
kernels through the C ABI against the CPU oracle, on the same seeded inputs.
Needs an MI355X; run with ``-m gpu``."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import batquant as ob
from tests import parity
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def w():
    import w4a4_bit_gemm_amd as w

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return w


def dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def run_act8(w, X_bits, A, B, alpha=None, beta=None):
    rh = None if alpha is None else dev_f32(w.clip_ratios(alpha))
    rl = None if beta is None else dev_f32(w.clip_ratios(beta))
    q, s = w.act_transform_quant_mxfp8(dev_bf16(X_bits), dev_f32(A), dev_f32(B), rh, rl)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _sample_rows(M, n, seed):
    if M <= n:
        return np.arange(M)
    return np.sort(np.random.default_rng(seed).choice(M, size=n, replace=False))


# ------------------------------------------------------ MXFP8 activation path


@pytest.mark.parametrize("M,K,a,seed", [(1, 32, 8, 1), (33, 96, 4, 2), (100, 224, 2, 3), (257, 512, 16, 4),
                                        (64, 256, 1, 5), (40, 288, 32, 6)])
def test_act8_ragged_shapes_and_factor_sizes(w, M, K, a, seed):
    note(f"case: act mxfp8 {M}x{K} a={a}")
    wl = gen.make_custom(M, K, 8, a=a, seed=seed)
    q, s = run_act8(w, wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    assert q.shape == (M, K)
    dec = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta, fmt="e4m3")
    parity.compare_quant(q, s, dec, label=f"mxfp8 {M}x{K}", fmt="e4m3")


def test_act8_identity_factors_exact_with_ties_and_saturation(w):
    """A = I, B_i = I, dyadic ratios: every fp32 step is exact, so the output
    must match bit for bit, including exact E4M3 midpoints and saturated
    block maxima (amax / 2^e in [448, 512))."""
    note("case: act mxfp8 identity factors, exact ties and saturation")
    rng = np.random.default_rng(51)
    M, K = 96, 512
    x = rng.integers(-255, 256, size=(M, K)) / 16.0
    x[:, 7] = 31.75   # block 0: amax 31.75 -> e = -4, 31.75 * 16 = 508 saturates to 448
    x[:, 40] = -30.0  # block 1: 30 * 16 = 480 saturates to -448
    wl = gen.make_custom(M, K, 8, seed=51)
    wl.X_bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1))
    lg = np.array([40.0, np.log(3.0), 0.0], dtype=np.float32)  # sigmoid exactly 1, 0.75, 0.5
    alpha = lg[np.arange(K // 32) % 3]
    beta = lg[(np.arange(K // 32) + 1) % 3]
    q, s = run_act8(w, wl.X_bits, A, B, alpha, beta)
    dec = ob.act_transform_quant(wl.X_bits, A, B, alpha, beta, exact=True, fmt="e4m3")
    assert np.array_equal(s, dec.scales)
    same = (q == dec.codes) | (dec.zero_sign_free & ((q & 0x7F) == 0) & ((dec.codes & 0x7F) == 0))
    assert same.all(), np.argwhere(~same)[:5].tolist()
    assert np.any((dec.codes & 0x7F) == 0x7E)  # saturation really exercised
    assert not np.any((q & 0x7F) == 0x7F)      # never a NaN code
    e = dec.scales.astype(np.int64) - 127
    v = np.abs(np.ldexp(dec.z32.astype(np.float64), -np.repeat(e, 32, axis=1)))
    mids = (ob.E4M3_GRID[1:] + ob.E4M3_GRID[:-1]) / 2
    assert np.isin(v, mids).sum() > 50  # ties really exercised


def test_act8_zero_tiny_and_single_sign_blocks(w):
    """All-zero blocks, blocks just above the smallest normal float (lowest
    scale byte, nonzero codes) and single-sign blocks, identity factors."""
    note("case: act mxfp8 zero, tiny and single-sign blocks")
    rng = np.random.default_rng(52)
    M, K = 40, 256
    x = rng.standard_normal((M, K))
    x[:, 0:32] = 0.0
    mags = np.array([1.0, 1.25, 1.5, 3.0, 7.0, 100.0, 255.0]) * 2.0 ** -126
    x[:, 32:64] = rng.choice(mags, size=(M, 32)) * np.where(rng.random((M, 32)) < 0.5, -1.0, 1.0)
    x[:, 64:96] = np.abs(x[:, 64:96]) + 1.0
    x[:, 96:128] = -np.abs(x[:, 96:128]) - 1.0
    wl = gen.make_custom(M, K, 8, seed=52)
    wl.X_bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1))
    alpha = np.full(K // 32, -1.0, np.float32)
    beta = np.full(K // 32, 2.0, np.float32)  # r_lo > r_hi: l > u on positive blocks
    q, s = run_act8(w, wl.X_bits, A, B, alpha, beta)
    dec = ob.act_transform_quant(wl.X_bits, A, B, alpha, beta, exact=True, fmt="e4m3")
    assert np.all(s[:, 0] == 0) and np.all(dec.scales[:, 1] == 0)
    assert np.any(dec.codes[:, 32:64] & 0x7F)
    assert np.array_equal(s, dec.scales)
    same = (q == dec.codes) | (dec.zero_sign_free & ((q & 0x7F) == 0) & ((dec.codes & 0x7F) == 0))
    assert same.all(), np.argwhere(~same)[:5].tolist()


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_act8_full_config(w, cfg):
    note(f"case: act mxfp8 full config {cfg}")
    wl = gen.make_workload(cfg, with_weights=False)
    q, s = run_act8(w, wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    rows = _sample_rows(wl.M, 1024, 60 + cfg)
    dec = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta, fmt="e4m3")
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"mxfp8 config {cfg}", fmt="e4m3")
    note(f"  {st}")


# ----------------------------------------------------------- W4A8 GEMM


def _rand_e4m3(rng, rows, K):
    codes = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 1  # no NaN codes
    scales = rng.integers(110, 135, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def _rand_e2m1(rng, rows, K):
    return (rng.integers(0, 16, size=(rows, K), dtype=np.uint8),
            rng.integers(110, 135, size=(rows, K // 32), dtype=np.uint8))


def run_gemm8(w, xc, xs, wc, ws, out_dtype):
    wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV))
    y = w.mxfp8_gemm_packed(torch.from_numpy(xc).to(DEV), torch.from_numpy(xs).to(DEV), wp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


# K / 256 in {1, 2, 4, 8, 16, 48}: unrolled kernels; 3, 6, 12, 13, 20: the looped
# one, whose body covers 4 stages (20 with four-stage scale groups, 13 without).
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (33, 47, 256), (128, 256, 512), (130, 250, 768),
                                   (257, 129, 1024), (40, 33, 1536), (200, 300, 2048), (64, 520, 3072),
                                   (64, 300, 4096), (129, 257, 12288), (40, 70, 3328), (66, 90, 5120)])
def test_w4a8_gemm_matches_oracle(w, M, N, K):
    """Random E4M3 activations (all finite codes, subnormals included) and E2M1
    weights, block scales over 2^-17 .. 2^7: every product is exact, so the
    error is the fp32 accumulation bound plus the MFMA's group window."""
    note(f"case: w4a8 gemm {M}x{N}x{K}")
    rng = np.random.default_rng(M * 13 + N * 7 + K)
    xc, xs = _rand_e4m3(rng, M, K)
    wc, ws = _rand_e2m1(rng, N, K)
    ref = ob.gemm(xc, xs, wc, ws, x_fmt="e4m3")
    bound = parity.w4a8_gemm_bound(xc, xs, wc, ws)
    y = run_gemm8(w, xc, xs, wc, ws, torch.float32)
    err = np.abs(y - ref)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.max() <= 1e-3 * np.abs(ref).max()
    yb = run_gemm8(w, xc, xs, wc, ws, torch.bfloat16)
    assert np.array_equal(yb, parity.bf16_rne(y.astype(np.float32)).astype(np.float64))


# More than 256 tiles of 128 x 256 with K / 256 in {4, 8, 16, 48}: the two-
# workgroups-per-CU kernel.  Rows are independent, so the output rows of a
# slice of X (few tiles: the one-workgroup-per-CU kernel) must equal the same
# rows of the full product bit for bit; sampled rows against the oracle.  N =
# 33001: output rows that are not whole 16-byte chunks (scalar stores).
@pytest.mark.parametrize("M,N,K", [(2000, 12200, 1024), (2100, 8300, 2048), (2100, 4200, 4096),
                                   (2100, 4200, 12288), (1000, 33001, 1024)])
def test_w4a8_gemm_two_workgroups_per_cu(w, M, N, K):
    note(f"case: w4a8 gemm two workgroups per CU {M}x{N}x{K}")
    assert w.packed_gemm_kernel(M, N, K, act_fp8=True) == 1
    rng = np.random.default_rng(M + 3 * N + 5 * K)
    xc, xs = _rand_e4m3(rng, M, K)
    wc, ws = _rand_e2m1(rng, N, K)
    wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV))
    X, XS = torch.from_numpy(xc).to(DEV), torch.from_numpy(xs).to(DEV)
    Y = w.mxfp8_gemm_packed(X, XS, wp, out_dtype=torch.float32)
    for r0, r1 in ((0, 128), (M - 100, M)):
        assert w.packed_gemm_kernel(r1 - r0, N, K, act_fp8=True) == 0
        Ys = w.mxfp8_gemm_packed(X[r0:r1].contiguous(), XS[r0:r1].contiguous(), wp, out_dtype=torch.float32)
        assert torch.equal(Ys.view(torch.int32), Y[r0:r1].view(torch.int32)), (r0, r1)
    rows = np.unique(np.concatenate([_sample_rows(M, 24, M + K), [M - 1]]))
    ref = ob.gemm(xc[rows], xs[rows], wc, ws, x_fmt="e4m3")
    bound = parity.w4a8_gemm_bound(xc[rows], xs[rows], wc, ws)
    y = Y.cpu().numpy().astype(np.float64)[rows]
    err = np.abs(y - ref)
    assert np.all(err <= bound), float((err - bound).max())
    Yb = w.mxfp8_gemm_packed(X, XS, wp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(Yb.float().cpu().numpy(), parity.bf16_rne(Y.cpu().numpy()))


@pytest.mark.parametrize("M,N,K", [(5, 9, 256), (70, 61, 1024), (129, 257, 3072)])
def test_w4a8_gemm_bit_exact_inside_the_window(w, M, N, K):
    """E4M3 exponent fields 6..9 (|x| in [0.5, 7.5]), unit scales: every product
    is a multiple of 2^-5 below 46, every partial sum fits 24 bits, and no group
    spans more than the window, so the result equals the exact sum bit for bit."""
    note(f"case: w4a8 gemm exact {M}x{N}x{K}")
    rng = np.random.default_rng(M + N + K)
    xc = ((rng.integers(6, 10, size=(M, K)) << 3) | rng.integers(0, 8, size=(M, K))
          | (rng.integers(0, 2, size=(M, K)) << 7)).astype(np.uint8)
    wc = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    ref = ob.gemm(xc, xs, wc, ws, x_fmt="e4m3")
    assert 45 * K * 2 ** 5 < 2 ** 24  # every partial sum is a multiple of 2^-5 below 45 K
    y = run_gemm8(w, xc, xs, wc, ws, torch.float32)
    assert np.array_equal(y, ref), float(np.abs(y - ref).max())


def test_w4a8_gemm_truncation_window_model(w):
    """The FP8 x FP4 MFMA's group window, pinned bit for bit (the model behind
    parity.f8f4_window_bound): inside each run of F8F4_GROUP consecutive k,
    every nonzero product is truncated toward zero to a multiple of
    2^(A - F8F4_WINDOW_BITS), A the run's largest exponent-field sum; the run
    sums then add like fp32.  Activations 2^-3 (1 + m/8) with random signs, and
    in a random half of the runs one +-448; weights +-1, +-1.5; unit scales.  A
    run with a 448 has A = 8, so its small products (multiples of 2^-7) lose
    their 2^-6 and 2^-7 bits toward zero; a run without one keeps them all.
    Every partial sum is a multiple of 2^-7 below 2^14 (21 bits), so the result
    is exact in fp32 and must equal the model exactly; the exact sum differs on
    almost every output, and so would a group of 16, a window of 12 or 14 bits,
    or flooring instead of truncation."""
    note("case: w4a8 gemm truncation window model 64x96x256")
    M, N, K = 64, 96, 256
    g = parity.F8F4_GROUP
    rng = np.random.default_rng(2024)
    xc = ((4 << 3) | rng.integers(0, 8, size=(M, K))).astype(np.uint8)  # 2^-3 (1 + m/8)
    big = rng.integers(0, 2, size=(M, K // g)).astype(bool)
    pos = rng.integers(0, g, size=(M, K // g))
    for m in range(M):
        for r in np.nonzero(big[m])[0]:
            xc[m, r * g + pos[m, r]] = 0x7E  # 448 = 1.75 x 2^8
    xc |= (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    wc = (rng.integers(2, 4, size=(N, K)) | (rng.integers(0, 2, size=(N, K)) << 3)).astype(np.uint8)  # +-1, +-1.5
    xs = np.full((M, K // 32), 127, np.uint8)
    ws = np.full((N, K // 32), 127, np.uint8)
    Xd = ob.dequantize(xc, xs, "e4m3")
    Wd = ob.dequantize(wc, ws)
    ex = np.maximum(np.floor(np.log2(np.abs(Xd))), -6.0)  # exponent fields (no zeros here)
    ew = np.maximum(np.floor(np.log2(np.abs(Wd))), 0.0)
    model = np.empty((M, N))
    for m in range(M):
        P = (Xd[m][None, :] * Wd).reshape(N, K // g, g)
        A = (ex[m][None, :] + ew).reshape(N, K // g, g).max(axis=2, keepdims=True)
        step = np.exp2(A - parity.F8F4_WINDOW_BITS)
        model[m] = (np.trunc(P / step) * step).sum(axis=(1, 2))
    assert np.all(np.abs(model) < 2.0 ** 14) and np.all(model * 128 == np.round(model * 128))
    assert np.all(np.abs(exact_sum := Xd @ Wd.T) < 2.0 ** 14)
    assert np.count_nonzero(exact_sum != model) > M * N // 2  # the window matters on most outputs
    assert np.all(np.abs(exact_sum - model) <= parity.f8f4_window_bound(Xd, Wd))
    y = run_gemm8(w, xc, xs, wc, ws, torch.float32)
    assert np.array_equal(y, model), f"{np.count_nonzero(y != model)} outputs off the model"


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_w4a8_end_to_end(w, cfg):
    """The W4A8 chain X, W -> Y in the benchmark's launch configuration,
    sampled outputs against the oracle chain."""
    note(f"case: w4a8 end to end config {cfg}")
    wl = gen.make_workload(cfg)
    xq, xs = w.act_transform_quant_mxfp8(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                         dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    wp = w.weight_pack(wq, ws)
    Y = w.mxfp8_gemm_packed(xq, xs, wp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.M, 16, 1000 + cfg)
    cols = _sample_rows(wl.N, 16, 1100 + cfg)
    x = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta, fmt="e4m3")
    wt = ob.weight_prep(wl.W_bits[cols], wl.A, wl.B, wl.walpha[cols], wl.wbeta[cols])
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales, x_fmt="e4m3")
    y = Y[rows][:, cols].cpu().numpy().astype(np.float64)
    rel = np.abs(y - ref).max() / np.abs(ref).max()
    note(f"  max rel err {rel:.3e}")
    assert rel <= 1e-3
    # W4A8 is closer to the unquantised layer than W4A4 on the same sample
    x4 = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    y4 = ob.gemm(x4.codes, x4.scales, wt.codes, wt.scales)
    exact = ob.unquantized_layer(wl.X_bits[rows], wl.W_bits[cols])
    assert np.abs(ref - exact).mean() < np.abs(y4 - exact).mean()
