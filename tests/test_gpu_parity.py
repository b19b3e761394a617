"""GPU parity: the HIP kernels through the C ABI against the CPU oracle, on the
same seeded inputs.  Needs an MI355X; run with ``-m gpu``."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import batquant as ob
from tests import parity
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def w():
    import w4a4_bit_gemm_amd as w

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return w


DEV = "cuda"


def dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def run_act(w, wl, A=None, B=None, alpha=None, beta=None, clip=True):
    A = wl.A if A is None else A
    B = wl.B if B is None else B
    alpha = wl.alpha if alpha is None else alpha
    beta = wl.beta if beta is None else beta
    X = dev_bf16(wl.X_bits)
    rh = dev_f32(w.clip_ratios(alpha)) if clip else None
    rl = dev_f32(w.clip_ratios(beta)) if clip else None
    Xq, Xs = w.act_transform_quant(X, dev_f32(A), dev_f32(B), rh, rl)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), Xs.cpu().numpy()


def run_weight(w, wl, clip=True):
    Wd = dev_bf16(wl.W_bits)
    if clip:
        Wq, Ws = w.prepare_weight(Wd, wl.A, wl.B, wl.walpha, wl.wbeta)
    else:
        Wq, Ws = w.prepare_weight(Wd, wl.A, wl.B)
    torch.cuda.synchronize()
    return Wq.cpu().numpy(), Ws.cpu().numpy()


# ------------------------------------------------------------ activation path


def test_act_tiny_matches_oracle(w):
    note("case: act tiny (config 1, 64x256, a=8)")
    wl = gen.make_workload(1)
    q, s = run_act(w, wl)
    dec = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    st = parity.compare_quant(q, s, dec, label="tiny")
    assert st["mismatches"] == 0, st


@pytest.mark.parametrize("M,K,a,seed", [(1, 32, 8, 1), (33, 96, 4, 2), (100, 224, 2, 3), (257, 512, 16, 4),
                                        (31, 64, 1, 5), (77, 128, 32, 6), (300, 4096, 8, 7)])
def test_act_ragged_shapes_and_factor_sizes(w, M, K, a, seed):
    note(f"case: act ragged M={M} K={K} a={a}")
    wl = gen.make_custom(M, K, 8, a=a, seed=seed)
    q, s = run_act(w, wl)
    dec = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    parity.compare_quant(q, s, dec, label=f"ragged {M}x{K} a={a}")


def test_act_no_clip(w):
    note("case: act without clipping")
    wl = gen.make_custom(70, 256, 8, seed=11)
    q, s = run_act(w, wl, clip=False)
    P = ob.block_matrices(wl.A, wl.B)
    X = ob.bf16_values(wl.X_bits)
    dec = ob.decisions(ob.transform(X, P), ob.transform_abs_sum(X, P), None, None)
    parity.compare_quant(q, s, dec, label="no clip")


def test_act_identity_factors_exact_with_ties(w):
    """A = I, B_i = I, dyadic ratios: every fp32 step is exact, so the whole
    output must match bit for bit, including values exactly on midpoints."""
    note("case: act identity factors, dyadic ratios, exact ties")
    rng = np.random.default_rng(21)
    M, K = 96, 512
    # values on a coarse dyadic grid put many elements exactly on E2M1 midpoints
    x = rng.integers(-48, 49, size=(M, K)) / 8.0
    x[:, 5] *= 64
    wl = gen.make_custom(M, K, 8, seed=21)
    wl.X_bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1))
    # logits whose float32 sigmoid is exactly 1, 0.75 or 0.5
    lg = np.array([40.0, np.log(3.0), 0.0], dtype=np.float32)
    alpha = lg[np.arange(K // 32) % 3]
    beta = lg[(np.arange(K // 32) + 1) % 3]
    assert set(ob.clip_ratio(lg).tolist()) == {1.0, 0.75, 0.5}
    q, s = run_act(w, wl, A=A, B=B, alpha=alpha, beta=beta)
    dec = ob.act_transform_quant(wl.X_bits, A, B, alpha, beta, exact=True)
    codes = ob.unpack_codes(q)
    assert np.array_equal(s, dec.scales)
    same = (codes == dec.codes) | (dec.zero_sign_free & ((codes & 7) == 0) & ((dec.codes & 7) == 0))
    assert same.all(), np.argwhere(~same)[:5].tolist()
    v = np.abs(np.ldexp(dec.z32.astype(np.float64), -(dec.scales.astype(np.int64) - 127).repeat(32, axis=1)))
    assert np.isin(v, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]).sum() > 100  # ties really exercised


def test_act_zero_and_single_sign_blocks(w):
    note("case: act zero blocks and single-sign blocks")
    wl = gen.make_custom(40, 256, 8, seed=31)
    x = ob.bf16_values(wl.X_bits)
    x[:, 0:32] = 0.0                    # all-zero block
    x[:, 32:64] = np.abs(x[:, 32:64]) + 1.0  # all-positive block
    x[:, 64:96] = -np.abs(x[:, 64:96]) - 1.0  # all-negative block
    wl.X_bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (8, 1, 1))
    alpha = np.full(8, -1.0, np.float32)  # r_hi ~ 0.27
    beta = np.full(8, 2.0, np.float32)    # r_lo ~ 0.88 > r_hi: l > u on positive blocks
    q, s = run_act(w, wl, A=A, B=B, alpha=alpha, beta=beta)
    dec = ob.act_transform_quant(wl.X_bits, A, B, alpha, beta, exact=True)
    codes = ob.unpack_codes(q)
    assert np.all(s[:, 0] == 0)
    assert np.all((codes[:, :32] & 7) == 0)
    assert np.array_equal(s, dec.scales)
    same = (codes == dec.codes) | (dec.zero_sign_free & ((codes & 7) == 0))
    assert same.all()


def test_act_tiny_blocks_lowest_scale(w):
    """Blocks whose maximum lies in [2^-126, 2^-124) take the lowest scale byte
    (e = -127) yet still quantise to nonzero codes; some blocks of the same
    rows are ordinary.  Identity factors keep every fp32 step exact."""
    note("case: act tiny blocks at the lowest scale byte")
    rng = np.random.default_rng(41)
    M, K = 64, 256
    x = rng.standard_normal((M, K))
    # normal float32 magnitudes just above the smallest normal number
    mags = np.array([1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5]) * 2.0 ** -126
    tiny = rng.choice(mags, size=(M, 96)) * np.where(rng.random((M, 96)) < 0.5, -1.0, 1.0)
    x[:, 32:128] = tiny
    x[::3, 160:192] = tiny[::3, :32]  # some waves mix tiny and ordinary blocks
    wl = gen.make_custom(M, K, 8, seed=41)
    wl.X_bits = gen.f64_to_bf16_bits(x)
    A = np.eye(8, dtype=np.float32)
    B = np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1))
    q, s = run_act(w, wl, A=A, B=B, clip=False)
    dec = ob.act_transform_quant(wl.X_bits, A, B, None, None, exact=True)
    codes = ob.unpack_codes(q)
    assert np.all(dec.scales[:, 1:4] == 0) and np.any(dec.codes[:, 32:128] & 7)
    assert np.array_equal(s, dec.scales)
    same = (codes == dec.codes) | (dec.zero_sign_free & ((codes & 7) == 0) & ((dec.codes & 7) == 0))
    assert same.all(), np.argwhere(~same)[:5].tolist()


def test_act_locality_and_determinism(w):
    note("case: act locality (re-randomised block) and determinism")
    wl = gen.make_custom(128, 1024, 8, seed=41)
    q0, s0 = run_act(w, wl)
    q1, s1 = run_act(w, wl)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
    x2 = wl.X_bits.copy()
    x2[:, 320:352] = gen.f64_to_bf16_bits(np.random.default_rng(5).standard_t(3, (128, 32)) * 20)
    wl2 = gen.make_custom(128, 1024, 8, seed=41)
    wl2.X_bits = x2
    q2, s2 = run_act(w, wl2)
    keep_q = np.ones(512, bool)
    keep_q[160:176] = False
    keep_s = np.ones(32, bool)
    keep_s[10] = False
    assert np.array_equal(q0[:, keep_q], q2[:, keep_q])
    assert np.array_equal(s0[:, keep_s], s2[:, keep_s])
    assert not np.array_equal(q0[:, ~keep_q], q2[:, ~keep_q])


def _sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist())
    rows.update([0, M - 1])
    return np.array(sorted(rows))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_act_full_config(w, cfg):
    """Full-size activation run (the shape the benchmark times); every code of a
    row sample (all rows up to 2048) is compared with the oracle."""
    note(f"case: act full config {cfg}")
    wl = gen.make_workload(cfg, with_weights=False)
    q, s = run_act(w, wl)
    rows = np.arange(wl.M) if wl.M <= 2048 else _sample_rows(wl.M, 1024, cfg)
    dec = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"config {cfg}")
    note(f"  {st}")


@pytest.mark.parametrize("fp8", [False, True])
def test_act_skewed_walk_equals_row_slices(w, fp8):
    """At 16384 x 4096 the transform runs two workgroups per CU with 16 tiles
    each, which takes the skewed tile walk (the first-dispatched half of the
    workgroups takes 17 consecutive tile rows, the second half 15).  Rows are
    independent, so the whole must equal the same rows transformed as 2048-row
    slices, which take the other instance (one workgroup per CU with a
    dedicated loader wave, strided walk)."""
    note(f"case: act skewed walk vs row slices fp8={fp8}")
    assert w.transform_kernel(16384, 4096) == 0 and w.transform_kernel(2048, 4096) == 1
    wl = gen.make_workload(5, with_weights=False)
    X = dev_bf16(wl.X_bits)
    A, B = dev_f32(wl.A), dev_f32(wl.B)
    rh, rl = dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta))
    fn = w.act_transform_quant_mxfp8 if fp8 else w.act_transform_quant
    q, s = fn(X, A, B, rh, rl)
    for r0 in range(0, wl.M, 2048):
        qs, ss = fn(X[r0:r0 + 2048], A, B, rh, rl)
        assert torch.equal(qs, q[r0:r0 + 2048]) and torch.equal(ss, s[r0:r0 + 2048]), r0
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["kv4", "kv8", "weight"])
def test_skewed_walk_cache_and_weight_modes_equal_row_slices(w, mode):
    """The KV-cache and per-row weight instances at the skewed-walk shape
    (16384 rows x 4096 channels) against the same rows as 2048-row slices,
    which take the one-workgroup-per-CU instance: bit for bit.  Cache slots are
    a permutation of the rows; the weight side gets per-row ratios."""
    note(f"case: skewed walk vs row slices, {mode}")
    assert w.transform_kernel(16384, 4096) == 0 and w.transform_kernel(2048, 4096) == 1
    wl = gen.make_workload(5, with_weights=False)
    X = dev_bf16(wl.X_bits)
    A, B = dev_f32(wl.A), dev_f32(wl.B)
    M, K = wl.M, wl.K
    rng = np.random.default_rng(77)
    if mode == "weight":
        wr_hi = dev_f32(rng.uniform(0.5, 1.0, size=(M, K // 32)))
        wr_lo = dev_f32(rng.uniform(0.5, 1.0, size=(M, K // 32)))
        q, s = w.weight_prep(X, A, B, wr_hi, wr_lo)
        for r0 in range(0, M, 2048):
            qs, ss = w.weight_prep(X[r0:r0 + 2048], A, B, wr_hi[r0:r0 + 2048], wr_lo[r0:r0 + 2048])
            assert torch.equal(qs, q[r0:r0 + 2048]) and torch.equal(ss, s[r0:r0 + 2048]), r0
    else:
        fmt = 4 if mode == "kv4" else 8
        rh, rl = dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta))
        slots = torch.from_numpy(rng.permutation(M).astype(np.int64)).to(DEV)
        qcols = K // 2 if fmt == 4 else K
        caches = []
        for sliced in (False, True):
            cq = torch.full((M, qcols), 0xA5, dtype=torch.uint8, device=DEV)
            cs = torch.full((M, K // 32), 0xA5, dtype=torch.uint8, device=DEV)
            spans = range(0, M, 2048) if sliced else [0]
            for r0 in spans:
                r1 = r0 + 2048 if sliced else M
                w.kv_cache_quant(X[r0:r1], A, B, rh, rl, slots[r0:r1], cq, cs, fmt=fmt)
            caches.append((cq, cs))
        assert torch.equal(caches[0][0], caches[1][0]) and torch.equal(caches[0][1], caches[1][1])
        # every row was written: no sentinel scale row is left
        assert not bool((caches[0][1] == 0xA5).all(dim=1).any())
    torch.cuda.synchronize()


@pytest.mark.parametrize("a", gen.SWEEP_A)
def test_act_shared_factor_sweep(w, a):
    note(f"case: act sweep a={a} (config 5 shape)")
    wl = gen.make_workload(5, a=a, with_weights=False)
    q, s = run_act(w, wl)
    rows = _sample_rows(wl.M, 256, 100 + a)
    dec = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"sweep a={a}")
    note(f"  {st}")


# --------------------------------------------------------------- weight side


@pytest.mark.parametrize("clip", [True, False])
def test_weight_prep_tiny(w, clip):
    note(f"case: weight prep tiny clip={clip}")
    wl = gen.make_workload(1)
    q, s = run_weight(w, wl, clip=clip)
    dec = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha if clip else None, wl.wbeta if clip else None)
    parity.compare_quant(q, s, dec, label=f"weight tiny clip={clip}")


@pytest.mark.parametrize("a", [a for a in gen.SWEEP_A])
def test_weight_prep_shared_factor_sweep(w, a):
    """The offline weight side (the per-row-ratio instance of the transform
    kernel) for every shared-factor size of the sweep, on the config 5 weight
    (4096 x 4096): sampled rows, every code and scale against the oracle."""
    note(f"case: weight prep sweep a={a} (config 5 weight)")
    wl = gen.make_workload(5, a=a)
    q, s = run_weight(w, wl)
    rows = _sample_rows(wl.N, 256, 40 + a)
    dec = ob.weight_prep(wl.W_bits[rows], wl.A, wl.B, wl.walpha[rows], wl.wbeta[rows])
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"weight sweep a={a}")
    note(f"  {st}")


@pytest.mark.parametrize("cfg", [2, 3])
def test_weight_prep_full_config(w, cfg):
    note(f"case: weight prep full config {cfg}")
    wl = gen.make_workload(cfg)
    q, s = run_weight(w, wl)
    rows = _sample_rows(wl.N, 512, 7 + cfg)
    dec = ob.weight_prep(wl.W_bits[rows], wl.A, wl.B, wl.walpha[rows], wl.wbeta[rows])
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"weight config {cfg}")
    note(f"  {st}")


# ---------------------------------------------------------------------- GEMM


def _rand_mx(rng, rows, K, lo=110, hi=135):
    codes = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def run_gemm(w, xc, xs, wc, ws, dtype):
    Y = w.mxfp4_gemm(torch.from_numpy(ob.pack_codes(xc)).to(DEV), torch.from_numpy(xs).to(DEV),
                     torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV), out_dtype=dtype)
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 16, 64), (33, 47, 96), (128, 128, 256), (130, 250, 288),
                                   (200, 64, 1024), (64, 300, 4096), (33, 47, 512), (257, 129, 768),
                                   (512, 512, 2048)])
def test_gemm_isolated_matches_oracle(w, M, N, K):
    """The same packed operands go to both sides (random codes and scales)."""
    note(f"case: gemm isolated {M}x{N}x{K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    xc, xs = _rand_mx(rng, M, K)
    wc, ws = _rand_mx(rng, N, K)
    ref = ob.gemm(xc, xs, wc, ws)
    bound = parity.gemm_bound(ob.gemm_abs(xc, xs, wc, ws), K)
    y32 = run_gemm(w, xc, xs, wc, ws, torch.float32)
    err = np.abs(y32 - ref)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.max() <= 1e-3 * np.abs(ref).max()
    yb = run_gemm(w, xc, xs, wc, ws, torch.bfloat16)
    assert np.array_equal(yb, parity.bf16_rne(y32).astype(np.float64))


def test_gemm_exact_on_tiny_chain(w):
    """Tiny operands from the oracle chain: fp32 accumulation of these small
    dyadic products is exact, so the GPU result equals the exact rational sum."""
    note("case: gemm tiny chain exact")
    wl = gen.make_workload(1)
    x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y32 = run_gemm(w, x.codes, x.scales, wt.codes, wt.scales, torch.float32)
    bound = parity.gemm_bound(ob.gemm_abs(x.codes, x.scales, wt.codes, wt.scales), wl.K)
    assert np.all(np.abs(y32 - ref) <= bound)


def test_end_to_end_tiny(w):
    note("case: end-to-end tiny")
    wl = gen.make_workload(1)
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                   dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Y = w.mxfp4_gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y = Y.cpu().numpy().astype(np.float64)
    assert np.abs(y - ref).max() <= 1e-3 * np.abs(ref).max()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_end_to_end_full_config(w, cfg):
    """Full-size chain X, W -> Y in the launch configuration the benchmark times;
    sampled outputs against the oracle chain computed one row/column at a time."""
    note(f"case: end-to-end full config {cfg}")
    wl = gen.make_workload(cfg)
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                   dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Y32 = w.mxfp4_gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    Yb = w.mxfp4_gemm(xq, xs, wq, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.M, 48, 500 + cfg)
    cols = _sample_rows(wl.N, 48, 600 + cfg)
    x = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits[cols], wl.A, wl.B, wl.walpha[cols], wl.wbeta[cols])
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y32 = Y32[rows][:, cols].cpu().numpy().astype(np.float64)
    rel = np.abs(y32 - ref).max() / np.abs(ref).max()
    note(f"  max rel err {rel:.3e}")
    assert rel <= 1e-3
    # isolated GEMM on the GPU's own operands: elementwise fp32 bound
    gx = ob.unpack_codes(xq[rows].cpu().numpy())
    gw = ob.unpack_codes(wq[cols].cpu().numpy())
    gxs, gws = xs[rows].cpu().numpy(), ws[cols].cpu().numpy()
    ref_g, abs_g = ob.gemm_rows_cols(gx, gxs, gw, gws, np.arange(len(rows)), np.arange(len(cols)))
    assert np.all(np.abs(y32 - ref_g) <= parity.gemm_bound(abs_g, wl.K))
    yb = Yb[rows][:, cols].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(yb, parity.bf16_rne(y32).astype(np.float64))


@pytest.mark.parametrize("a", gen.SWEEP_A)
def test_end_to_end_shared_factor_sweep(w, a):
    """Config 5 (16384 x 4096 x 4096) end to end for every shared-factor size,
    through the path the benchmark times (transform kernel, offline weight
    prep and packing, the packed GEMM): sampled outputs against the oracle
    chain (1e-3 relative, fp32 output), the fp32 bound elementwise on the
    GPU's own operands, and bf16 = RNE(fp32)."""
    note(f"case: end-to-end sweep a={a} (config 5)")
    wl = gen.make_workload(5, a=a)
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                   dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    wp = w.weight_pack(wq, ws)
    Y32 = w.mxfp4_gemm_packed(xq, xs, wp, out_dtype=torch.float32)
    Yb = w.mxfp4_gemm_packed(xq, xs, wp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.M, 40, 1500 + a)
    cols = _sample_rows(wl.N, 40, 1600 + a)
    x = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits[cols], wl.A, wl.B, wl.walpha[cols], wl.wbeta[cols])
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y32 = Y32[rows][:, cols].cpu().numpy().astype(np.float64)
    rel = np.abs(y32 - ref).max() / np.abs(ref).max()
    note(f"  max rel err {rel:.3e}")
    assert rel <= 1e-3
    gx = ob.unpack_codes(xq[rows].cpu().numpy())
    gw = ob.unpack_codes(wq[cols].cpu().numpy())
    ref_g, abs_g = ob.gemm_rows_cols(gx, xs[rows].cpu().numpy(), gw, ws[cols].cpu().numpy(),
                                     np.arange(len(rows)), np.arange(len(cols)))
    assert np.all(np.abs(y32 - ref_g) <= parity.gemm_bound(abs_g, wl.K))
    yb = Yb[rows][:, cols].float().cpu().numpy()
    assert np.array_equal(yb, parity.bf16_rne(y32.astype(np.float32)))


# ------------------------------------------------------- packed-weight GEMM


def _packed_layout(wq_bytes: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """The byte layout batq_weight_pack documents, written out with numpy."""
    N, K2 = wq_bytes.shape
    K = 2 * K2
    G, S = (N + 31) // 32, K // 256
    codes = np.zeros((G * 32, K2), np.uint8)
    codes[:N] = wq_bytes
    scales = np.full((G * 32, K // 32), 127, np.uint8)
    scales[:N] = ws
    out = np.zeros((G, S, 4352), np.uint8)
    lanes = np.arange(64)
    for g in range(G):
        rows = 32 * g + lanes % 32
        for s in range(S):
            first = 8 * s + 4 * (lanes // 32)  # MX block of sub-step 0, per lane
            for j in range(4):
                blk = first + j
                out[g, s, 1024 * j:1024 * (j + 1)] = np.stack(
                    [codes[rows[l], 16 * blk[l]:16 * blk[l] + 16] for l in range(64)]).reshape(-1)
            out[g, s, 4096:] = np.stack([scales[rows[l], first[l]:first[l] + 4] for l in range(64)]).reshape(-1)
    return out.reshape(-1)


@pytest.mark.parametrize("N,K", [(1, 256), (32, 512), (47, 768), (300, 256)])
def test_weight_pack_layout(w, N, K):
    note(f"case: weight pack layout {N}x{K}")
    rng = np.random.default_rng(N + K)
    wc, ws = _rand_mx(rng, N, K)
    wq = ob.pack_codes(wc)
    P = w.weight_pack(torch.from_numpy(wq).to(DEV), torch.from_numpy(ws).to(DEV))
    torch.cuda.synchronize()
    got = P.data.cpu().numpy()
    assert got.size == w.weight_packed_bytes(N, K)
    assert np.array_equal(got, _packed_layout(wq, ws))


def run_gemm_packed(w, xc, xs, wc, ws, dtype):
    wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV))
    Y = w.mxfp4_gemm_packed(torch.from_numpy(ob.pack_codes(xc)).to(DEV), torch.from_numpy(xs).to(DEV), wp,
                            out_dtype=dtype)
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64)


# K / 256 in {1, 2, 4, 8, 16, 48} take the fully unrolled kernels; 3, 6, 12, 13,
# 20, 25 the looped one, whose body covers 12 stages (13, 20 and 25 end inside
# a second or third pass, 20 with four-stage scale groups, 13 and 25 without).
# M and N cover partial row and column tiles.  The last five
# shapes have more than 256 tiles of 128 x 256 with K / 256 in {4, 8, 48}: they
# run the two-workgroups-per-CU kernel (direct-to-LDS activation loads); N =
# 33001 gives output rows that are not whole 16-byte chunks (scalar stores).
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (33, 47, 256), (128, 256, 512), (130, 250, 768),
                                   (257, 129, 1024), (40, 33, 1536), (200, 300, 2048), (64, 520, 3072),
                                   (64, 300, 4096), (129, 257, 12288), (96, 200, 3328), (130, 300, 5120),
                                   (64, 96, 6400), (2000, 12200, 1024),
                                   (4000, 8000, 1024), (2100, 8300, 2048), (2100, 4200, 12288),
                                   (1000, 33001, 1024)])
def test_packed_gemm_matches_oracle_and_unpacked(w, M, N, K):
    note(f"case: packed gemm {M}x{N}x{K}")
    rng = np.random.default_rng(M * 5 + N * 11 + K)
    xc, xs = _rand_mx(rng, M, K)
    wc, ws = _rand_mx(rng, N, K)
    ref = ob.gemm(xc, xs, wc, ws)
    bound = parity.gemm_bound(ob.gemm_abs(xc, xs, wc, ws), K)
    y32 = run_gemm_packed(w, xc, xs, wc, ws, torch.float32)
    err = np.abs(y32 - ref)
    assert np.all(err <= bound), float((err - bound).max())
    # same MFMA sequence per output as the unpacked kernel: identical bits
    assert np.array_equal(y32, run_gemm(w, xc, xs, wc, ws, torch.float32))
    yb = run_gemm_packed(w, xc, xs, wc, ws, torch.bfloat16)
    assert np.array_equal(yb, parity.bf16_rne(y32).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(2048, 12288, 4096), (16384, 4096, 4096)])
def test_timed_gemm_instance_matches_oracle(w, M, N, K):
    """The kernel the benchmark times (two workgroups per CU, K / 256 = 16,
    more than 256 tiles) at the up/gate and large-prefill shapes, on random
    MXFP4 operands: sampled rows with every column against the oracle, the
    fp32 bound elementwise, 1e-3 relative, and bf16 = RNE(fp32)."""
    note(f"case: timed GEMM instance {M}x{N}x{K}")
    assert w.packed_gemm_kernel(M, N, K) == 1
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    xc, xs = _rand_mx(rng, M, K)
    wc, ws = _rand_mx(rng, N, K)
    wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV))
    xq_d, xs_d = torch.from_numpy(ob.pack_codes(xc)).to(DEV), torch.from_numpy(xs).to(DEV)
    y32 = w.mxfp4_gemm_packed(xq_d, xs_d, wp, out_dtype=torch.float32)
    yb = w.mxfp4_gemm_packed(xq_d, xs_d, wp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # rows of every 128-row tile position, the first and last tiles included
    rows = np.unique(np.concatenate([_sample_rows(M, 40, M + K), np.arange(120, 136), [M - 129, M - 128]]))
    ref, absum = ob.gemm_rows_cols(xc, xs, wc, ws, rows, np.arange(N))
    got = y32[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = parity.gemm_bound(absum, K)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.max() <= 1e-3 * np.abs(ref).max()
    gotb = yb[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    assert np.array_equal(gotb, parity.bf16_rne(got.astype(np.float32)))
    note(f"  rows {len(rows)}, max err / bound {float((err / np.maximum(bound, 1e-300)).max()):.3f}")


def test_packed_gemm_unaligned_output(w):
    """Y rows not a whole number of 16-byte chunks: scalar store path."""
    note("case: packed gemm unaligned output")
    rng = np.random.default_rng(77)
    M, N, K = 70, 61, 512
    xc, xs = _rand_mx(rng, M, K)
    wc, ws = _rand_mx(rng, N, K)
    ref = ob.gemm(xc, xs, wc, ws)
    bound = parity.gemm_bound(ob.gemm_abs(xc, xs, wc, ws), K)
    for dt in (torch.float32, torch.bfloat16):
        y = run_gemm_packed(w, xc, xs, wc, ws, dt)
        lim = bound if dt == torch.float32 else bound + np.abs(ref) * 2.0 ** -8
        assert np.all(np.abs(y - ref) <= lim)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_packed_end_to_end_full_config(w, cfg):
    """The chain the benchmark times (prepared weight packed offline): equal to
    the unpacked GEMM on the same operands, bit for bit, over the whole output;
    the unpacked path is held to the oracle by the tests above."""
    note(f"case: packed end-to-end config {cfg}")
    wl = gen.make_workload(cfg)
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                   dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    wp = w.weight_pack(wq, ws)
    Yp = w.mxfp4_gemm_packed(xq, xs, wp, out_dtype=torch.bfloat16)
    Yu = w.mxfp4_gemm(xq, xs, wq, ws, out_dtype=torch.bfloat16)
    Y32 = w.mxfp4_gemm_packed(xq, xs, wp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Yp, Yu)
    rows = _sample_rows(wl.M, 16, 700 + cfg)
    cols = _sample_rows(wl.N, 16, 800 + cfg)
    x = ob.act_transform_quant(wl.X_bits[rows], wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits[cols], wl.A, wl.B, wl.walpha[cols], wl.wbeta[cols])
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y = Y32[rows][:, cols].cpu().numpy().astype(np.float64)
    rel = np.abs(y - ref).max() / np.abs(ref).max()
    note(f"  max rel err {rel:.3e}")
    assert rel <= 1e-3
    yb = Yp[rows][:, cols].float().cpu().numpy()
    assert np.array_equal(yb, parity.bf16_rne(y.astype(np.float32)))




@pytest.mark.parametrize("M,N,K", [(2048, 4200, 1024), (100, 300, 512)])
def test_step_graph_replays_match_eager(w, M, N, K):
    """The online step (transform + clip + MXFP4 quantisation, then the packed
    GEMM) captured in a HIP graph: every one of several replays, with eager
    work and synchronisations between them, equals the eager result bit for
    bit (no library call records a memset).  The first shape runs the
    two-workgroups-per-CU GEMM, the second the one-per-CU kernel."""
    note(f"case: step graph replay {M}x{N}x{K}")
    assert w.packed_gemm_kernel(M, N, K) == (1 if M == 2048 else 0)
    wl = gen.make_custom(M, K, N, seed=M + N)
    X = dev_bf16(wl.X_bits)
    A, B = dev_f32(wl.A), dev_f32(wl.B)
    rh, rl = dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta))
    wq, wsc = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    Xs = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        w.act_transform_quant(X, A, B, rh, rl, out=(Xq, Xs))
        w.mxfp4_gemm_packed(Xq, Xs, Wp, out=Y)

    step()
    torch.cuda.synchronize()
    eager = Y.clone()
    other = dev_bf16(np.ascontiguousarray(wl.X_bits[::-1]))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        Y.fill_(float("nan"))
        Xq.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), eager.view(torch.int16)), rep
        oq, os_ = w.act_transform_quant(other, A, B, rh, rl)  # eager work between replays
        w.mxfp4_gemm_packed(oq, os_, Wp, out_dtype=torch.float32)
        torch.cuda.synchronize()

# ------------------------------------------- block-Hadamard (BRQ) special case


@pytest.mark.parametrize("cfg,clip", [(1, False), (2, False), (2, True), (3, False)])
def test_act_block_hadamard(w, cfg, clip):
    """The block rotation of the BRQ article is the GPK transform with
    A = H_8 / sqrt(8), B_i = H_4 / 2 (P_i = H_32 / sqrt(32)); same kernel, same
    parity rules, with and without the block-wise clipping."""
    note(f"case: act block-Hadamard config {cfg} clip={clip}")
    wl = gen.make_workload(cfg, with_weights=False)
    A, B = gen.hadamard_factors(wl.K)
    q, s = run_act(w, wl, A=A, B=B, clip=clip)
    rows = np.arange(wl.M) if wl.M <= 1024 else _sample_rows(wl.M, 1024, 300 + cfg)
    dec = ob.act_transform_quant(wl.X_bits[rows], A, B, wl.alpha if clip else None, wl.beta if clip else None)
    st = parity.compare_quant(q[rows], s[rows], dec, label=f"hadamard config {cfg} clip={clip}")
    note(f"  {st}")


def test_block_hadamard_end_to_end(w):
    """Block-Hadamard chain X, W -> Y: the weight side uses P^-T = P (orthogonal,
    symmetric); sampled outputs against the oracle chain, and the packed GEMM
    equals the unpacked one."""
    note("case: block-Hadamard end to end (config 2)")
    wl = gen.make_workload(2)
    A, B = gen.hadamard_factors(wl.K)
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(A), dev_f32(B), None, None)
    wq, ws = w.prepare_weight(dev_bf16(wl.W_bits), A, B, None, None)
    wp = w.weight_pack(wq, ws)
    Yp = w.mxfp4_gemm_packed(xq, xs, wp, out_dtype=torch.float32)
    Yu = w.mxfp4_gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Yp, Yu)
    rows = _sample_rows(wl.M, 16, 901)
    cols = _sample_rows(wl.N, 16, 902)
    x = ob.act_transform_quant(wl.X_bits[rows], A, B, None, None)
    wt = ob.weight_prep(wl.W_bits[cols], A, B, None, None)
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y = Yp[rows][:, cols].cpu().numpy().astype(np.float64)
    rel = np.abs(y - ref).max() / np.abs(ref).max()
    note(f"  max rel err {rel:.3e}")
    assert rel <= 1e-3
