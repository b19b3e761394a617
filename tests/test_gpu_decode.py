"""GPU parity of the fused decode step (transform + clip + MXFP4 quantisation
inside the packed-weight GEMM, one launch): the HIP kernel through the C ABI
against the CPU oracle on the same seeded inputs.  Needs an MI355X; run with
``-m gpu``."""
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


def run_decode(w, wl, Wp, clip=True, out_dtype=None):
    M, K = wl.X_bits.shape
    rh = dev_f32(w.clip_ratios(wl.alpha)) if clip else None
    rl = dev_f32(w.clip_ratios(wl.beta)) if clip else None
    ws = w.decode_workspace(M, Wp.N, K, DEV)
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    Y = w.w4a4_decode(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B), rh, rl, Wp, ws,
                      out_dtype=out_dtype or torch.float32, quantized_out=(xq, xs))
    torch.cuda.synchronize()
    return Y, xq, xs, ws


# M = 1 .. 32 tokens; K / 256 = 1 .. 16 stages; N with partial 256-column chunks.
@pytest.mark.parametrize("M,K,N,a,seed", [(1, 256, 256, 8, 1), (5, 1024, 300, 4, 2), (16, 4096, 4096, 8, 3),
                                          (17, 512, 1000, 2, 4), (32, 2048, 520, 16, 5), (3, 768, 33, 1, 6),
                                          (5, 768, 128, 32, 7)])
def test_decode_codes_match_oracle_and_transform_kernel(w, M, K, N, a, seed):
    """The activation codes the fused kernel quantises are the oracle's (decision
    rules) and bit-identical to the separate transform kernel's."""
    note(f"case: decode codes {M}x{K} N={N} a={a}")
    wl = gen.make_custom(M, K, N, a=a, seed=seed)
    wq, wsc = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    _, xq, xs, ws = run_decode(w, wl, Wp)
    q_ref, s_ref = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                         dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    assert torch.equal(xq, q_ref) and torch.equal(xs, s_ref)
    dec = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    parity.compare_quant(xq.cpu().numpy(), xs.cpu().numpy(), dec, label=f"decode {M}x{K}")


# K splits of two 256-k stages: the first shape is one split (Y written
# directly), 1024 is two, 1280 ends in a split of one stage, the others are 6
# to 24 splits added by the last-arriving workgroup of each chunk; N covers
# partial 128-column chunks.
@pytest.mark.parametrize("M,K,N,seed", [(1, 256, 256, 11), (7, 1024, 300, 12), (16, 4096, 4096, 13),
                                        (32, 3072, 777, 14), (32, 4096, 12288, 15), (17, 12288, 4096, 16),
                                        (9, 1280, 200, 17)])
def test_decode_gemm_exact_operands(w, M, K, N, seed):
    """Identity factors, no clipping and activations that are exact MXFP4 values
    (every block holds a +-6 code): the quantisation has no free decision, so
    the oracle's codes are the operands, and Y must meet the fp32 accumulation
    bound elementwise (the stage split only reorders the sum)."""
    note(f"case: decode exact {M}x{K} N={N}")
    rng = np.random.default_rng(seed)
    nb = K // 32
    codes = rng.integers(0, 16, size=(M, K), dtype=np.uint8)
    codes[:, ::32] = np.where(rng.random((M, nb)) < 0.5, 0x7, 0xF)  # one +-6 per block fixes the scale
    sc = rng.integers(115, 140, size=(M, nb), dtype=np.uint8)
    x = ob.dequantize(codes, sc)
    wl = gen.make_custom(M, K, 8, seed=seed)
    wl.X_bits = gen.f64_to_bf16_bits(x)
    assert np.array_equal(gen.bf16_bits_to_f32(wl.X_bits).astype(np.float64), x)
    wl.A = np.eye(8, dtype=np.float32)
    wl.B = np.tile(np.eye(4, dtype=np.float32), (nb, 1, 1))
    dec = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, None, None, exact=True)
    assert dec.n_exempt == 0 and np.array_equal(dec.scales, sc)
    wc = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    wsc = rng.integers(115, 140, size=(N, nb), dtype=np.uint8)
    Wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(wsc).to(DEV))
    ref = ob.gemm(dec.codes, dec.scales, wc, wsc)
    bound = parity.gemm_bound(ob.gemm_abs(dec.codes, dec.scales, wc, wsc), K)
    Y, xq, xs, ws = run_decode(w, wl, Wp, clip=False)
    assert np.array_equal(xq.cpu().numpy(), ob.pack_codes(dec.codes))
    y = Y.cpu().numpy().astype(np.float64)
    err = np.abs(y - ref)
    assert np.all(err <= bound), float((err - bound).max())
    Yb, _, _, _ = run_decode(w, wl, Wp, clip=False, out_dtype=torch.bfloat16)
    assert np.array_equal(Yb.float().cpu().numpy(), parity.bf16_rne(Y.cpu().numpy()))


COUNTER_BYTES = 16384  # the workspace's leading arrival counters


def test_decode_deterministic_and_reusable_workspace(w):
    """Two calls on one workspace, the first over partial tiles full of junk
    (zero arrival counters), give the same bits (the K splits are summed in a
    fixed order), and each call leaves the counters at zero."""
    note("case: decode determinism")
    wl = gen.make_workload(4)
    wq, wsc = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    M, K = wl.X_bits.shape
    ws = w.decode_workspace(M, Wp.N, K, DEV)
    ws.fill_(0xA5)
    ws[:COUNTER_BYTES].zero_()
    args = (dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B), dev_f32(w.clip_ratios(wl.alpha)),
            dev_f32(w.clip_ratios(wl.beta)), Wp, ws)
    y1 = w.w4a4_decode(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    y2 = w.w4a4_decode(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0


def test_decode_workspace_reused_across_shapes(w):
    """One workspace, sized for the largest call, with junk past its zeroed
    counters, serves calls of different M, N and K in turn (each call's
    partial area overlaps the earlier calls' data); each matches a call on a
    fresh workspace bit for bit."""
    note("case: decode workspace reuse across shapes")
    rng = np.random.default_rng(7)
    shapes = [(32, 12288, 4096), (3, 300, 512), (16, 4096, 12288), (1, 8192, 256), (32, 12288, 4096)]
    big = max(w.decode_workspace_bytes(M, N, K) for M, N, K in shapes)
    ws = torch.full((big,), 0x5A, dtype=torch.uint8, device=DEV)
    ws[:COUNTER_BYTES].zero_()
    for M, N, K in shapes:
        note(f"  shape M={M} N={N} K={K}")
        Wq = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)).to(DEV)
        Ws = torch.from_numpy(rng.integers(118, 124, (N, K // 32), dtype=np.uint8)).to(DEV)
        Wp = w.weight_pack(Wq, Ws)
        X = dev_bf16(np.ascontiguousarray(
            (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)))
        A = dev_f32(np.eye(8, dtype=np.float32) + 0.05 * rng.standard_normal((8, 8)).astype(np.float32))
        B = dev_f32(np.tile(np.eye(4, dtype=np.float32), (K // 32, 1, 1)))
        ref = w.w4a4_decode(X, A, B, None, None, Wp, w.decode_workspace(M, N, K, DEV), out_dtype=torch.float32)
        got = w.w4a4_decode(X, A, B, None, None, Wp, ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


@pytest.mark.parametrize("cfg", [1, 4])
def test_decode_end_to_end(w, cfg):
    """The chain X, W -> Y in one fused launch against the oracle chain (config
    1 on its first 32 tokens): within 1e-3 of max |Y| plus, per output, the
    change that the oracle's free decisions (activation or weight codes on a
    decision boundary) allow; and against the separate GPU path."""
    note(f"case: decode end to end config {cfg}")
    wl = gen.make_workload(cfg)
    if wl.M > 32:
        wl.X_bits = wl.X_bits[:32]
        wl.M = 32
    wq, wsc = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    Y, _, _, _ = run_decode(w, wl, Wp)
    x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    wt = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)
    ref = ob.gemm(x.codes, x.scales, wt.codes, wt.scales)
    y = Y.cpu().numpy().astype(np.float64)
    free = parity.free_decision_bound(x, wt)
    err = np.abs(y - ref)
    note(f"  max rel err {err.max() / np.abs(ref).max():.3e}; outputs touched by free decisions "
         f"{int((free > 0).sum())} of {free.size}")
    assert np.all(err <= 1e-3 * np.abs(ref).max() + free)
    assert (err[free == 0]).max() <= 1e-3 * np.abs(ref).max()
    xq, xs = w.act_transform_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B),
                                   dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta)))
    Ysep = w.mxfp4_gemm_packed(xq, xs, Wp, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert np.abs(y - Ysep).max() <= 1e-5 * np.abs(Ysep).max()


def test_decode_graph_replays_match_eager(w):
    """The fused decode step captured in a HIP graph: each of several replays,
    with eager work and synchronisations between them, equals the eager result
    bit for bit (the step records no memset; its workspace needs no clearing)."""
    note("case: decode graph replay")
    wl = gen.make_workload(4)
    wq, wsc = w.prepare_weight(dev_bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    M, K = wl.X_bits.shape
    X = dev_bf16(wl.X_bits)
    A, B = dev_f32(wl.A), dev_f32(wl.B)
    rh, rl = dev_f32(w.clip_ratios(wl.alpha)), dev_f32(w.clip_ratios(wl.beta))
    ws = w.decode_workspace(M, Wp.N, K, DEV)
    Y = torch.empty((M, Wp.N), dtype=torch.float32, device=DEV)
    eager = w.w4a4_decode(X, A, B, rh, rl, Wp, ws, out=Y).clone()
    other = dev_bf16(np.ascontiguousarray(wl.X_bits[::-1]))
    ws2 = w.decode_workspace(M, Wp.N, K, DEV)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w.w4a4_decode(X, A, B, rh, rl, Wp, ws, out=Y)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            w.w4a4_decode(X, A, B, rh, rl, Wp, ws, out=Y)
    torch.cuda.synchronize()
    for rep in range(4):
        Y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), eager.view(torch.int32)), rep
        w.w4a4_decode(other, A, B, rh, rl, Wp, ws2, out_dtype=torch.float32)  # eager work between replays
        torch.cuda.synchronize()
