"""Row-strided activations (the C ABI's leading dimension ld > K): a column
slice of a wider matrix must give the same bits as its contiguous copy, on
every entry point that takes ld.  The columns past K hold huge values, so any
read of them would change a block's range and its scale.  Needs an MI355X;
run with ``-m gpu``."""
from __future__ import annotations

import sys

import numpy as np
import pytest

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


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def strided(bits: np.ndarray, pad: int):
    """(contiguous X, the same values as a column slice of rows K + pad long)."""
    rows, K = bits.shape
    wide = np.full((rows, K + pad), 0x7E80, dtype=np.uint16)  # bf16 2^126 past column K
    wide[:, :K] = bits
    Xw = torch.from_numpy(wide.view(np.int16)).to(DEV).view(torch.bfloat16)
    Xc = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)
    Xs = Xw[:, :K]
    assert Xs.stride(0) == K + pad and not Xs.is_contiguous()
    return Xc, Xs


@pytest.mark.parametrize("M,K,a,pad", [(37, 800, 4, 64), (300, 4096, 8, 128), (5, 288, 1, 8)])
def test_transform_row_strided_equals_contiguous(w, M, K, a, pad):
    note(f"case: strided transform {M}x{K} a={a} ld={K + pad}")
    wl = gen.make_custom(M, K, 8, a=a, seed=M + K)
    Xc, Xs = strided(wl.X_bits, pad)
    A, B = f32(wl.A), f32(wl.B)
    rh, rl = f32(w.clip_ratios(wl.alpha)), f32(w.clip_ratios(wl.beta))
    for fn in (w.act_transform_quant, w.act_transform_quant_mxfp8):
        q0, s0 = fn(Xc, A, B, rh, rl)
        q1, s1 = fn(Xs, A, B, rh, rl)
        torch.cuda.synchronize()
        assert torch.equal(q0, q1) and torch.equal(s0, s1), fn.__name__


@pytest.mark.parametrize("N,K,pad", [(64, 800, 32), (300, 1024, 64)])
def test_weight_prep_row_strided_equals_contiguous(w, N, K, pad):
    note(f"case: strided weight prep {N}x{K} ld={K + pad}")
    wl = gen.make_custom(N, K, 8, a=8, seed=N + 3 * K)
    Wc, Ws = strided(wl.X_bits, pad)
    wa = np.random.default_rng(N).normal(3, 0.5, (N, K // 32))
    wb = np.random.default_rng(K).normal(3, 0.5, (N, K // 32))
    q0, s0 = w.prepare_weight(Wc, wl.A, wl.B, wa, wb)
    q1, s1 = w.prepare_weight(Ws, wl.A, wl.B, wa, wb)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1)


@pytest.mark.parametrize("M,K,N,pad", [(16, 1280, 300, 64), (2, 4096, 512, 256), (32, 512, 1000, 8)])
def test_decode_row_strided_equals_contiguous(w, M, K, N, pad):
    note(f"case: strided decode {M}x{K} N={N} ld={K + pad}")
    wl = gen.make_custom(M, K, N, a=8, seed=M + K + N)
    Xc, Xs = strided(wl.X_bits, pad)
    Wd = torch.from_numpy(np.ascontiguousarray(wl.W_bits).view(np.int16)).to(DEV).view(torch.bfloat16)
    wq, wsc = w.prepare_weight(Wd, wl.A, wl.B, wl.walpha, wl.wbeta)
    Wp = w.weight_pack(wq, wsc)
    A, B = f32(wl.A), f32(wl.B)
    rh, rl = f32(w.clip_ratios(wl.alpha)), f32(w.clip_ratios(wl.beta))
    ys = []
    for X in (Xc, Xs):
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
        xs = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
        y = w.w4a4_decode(X, A, B, rh, rl, Wp, w.decode_workspace(M, N, K, DEV), out_dtype=torch.float32,
                          quantized_out=(xq, xs))
        ys.append((y, xq, xs))
    y2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    w.w4a4_decode_noalloc(Xs, A, B, rh, rl, Wp, y2)
    torch.cuda.synchronize()
    (y0, q0, s0), (y1, q1, s1) = ys
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    assert torch.equal(q0, q1) and torch.equal(s0, s1)
    assert torch.equal(y0.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("fmt", [4, 8])
def test_kv_cache_row_strided_equals_contiguous(w, fmt):
    T, HD, pad, rows = 45, 256, 64, 128
    note(f"case: strided kv{fmt} {T}x{HD} ld={HD + pad}")
    wl = gen.make_custom(T, HD, 8, a=8, seed=fmt)
    Xc, Xs = strided(wl.X_bits, pad)
    A, B = f32(wl.A), f32(wl.B)
    rh, rl = f32(w.clip_ratios(wl.alpha)), f32(w.clip_ratios(wl.beta))
    slots = torch.from_numpy(np.random.default_rng(fmt).permutation(rows)[:T].astype(np.int64)).to(DEV)
    outs = []
    for X in (Xc, Xs):
        cq = torch.full((rows, HD // 2 if fmt == 4 else HD), 0x5A, dtype=torch.uint8, device=DEV)
        cs = torch.full((rows, HD // 32), 0x33, dtype=torch.uint8, device=DEV)
        w.kv_cache_quant(X, A, B, rh, rl, slots, cq, cs, fmt=fmt)
        outs.append((cq, cs))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
