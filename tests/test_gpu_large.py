"""GPU parity at the size limits: operands past 2 GiB, where every byte offset
must be 64-bit or stay inside a buffer descriptor's 32-bit range.

* Activations of 262192 and 263168 tokens x 4096 channels (2.15 GB of bf16):
  the transform kernel's strided walk with a ragged last tile, and its skewed
  walk.
* MXFP4 codes past 2 GiB (262200 x 16384): the packed GEMM leaves its
  direct-to-LDS kernel, whose descriptors hold 32-bit offsets, for the
  one-workgroup-per-CU kernel with 64-bit addresses.
* Codes just under 2 GiB (1048000 x 4096, E2M1; 524000 x 4096, E4M3): the
  direct-to-LDS kernel at the largest offsets it accepts.

Inputs come from the seeded generators: a base of 4096 rows, expanded on the
device by whole-block column rotations per group of 4096 rows
(``workloads.gen.large_rows``), so that rows of different groups differ.  The
oracle takes the sampled rows, rebuilt on the host from the same base."""
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
R0 = 4096  # base rows
TWO_GIB = 1 << 31


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def w():
    import w4a4_bit_gemm_amd as w

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return w


def expand(base: np.ndarray, rows: int, unit: int, period: int):
    """The large operand on the device: row r = base row r % R0 rotated by
    gen.large_group_shift(r // R0, unit, period) columns."""
    src = torch.from_numpy(np.ascontiguousarray(base)).to(DEV)
    out = torch.empty((rows, base.shape[1]), dtype=src.dtype, device=DEV)
    for g in range((rows + R0 - 1) // R0):
        n = min(R0, rows - g * R0)
        out[g * R0:g * R0 + n] = torch.roll(src[:n], gen.large_group_shift(g, unit, period), dims=1)
    return out


def sample(rows: int, boundary_row: int, seed: int) -> np.ndarray:
    """The first 32 rows, 80 rows around the row where the byte offset reaches
    2 GiB (or the last 80 rows, if it is never reached), the last 48 rows and
    64 random rows."""
    rng = np.random.default_rng(seed)
    b = min(boundary_row, rows - 40)
    picks = [np.arange(32), np.arange(b - 40, min(b + 40, rows)), np.arange(rows - 48, rows),
             rng.choice(rows, size=64, replace=False)]
    return np.unique(np.concatenate(picks))


@pytest.mark.parametrize("rows", [262192, 263168])
def test_act_past_2gib(w, rows):
    K = 4096
    note(f"case: act transform {rows}x{K} bf16 ({rows * K * 2 / 1e9:.2f} GB)")
    assert rows * K * 2 > TWO_GIB
    base = gen.make_custom(R0, K, 8, a=8, seed=rows % 1000)
    nb = K // 32
    X = expand(base.X_bits.view(np.int16), rows, 32, nb).view(torch.bfloat16)
    rh = torch.from_numpy(w.clip_ratios(base.alpha)).to(DEV)
    rl = torch.from_numpy(w.clip_ratios(base.beta)).to(DEV)
    q, s = w.act_transform_quant(X, torch.from_numpy(base.A).to(DEV), torch.from_numpy(base.B).to(DEV), rh, rl)
    torch.cuda.synchronize()
    del X
    rows_s = sample(rows, TWO_GIB // (K * 2), rows)
    idx = torch.from_numpy(rows_s).to(DEV)
    q_s, s_s = q[idx].cpu().numpy(), s[idx].cpu().numpy()
    x_s = gen.large_rows(base.X_bits, rows_s, 32, nb)
    dec = ob.act_transform_quant(x_s, base.A, base.B, base.alpha, base.beta)
    st = parity.compare_quant(q_s, s_s, dec, label=f"act {rows}x{K} sampled")
    note(f"  rows {len(rows_s)}, mismatches {st['mismatches']}")


def _gemm_case(w, M, N, K, fp8, expect_kernel, seed):
    rng = np.random.default_rng(seed)
    if fp8:
        xc_base = rng.integers(0, 256, size=(R0, K), dtype=np.uint8)
        xc_base[(xc_base & 0x7F) == 0x7F] ^= 1  # no NaN codes
        Xq = expand(xc_base, M, 32, K // 32)
    else:
        xc_base = rng.integers(0, 16, size=(R0, K), dtype=np.uint8)
        Xq = expand(ob.pack_codes(xc_base), M, 16, K // 32)
    xs_base = rng.integers(110, 135, size=(R0, K // 32), dtype=np.uint8)
    Xs = expand(xs_base, M, 1, K // 32)
    wc = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    ws = rng.integers(110, 135, size=(N, K // 32), dtype=np.uint8)
    assert w.packed_gemm_kernel(M, N, K, act_fp8=fp8) == expect_kernel
    wp = w.weight_pack(torch.from_numpy(ob.pack_codes(wc)).to(DEV), torch.from_numpy(ws).to(DEV))
    gemm = w.mxfp8_gemm_packed if fp8 else w.mxfp4_gemm_packed
    y32 = gemm(Xq, Xs, wp, out_dtype=torch.float32)
    yb = gemm(Xq, Xs, wp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del Xq, Xs
    row_bytes = K if fp8 else K // 2
    rows_s = sample(M, TWO_GIB // row_bytes, seed)
    idx = torch.from_numpy(rows_s).to(DEV)
    got = y32[idx].cpu().numpy().astype(np.float64)
    gotb = yb[idx].float().cpu().numpy()
    fmt = "e4m3" if fp8 else "e2m1"
    xc_s = gen.large_rows(xc_base, rows_s, 32, K // 32)
    xs_s = gen.large_rows(xs_base, rows_s, 1, K // 32)
    sel = np.arange(len(rows_s))
    ref, absum = ob.gemm_rows_cols(xc_s, xs_s, wc, ws, sel, np.arange(N), x_fmt=fmt)
    bound = parity.gemm_bound(absum, K)
    if fp8:
        bound = bound + parity.f8f4_window_bound(ob.dequantize(xc_s, xs_s, fmt), ob.dequantize(wc, ws))
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.max() <= 1e-3 * np.abs(ref).max()
    assert np.array_equal(gotb, parity.bf16_rne(got.astype(np.float32)))
    note(f"  rows {len(rows_s)}, max err / bound {float((err / np.maximum(bound, 1e-300)).max()):.3f}")


@pytest.mark.parametrize("M,N,K,fp8", [(262200, 96, 16384, False), (524400, 256, 4096, True)])
def test_gemm_codes_past_2gib(w, M, N, K, fp8):
    """More than 2 GiB of activation codes: the one-workgroup-per-CU kernel."""
    note(f"case: packed gemm {M}x{N}x{K} {'E4M3' if fp8 else 'E2M1'} codes past 2 GiB")
    assert M * (K if fp8 else K // 2) >= TWO_GIB
    _gemm_case(w, M, N, K, fp8, 0, M + K)


@pytest.mark.parametrize("M,N,K,fp8", [(1048000, 256, 4096, False), (524000, 256, 4096, True)])
def test_gemm_codes_just_under_2gib(w, M, N, K, fp8):
    """Activation codes just under 2 GiB: the direct-to-LDS kernel at the
    largest offsets its descriptors accept."""
    note(f"case: packed gemm {M}x{N}x{K} {'E4M3' if fp8 else 'E2M1'} codes just under 2 GiB")
    assert M * (K if fp8 else K // 2) < TWO_GIB
    _gemm_case(w, M, N, K, fp8, 1, M + 7 * K)
