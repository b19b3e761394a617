"""GPU parity of KV-cache quantisation (per-head block transform, clipping and
MXFP4 / MXFP8 quantisation of new K or V rows, written to their cache slots):
the HIP kernel through the C ABI against the CPU oracle.  Needs an MI355X;
run with ``-m gpu``."""
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
SENTINEL = 0xA5


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


# T new tokens, H heads x D head_dim, cache rows; slots include two out of range.
@pytest.mark.parametrize("T,H,D,rows,fmt,clip,seed", [(37, 8, 128, 100, 4, True, 1), (37, 8, 128, 100, 8, True, 2),
                                                       (1, 8, 128, 16, 4, False, 3), (70, 2, 64, 200, 8, False, 4),
                                                       (300, 8, 128, 512, 4, True, 5)])
def test_kv_cache_quant_matches_oracle(w, T, H, D, rows, fmt, clip, seed):
    note(f"case: kv cache T={T} HD={H * D} rows={rows} fmt={fmt} clip={clip}")
    HD = H * D
    wl = gen.make_custom(T, HD, 8, seed=seed)
    rng = np.random.default_rng(seed)
    slots = rng.choice(rows, size=T, replace=False).astype(np.int64)
    if T >= 3:
        slots[1], slots[2] = -1, rows  # skipped
    qcols = HD // 2 if fmt == 4 else HD
    cq = torch.full((rows, qcols), SENTINEL, dtype=torch.uint8, device=DEV)
    cs = torch.full((rows, HD // 32), SENTINEL, dtype=torch.uint8, device=DEV)
    rh = dev_f32(w.clip_ratios(wl.alpha)) if clip else None
    rl = dev_f32(w.clip_ratios(wl.beta)) if clip else None
    w.kv_cache_quant(dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B), rh, rl, torch.from_numpy(slots).to(DEV),
                     cq, cs, fmt=fmt)
    torch.cuda.synchronize()
    q, s = cq.cpu().numpy(), cs.cpu().numpy()
    f = "e2m1" if fmt == 4 else "e4m3"
    dec = ob.kv_cache_quant(wl.X_bits, wl.A, wl.B, wl.alpha if clip else None, wl.beta if clip else None, fmt=f)
    src = ob.kv_cache_rows(slots, rows)
    written = src >= 0
    assert np.all(q[~written] == SENTINEL) and np.all(s[~written] == SENTINEL)
    order = src[written]
    sub = ob.Decisions(dec.codes[order], dec.scales[order], dec.block_free[order], dec.elem_free[order],
                       dec.zero_sign_free[order], dec.y64[order], dec.z32[order])
    parity.compare_quant(q[written], s[written], sub, label=f"kv fmt {fmt}", fmt=f)


def test_kv_cache_quant_equals_activation_path(w):
    """The cache rows hold exactly what the activation path produces for the
    same rows (same kernel, same arithmetic), in slot order."""
    note("case: kv cache equals activation path")
    T, HD, rows = 64, 1024, 96
    wl = gen.make_custom(T, HD, 8, seed=9)
    slots = np.random.default_rng(9).permutation(rows)[:T].astype(np.int64)
    cq = torch.zeros((rows, HD // 2), dtype=torch.uint8, device=DEV)
    cs = torch.zeros((rows, HD // 32), dtype=torch.uint8, device=DEV)
    args = (dev_bf16(wl.X_bits), dev_f32(wl.A), dev_f32(wl.B), dev_f32(w.clip_ratios(wl.alpha)),
            dev_f32(w.clip_ratios(wl.beta)))
    w.kv_cache_quant(*args, torch.from_numpy(slots).to(DEV), cq, cs, fmt=4)
    xq, xs = w.act_transform_quant(*args)
    torch.cuda.synchronize()
    idx = torch.from_numpy(slots).to(DEV)
    assert torch.equal(cq[idx], xq) and torch.equal(cs[idx], xs)
