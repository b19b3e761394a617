"""The no-allocation decode entry point (batq_w4a4_decode_noalloc) against the
workspace entry point (batq_w4a4_decode), through the C ABI: identical bits
on two calls in a row, the second with a smaller input, and the size limit."""
from __future__ import annotations

import numpy as np
import pytest

from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w():
    import w4a4_bit_gemm_amd as w

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return w


DEV = "cuda"


def _inputs(w, M, K, N, seed):
    wl = gen.make_custom(M, K, N, seed=seed)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)

    wq, ws = w.prepare_weight(bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    return dict(X=bf16(wl.X_bits), A=f32(wl.A), B=f32(wl.B), rh=f32(w.clip_ratios(wl.alpha)),
                rl=f32(w.clip_ratios(wl.beta)), Wp=w.weight_pack(wq, ws), M=M, K=K, N=N)


def _both(w, d, dtype):
    M, K, N = d["M"], d["K"], d["N"]
    ref = torch.empty((M, N), dtype=dtype, device=DEV)
    w.w4a4_decode(d["X"], d["A"], d["B"], d["rh"], d["rl"], d["Wp"], w.decode_workspace(M, N, K, DEV), out=ref)
    got = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
    xq = torch.zeros((M, K // 2), dtype=torch.uint8, device=DEV)
    xs = torch.zeros((M, K // 32), dtype=torch.uint8, device=DEV)
    w.w4a4_decode_noalloc(d["X"], d["A"], d["B"], d["rh"], d["rl"], d["Wp"], got, quantized_out=(xq, xs))
    torch.cuda.synchronize()
    return ref, got, xq, xs


def test_noalloc_decode_equals_workspace_decode_on_two_calls(w):
    """A large call, then a smaller one reusing the same device array: both
    equal the workspace entry point bit for bit (float and bf16 outputs), and
    the quantised activations equal the separate transform kernel's."""
    print("case: no-alloc decode 32x4096x4096 then 5x1024x768", flush=True)
    assert w.decode_workspace_bytes(32, 4096, 4096) <= w.decode_noalloc_scratch_bytes()
    for (M, K, N), seed, dtype in (((32, 4096, 4096), 1, torch.float32), ((5, 1024, 768), 2, torch.bfloat16)):
        d = _inputs(w, M, K, N, seed)
        ref, got, xq, xs = _both(w, d, dtype)
        assert torch.equal(ref.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)), (M, K, N)
        q, s = w.act_transform_quant(d["X"], d["A"], d["B"], d["rh"], d["rl"])
        torch.cuda.synchronize()
        assert torch.equal(q, xq) and torch.equal(s, xs)


def test_noalloc_decode_rejects_problems_beyond_its_array(w):
    """(32, 12288, 12288) needs more partial-tile scratch than the array holds:
    a clear error before anything is launched, and the output is untouched."""
    print("case: no-alloc decode size limit", flush=True)
    M, K, N = 32, 12288, 12288
    assert w.decode_workspace_bytes(M, N, K) > w.decode_noalloc_scratch_bytes()
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    A = torch.eye(8, dtype=torch.float32, device=DEV)
    B = torch.eye(4, dtype=torch.float32, device=DEV).repeat(K // 32, 1, 1)
    Wp = w.PackedWeight(torch.zeros(w.weight_packed_bytes(N, K), dtype=torch.uint8, device=DEV), N, K)
    out = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(w.BatqError, match="scratch"):
        w.w4a4_decode_noalloc(X, A, B, None, None, Wp, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
