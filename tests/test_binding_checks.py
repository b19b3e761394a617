"""The Python binding rejects every wrongly typed or sized buffer before it
calls into the library (CPU only: the shape checks run before the device
check, so CPU tensors reach each of them, and a CPU tensor of the right shape
is then refused as not being on a HIP device)."""
import pytest

torch = pytest.importorskip("torch")

from w4a4_bit_gemm_amd import binding as bd  # noqa: E402

M, K, N = 4, 256, 64


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def good_act():
    return dict(X=bf16(M, K), A=f32(8, 8), B=f32(K // 32, 4, 4), r_hi=f32(K // 32), r_lo=f32(K // 32))


def refused(fn, *args, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_act_transform_quant_rejections():
    g = good_act()
    f = bd.act_transform_quant
    refused(f, bf16(M, K, 1), g["A"], g["B"], match="2-D")
    refused(f, g["X"].float(), g["A"], g["B"], match="bfloat16")
    refused(f, g["X"], f32(8, 4), g["B"], match=r"\[a, a\]")
    refused(f, g["X"], f32(3, 3), f32(K // 32, 4, 4), match=r"\[a, a\]")
    refused(f, g["X"], g["A"], f32(K // 32 - 1, 4, 4), match="B must be")
    refused(f, g["X"], g["A"], f32(K // 32, 8, 8), match="B must be")
    refused(f, g["X"], g["A"], g["B"], f32(K // 32), None, match="both")
    refused(f, g["X"], g["A"], g["B"], f32(K // 32 + 1), f32(K // 32 + 1), match="r_hi must have shape")
    refused(f, g["X"], g["A"], g["B"], f32(K // 32), f32(1, K // 32), match="r_lo must have shape")
    refused(f, g["X"], g["A"], g["B"], out=(u8(M, K // 2 - 1), u8(M, K // 32)), match="Xq")
    refused(f, g["X"], g["A"], g["B"], out=(u8(M, K // 2), u8(M + 1, K // 32)), match="Xs")
    refused(f, g["X"], g["A"], g["B"], out=(u8(M, K // 2).float(), u8(M, K // 32)), match="uint8")
    # the MXFP8 variant wants one byte per element
    refused(bd.act_transform_quant_mxfp8, g["X"], g["A"], g["B"], out=(u8(M, K // 2), u8(M, K // 32)), match="Xq")
    # activations may be a column slice of a wider matrix (row stride > K), but
    # not a transposed or column-strided view
    refused(f, bf16(K, M).t(), g["A"], g["B"], match="unit column stride")
    refused(f, bf16(M, 2 * K)[:, ::2], g["A"], g["B"], match="unit column stride")
    refused(f, bf16(M, K + 64)[:, :K], g["A"], g["B"], match="CUDA")  # accepted up to the device check
    # right shapes, wrong device
    refused(f, g["X"], g["A"], g["B"], g["r_hi"], g["r_lo"], match="CUDA")
    refused(f, g["X"], g["A"], g["B"], out=(u8(M, K // 2), u8(M, K // 32)), match="CUDA")


def test_weight_prep_rejections():
    W = bf16(N, K)
    A, B = f32(4, 4), f32(K // 32, 8, 8)
    f = bd.weight_prep
    refused(f, W, A, f32(K // 32, 4, 4), match="BinvT must be")
    refused(f, W, A, B, f32(K // 32), f32(K // 32), match="wr_hi must have shape")
    refused(f, W, A, B, out=(u8(N, K // 2), u8(N, K // 16)), match="Ws")
    refused(f, W, A, B, out=(u8(N + 1, K // 2), u8(N, K // 32)), match="Wq")
    refused(f, W, A, B, f32(N, K // 32), f32(N, K // 32), match="CUDA")


def test_gemm_rejections():
    Xq, Xs, Wq, Ws = u8(M, K // 2), u8(M, K // 32), u8(N, K // 2), u8(N, K // 32)
    f = bd.mxfp4_gemm
    refused(f, Xq, u8(M, K // 16), Wq, Ws, match="shapes")
    refused(f, Xq, Xs, u8(N, K // 4), Ws, match="shapes")
    refused(f, Xq, Xs, Wq, Ws, out=f32(M, N + 1), match="out must have shape")
    refused(f, Xq, Xs, Wq, Ws, out=f32(M, N).double(), match="bfloat16 or float32")
    refused(f, Xq, Xs, Wq, Ws, out_dtype=torch.float16, match="bfloat16 or float32")
    refused(f, Xq, Xs, Wq, Ws, match="CUDA")


def test_packed_rejections():
    # packed sizes come from the library's own formula (a host-only call)
    Wp = bd.PackedWeight(u8(bd.weight_packed_bytes(N, K)), N, K)
    short = bd.PackedWeight(u8(bd.weight_packed_bytes(N, K) - 16), N, K)
    Xq, Xs = u8(M, K // 2), u8(M, K // 32)
    refused(bd.weight_pack, u8(N, K // 2), u8(N, K // 32), out=u8(10), match="out must have shape")
    refused(bd.weight_pack, u8(N, K // 2), u8(N + 1, K // 32), match="Ws must have shape")
    for fn, xq in ((bd.mxfp4_gemm_packed, Xq), (bd.mxfp8_gemm_packed, u8(M, K))):
        refused(fn, xq, Xs, short, match="Wp.data must have shape")
        refused(fn, xq, Xs, Wp.data, match="PackedWeight")
        refused(fn, xq, u8(M, K // 16), Wp, match="Xs must have shape")
        refused(fn, xq, Xs, Wp, out=f32(M - 1, N), match="out must have shape")
        refused(fn, xq, Xs, Wp, match="CUDA")


def test_decode_rejections():
    g = good_act()
    Wp = bd.PackedWeight(u8(bd.weight_packed_bytes(N, K)), N, K)
    ws = u8(bd.decode_workspace_bytes(M, N, K))
    f = bd.w4a4_decode
    refused(f, g["X"], g["A"], f32(K // 32, 2, 2), g["r_hi"], g["r_lo"], Wp, ws, match="B must be")
    refused(f, g["X"], g["A"], g["B"], f32(3), f32(3), Wp, ws, match="r_hi must have shape")
    refused(f, g["X"], g["A"], g["B"], g["r_hi"], g["r_lo"], bd.PackedWeight(u8(8), N, K), ws,
            match="Wp.data must have shape")
    refused(f, g["X"], g["A"], g["B"], g["r_hi"], g["r_lo"], Wp, ws, out=f32(M, N - 1), match="out must have shape")
    refused(f, g["X"], g["A"], g["B"], g["r_hi"], g["r_lo"], Wp, ws,
            quantized_out=(u8(M, K // 2), u8(M, K // 16)), match="Xs")
    refused(f, g["X"], g["A"], g["B"], g["r_hi"], g["r_lo"], Wp, ws, match="CUDA")


def test_kv_cache_rejections():
    T, HD, rows = 4, 256, 16
    KV, A, B = bf16(T, HD), f32(8, 8), f32(HD // 32, 4, 4)
    slots = torch.zeros(T, dtype=torch.int64)
    cq, cs = u8(rows, HD // 2), u8(rows, HD // 32)
    f = bd.kv_cache_quant
    refused(f, KV, A, B, f32(HD // 32), None, slots, cq, cs, match="both")
    refused(f, KV, A, B, f32(1), f32(1), slots, cq, cs, match="r_hi must have shape")
    refused(f, KV, A, B, None, None, torch.zeros(T + 1, dtype=torch.int64), cq, cs, match="slots")
    refused(f, KV, A, B, None, None, slots.int(), cq, cs, match="int64")
    refused(f, KV, A, B, None, None, slots, cq, cs, fmt=8, match="cache_q")
    refused(f, KV, A, B, None, None, slots, cq, u8(rows, HD // 16), match="cache_s")
    refused(f, KV, A, B, None, None, slots, cq, cs, fmt=6, match="fmt")
    refused(f, KV, A, B, f32(HD // 32), f32(HD // 32), slots, cq, cs, match="CUDA")
