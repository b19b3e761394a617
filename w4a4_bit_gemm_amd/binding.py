"""ctypes binding over libbatq.so (argument marshalling only).

Every function here checks tensor dtype, device, shape and contiguity, passes raw
pointers plus ``torch.cuda.current_stream()`` to the C ABI, and raises
:class:`BatqError` with the library's message on a non-OK status.  No step of
the path runs in Python.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libbatq.so")
_lib = None

BATQ_OUT_BF16 = 0
BATQ_OUT_F32 = 1


class BatqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"batq status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m w4a4_bit_gemm_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    lib.batq_abi_version.restype = ctypes.c_int
    lib.batq_abi_version.argtypes = []
    lib.batq_status_str.restype = ctypes.c_char_p
    lib.batq_status_str.argtypes = [ctypes.c_int]
    lib.batq_clip_ratios.restype = ctypes.c_int
    lib.batq_clip_ratios.argtypes = [P, P, I64]
    lib.batq_gpk_invert.restype = ctypes.c_int
    lib.batq_gpk_invert.argtypes = [I32, I32, I64, P, P, P, P]
    lib.batq_act_transform_quant.restype = ctypes.c_int
    lib.batq_act_transform_quant.argtypes = [P, I64, I64, I64, I32, I32, P, P, P, P, P, P, P]
    lib.batq_weight_prep.restype = ctypes.c_int
    lib.batq_weight_prep.argtypes = [P, I64, I64, I64, I32, I32, P, P, P, P, P, P, P]
    lib.batq_mxfp4_gemm.restype = ctypes.c_int
    lib.batq_mxfp4_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, ctypes.c_int, P]
    lib.batq_weight_packed_bytes.restype = I64
    lib.batq_weight_packed_bytes.argtypes = [I64, I64]
    lib.batq_weight_pack.restype = ctypes.c_int
    lib.batq_weight_pack.argtypes = [P, P, I64, I64, P, P]
    lib.batq_mxfp4_gemm_packed.restype = ctypes.c_int
    lib.batq_mxfp4_gemm_packed.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_int, P]
    lib.batq_packed_gemm_kernel.restype = I32
    lib.batq_packed_gemm_kernel.argtypes = [I64, I64, I64, I32]
    lib.batq_act_transform_quant_mxfp8.restype = ctypes.c_int
    lib.batq_act_transform_quant_mxfp8.argtypes = [P, I64, I64, I64, ctypes.c_int32, ctypes.c_int32, P, P, P, P,
                                                    P, P, P]
    lib.batq_mxfp8_gemm_packed.restype = ctypes.c_int
    lib.batq_mxfp8_gemm_packed.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_int, P]
    lib.batq_kv_cache_quant.restype = ctypes.c_int
    lib.batq_kv_cache_quant.argtypes = [P, I64, I64, I64, I32, I32, P, P, P, P, P, I64, I32, P, P, P]
    lib.batq_decode_workspace_bytes.restype = I64
    lib.batq_decode_workspace_bytes.argtypes = [I64, I64, I64]
    lib.batq_w4a4_decode.restype = ctypes.c_int
    lib.batq_w4a4_decode.argtypes = [P, I64, I64, I64, I32, I32, P, P, P, P, P, I64, P, ctypes.c_int, P, P, P, I64,
                                     P]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise BatqError(status, _load().batq_status_str(status).decode())


def abi_version() -> int:
    return _load().batq_abi_version()


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def clip_ratios(logits) -> np.ndarray:
    """Host helper: float32 sigmoid ratios of float32 logits (C ABI)."""
    x = np.ascontiguousarray(np.asarray(logits, dtype=np.float32))
    out = np.empty_like(x)
    _check(_load().batq_clip_ratios(_np_ptr(x), _np_ptr(out), x.size))
    return out


def gpk_invert(A, B) -> Tuple[np.ndarray, np.ndarray]:
    """Host helper: (A^-T, B_i^-T) as float32 (C ABI, double-precision inversion)."""
    A = np.ascontiguousarray(np.asarray(A, dtype=np.float32))
    B = np.ascontiguousarray(np.asarray(B, dtype=np.float32))
    a = A.shape[0]
    b = B.shape[-1]
    AinvT = np.empty_like(A)
    BinvT = np.empty_like(B)
    _check(_load().batq_gpk_invert(a, b, B.shape[0], _np_ptr(A), _np_ptr(B), _np_ptr(AinvT), _np_ptr(BinvT)))
    return AinvT, BinvT


def _torch():
    import torch
    return torch


def _stream_ptr(torch, dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _req(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def act_transform_quant(X, A, B, r_hi=None, r_lo=None, out: Optional[tuple] = None):
    """Fused block transform + clip + MXFP4 quantisation of bf16 activations.

    X: [M, K] bf16; A: [a, a] f32; B: [K/32, b, b] f32; r_hi, r_lo: [K/32] f32
    ratios or None (no clip).  Returns (Xq uint8 [M, K/2], Xs uint8 [M, K/32]).
    """
    return _act(X, A, B, r_hi, r_lo, out, fp8=False)


def act_transform_quant_mxfp8(X, A, B, r_hi=None, r_lo=None, out: Optional[tuple] = None):
    """The same transform and clipping with MXFP8 (E4M3) output, the W4A8
    setting.  Returns (Xq8 uint8 [M, K], Xs uint8 [M, K/32])."""
    return _act(X, A, B, r_hi, r_lo, out, fp8=True)


def _act(X, A, B, r_hi, r_lo, out, fp8: bool):
    torch = _torch()
    _req(X, torch.bfloat16, "X")
    _req(A, torch.float32, "A")
    _req(B, torch.float32, "B")
    if (r_hi is None) != (r_lo is None):
        raise ValueError("r_hi and r_lo must both be given or both be None")
    if r_hi is not None:
        _req(r_hi, torch.float32, "r_hi")
        _req(r_lo, torch.float32, "r_lo")
    M, K = X.shape
    a, b = A.shape[0], B.shape[-1]
    if B.shape[0] != K // 32 or (r_hi is not None and r_hi.numel() != K // 32):
        raise ValueError("B / ratio shapes must match K/32 blocks")
    if out is None:
        Xq = torch.empty((M, K if fp8 else K // 2), dtype=torch.uint8, device=X.device)
        Xs = torch.empty((M, K // 32), dtype=torch.uint8, device=X.device)
    else:
        Xq, Xs = out
    fn = _load().batq_act_transform_quant_mxfp8 if fp8 else _load().batq_act_transform_quant
    st = fn(_ptr(X), M, K, X.stride(0), a, b, _ptr(A), _ptr(B), _ptr(r_hi), _ptr(r_lo), _ptr(Xq), _ptr(Xs),
            _stream_ptr(torch, X.device))
    _check(st)
    return Xq, Xs


def weight_prep(W, AinvT, BinvT, wr_hi=None, wr_lo=None, out: Optional[tuple] = None):
    """Offline weight side with already inverted-transposed factors.

    W: [N, K] bf16; AinvT: [a, a]; BinvT: [K/32, b, b]; wr_hi, wr_lo: [N, K/32]
    ratios or None.  Returns (Wq uint8 [N, K/2], Ws uint8 [N, K/32]).
    """
    torch = _torch()
    _req(W, torch.bfloat16, "W")
    _req(AinvT, torch.float32, "AinvT")
    _req(BinvT, torch.float32, "BinvT")
    if (wr_hi is None) != (wr_lo is None):
        raise ValueError("wr_hi and wr_lo must both be given or both be None")
    N, K = W.shape
    if wr_hi is not None:
        _req(wr_hi, torch.float32, "wr_hi")
        _req(wr_lo, torch.float32, "wr_lo")
        if tuple(wr_hi.shape) != (N, K // 32) or tuple(wr_lo.shape) != (N, K // 32):
            raise ValueError("weight ratios must be [N, K/32]")
    if BinvT.shape[0] != K // 32:
        raise ValueError("BinvT must have K/32 blocks")
    if out is None:
        Wq = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
        Ws = torch.empty((N, K // 32), dtype=torch.uint8, device=W.device)
    else:
        Wq, Ws = out
    st = _load().batq_weight_prep(_ptr(W), N, K, W.stride(0), AinvT.shape[0], BinvT.shape[-1], _ptr(AinvT),
                                  _ptr(BinvT), _ptr(wr_hi), _ptr(wr_lo), _ptr(Wq), _ptr(Ws),
                                  _stream_ptr(torch, W.device))
    _check(st)
    return Wq, Ws


def prepare_weight(W, A_host, B_host, walpha_host=None, wbeta_host=None):
    """Convenience for the offline step: invert the factors and map the weight
    clip logits to ratios on the host (C ABI helpers), copy them to the device
    and run :func:`weight_prep`."""
    torch = _torch()
    AinvT, BinvT = gpk_invert(A_host, B_host)
    dev = W.device
    rh = rl = None
    if walpha_host is not None:
        rh = torch.from_numpy(clip_ratios(walpha_host)).to(dev)
        rl = torch.from_numpy(clip_ratios(wbeta_host)).to(dev)
    return weight_prep(W, torch.from_numpy(AinvT).to(dev), torch.from_numpy(BinvT).to(dev), rh, rl)


def mxfp4_gemm(Xq, Xs, Wq, Ws, out_dtype=None, out=None):
    """Y = deq(Xq, Xs) deq(Wq, Ws)^T with FP32 accumulation; bf16 (default) or f32 out."""
    torch = _torch()
    for t, n in ((Xq, "Xq"), (Xs, "Xs"), (Wq, "Wq"), (Ws, "Ws")):
        _req(t, torch.uint8, n)
    M, K2 = Xq.shape
    N = Wq.shape[0]
    K = 2 * K2
    if Wq.shape[1] != K2 or tuple(Xs.shape) != (M, K // 32) or tuple(Ws.shape) != (N, K // 32):
        raise ValueError("operand shapes do not match")
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Xq.device)
    else:
        _req(out, out_dtype, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    code = BATQ_OUT_F32 if out_dtype == torch.float32 else BATQ_OUT_BF16
    st = _load().batq_mxfp4_gemm(_ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), M, N, K, _ptr(out), code,
                                 _stream_ptr(torch, Xq.device))
    _check(st)
    return out


def weight_packed_bytes(N: int, K: int) -> int:
    """Bytes of the packed weight form (C ABI; -1 for unsupported shapes)."""
    return int(_load().batq_weight_packed_bytes(N, K))


class PackedWeight:
    """A weight in the matrix-core lane order produced by :func:`weight_pack`."""

    def __init__(self, data, N: int, K: int):
        self.data = data
        self.N = N
        self.K = K


def weight_pack(Wq, Ws, out=None) -> PackedWeight:
    """Offline: repack MXFP4 weights (from :func:`weight_prep`) for
    :func:`mxfp4_gemm_packed`.  Needs K % 256 == 0."""
    torch = _torch()
    _req(Wq, torch.uint8, "Wq")
    _req(Ws, torch.uint8, "Ws")
    N, K2 = Wq.shape
    K = 2 * K2
    nbytes = weight_packed_bytes(N, K)
    if nbytes < 0:
        raise ValueError("packed weights need K to be a positive multiple of 256")
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=Wq.device)
    _check(_load().batq_weight_pack(_ptr(Wq), _ptr(Ws), N, K, _ptr(out), _stream_ptr(torch, Wq.device)))
    return PackedWeight(out, N, K)


def mxfp4_gemm_packed(Xq, Xs, Wp: PackedWeight, out_dtype=None, out=None):
    """Y = deq(Xq, Xs) deq(W)^T with W packed by :func:`weight_pack`; same
    result as :func:`mxfp4_gemm` on the unpacked weight."""
    torch = _torch()
    _req(Xq, torch.uint8, "Xq")
    _req(Xs, torch.uint8, "Xs")
    M, K2 = Xq.shape
    K = 2 * K2
    if K != Wp.K or tuple(Xs.shape) != (M, K // 32):
        raise ValueError("operand shapes do not match")
    N = Wp.N
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Xq.device)
    else:
        _req(out, out_dtype, "out")
    code = BATQ_OUT_F32 if out_dtype == torch.float32 else BATQ_OUT_BF16
    st = _load().batq_mxfp4_gemm_packed(_ptr(Xq), _ptr(Xs), _ptr(Wp.data), M, N, K, _ptr(out), code,
                                        _stream_ptr(torch, Xq.device))
    _check(st)
    return out


def mxfp8_gemm_packed(Xq8, Xs, Wp: PackedWeight, out_dtype=None, out=None):
    """W4A8: Y = deq8(Xq8, Xs) deq4(W)^T with W packed by :func:`weight_pack`
    and MXFP8 (E4M3) activation codes from :func:`act_transform_quant_mxfp8`."""
    torch = _torch()
    _req(Xq8, torch.uint8, "Xq8")
    _req(Xs, torch.uint8, "Xs")
    M, K = Xq8.shape
    if K != Wp.K or tuple(Xs.shape) != (M, K // 32):
        raise ValueError("operand shapes do not match")
    N = Wp.N
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Xq8.device)
    else:
        _req(out, out_dtype, "out")
    code = BATQ_OUT_F32 if out_dtype == torch.float32 else BATQ_OUT_BF16
    st = _load().batq_mxfp8_gemm_packed(_ptr(Xq8), _ptr(Xs), _ptr(Wp.data), M, N, K, _ptr(out), code,
                                        _stream_ptr(torch, Xq8.device))
    _check(st)
    return out


def packed_gemm_kernel(M: int, N: int, K: int, act_fp8: bool = False) -> int:
    """Which kernel the packed GEMM launches for this shape (host-only query):
    0 one workgroup per CU, 1 two per CU (same results); -1 bad shape."""
    return int(_load().batq_packed_gemm_kernel(M, N, K, 1 if act_fp8 else 0))


DECODE_MAX_M = 32


def decode_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of workspace :func:`w4a4_decode` needs (-1 for unsupported shapes)."""
    return int(_load().batq_decode_workspace_bytes(M, N, K))


def decode_workspace(M: int, N: int, K: int, device):
    """A workspace for :func:`w4a4_decode` (256-byte aligned as allocated by the
    PyTorch caching allocator; one per stream)."""
    torch = _torch()
    n = decode_workspace_bytes(M, N, K)
    if n < 0:
        raise ValueError(f"unsupported decode shape M={M} N={N} K={K}")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def w4a4_decode(X, A, B, r_hi, r_lo, Wp: PackedWeight, workspace, out_dtype=None, out=None,
                quantized_out: Optional[tuple] = None):
    """Fused decode step: transform + clip + MXFP4 quantisation of X (M <= 32
    tokens) inside the GEMM against packed weights, one launch.

    X: [M, K] bf16; A, B, r_hi, r_lo as for :func:`act_transform_quant`;
    workspace: from :func:`decode_workspace` (one per stream).
    quantized_out: optional (Xq [M, K/2], Xs [M, K/32]) uint8 tensors that also
    receive the quantised activations.  Returns Y [M, N].
    """
    torch = _torch()
    _req(X, torch.bfloat16, "X")
    _req(A, torch.float32, "A")
    _req(B, torch.float32, "B")
    if (r_hi is None) != (r_lo is None):
        raise ValueError("r_hi and r_lo must both be given or both be None")
    if r_hi is not None:
        _req(r_hi, torch.float32, "r_hi")
        _req(r_lo, torch.float32, "r_lo")
    _req(workspace, torch.uint8, "workspace")
    M, K = X.shape
    if K != Wp.K:
        raise ValueError("X and the packed weight disagree on K")
    N = Wp.N
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    else:
        _req(out, out_dtype, "out")
    Xq, Xs = quantized_out if quantized_out is not None else (None, None)
    code = BATQ_OUT_F32 if out_dtype == torch.float32 else BATQ_OUT_BF16
    st = _load().batq_w4a4_decode(_ptr(X), M, K, X.stride(0), A.shape[0], B.shape[-1], _ptr(A), _ptr(B),
                                  _ptr(r_hi), _ptr(r_lo), _ptr(Wp.data), N, _ptr(out), code, _ptr(Xq), _ptr(Xs),
                                  _ptr(workspace), workspace.numel(), _stream_ptr(torch, X.device))
    _check(st)
    return out


def kv_cache_quant(KV, A, B, r_hi, r_lo, slots, cache_q, cache_s, fmt: int = 4):
    """Quantise new K or V rows into a cache: KV [T, H*D] bf16 (head_dim a
    multiple of 32), slots [T] int64 cache rows, cache_q [rows, H*D/2] (fmt 4,
    MXFP4) or [rows, H*D] (fmt 8, MXFP8 E4M3) uint8, cache_s [rows, H*D/32]
    uint8.  Rows of the cache not named by a slot are left untouched."""
    torch = _torch()
    _req(KV, torch.bfloat16, "KV")
    _req(A, torch.float32, "A")
    _req(B, torch.float32, "B")
    _req(slots, torch.int64, "slots")
    _req(cache_q, torch.uint8, "cache_q")
    _req(cache_s, torch.uint8, "cache_s")
    if (r_hi is None) != (r_lo is None):
        raise ValueError("r_hi and r_lo must both be given or both be None")
    T, HD = KV.shape
    rows = cache_q.shape[0]
    if fmt not in (4, 8) or tuple(cache_q.shape) != (rows, HD if fmt == 8 else HD // 2) \
            or tuple(cache_s.shape) != (rows, HD // 32) or slots.numel() != T:
        raise ValueError("cache / slot shapes do not match")
    st = _load().batq_kv_cache_quant(_ptr(KV), T, HD, KV.stride(0), A.shape[0], B.shape[-1], _ptr(A), _ptr(B),
                                     _ptr(r_hi), _ptr(r_lo), _ptr(slots), rows, fmt, _ptr(cache_q), _ptr(cache_s),
                                     _stream_ptr(torch, KV.device))
    _check(st)
