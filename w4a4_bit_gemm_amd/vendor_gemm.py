"""ctypes binding over libbatq_vendor.so: hipBLASLt's block-scaled MXFP4 GEMM
on the operands of :func:`w4a4_bit_gemm_amd.mxfp4_gemm` (include/batq_vendor.h).

A comparison for the benchmark, not part of the path: the package never
imports this module.  Argument marshalling only; the checks mirror the main
binding's.
"""
from __future__ import annotations

import ctypes
import os

from . import binding as _b

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbatq_vendor.so")
_lib = None

_ERRORS = {-1: "bad arguments", -2: "a hipBLASLt call failed", -3: "no hipBLASLt algorithm for this shape"}


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
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.batq_vendor_gemm_create.restype = ctypes.c_int
    lib.batq_vendor_gemm_create.argtypes = [I64, I64, I64, I32, ctypes.c_size_t, ctypes.POINTER(P)]
    lib.batq_vendor_gemm_algos.restype = I32
    lib.batq_vendor_gemm_algos.argtypes = [P]
    lib.batq_vendor_gemm_run.restype = ctypes.c_int
    lib.batq_vendor_gemm_run.argtypes = [P, I32, P, P, P, P, P, P, P]
    lib.batq_vendor_gemm_destroy.restype = None
    lib.batq_vendor_gemm_destroy.argtypes = [P]
    lib.batq_vendor_version.restype = I32
    lib.batq_vendor_version.argtypes = []
    lib.batq_vendor_last_status.restype = I32
    lib.batq_vendor_last_status.argtypes = []
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        extra = f" (hipBLASLt status {_load().batq_vendor_last_status()})" if rc == -2 else ""
        raise RuntimeError(f"batq_vendor: {_ERRORS.get(rc, f'error {rc}')}{extra}")


def version() -> int:
    return int(_load().batq_vendor_version())


class VendorGemm:
    """A hipBLASLt plan for Y = X W^T (M x N x K), with its own workspace.
    :meth:`run` takes the operands of the W4A4 GEMM: E2M1 codes [rows][K/2],
    UE8M0 scales [rows][K/32], bf16 output [M][N]."""

    def __init__(self, M: int, N: int, K: int, device, max_algos: int = 16, workspace_bytes: int = 256 << 20):
        torch = _b._torch()
        self.M, self.N, self.K = M, N, K
        self.workspace = torch.empty(workspace_bytes, dtype=torch.uint8, device=device)
        plan = ctypes.c_void_p()
        _check(_load().batq_vendor_gemm_create(M, N, K, max_algos, workspace_bytes, ctypes.byref(plan)))
        self._plan = plan

    @property
    def algos(self) -> int:
        return int(_load().batq_vendor_gemm_algos(self._plan))

    def run(self, algo: int, Xq, Xs, Wq, Ws, Y) -> None:
        torch = _b._torch()
        M, N, K = self.M, self.N, self.K
        _b._req_shape(Xq, torch.uint8, (M, K // 2), "Xq")
        _b._req_shape(Xs, torch.uint8, (M, K // 32), "Xs")
        _b._req_shape(Wq, torch.uint8, (N, K // 2), "Wq")
        _b._req_shape(Ws, torch.uint8, (N, K // 32), "Ws")
        _b._req_shape(Y, torch.bfloat16, (M, N), "Y")
        _b._dev(Xq, Xs, Wq, Ws, Y, self.workspace)
        _check(_load().batq_vendor_gemm_run(self._plan, algo, Xq.data_ptr(), Xs.data_ptr(), Wq.data_ptr(),
                                            Ws.data_ptr(), Y.data_ptr(), self.workspace.data_ptr(),
                                            _b._stream_ptr(torch, Y.device)))

    def close(self) -> None:
        if self._plan is not None and self._plan.value:
            _load().batq_vendor_gemm_destroy(self._plan)
        self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
