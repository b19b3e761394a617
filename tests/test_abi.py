"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, validates arguments before any HIP call, and its host helpers
agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import batquant as ob
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "batq.h")

OK, NULL, SHAPE, ALIGN, UNSUP, SINGULAR, HIP, TOO_LARGE = range(8)
FAKE = 0x10000  # aligned address never dereferenced: every case below fails a check first


@pytest.fixture(scope="module")
def lib():
    from w4a4_bit_gemm_amd import binding

    return binding._load()


PROBE_HEADER = os.path.join(ROOT, "include", "batq_probe.h")


def declared_functions(headers=(HEADER, PROBE_HEADER)):
    names = set()
    for h in headers:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(batq_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("batq_act_transform_quant", "batq_weight_prep", "batq_mxfp4_gemm", "batq_gpk_invert",
              "batq_clip_ratios", "batq_abi_version", "batq_status_str", "batq_weight_packed_bytes",
              "batq_weight_pack", "batq_mxfp4_gemm_packed", "batq_act_transform_quant_mxfp8",
              "batq_mxfp8_gemm_packed", "batq_decode_workspace_bytes", "batq_w4a4_decode",
              "batq_kv_cache_quant", "batq_packed_gemm_kernel", "batq_transform_kernel", "batq_probe_mfma_fp4", "batq_probe_hbm_read",
              "batq_probe_hbm_copy", "batq_probe_stream_granule", "batq_probe_hbm_stream"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.batq_abi_version() == 5
    for s in range(8):
        assert lib.batq_status_str(s) and lib.batq_status_str(s) != b"unknown status"
    assert lib.batq_status_str(99) == b"unknown status"


def _tq(lib, fn, x=FAKE, M=4, K=64, ld=64, a=8, b=4, A=FAKE, B=FAKE, rh=0, rl=0, q=FAKE, s=FAKE):
    return getattr(lib, fn)(x, M, K, ld, a, b, A, B, rh, rl, q, s, None)


@pytest.mark.parametrize("fn", ["batq_act_transform_quant", "batq_weight_prep", "batq_act_transform_quant_mxfp8"])
def test_transform_argument_checks(lib, fn):
    assert _tq(lib, fn, x=0) == NULL
    assert _tq(lib, fn, A=0) == NULL
    assert _tq(lib, fn, B=0) == NULL
    assert _tq(lib, fn, q=0) == NULL
    assert _tq(lib, fn, s=0) == NULL
    assert _tq(lib, fn, rh=FAKE, rl=0) == NULL
    assert _tq(lib, fn, K=48, ld=64) == SHAPE
    assert _tq(lib, fn, K=0, ld=0) == SHAPE
    assert _tq(lib, fn, M=-1) == SHAPE
    assert _tq(lib, fn, ld=32) == SHAPE
    assert _tq(lib, fn, a=8, b=8) == SHAPE
    assert _tq(lib, fn, a=-1, b=-32) == UNSUP
    assert _tq(lib, fn, x=FAKE + 2) == ALIGN
    assert _tq(lib, fn, q=FAKE + 8) == ALIGN
    assert _tq(lib, fn, ld=68) == ALIGN
    # empty input: a no-op that returns before touching the GPU
    assert _tq(lib, fn, M=0) == OK


def test_gemm_argument_checks(lib):
    f = lib.batq_mxfp4_gemm
    assert f(0, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, 0, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 48, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, -4, 4, 64, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 7, None) == UNSUP
    assert f(FAKE + 4, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, FAKE + 2, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 4, 64, FAKE, 0, None) == OK
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 0, 64, FAKE, 1, None) == OK


def test_packed_size(lib):
    f = lib.batq_weight_packed_bytes
    assert f(12288, 4096) == 384 * 16 * 4352
    assert f(33, 512) == 2 * 2 * 4352
    assert f(0, 256) == 0
    assert f(4, 100) == -1 and f(4, 0) == -1 and f(-1, 256) == -1 and f(4, 288) == -1


def test_pack_argument_checks(lib):
    f = lib.batq_weight_pack
    assert f(FAKE, FAKE, 4, 288, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, -1, 256, FAKE, None) == SHAPE
    assert f(0, FAKE, 4, 256, FAKE, None) == NULL
    assert f(FAKE, FAKE, 4, 256, 0, None) == NULL
    assert f(FAKE + 8, FAKE, 4, 256, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, 4, 256, FAKE + 4, None) == ALIGN
    assert f(FAKE, FAKE, 0, 256, FAKE, None) == OK


@pytest.mark.parametrize("name", ["batq_mxfp4_gemm_packed", "batq_mxfp8_gemm_packed"])
def test_packed_gemm_argument_checks(lib, name):
    f = getattr(lib, name)
    assert f(FAKE, FAKE, FAKE, 4, 4, 288, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 4, -1, 256, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 4, 256, FAKE, 3, None) == UNSUP
    assert f(FAKE, 0, FAKE, 4, 4, 256, FAKE, 0, None) == NULL
    assert f(FAKE, FAKE, 0, 4, 4, 256, FAKE, 0, None) == NULL
    assert f(FAKE + 8, FAKE, FAKE, 4, 4, 256, FAKE, 0, None) == ALIGN
    assert f(FAKE, FAKE + 2, FAKE, 4, 4, 256, FAKE, 0, None) == ALIGN
    assert f(FAKE, FAKE + 4, FAKE, 4, 4, 256, FAKE, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE + 4, 4, 4, 256, FAKE, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 4, 256, FAKE + 2, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 0, 4, 256, FAKE, 0, None) == OK
    assert f(FAKE, FAKE, FAKE, 4, 0, 256, FAKE, 1, None) == OK


def test_packed_gemm_kernel_choice(lib):
    """Two workgroups per CU only with more than 256 tiles of 128 x 256, a
    compiled stage count (K / 256 in 4, 8, 16, 48) and activation codes under
    2 GiB."""
    f = lib.batq_packed_gemm_kernel
    assert f(2048, 12288, 4096, 0) == 1                     # 16 x 48 tiles
    assert f(16384, 4096, 4096, 0) == 1
    assert f(2100, 4200, 12288, 0) == 1                     # 17 x 17 tiles
    assert f(2048, 4096, 12288, 0) == 0                     # 16 x 16 = 256 tiles: one per CU
    assert f(2048, 12288, 4096, 1) == 1 and f(2100, 8300, 2048, 1) == 1  # E4M3 activations
    assert f(2100, 4200, 12288, 1) == 1                     # E4M3 with 48 stages
    assert f(2048, 1 << 20, 4096, 0) == 1                   # 2.2 GB of packed weights: per-group descriptors
    assert f(2048, 12288, 3072, 0) == 0 and f(2048, 12288, 512, 0) == 0  # runtime / small stage counts
    assert f(1 << 20, 4096, 4096, 0) == 0                   # 2 GiB of activation codes
    assert f(1 << 19, 4096, 4096, 1) == 0 and f((1 << 19) - 128, 4096, 4096, 1) == 1
    assert f(0, 12288, 4096, 0) == 0
    assert f(4, 4, 100, 0) == -1 and f(-1, 4, 256, 0) == -1 and f(4, 4, 0, 0) == -1


def test_transform_kernel_choice(lib):
    """Two workgroups per CU where that grid holds 512 workgroups (16 column
    groups x 32 tile rows at K = 4096, each walking 4 or more tiles); one
    workgroup per CU with a dedicated loader wave for smaller grids."""
    f = lib.batq_transform_kernel
    assert f(16384, 4096) == 0                              # 512 workgroups of 16 tiles: skewed walk
    assert f(263168, 4096) == 0 and f(262192, 4096) == 0    # 257 tiles each; ragged
    assert f(16383, 4096) == 0 and f(8192, 4096) == 0       # 512 workgroups of 16, of 8 tiles
    assert f(16384, 1024) == 0                              # 4 column groups x 128 tile rows
    assert f(2048, 4096) == 1                               # capped at 4 tiles each: 256 workgroups
    assert f(2048, 12288) == 1                              # 48 column groups x 8: 384 workgroups
    assert f(32, 4096) == 1 and f(0, 4096) == 1 and f(4096, 1024) == 1
    assert f(-1, 4096) == -1 and f(16, 0) == -1 and f(16, 100) == -1


def test_decode_workspace_bytes(lib):
    """16 KiB of arrival counters, then fp32 partial tiles: one per 128-column
    chunk, K split of two 256-k stages and token; none when K is a single
    split (Y is written directly)."""
    f = lib.batq_decode_workspace_bytes
    C = 16384
    assert f(16, 4096, 4096) == C + 32 * 8 * 16 * 128 * 4    # 8 splits of 2 stages
    assert f(1, 300, 512) == 0                                # 2 stages: one split
    assert f(4, 12288, 4096) == C + 96 * 8 * 4 * 128 * 4
    assert f(8, 12288, 12288) == C + 96 * 24 * 8 * 128 * 4
    assert f(32, 4096, 4096) == C + 32 * 8 * 32 * 128 * 4
    assert f(17, 4096, 12288) == C + 32 * 24 * 17 * 128 * 4
    assert f(3, 100, 1280) == C + 1 * 3 * 3 * 128 * 4        # 5 stages: splits of 2, 2 and 1
    assert f(1, 524288, 1024) == C + 4096 * 2 * 1 * 128 * 4 and f(1, 524289, 1024) == -1
    assert f(0, 256, 256) == 0
    assert f(33, 256, 256) == -1 and f(-1, 256, 256) == -1
    assert f(4, 256, 100) == -1 and f(4, 256, 0) == -1 and f(4, -1, 256) == -1


def _dec(lib, x=FAKE, M=4, K=256, ld=256, a=8, b=4, A=FAKE, B=FAKE, rh=0, rl=0, wp=FAKE, N=256, y=FAKE, out=0,
         xq=0, xs=0, ws=FAKE, wsb=1 << 30):
    return lib.batq_w4a4_decode(x, M, K, ld, a, b, A, B, rh, rl, wp, N, y, out, xq, xs, ws, wsb, None)


def test_decode_limits_match_the_header():
    import re
    from w4a4_bit_gemm_amd import binding as bd
    h = open(os.path.join(ROOT, "include", "batq.h")).read()
    assert int(re.search(r"#define BATQ_DECODE_MAX_M (\d+)", h).group(1)) == bd.DECODE_MAX_M
    assert int(re.search(r"#define BATQ_DECODE_MAX_K (\d+)", h).group(1)) == bd.DECODE_MAX_K == 8191 * 512


def test_decode_argument_checks(lib):
    assert _dec(lib, K=8191 * 512 + 256, ld=8191 * 512 + 256) == SHAPE  # more K splits than the kernel counts
    assert lib.batq_decode_workspace_bytes(4, 256, 8191 * 512 + 256) == -1
    assert lib.batq_decode_workspace_bytes(4, 256, 8191 * 512) > 0
    assert _dec(lib, M=33) == SHAPE
    assert _dec(lib, M=-1) == SHAPE
    assert _dec(lib, K=224, ld=256) == SHAPE
    assert _dec(lib, K=0, ld=0) == SHAPE
    assert _dec(lib, ld=128) == SHAPE
    assert _dec(lib, a=8, b=8) == SHAPE
    assert _dec(lib, wsb=lib.batq_decode_workspace_bytes(4, 256, 256) - 1) == SHAPE
    assert _dec(lib, a=-1, b=-32) == UNSUP
    assert _dec(lib, out=5) == UNSUP
    for kw in ("x", "A", "B", "wp", "y", "ws"):
        assert _dec(lib, **{kw: 0}) == NULL, kw
    assert _dec(lib, rh=FAKE) == NULL
    assert _dec(lib, xq=FAKE) == NULL
    assert _dec(lib, x=FAKE + 2) == ALIGN
    assert _dec(lib, ld=260, K=256) == ALIGN
    assert _dec(lib, wp=FAKE + 8) == ALIGN
    assert _dec(lib, y=FAKE + 2) == ALIGN
    assert _dec(lib, ws=FAKE + 16) == ALIGN
    assert _dec(lib, xq=FAKE + 4, xs=FAKE) == ALIGN
    # empty batch or no columns: no-ops that return before touching the GPU
    assert _dec(lib, M=0) == OK
    assert _dec(lib, N=0) == OK


def _kv(lib, x=FAKE, T=4, HD=256, ld=256, a=8, b=4, A=FAKE, B=FAKE, rh=0, rl=0, slots=FAKE, rows=16, fmt=4,
        q=FAKE, s=FAKE):
    return lib.batq_kv_cache_quant(x, T, HD, ld, a, b, A, B, rh, rl, slots, rows, fmt, q, s, None)


def test_kv_cache_argument_checks(lib):
    assert _kv(lib, fmt=6) == UNSUP
    assert _kv(lib, rows=-1) == SHAPE
    assert _kv(lib, HD=48, ld=64) == SHAPE
    assert _kv(lib, T=-1) == SHAPE
    assert _kv(lib, a=8, b=8) == SHAPE
    assert _kv(lib, slots=0) == NULL
    assert _kv(lib, q=0) == NULL
    assert _kv(lib, s=0) == NULL
    assert _kv(lib, rh=FAKE) == NULL
    assert _kv(lib, slots=FAKE + 4) == ALIGN
    assert _kv(lib, q=FAKE + 8) == ALIGN
    assert _kv(lib, x=FAKE + 2) == ALIGN
    assert _kv(lib, T=0, slots=0) == OK


def test_clip_ratios_match_oracle():
    from w4a4_bit_gemm_amd import binding

    x = np.random.default_rng(0).normal(3, 3, 4096).astype(np.float32)
    assert np.array_equal(binding.clip_ratios(x), ob.clip_ratio(x))


def test_clip_ratios_errors(lib):
    assert lib.batq_clip_ratios(None, None, 0) == OK
    assert lib.batq_clip_ratios(None, FAKE, 3) == NULL
    assert lib.batq_clip_ratios(FAKE, FAKE, -1) == SHAPE


@pytest.mark.parametrize("a", [1, 2, 4, 8, 16, 32])
def test_gpk_invert_matches_oracle_inverse(a):
    from w4a4_bit_gemm_amd import binding
    from workloads import gen

    A, B = gen.make_factors(5, 256, a, sweep=True)
    AinvT, BinvT = binding.gpk_invert(A, B)
    PinvT = ob.inverse_transpose_blocks(A, B)
    for i in range(B.shape[0]):
        got = np.kron(BinvT[i].astype(np.float64), AinvT.astype(np.float64))
        # each factor is the double inverse rounded once to float
        assert np.allclose(got, PinvT[i], rtol=4e-7, atol=4e-7 * np.abs(PinvT[i]).max())


def test_gpk_invert_rejects_singular(lib):
    A = np.eye(8, dtype=np.float32)
    A[3] = A[2]
    B = np.tile(np.eye(4, dtype=np.float32), (2, 1, 1))
    out_a = np.empty_like(A)
    out_b = np.empty_like(B)
    st = lib.batq_gpk_invert(8, 4, 2, A.ctypes.data, B.ctypes.data, out_a.ctypes.data, out_b.ctypes.data)
    assert st == SINGULAR
    B[1] = np.diag([1.0, 1e-9, 1.0, 1.0]).astype(np.float32)  # ill-conditioned private factor
    A = np.eye(8, dtype=np.float32)
    st = lib.batq_gpk_invert(8, 4, 2, A.ctypes.data, B.ctypes.data, out_a.ctypes.data, out_b.ctypes.data)
    assert st == SINGULAR
    assert lib.batq_gpk_invert(8, 8, 2, A.ctypes.data, B.ctypes.data, out_a.ctypes.data,
                               out_b.ctypes.data) == SHAPE


def test_probe_argument_checks(lib):
    g = lib.batq_probe_stream_granule()
    assert g == 256 * 8 * 16
    assert lib.batq_probe_mfma_fp4(0, 10, 1, 7, FAKE, FAKE, None) == SHAPE
    assert lib.batq_probe_mfma_fp4(4, 0, 1, 7, FAKE, FAKE, None) == SHAPE
    assert lib.batq_probe_mfma_fp4(4, 10, 1, 7, 0, FAKE, None) == NULL
    assert lib.batq_probe_mfma_fp4(4, 10, 1, 7, FAKE, FAKE + 4, None) == ALIGN
    assert lib.batq_probe_hbm_read(FAKE, g + 16, FAKE, None) == SHAPE
    assert lib.batq_probe_hbm_read(FAKE, 0, FAKE, None) == SHAPE
    assert lib.batq_probe_hbm_read(0, g, FAKE, None) == NULL
    assert lib.batq_probe_hbm_read(FAKE + 8, g, FAKE, None) == ALIGN
    assert lib.batq_probe_hbm_copy(FAKE, FAKE, 0, None) == SHAPE
    assert lib.batq_probe_hbm_copy(FAKE, 0, g, None) == NULL
    assert lib.batq_probe_hbm_copy(FAKE, FAKE + 4, g, None) == ALIGN
    assert lib.batq_probe_hbm_stream(FAKE, g, FAKE, 3, None) == UNSUP
    assert lib.batq_probe_hbm_stream(FAKE, g - 16, FAKE, 4, None) == SHAPE
    assert lib.batq_probe_hbm_stream(FAKE, g, 0, 4, None) == NULL


VENDOR_HEADER = os.path.join(ROOT, "include", "batq_vendor.h")


@pytest.fixture(scope="module")
def vendor_lib():
    from w4a4_bit_gemm_amd import vendor_gemm

    return vendor_gemm._load()


def test_vendor_library_exports_every_declared_symbol(vendor_lib):
    names = declared_functions((VENDOR_HEADER,))
    assert {"batq_vendor_gemm_create", "batq_vendor_gemm_run", "batq_vendor_gemm_algos",
            "batq_vendor_gemm_destroy", "batq_vendor_version", "batq_vendor_last_status"} <= set(names)
    for name in names:
        assert hasattr(vendor_lib, name), name


def test_vendor_library_is_separate_from_the_path(lib):
    # the comparison GEMM is not in libbatq.so, and libbatq.so does not link hipBLASLt
    assert not hasattr(lib, "batq_vendor_gemm_create")
    from w4a4_bit_gemm_amd import binding

    with open(binding.library_path(), "rb") as f:
        assert b"libhipblaslt" not in f.read()


def test_vendor_argument_checks_before_any_library_call(vendor_lib):
    plan = ctypes.c_void_p(FAKE)
    for M, N, K, algos in ((0, 16, 64, 4), (16, -1, 64, 4), (16, 16, 48, 4), (16, 16, 64, 0), (16, 16, 64, 65)):
        assert vendor_lib.batq_vendor_gemm_create(M, N, K, algos, 0, ctypes.byref(plan)) == -1
        assert plan.value is None  # cleared on failure
        plan = ctypes.c_void_p(FAKE)
    assert vendor_lib.batq_vendor_gemm_create(16, 16, 64, 4, 0, None) == -1
    assert vendor_lib.batq_vendor_gemm_algos(None) == -1
    assert vendor_lib.batq_vendor_gemm_run(None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    vendor_lib.batq_vendor_gemm_destroy(None)
