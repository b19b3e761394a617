"""BATQuant W4A4 deployment path on MI355X (gfx950).

The compute lives in ``libbatq.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/batq.h``); :mod:`w4a4_bit_gemm_amd.binding` marshals
PyTorch device tensors and streams to it.  There is no fallback: importing the
binding raises if the library has not been built.
"""
from .binding import (  # noqa: F401
    BatqError,
    abi_version,
    act_transform_quant,
    clip_ratios,
    gpk_invert,
    library_path,
    native_library,
    mxfp4_gemm,
    mxfp4_gemm_packed,
    packed_gemm_kernel,
    transform_kernel,
    mxfp8_gemm_packed,
    act_transform_quant_mxfp8,
    PackedWeight,
    weight_pack,
    weight_packed_bytes,
    prepare_weight,
    weight_prep,
    DECODE_MAX_K,
    DECODE_MAX_M,
    decode_workspace,
    decode_workspace_bytes,
    w4a4_decode,
    w4a4_decode_noalloc,
    decode_noalloc_scratch_bytes,
    kv_cache_quant,
    probe_mfma_fp4,
    probe_stream_granule,
    probe_hbm_read,
    probe_hbm_copy,
    probe_hbm_stream,
)
