"""CPU model of the direct-to-LDS activation loads of the transform kernel and
of the two-workgroups-per-CU GEMMs: for ragged sizes, every 16-byte load that
the buffer range check lets through reads bytes inside its buffer.

The hardware range check of a raw buffer load covers the vector offset (plus
the instruction offset); the kernels put every row offset there and keep the
scalar offset to a position inside a row.  The model restates each kernel's
index formulas (transform_quant.hip: the loader wave; mxfp4_gemm_packed_dma.hip:
the code and scale loads of both kernels) and asserts, for every lane of every
load, that an in-range vector offset (offset < range) implies
base + offset + scalar offset + 16 <= the buffer's size.  A load that is out of
range reads zeros without touching memory.
"""
import numpy as np
import pytest

LANES = np.arange(64)


def _check(base, voff, soff, nrec, size, what):
    voff = np.asarray(voff, dtype=np.int64)
    live = voff < nrec
    end = base + voff[live] + soff + 16
    assert np.all(end <= size), f"{what}: read past the buffer end ({int(end.max())} > {size})"
    return int(live.sum())


def transform_loads(rows, K, ldx):
    """The loader of transform_quant_tiles: per tile and half tile, one
    descriptor based at the half's first row with range = bytes to the end of
    X; eight loads of 64 lanes (two rows each)."""
    ld2 = 2 * ldx
    size = rows * ld2
    tiles = (rows + 31) // 32
    live = 0
    for blk0 in range(0, K // 32, 8):
        voff = []
        for q in range(8):
            row = 2 * q + (LANES >> 5)
            c = (LANES & 31) ^ (row & 15)
            col = blk0 * 32 + 8 * c
            voff.append(row * ld2 + np.where(col < K, col * 2, 0))
        for t in range(tiles):
            for half in range(2):
                row0 = 32 * t + 16 * half
                left = (rows - row0) * ld2 if row0 < rows else 0
                nrec = min(left, 0x7FFFFFFF)
                for q in range(8):
                    live += _check(row0 * ld2, voff[q], 0, nrec, size, f"transform rows={rows} t={t} h={half}")
    return live


def w4a4_dma_loads(M, K):
    """mxfp4_gemm_packed_dma_kernel: codes (rows clamped to M - 1, stage in the
    scalar offset) and scale groups (rows clamped, group in the scalar offset)."""
    krow, srow, nst = K // 2, K // 32, K // 256
    live = 0
    for m0 in range(0, M, 128):
        for wave in range(4):
            for q in range(4):
                row = 8 * (4 * wave + q) + (LANES >> 3)
                gr = np.minimum(m0 + row, M - 1)
                swz = (row & 7) ^ ((row >> 3) & 1)
                qoff = gr * krow + 16 * ((LANES & 7) ^ swz)
                for st in range(nst):
                    live += _check(0, qoff, st * 128, M * krow, M * krow, f"w4a4 codes M={M}")
            row = 32 * wave + (LANES & 31)
            gr = np.minimum(m0 + row, M - 1)
            soff = gr * srow + 16 * (LANES >> 5)
            for g in range(nst // 4):
                live += _check(0, soff, 32 * g, M * srow, M * srow, f"w4a4 scales M={M}")
    return live


def w4a8_dma_loads(M, K):
    """w4a8_gemm_packed_dma_kernel: four lane offsets serve eight loads; loads
    4..7 (rows 16 further on) use a second descriptor based 16 rows later."""
    krow, nst = K, K // 256
    live = 0
    for m0 in range(0, M, 128):
        for wave in range(4):
            qoff = []
            for q in range(4):
                row = 4 * (8 * wave + q) + (LANES >> 4)
                qoff.append((m0 + row) * krow + 16 * ((LANES & 15) ^ (row & 15)))
            for q in range(8):
                base, nrec = (0, M * krow) if q < 4 else (16 * krow, max(M - 16, 0) * krow)
                for st in range(nst):
                    live += _check(base, qoff[q & 3], st * 256, nrec, M * krow, f"w4a8 codes M={M}")
    return live


@pytest.mark.parametrize("rows,K,ldx", [(1, 256, 256), (15, 256, 264), (16, 512, 512), (17, 256, 256),
                                        (31, 96, 96), (33, 4096, 4096), (100, 224, 224), (257, 768, 776)])
def test_transform_loads_stay_in_bounds(rows, K, ldx):
    live = transform_loads(rows, K, ldx)
    # every element of X is read by some in-range lane
    assert live >= rows * ((K + 255) // 256)


@pytest.mark.parametrize("M,K", [(1, 1024), (17, 1024), (130, 2048), (2000, 1024), (2100, 4096), (257, 12288)])
def test_w4a4_gemm_loads_stay_in_bounds(M, K):
    assert w4a4_dma_loads(M, K) > 0


@pytest.mark.parametrize("M,K", [(1, 1024), (15, 1024), (16, 1024), (17, 1024), (130, 2048), (2000, 1024),
                                 (2100, 2048)])
def test_w4a8_gemm_loads_stay_in_bounds(M, K):
    assert w4a8_dma_loads(M, K) > 0


def test_model_catches_the_scalar_row_offset():
    """The earlier form of the W4A8 loads (rows 16 further on through the
    scalar offset, against one descriptor of range M K) reads past the end for
    a ragged M: the check above would have failed on it."""
    M, K = 130, 1024
    m0, wave, q = 128, 0, 0
    row = 4 * (8 * wave + q) + (LANES >> 4)
    qoff = (m0 + row) * K + 16 * ((LANES & 15) ^ (row & 15))
    with pytest.raises(AssertionError, match="past the buffer end"):
        _check(0, qoff, 16 * K, M * K, M * K, "scalar row offset")
