"""The C ABI library on the host: it loads, exports what include/sgemm.h
declares, and rejects bad arguments before any GPU call (no GPU needed)."""

import ctypes
import os
import re

import pytest

import dense_fp32_matrix_sgemm_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")

A, B, C = 0x10000, 0x20000000, 0x40000000  # distinct fake addresses, never touched


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sg.load_library()


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(sg.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    codes = [sg.SGEMM_OK, sg.SGEMM_ERR_DIM, sg.SGEMM_ERR_LD, sg.SGEMM_ERR_NULL,
             sg.SGEMM_ERR_VARIANT, sg.SGEMM_ERR_LAUNCH, sg.SGEMM_ERR_DEVICE, sg.SGEMM_ERR_ALIAS,
             sg.SGEMM_ERR_OP, sg.SGEMM_ERR_DTYPE, sg.SGEMM_ERR_SCRATCH]
    texts = [sg.sgemm_status_string(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert "unknown status" not in texts
    assert sg.sgemm_status_string(12345) == "unknown status"


def test_variant_names(lib):
    for name, code in sg.VARIANTS.items():
        assert sg.sgemm_variant_name(code) == name
    assert sg.sgemm_variant_name(7) is None
    assert sg.sgemm_variant_name(-2) is None
    assert sg.sgemm_best_variant(4096, 4096, 4096) in (0, 1, 2, 3)


CASES = [
    # (M, N, K, A, lda, B, ldb, C, ldc, variant) -> status
    ((-1, 4, 4, A, 4, B, 4, C, 4, 0), sg.SGEMM_ERR_DIM),
    ((4, -1, 4, A, 4, B, 4, C, 4, 0), sg.SGEMM_ERR_DIM),
    ((4, 4, -1, A, 4, B, 4, C, 4, 0), sg.SGEMM_ERR_DIM),
    ((4, 4, 4, A, 3, B, 4, C, 4, 0), sg.SGEMM_ERR_LD),
    ((4, 4, 4, A, 4, B, 3, C, 4, 0), sg.SGEMM_ERR_LD),
    ((4, 4, 4, A, 4, B, 4, C, 3, 0), sg.SGEMM_ERR_LD),
    ((4, 4, 0, A, 0, B, 4, C, 4, 0), sg.SGEMM_ERR_LD),      # lda >= max(1, K)
    ((0, 0, 0, None, 1, None, 1, None, 1, 0), sg.SGEMM_OK),  # empty, NULLs fine
    ((4, 4, 4, A, 4, B, 4, C, 4, 7), sg.SGEMM_ERR_VARIANT),
    ((4, 4, 4, A, 4, B, 4, C, 4, -2), sg.SGEMM_ERR_VARIANT),
    ((4, 4, 4, A, 4, B, 4, C, 4, 6), sg.SGEMM_OK),          # tiled rung with T = 32
    ((0, 4, 4, A, 4, B, 4, C, 4, 7), sg.SGEMM_ERR_VARIANT),  # variant checked first
    ((0, 4, 4, None, 4, None, 4, None, 4, 3), sg.SGEMM_OK),  # M == 0
    ((4, 0, 4, None, 4, None, 1, None, 1, 3), sg.SGEMM_OK),  # N == 0
    ((4, 4, 4, None, 4, B, 4, C, 4, 0), sg.SGEMM_ERR_NULL),
    ((4, 4, 4, A, 4, None, 4, C, 4, 0), sg.SGEMM_ERR_NULL),
    ((4, 4, 4, A, 4, B, 4, None, 4, 0), sg.SGEMM_ERR_NULL),
    ((4, 4, 0, None, 1, None, 4, C, 4, 0), sg.SGEMM_OK),     # K == 0: A, B unused
    ((4, 4, 0, None, 1, None, 4, None, 4, 0), sg.SGEMM_ERR_NULL),
    # C overlapping A or B
    ((4, 4, 4, A, 4, B, 4, A + 4 * 15, 4, 0), sg.SGEMM_ERR_ALIAS),   # C starts in A's last element
    ((4, 4, 4, A, 4, B, 4, A + 4 * 16, 4, 0), sg.SGEMM_OK),          # C starts right after A
    ((4, 4, 4, A, 4, B, 4, B - 4 * 16, 4, 0), sg.SGEMM_OK),          # C ends right before B
    ((4, 4, 4, A, 4, B, 4, B - 4 * 15, 4, 0), sg.SGEMM_ERR_ALIAS),
    ((4, 4, 0, A, 1, B, 4, A, 4, 0), sg.SGEMM_OK),                   # K == 0: A not read
    # Large, overflow-prone extents are handled in 64 bits
    ((2**31 - 1, 2, 2, A, 2, B, 2, C, 2**31 - 1, 0), sg.SGEMM_ERR_ALIAS),
]


@pytest.mark.parametrize("args,want", CASES)
def test_check_args(lib, args, want):
    assert sg.sgemm_check_args(*args) == want


@pytest.mark.parametrize("args,want", [c for c in CASES if c[1] != sg.SGEMM_OK])
def test_sgemm_rejects_before_touching_the_gpu(lib, args, want):
    M, N, K, pa, lda, pb, ldb, pc, ldc, variant = args
    assert sg.sgemm(M, N, K, pa, lda, pb, ldb, pc, ldc, None, variant) == want


def test_empty_product_returns_ok_without_gpu(lib):
    assert sg.sgemm(0, 5, 5, None, 5, None, 5, None, 5, None, 3) == sg.SGEMM_OK
    assert sg.sgemm(5, 0, 5, None, 5, None, 1, None, 1, None, 3) == sg.SGEMM_OK


def test_no_device_is_reported_not_crashed(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    rc = sg.sgemm(4, 4, 4, A, 4, B, 4, C, 4, None, 0)
    assert rc == sg.SGEMM_ERR_DEVICE


N_, T_ = sg.SGEMM_OP_N, sg.SGEMM_OP_T

EX_CASES = [
    # (transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant) -> status
    ((2, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_ERR_OP),
    ((N_, -1, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_ERR_OP),
    ((2, N_, -1, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_ERR_OP),    # flags checked first
    ((T_, T_, -1, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_ERR_DIM),
    # Leading dimensions follow the stored shapes.
    ((T_, N_, 6, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_ERR_LD),     # A^T stored 4 x 6
    ((T_, N_, 6, 4, 4, 1.0, A, 6, B, 4, 0.0, C, 4, 0), sg.SGEMM_OK),
    ((N_, N_, 6, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0), sg.SGEMM_OK),
    ((N_, T_, 4, 6, 3, 1.0, A, 3, B, 2, 0.0, C, 6, 0), sg.SGEMM_ERR_LD),     # B^T stored 6 x 3
    ((N_, T_, 4, 6, 3, 1.0, A, 3, B, 3, 0.0, C, 6, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 6, 3, 1.0, A, 3, B, 3, 0.0, C, 6, 0), sg.SGEMM_ERR_LD),     # B stored 3 x 6
    ((T_, T_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 3, 0), sg.SGEMM_ERR_LD),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 9), sg.SGEMM_ERR_VARIANT),
    # alpha == 0 or K == 0: A and B are not read (NULL or overlapping is fine).
    ((N_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 2.0, C, 4, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 0.0, A, 4, B, 4, 2.0, A, 4, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 1.0, None, 4, B, 4, 2.0, C, 4, 0), sg.SGEMM_ERR_NULL),
    ((N_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 2.0, None, 4, 0), sg.SGEMM_ERR_NULL),
    # Overlap is measured on the stored extents: A^T stored 8 x 2 spans 16 floats.
    ((T_, N_, 2, 4, 8, 1.0, A, 2, B, 4, 0.0, A + 4 * 15, 4, 0), sg.SGEMM_ERR_ALIAS),
    ((T_, N_, 2, 4, 8, 1.0, A, 2, B, 4, 0.0, A + 4 * 16, 4, 0), sg.SGEMM_OK),
    ((N_, T_, 4, 2, 8, 1.0, A, 8, B, 8, 0.0, B - 4 * 8, 2, 0), sg.SGEMM_OK),      # C ends where B^T starts
    ((N_, T_, 4, 2, 8, 1.0, A, 8, B, 8, 0.0, B - 4 * 7, 2, 0), sg.SGEMM_ERR_ALIAS),
]


@pytest.mark.parametrize("args,want", EX_CASES)
def test_ex_check_args(lib, args, want):
    assert sg.sgemm_ex_check_args(*args) == want


@pytest.mark.parametrize("args,want", [c for c in EX_CASES if c[1] != sg.SGEMM_OK])
def test_ex_rejects_before_touching_the_gpu(lib, args, want):
    ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc, variant = args
    assert sg.sgemm_ex(ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc, None, variant) == want


@pytest.mark.parametrize("args,want", CASES)
def test_plain_checks_are_the_general_checks(lib, args, want):
    M, N, K, pa, lda, pb, ldb, pc, ldc, variant = args
    assert sg.sgemm_ex_check_args(N_, N_, M, N, K, 1.0, pa, lda, pb, ldb, 0.0, pc, ldc, variant) == want


def test_ex_nothing_to_do_returns_ok_without_gpu(lib):
    # Empty C, and C = 1 * C (alpha == 0 or K == 0 with beta == 1).
    assert sg.sgemm_ex(N_, N_, 0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5, None, 3) == sg.SGEMM_OK
    assert sg.sgemm_ex(T_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, C, 4, None, 3) == sg.SGEMM_OK
    assert sg.sgemm_ex(N_, T_, 4, 4, 0, 2.0, None, 1, None, 1, 1.0, C, 4, None, 3) == sg.SGEMM_OK


def test_ex_no_device_is_reported_not_crashed(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert sg.sgemm_ex(T_, T_, 4, 4, 4, 1.0, A, 4, B, 4, 0.5, C, 4, None, 3) == sg.SGEMM_ERR_DEVICE
    assert sg.sgemm_ex(N_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 0.0, C, 4, None, 3) == sg.SGEMM_ERR_DEVICE


def test_storage_order_of_tensor_views():
    import torch
    x = torch.zeros(5, 7)
    assert sg._storage(x, "x") == (N_, 7)
    assert sg._storage(x.t(), "x") == (T_, 7)          # 7 x 5 view of 5 x 7 storage
    assert sg._storage(x[:, :3], "x") == (N_, 7)
    assert sg._storage(x[:3].t(), "x") == (T_, 7)
    assert sg._storage(x[:, 1:2].t(), "x") == (T_, 7)  # one row, elements 7 apart
    assert sg._storage(x[1:2].t(), "x") == (N_, 1)     # one column, elements adjacent
    with pytest.raises(ValueError):
        sg._storage(x[:, 0:1].expand(5, 4), "x")
    with pytest.raises(ValueError):
        sg._storage(x[::2, ::2], "x")


def test_sizes_beyond_int_are_refused_not_wrapped():
    # ctypes passes 2**32 + 8 to a C int as 8; the binding refuses such sizes.
    sg._check_int32(M=0, N=1, K=2**31 - 1, lda=7)
    for bad in (2**31, 2**32 + 8, -1):
        with pytest.raises(ValueError, match="int range"):
            sg._check_int32(M=4, N=4, K=4, lda=bad)
    # A stride past int range (a meta tensor: shape and strides, no storage).
    import torch
    x = torch.empty_strided((2, 3), (2**32 + 8, 1), device="meta")
    assert sg._storage(x, "x") == (N_, 2**32 + 8)


def test_matmul_rejects_bad_tensors():
    import torch
    a = torch.zeros(3, 4)
    with pytest.raises(ValueError):
        sg.matmul(a, torch.zeros(4, 2))          # CPU tensors: no CPU path
    with pytest.raises(TypeError):
        sg.matmul(a.double(), torch.zeros(4, 2))
    with pytest.raises(TypeError):
        sg.matmul(torch.zeros(3), torch.zeros(3, 2))
    with pytest.raises(ValueError):
        sg._variant_code("nope")
    with pytest.raises(ValueError):
        sg.gemm(a, torch.zeros(4, 2), beta=1.0)    # beta != 0 needs C


def test_mfma_tile_choice(lib):
    # 128x128 tiles split over their waves where they fill whole rounds of
    # the compute units with K >= 2048 (4096^3: four rounds) or give one per
    # compute unit (2048^2); 256x256 tiles at 4096^2 with a short K; 64x64
    # for the mid sizes and 32x32 for the smallest products.
    assert sg.sgemm_mfma_tile(4096, 4096, 4096) == (128, 128)
    assert sg.sgemm_mfma_tile(8192, 8192, 8192) == (128, 128)
    assert sg.sgemm_mfma_tile(4096, 4096, 1024) == (256, 256)
    assert sg.sgemm_mfma_tile(5000, 3000, 2000) == (256, 256)
    assert sg.sgemm_mfma_tile(2048, 2048, 2048) == (128, 128)
    assert sg.sgemm_mfma_tile(1024, 1024, 1024) == (64, 64)
    assert sg.sgemm_mfma_tile(3001, 2047, 4093) == (192, 128)   # 16 x 16 tiles: one per compute unit
    assert sg.sgemm_mfma_tile(3072, 2048, 4096) == (192, 128)
    assert sg.sgemm_mfma_tile(2047, 3001, 4093) == (128, 192)   # the same, turned round
    assert sg.sgemm_mfma_tile(2048, 3072, 4096) == (128, 192)
    assert sg.sgemm_mfma_tile(128, 128, 128) == (32, 32)     # at most one 32 x 32 tile per compute unit
    assert sg.sgemm_mfma_tile(512, 512, 512) == (32, 32)
    assert sg.sgemm_mfma_tile(640, 640, 640) == (64, 64)     # two 32 x 32 tiles per compute unit
    # Fewer compute units shift the choice toward larger tiles.
    assert sg.sgemm_mfma_tile(2048, 2048, 1024, cus=64) == (256, 256)
    assert sg.sgemm_mfma_tile(4096, 4096, 4096, cus=0) == sg.sgemm_mfma_tile(4096, 4096, 4096, cus=256)


WSPLIT = (64, 64, 32, 1, 1, 4)    # K split over four waves, each holding the whole tile
WSPLIT96 = (96, 96, 32, 1, 1, 4)  # the same on 96x96 and 128x128 tiles, one work-group per compute unit
WSPLIT128 = (128, 128, 16, 1, 1, 4)
MID = (128, 128, 32, 2, 4, 1)     # eight waves staged through LDS
KSPLIT32 = (32, 32, 32, 1, 1, 2)  # two single-wave sets sharing each slab
SMALL = (64, 64, 16, 2, 2, 1)     # plain 64x64, up to four work-groups per compute unit


def test_mfma_shape_choice(lib):
    # Up to two 64x64 tiles per compute unit take the tile whose K range is
    # split over its four waves, whatever K; three too when K is a multiple of
    # 32 (its chunk), else the 64x64 tiles that hold three or four per compute
    # unit at once. Products that leave most compute units without a 64x64
    # tile, or under 64 wide, take the 32x32 tile; under 64 rows with two
    # 64x64 tiles per compute unit, the two-set 64x64 tile.
    assert sg.sgemm_mfma_shape(1024, 1024, 1024) == WSPLIT
    assert sg.sgemm_mfma_shape(1000, 1000, 1000) == WSPLIT
    assert sg.sgemm_mfma_shape(640, 640, 640) == WSPLIT
    # One 96x96 or 128x128 tile per compute unit: the larger split tiles.
    assert sg.sgemm_mfma_shape(1536, 1536, 1536) == WSPLIT96
    assert sg.sgemm_mfma_shape(1500, 1500, 1500) == WSPLIT96
    assert sg.sgemm_mfma_shape(2048, 2048, 2048) == WSPLIT128
    assert sg.sgemm_mfma_shape(2000, 2040, 77) == WSPLIT128
    assert sg.sgemm_mfma_shape(8192, 512, 4096) == WSPLIT128
    # Under 128 rows, the eight-wave 128x128 tile.
    assert sg.sgemm_mfma_shape(120, 30000, 100) == MID
    assert sg.sgemm_mfma_shape(48, 12000, 1000) == (64, 64, 32, 2, 2, 2)
    assert sg.sgemm_mfma_shape(2048, 1024, 1024) == WSPLIT
    assert sg.sgemm_mfma_shape(4000, 70, 4000) == WSPLIT
    assert sg.sgemm_mfma_shape(1024, 1024, 1) == WSPLIT
    # Ragged K: up to two 64x64 tiles per compute unit, not three.
    assert sg.sgemm_mfma_shape(2048, 1024, 1000) == WSPLIT
    assert sg.sgemm_mfma_shape(1200, 1200, 1200) == WSPLIT
    assert sg.sgemm_mfma_shape(1200, 2400, 1200) == SMALL
    assert sg.sgemm_mfma_shape(1536, 1500, 1000) == WSPLIT96
    assert sg.sgemm_mfma_shape(1536, 1500, 1024) == WSPLIT96
    # More than three tiles per compute unit.
    assert sg.sgemm_mfma_shape(2200, 2200, 2208) != WSPLIT
    assert sg.sgemm_mfma_shape(2560, 2560, 2560) == SMALL
    # Under 64 wide.
    assert sg.sgemm_mfma_shape(16000, 8, 1000) != WSPLIT
    assert sg.sgemm_mfma_shape(16384, 5, 64) != WSPLIT
    assert sg.sgemm_mfma_shape(512, 512, 512) == KSPLIT32
    assert sg.sgemm_mfma_shape(128, 128, 128) == KSPLIT32
    assert sg.sgemm_mfma_shape(300, 257, 513) == KSPLIT32
    assert sg.sgemm_mfma_shape(3001, 2047, 4093) == (192, 128, 16, 2, 2, 1)
    assert sg.sgemm_mfma_shape(2047, 3001, 4093) == (128, 192, 16, 2, 2, 1)
    assert sg.sgemm_mfma_shape(4096, 4096, 4096) == WSPLIT128
    assert sg.sgemm_mfma_shape(6144, 6144, 4096) == WSPLIT128
    assert sg.sgemm_mfma_shape(4096, 4096, 1024) == (256, 256, 16, 4, 2, 1)    # short K
    assert sg.sgemm_mfma_shape(3072, 3072, 3072) == SMALL                      # rounds 75% full
    # Two or more 128 x 128 tiles per compute unit: the four-wave tile, two
    # work-groups to a compute unit; one per compute unit: the eight-wave one.
    # (unless the split 128x128 tile fills whole rounds with K >= 2048).
    assert sg.sgemm_mfma_shape(2048, 4096, 1024) == (128, 128, 16, 2, 2, 1)
    assert sg.sgemm_mfma_shape(4000, 5000, 2000) == (128, 128, 16, 2, 2, 1)
    assert sg.sgemm_mfma_shape(16384, 512, 1024) == (128, 128, 16, 2, 2, 1)
    assert sg.sgemm_mfma_shape(2048, 4096, 2048) == WSPLIT128
    assert sg.sgemm_mfma_shape(16384, 512, 4096) == WSPLIT128
    for shape in [(7, 9, 5), (128, 128, 128), (1024, 1024, 1024), (3001, 2047, 4093), (4096, 4096, 4096),
                  (8192, 300, 100), (2048, 4096, 2048), (1536, 1500, 1000)]:
        assert sg.sgemm_mfma_shape(*shape)[:2] == sg.sgemm_mfma_tile(*shape)
    shp = (ctypes.c_int * 6)()
    assert lib.sgemm_mfma_shape(-1, 4, 4, 0, shp) == sg.SGEMM_ERR_DIM
    assert lib.sgemm_mfma_shape(4, 4, -1, 0, shp) == sg.SGEMM_ERR_DIM
    assert lib.sgemm_mfma_shape(4, 4, 4, 0, None) == sg.SGEMM_ERR_NULL


def test_mfma_tile_errors(lib):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    assert lib.sgemm_mfma_tile(-1, 4, 4, 0, ctypes.byref(bm), ctypes.byref(bn)) == sg.SGEMM_ERR_DIM
    assert lib.sgemm_mfma_tile(4, 4, -1, 0, ctypes.byref(bm), ctypes.byref(bn)) == sg.SGEMM_ERR_DIM
    assert lib.sgemm_mfma_tile(4, 4, 4, 0, None, ctypes.byref(bn)) == sg.SGEMM_ERR_NULL
    assert lib.sgemm_mfma_tile(0, 0, 0, 0, ctypes.byref(bm), ctypes.byref(bn)) == sg.SGEMM_OK


def test_regblock_tile_choice(lib):
    # The pages' 128 x 128 tile where C holds at least 1.5 of them per compute
    # unit, 64 x 64 where it holds at least one per two compute units, 32 x 32
    # where it holds at least one of those per two compute units, else 16 x 16.
    assert sg.sgemm_regblock_tile(4096, 4096) == 128
    assert sg.sgemm_regblock_tile(3001, 2047) == 128     # 24 x 16 = 384 tiles: exactly 1.5 per CU
    assert sg.sgemm_regblock_tile(3001, 1919) == 64      # 24 x 15 = 360
    assert sg.sgemm_regblock_tile(2048, 2048) == 64      # 256: one per CU
    assert sg.sgemm_regblock_tile(1024, 1024) == 64
    assert sg.sgemm_regblock_tile(768, 768) == 64        # 12 x 12 = 144 tiles of 64
    assert sg.sgemm_regblock_tile(768, 640) == 32        # 12 x 10 = 120 < 128
    assert sg.sgemm_regblock_tile(512, 512) == 32        # 64 tiles of 64
    assert sg.sgemm_regblock_tile(384, 384) == 32        # 12 x 12 = 144 tiles of 32
    assert sg.sgemm_regblock_tile(384, 320) == 16        # 12 x 10 = 120 < 128
    assert sg.sgemm_regblock_tile(256, 256) == 16        # 64 tiles of 32
    assert sg.sgemm_regblock_tile(128, 128) == 16
    assert sg.sgemm_regblock_tile(1, 1) == 16
    assert sg.sgemm_regblock_tile(0, 0) == 16
    assert sg.sgemm_regblock_tile(2048, 2048, cus=64) == 128
    assert sg.sgemm_regblock_tile(4096, 4096, cus=0) == sg.sgemm_regblock_tile(4096, 4096, cus=256)
    assert lib.sgemm_regblock_tile(-1, 4, 0) == sg.SGEMM_ERR_DIM
    assert lib.sgemm_regblock_tile(4, -1, 0) == sg.SGEMM_ERR_DIM


BF, F16 = sg.SGEMM_LP_BF16, sg.SGEMM_LP_F16

LP_CASES = [
    # (dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) -> status
    ((0, N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_DTYPE),
    ((3, 2, N_, -1, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_DTYPE),     # type checked first
    ((BF, 2, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_OP),
    ((F16, N_, N_, 4, -1, 4, 1.0, A, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_DIM),
    ((BF, T_, N_, 6, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_LD),      # A^T stored 4 x 6
    ((BF, T_, N_, 6, 4, 4, 1.0, A, 6, B, 4, 0.0, C, 4), sg.SGEMM_OK),
    ((F16, N_, T_, 4, 6, 3, 1.0, A, 3, B, 2, 0.0, C, 6), sg.SGEMM_ERR_LD),     # B^T stored 6 x 3
    ((F16, N_, N_, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4), sg.SGEMM_OK),
    ((BF, N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, None, 4), sg.SGEMM_ERR_NULL),
    ((BF, N_, N_, 4, 4, 4, 1.0, None, 4, B, 4, 0.0, C, 4), sg.SGEMM_ERR_NULL),
    ((BF, N_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 2.0, C, 4), sg.SGEMM_OK),    # alpha = 0: A, B unread
    # Overlap on 2-byte elements: A (4 x 4 bf16) spans 32 bytes.
    ((BF, N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, A + 30, 4), sg.SGEMM_ERR_ALIAS),
    ((BF, N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, A + 32, 4), sg.SGEMM_OK),
]


@pytest.mark.parametrize("args,want", LP_CASES)
def test_lp_check_args(lib, args, want):
    assert sg.sgemm_lp_check_args(*args) == want


@pytest.mark.parametrize("args,want", [c for c in LP_CASES if c[1] != sg.SGEMM_OK])
def test_lp_rejects_before_touching_the_gpu(lib, args, want):
    assert sg.sgemm_lp(*args, None) == want


def test_lp_no_device_is_reported_not_crashed(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert sg.sgemm_lp(BF, N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, None) == sg.SGEMM_ERR_DEVICE
    assert sg.sgemm_lp(F16, N_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, C, 4, None) == sg.SGEMM_OK


WS = 0x7000_0000   # a fake workspace address, far from A, B and C

WS_CASES = [
    # (transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, bytes, variant) -> status
    # sgemm_ex's checks come first, in its order.
    ((2, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, WS, 64, 0), sg.SGEMM_ERR_OP),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, A, 64, 9), sg.SGEMM_ERR_VARIANT),
    ((N_, N_, 4, 4, 4, 1.0, None, 4, B, 4, 0.0, C, 4, WS, 64, 0), sg.SGEMM_ERR_NULL),
    # Then the workspace, when it is non-empty: it must not overlap C, or A and
    # B when they are read.
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, WS, 64, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, None, 0, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, A, 0, 0), sg.SGEMM_OK),       # empty: never used
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, C + 4 * 15, 4, 0), sg.SGEMM_ERR_ALIAS),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, C + 4 * 16, 4, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, C - 4, 4, 0), sg.SGEMM_OK),    # ends where C starts
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, C - 4, 5, 0), sg.SGEMM_ERR_ALIAS),
    ((T_, N_, 2, 4, 8, 1.0, A, 2, B, 4, 0.0, C, 4, A + 4 * 15, 4, 0), sg.SGEMM_ERR_ALIAS),   # A^T: 16 floats
    ((T_, N_, 2, 4, 8, 1.0, A, 2, B, 4, 0.0, C, 4, A + 4 * 16, 4, 0), sg.SGEMM_OK),
    ((N_, N_, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, B + 8, 4, 0), sg.SGEMM_ERR_ALIAS),
    ((N_, N_, 4, 4, 4, 0.0, A, 4, B, 4, 2.0, C, 4, B + 8, 4, 0), sg.SGEMM_OK),    # alpha 0: B not read
    ((N_, N_, 0, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, C, 64, 0), sg.SGEMM_OK),       # empty C: nothing checked
]


@pytest.mark.parametrize("args,want", WS_CASES)
def test_ws_check_args(lib, args, want):
    assert sg.sgemm_ex_ws_check_args(*args) == want


@pytest.mark.parametrize("args,want", [c for c in WS_CASES if c[1] != sg.SGEMM_OK])
def test_ws_rejects_before_touching_the_gpu(lib, args, want):
    *head, ws, nbytes, variant = args
    assert sg.sgemm_ex_ws(*head, ws, nbytes, None, variant) == want


def test_ws_nothing_to_do_returns_ok_without_gpu(lib):
    assert sg.sgemm_ex_ws(N_, N_, 0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5, WS, 64, None, 3) == sg.SGEMM_OK
    assert sg.sgemm_ex_ws(T_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, C, 4, WS, 64, None, 3) == sg.SGEMM_OK


def test_split_workspace_size(lib):
    # Uneven tile loads take the split schedule: two partial tiles per
    # work-group, one 256x256 work-group per compute unit or two 128x128.
    big, mid = 2 * 256 * 256 * 256 * 4, 2 * 512 * 128 * 128 * 4
    assert sg.sgemm_ex_workspace_size(N_, N_, 2047, 2560, 4093, 256) == big
    assert sg.sgemm_ex_workspace_size(T_, T_, 3072, 3072, 3072, 0) == big
    # 3001 x 2047 fits 16 x 16 tiles of 192 x 128, one per compute unit, and
    # 2047 x 3001 as many of 128 x 192: whole tiles.
    assert sg.sgemm_ex_workspace_size(N_, N_, 3001, 2047, 4093, 256) == 0
    assert sg.sgemm_ex_workspace_size(N_, N_, 2047, 3001, 4093, 256) == 0
    assert sg.sgemm_ex_workspace_size(T_, T_, 3072, 2048, 4096, 0) == 0
    assert sg.sgemm_ex_workspace_size(N_, T_, 512, 512, 16384, 256) == mid
    for cus in (64, 128, 304):   # sized for the device's compute units when used
        assert sg.sgemm_ex_workspace_size(N_, N_, 3001, 2047, 4093, cus) in (0, 2 * cus * 256 * 256 * 4,
                                                                              2 * 2 * cus * 128 * 128 * 4)
    # Products that whole tiles already spread evenly keep them.
    for shape in [(4096, 4096, 4096), (8192, 8192, 8192), (2048, 2048, 2048), (1024, 1024, 1024), (128, 128, 128)]:
        assert sg.sgemm_ex_workspace_size(N_, N_, *shape, 256) == 0, shape
    # Invalid or empty products, and operands too narrow for the fast tiles.
    assert sg.sgemm_ex_workspace_size(2, N_, 3001, 2047, 4093, 256) == 0
    assert sg.sgemm_ex_workspace_size(N_, N_, -1, 2047, 4093, 256) == 0
    assert sg.sgemm_ex_workspace_size(N_, N_, 3001, 2047, 0, 256) == 0
    assert sg.sgemm_ex_workspace_size(N_, N_, 4096, 3, 1 << 20, 256) == 0
    assert sg.sgemm_ex_workspace_size(T_, T_, 3, 4096, 1 << 20, 256) == 0


@pytest.mark.parametrize("args,want", EX_CASES)
def test_noalloc_checks_are_the_general_checks(lib, args, want):
    # sgemm_ex_noalloc checks what sgemm_ex checks, in the same order.
    assert sg.sgemm_ex_noalloc_check_args(*args, 256) == want


@pytest.mark.parametrize("args,want", [c for c in EX_CASES if c[1] != sg.SGEMM_OK])
def test_noalloc_rejects_before_touching_the_gpu(lib, args, want):
    assert sg.sgemm_ex_noalloc(*args[:13], None, args[13]) == want


def test_noalloc_scratch_limit(lib):
    # The static buffer holds the largest split workspace on 256 compute units;
    # a device with more would need more for some products, which is a clear
    # error, and only where the matrix-core variant would split.
    limit = sg.sgemm_ex_noalloc_scratch_bytes()
    assert limit == 128 << 20 == sg.sgemm_ex_workspace_size(N_, N_, 2047, 2560, 4093, 256)
    ragged = (N_, N_, 2047, 2560, 16384, 1.0, A, 16384, B, 2560, 0.0, C, 2560)
    for cus in (0, 64, 128, 256):
        assert sg.sgemm_ex_noalloc_check_args(*ragged, sg.SGEMM_MFMA, cus) == sg.SGEMM_OK
    for cus in (512, 1024):
        assert sg.sgemm_ex_workspace_size(N_, N_, 2047, 2560, 16384, cus) > limit
        assert sg.sgemm_ex_noalloc_check_args(*ragged, sg.SGEMM_MFMA, cus) == sg.SGEMM_ERR_SCRATCH
        assert sg.sgemm_ex_noalloc_check_args(*ragged, sg.SGEMM_BEST, cus) == sg.SGEMM_ERR_SCRATCH
        for v in (sg.SGEMM_NAIVE, sg.SGEMM_TILED, sg.SGEMM_REGBLOCK):   # never split
            assert sg.sgemm_ex_noalloc_check_args(*ragged, v, cus) == sg.SGEMM_OK
        # Nothing to multiply: nothing to split.
        assert sg.sgemm_ex_noalloc_check_args(*ragged[:5], 0.0, *ragged[6:], sg.SGEMM_MFMA, cus) == sg.SGEMM_OK
    assert "scratch" in sg.sgemm_status_string(sg.SGEMM_ERR_SCRATCH)


def test_noalloc_nothing_to_do_returns_ok_without_gpu(lib):
    assert sg.sgemm_ex_noalloc(N_, N_, 0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5, None, 3) == sg.SGEMM_OK
    assert sg.sgemm_ex_noalloc(T_, N_, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, C, 4, None, 3) == sg.SGEMM_OK
