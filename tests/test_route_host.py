"""Kernel selection, checked on the host (no GPU): the tiled kernels address
a tile's rows with 32-bit byte offsets, so aligned calls whose offsets could
reach 2^32 bytes must take the generic kernel (64-bit row addresses)."""
import ctypes

import pytest

import norm_gemm_amd as ng

DECODE_ELEM, DECODE_WIDE, DECODE_LDS, PREFILL_LDS, PREFILL_GENERIC = range(5)


@pytest.fixture(scope="module")
def L():
    lib = ctypes.CDLL(ng.LIBRARY_PATH)
    i64, ci = ctypes.c_int64, ctypes.c_int
    lib.ng_tile_offsets_fit.argtypes = [i64, i64]
    lib.ng_tile_offsets_fit.restype = ci
    lib.ng_route_gemm.argtypes = [i64, i64, i64, ci, ci]
    lib.ng_route_gemm.restype = ci
    lib.ng_decode_wide_row_blocks.argtypes = [i64, ci]
    lib.ng_decode_wide_row_blocks.restype = ci
    lib.ng_gated_tiled_fits.argtypes = [i64, i64, i64, ci]
    lib.ng_gated_tiled_fits.restype = ci
    lib.ng_wide_tiles_fit.argtypes = [i64, i64, i64, ci]
    lib.ng_wide_tiles_fit.restype = ci
    lib.ng_wide_tiles_pay.argtypes = [i64, i64, ci]
    lib.ng_wide_tiles_pay.restype = ci
    return lib


def last_offset(rows, K):
    """Largest byte offset a lane forms inside a tile: the last row's last
    16-byte chunk, relative to the tile's first row."""
    return ((rows - 1) * K + ((K + 7) // 8) * 8) * 2


@pytest.mark.parametrize("K", [8, 64, 14336, 8388600, 8388608, 8421504, 8421512, 2 ** 31 - 1])
def test_tile_offsets_fit_matches_32_bit_range(L, K):
    assert L.ng_tile_offsets_fit(256, K) == (last_offset(256, K) <= 2 ** 32 - 1)


def test_largest_aligned_k_of_the_tiled_kernel(L):
    # 256 rows of K elements: 512 K bytes must stay below 2^32
    assert L.ng_tile_offsets_fit(256, 8388600) == 1
    assert L.ng_tile_offsets_fit(256, 8388608) == 0
    # the K at which the previous unchecked offsets wrapped is now refused
    assert L.ng_tile_offsets_fit(256, 8421512) == 0


@pytest.mark.parametrize("M,N,K,vec,route", [
    (1024, 8192, 8192, 1, PREFILL_LDS),
    (512, 49152, 14336, 1, PREFILL_LDS),
    (513, 49152, 14337, 0, PREFILL_GENERIC),       # K % 8 != 0
    (64, 256, 8388600, 1, PREFILL_LDS),
    (64, 256, 8388608, 1, PREFILL_GENERIC),        # offsets would pass 2^32
    (33, 16, 2 ** 31 - 8, 1, PREFILL_GENERIC),
    (1, 28672, 8192, 1, DECODE_WIDE),
    (8, 28672, 8192, 1, DECODE_WIDE),
    (16, 28672, 8192, 1, DECODE_WIDE),
    (17, 28672, 8192, 1, DECODE_LDS),
    (32, 28672, 8192, 1, DECODE_LDS),
    (16, 8, 8192, 1, DECODE_LDS),                  # fewer rows than one wide slab
    (16, 28672, 9586976, 1, DECODE_WIDE),          # 112-row slab: 2^31 - 6 KB
    (16, 28672, 9586984, 1, DECODE_LDS),           # slab offsets past 2^31
    (32, 28672, 8191, 0, DECODE_ELEM),
])
def test_route(L, M, N, K, vec, route):
    assert L.ng_route_gemm(M, N, K, vec, 256) == route


def test_decode_wide_row_blocks(L):
    assert L.ng_decode_wide_row_blocks(28672, 256) == 7      # 1792 blocks over 256 CUs
    assert L.ng_decode_wide_row_blocks(8, 256) == 0
    assert L.ng_decode_wide_row_blocks(100000, 256) == 8      # capped
    assert L.ng_decode_wide_row_blocks(28672, 0) == 7         # unknown CU count: 256


def test_gated_tiled_fits(L):
    assert L.ng_gated_tiled_fits(512, 28672, 8192, 1) == 1
    assert L.ng_gated_tiled_fits(32, 28672, 8192, 1) == 0      # decode range
    assert L.ng_gated_tiled_fits(512, 28672, 8192, 0) == 0     # unaligned
    assert L.ng_gated_tiled_fits(512, 2 ** 20, 8192, 1) == 0   # W rows past 2^32 bytes


def test_wide_tiles_fit(L):
    assert L.ng_wide_tiles_fit(512, 49152, 14336, 1) == 1
    assert L.ng_wide_tiles_fit(512, 49152, 14337, 1) == 0      # K not whole 64-element steps
    assert L.ng_wide_tiles_fit(512, 49152, 14336, 0) == 0      # unaligned
    assert L.ng_wide_tiles_fit(32, 49152, 14336, 1) == 0       # decode range
    assert L.ng_wide_tiles_fit(512, 49152, 8388608, 1) == 0    # tile offsets past 2^32


def wide_pays(M, N, cus):
    """Rounds of tiles times the rows moved per K step (256 + 192 against
    128 + 256), the wide tiles saving at least 10 %."""
    tw = -(-M // 256) * -(-N // 192)
    tn = -(-M // 128) * -(-N // 256)
    return -(-tw // cus) * 448 * 10 < -(-tn // cus) * 384 * 9


@pytest.mark.parametrize("M,N,cus,want", [
    (512, 49152, 256, 1),     # 512 wide tiles (2 rounds) against 768 (3 rounds)
    (1024, 8192, 256, 0),     # 172 against 256 tiles: one round each
    (512, 14336, 256, 0),     # 150 against 224: one round each
    (512, 8192, 256, 0),
    (129, 32776, 256, 1), (300, 21768, 256, 1), (400, 16392, 256, 1),
    (512, 49152, 304, 1), (512, 49152, 0, 1)])
def test_wide_tiles_pay(L, M, N, cus, want):
    assert L.ng_wide_tiles_pay(M, N, cus) == want
    assert wide_pays(M, N, cus if cus > 0 else 256) == bool(want)
