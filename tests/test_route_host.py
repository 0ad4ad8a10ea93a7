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
    lib.ng_skip_slice_plan.argtypes = [i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
    lib.ng_skip_slice_plan.restype = ci
    lib.ng_gated_split_tiles.argtypes = [i64, i64, i64, ci]
    lib.ng_gated_split_tiles.restype = ci
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


def skip_plan(L, M, N, K, cus):
    t, ln = ctypes.c_int(0), ctypes.c_int(0)
    ok = L.ng_skip_slice_plan(M, N, K, cus, ctypes.byref(t), ctypes.byref(ln))
    return (t.value, ln.value) if ok else None


def skip_slice_segments(M, N, K, tails, ln):
    """The segments of every workgroup of the skipped-slice split K, as the
    tiled kernel derives them from its workgroup index: (workgroup, row block,
    column block, plane, list of K steps). Workgroups are dealt to the 8 XCDs
    round-robin; the j-th of XCD xc with j < T / 8 owns local tile j and skips
    the len steps of slot j // tails; the others run the skipped slices of
    local tiles i tails + (j - T / 8), slot i after slot i."""
    tm, tn, nkt = -(-M // 128), -(-N // 256), -(-K // 64)
    T = tm * tn
    tx = T // 8
    segs = []
    for b in range(T + 8 * tails):
        xc, j = b % 8, b // 8
        units = [j] if j < tx else [i * tails + j - tx for i in range(tx // tails)]
        for sg, u in enumerate(units):
            mb, nt = u % tm, xc * (tn // 8) + u // tm
            if j < tx:
                gap_at = (u // tails) * ln
                nk = nkt - ln
                steps = [kt + ln if kt >= gap_at else kt for kt in range(nk)]
                segs.append((b, mb, nt, 0, steps))
            else:
                segs.append((b, mb, nt, 1, list(range(sg * ln, sg * ln + ln))))
    return segs


@pytest.mark.parametrize("M,N,K,cus,want", [
    (512, 14336, 49152, 256, (4, 88)),     # FFN second GEMM: 224 tiles, 768 K steps
    (512, 14336, 14336, 256, (4, 25)),
    (512, 12288, 49152, 256, (8, 178)),    # 192 tiles: 24 per XCD, 8 spare CUs each, 3 slots
    (300, 12288, 1792, 256, (9, 8)),       # 144 tiles (ragged rows): 18 per XCD, 9 of 14 spare CUs used
    (512, 14336, 4096, 256, None),         # 64 K steps: slices under 8 steps
    (512, 8192, 49152, 256, None),         # 128 tiles: half of the CUs, two equal ranges instead
    (1024, 8192, 8192, 256, None),         # 256 tiles fill the CUs
    (512, 13824, 49152, 256, None),        # 54 column blocks, not a multiple of 8
    (512, 14336, 49152, 240, (2, 46)),     # 224 tiles on 240 CUs: 2 spare per XCD, 14 slots
    (512, 14336, 49152, 0, None),
])
def test_skip_slice_plan(L, M, N, K, cus, want):
    assert skip_plan(L, M, N, K, cus) == want


@pytest.mark.parametrize("M,N,K,cus", [
    (512, 14336, 49152, 256), (512, 14336, 14336, 256), (512, 12288, 49152, 256),
    (300, 12288, 1792, 256), (300, 12288, 1800, 256), (129, 18432, 3000, 256),
    (640, 8192, 5000, 256), (512, 14336, 49152, 240), (200, 20480, 20000, 304),
])
def test_skip_slice_segments_cover_every_step_once(L, M, N, K, cus):
    """Every (tile, K step) is computed by exactly one segment; every tile has
    one part in plane 0 and one in plane 1 (the two planes the sum kernel
    adds); every step index is inside K and only the main parts hold the
    last (possibly ragged) step; the grid fits the CUs."""
    plan = skip_plan(L, M, N, K, cus)
    assert plan is not None, (M, N, K, cus)
    tails, ln = plan
    tm, tn, nkt = -(-M // 128), -(-N // 256), -(-K // 64)
    T = tm * tn
    assert cus // 2 < T < cus and tn % 8 == 0 and (T // 8) % tails == 0
    assert T + 8 * tails <= cus
    assert (T // 8 // tails + 1) * ln <= nkt          # the launcher's check
    cover = {}
    planes = {}
    for b, mb, nt, plane, steps in skip_slice_segments(M, N, K, tails, ln):
        assert 0 <= mb < tm and 0 <= nt < tn
        assert len(steps) >= 1 and all(0 <= k < nkt for k in steps)
        assert len(set(steps)) == len(steps)
        if plane == 1:
            assert nkt - 1 not in steps and steps == list(range(steps[0], steps[0] + ln))
        for k in steps:
            cover[(mb, nt, k)] = cover.get((mb, nt, k), 0) + 1
        planes.setdefault((mb, nt), []).append(plane)
    assert len(cover) == T * nkt and set(cover.values()) == {1}
    assert len(planes) == T and all(sorted(p) == [0, 1] for p in planes.values())


def test_skip_slice_spare_workgroups_run_the_slot_being_skipped(L):
    """At slot i the spare workgroups of an XCD compute exactly the slices
    that the XCD's tiles of slot i skip, and those are the same K steps for
    every tile of the slot (so the spare and the skipping workgroups read the
    same steps of x at about the same time)."""
    M, N, K = 512, 14336, 49152
    tails, ln = skip_plan(L, M, N, K, 256)
    segs = skip_slice_segments(M, N, K, tails, ln)
    tx = 224 // 8
    for xc in range(8):
        spare = [s for s in segs if s[0] % 8 == xc and s[0] // 8 >= tx]
        main = [s for s in segs if s[0] % 8 == xc and s[0] // 8 < tx]
        for i in range(tx // tails):
            at_slot = {(s[1], s[2]) for s in spare if s[4][0] == i * ln}
            skipping = {(s[1], s[2]) for s in main if (s[0] // 8) // tails == i}
            assert at_slot == skipping and len(at_slot) == tails
            # the tiles of a slot share their W column block (tails = row blocks)
            assert len({nt for _, nt in at_slot}) == 1


@pytest.mark.parametrize("M,F,K,cus,want", [
    (512, 28672, 8192, 256, 128),   # SwiGLU 512 x 28672: 896 tiles, last round 128 of 256
    (512, 9216, 320, 256, 32),      # 288 tiles
    (300, 11500, 264, 256, 14),     # 3 row blocks x 90 column blocks = 270 tiles
    (512, 12288, 8192, 256, 128),   # 384 tiles: the last round exactly half of the CUs
    (512, 14336, 8192, 256, 0),     # 448 tiles: last round 192 > 128
    (512, 16384, 8192, 256, 0),     # 512 tiles: two whole rounds
    (512, 8192, 8192, 256, 0),      # 256 tiles: one round
    (512, 28672, 192, 256, 0),      # 3 K steps: halves under 2 steps
    (512, 28672, 8192, 0, 0),
])
def test_gated_split_tiles(L, M, F, K, cus, want):
    assert L.ng_gated_split_tiles(M, F, K, cus) == want


def test_gated_split_covers_every_tile_and_step_once(L):
    """The gated kernel's workgroups (T - S whole tiles, then the two K halves
    of each of the last S tiles) compute every K step of every tile exactly
    once, each half at least two steps, and fit one round of the CUs."""
    for M, F, K, cus in [(512, 28672, 8192, 256), (512, 9216, 320, 256), (300, 11500, 264, 256),
                         (129, 20000, 1000, 240)]:
        T = -(-M // 128) * -(-F // 128)
        S = L.ng_gated_split_tiles(M, F, K, cus)
        nkt = -(-K // 64)
        if S == 0:
            continue
        assert 2 * S <= cus and S <= T - cus
        first = T - S
        cover = {}
        for b in range(T + S):
            if b < first:
                tile, steps = b, range(nkt)
            else:
                hw = b - first
                k1 = (nkt + 1) // 2
                tile = first + hw // 2
                steps = range(k1, nkt) if hw & 1 else range(0, k1)
                assert len(steps) >= 2
            for k in steps:
                cover[(tile, k)] = cover.get((tile, k), 0) + 1
        assert len(cover) == T * nkt and set(cover.values()) == {1}
