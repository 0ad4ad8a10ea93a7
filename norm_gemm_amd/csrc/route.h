/* route.h -- which kernel serves a request: pure host logic, no HIP calls,
 * so that every dispatch decision can be checked without a GPU. */
#ifndef NG_ROUTE_H
#define NG_ROUTE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NG_ROUTE_DECODE_ELEM = 0,   /* element-load skinny kernel: any alignment, M <= 32  */
    NG_ROUTE_DECODE_WIDE = 1,   /* 512-byte W pieces: aligned, M <= 16                 */
    NG_ROUTE_DECODE_LDS = 2,    /* 128-byte W lines: aligned, M <= 32                  */
    NG_ROUTE_PREFILL_LDS = 3,   /* tiled MFMA kernel with 32-bit tile offsets          */
    NG_ROUTE_PREFILL_GENERIC = 4 /* generic tiled kernel: element loads or 64-bit rows */
} ng_route_t;

/* Largest M served by the skinny (decode) kernels. */
#define NG_DECODE_MAX_M 32

/* Rows of W per tile of the tiled MFMA kernel (its largest operand tile). */
#define NG_TILE_ROWS 256

/* 1 when byte offsets within a tile of `rows` rows of a K-element row-major
 * operand (row r, 16-byte chunk c < K / 8) stay below 2^32: the tiled
 * kernels address every tile row from one base with 32-bit offsets. */
int ng_tile_offsets_fit(int64_t rows, int64_t K);

/* 16-row blocks of W per workgroup of the 512-byte-piece decode kernel on a
 * device with `cus` compute units (about one workgroup per CU, 1..8), or 0
 * when N has fewer rows than one such slab. */
int ng_decode_wide_row_blocks(int64_t N, int cus);

/* Kernel for y[M,N] = act(norm(x)[M,K] . W[N,K]^T + bias); vec = 1 when K % 8
 * == 0 and x, W, gamma, beta are 16-byte aligned. */
int ng_route_gemm(int64_t M, int64_t N, int64_t K, int vec, int cus);

/* 1 when the gated tiled kernel can serve W1 = [W_gate; W_up] of 2F rows:
 * aligned, M above the decode range, and its W row offsets (up to F + 255
 * rows past a tile's first gate row) within 32 bits. */
int ng_gated_tiled_fits(int64_t M, int64_t F, int64_t K, int vec);

/* 1 when the 256 x 192 tiled kernel can serve the request: aligned, M above
 * the decode range, K a whole number of 64-element steps, and its x and W
 * tile offsets (256 rows) within 32 bits. */
int ng_wide_tiles_fit(int64_t M, int64_t N, int64_t K, int vec);

/* 1 when 256 x 192 tiles move fewer bytes per CU than 128 x 256 tiles over
 * the whole call on `cus` compute units: rounds of tiles times the bytes of
 * one 64-element K step of one tile (56 KB against 48 KB). The K step of the
 * tiled kernels is bound by the L2 bytes a CU can have in flight. */
int ng_wide_tiles_pay(int64_t M, int64_t N, int cus);

/* Skipped-slice schedule of a plain GEMM (no normalization) whose 128 x 256
 * tiles fill more than half but not all of the CUs in one round: T tiles
 * with T / 8 on each of the 8 XCDs (tn % 8 == 0, cus % 8 == 0, cus / 2 < T <
 * cus). On each XCD, every tile keeps its own workgroup, which skips one
 * slice of `len` K steps (the slice of the tile's slot, see the kernel); the
 * XCD's `tails` spare workgroups compute the skipped slices, T / 8 / tails
 * slots one after another, so every tile ends with two fp32 partial sums.
 * tails is the largest divisor of T / 8 that the spare CUs hold, and len
 * balances the spare workgroups (slots x len steps, each taking about 1.1
 * times a main workgroup's step) against the others (K steps - len). Returns 1 and
 * sets *tails and *len when the schedule applies (len >= 8), else 0. */
int ng_skip_slice_plan(int64_t M, int64_t N, int64_t K, int cus, int *tails, int *len);

/* Tiles of the gated tiled kernel's last round whose K steps are split over
 * two workgroups: T = ceil(M / 128) ceil(F / 128) tiles on `cus` CUs take
 * more than one round, and when the last round holds at most cus / 2 tiles
 * each of them is computed as two halves of its K steps (at least 4 steps),
 * so that the last round takes half the time. Returns that tile count, or 0.
 * The partial sums take 262144 bytes per split tile (two fp32 planes of
 * 128 rows x 256 gate and up columns). */
int ng_gated_split_tiles(int64_t M, int64_t F, int64_t K, int cus);

#ifdef __cplusplus
}
#endif

#endif
