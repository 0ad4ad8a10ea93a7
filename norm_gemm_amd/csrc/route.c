/* route.c -- kernel selection (pure host C, no HIP). */
#include "route.h"

int ng_tile_offsets_fit(int64_t rows, int64_t K)
{
    if (rows < 1 || K < 1 || K > ((int64_t)1 << 40))
        return 0;
    /* last byte a lane may address: row rows-1, chunk (K/8 rounded up) - 1 */
    const int64_t last = ((rows - 1) * K + ((K + 7) / 8) * 8) * 2;
    return last <= (int64_t)0xffffffffLL;
}

int ng_decode_wide_row_blocks(int64_t N, int cus)
{
    if (N < 1)
        return 0;
    if (cus < 1)
        cus = 256;
    const int64_t blocks = (N + 15) / 16;
    int64_t nbk = (blocks + cus - 1) / cus;
    nbk = nbk < 1 ? 1 : (nbk > 8 ? 8 : nbk);
    while (nbk > 1 && N < 16 * nbk)
        --nbk;
    return N >= 16 * nbk ? (int)nbk : 0;
}

int ng_route_gemm(int64_t M, int64_t N, int64_t K, int vec, int cus)
{
    if (M <= NG_DECODE_MAX_M) {
        if (!vec)
            return NG_ROUTE_DECODE_ELEM;
        const int nbk = ng_decode_wide_row_blocks(N, cus);
        /* the wide kernel addresses a slab of 16 nbk rows with 32-bit offsets;
         * the line kernel forms 64-bit row addresses */
        if (M <= 16 && nbk > 0 && ng_tile_offsets_fit(16 * (int64_t)nbk, K) &&
            (int64_t)nbk * 16 * K * 2 <= 0x7fffffffLL)
            return NG_ROUTE_DECODE_WIDE;
        return NG_ROUTE_DECODE_LDS;
    }
    if (vec && ng_tile_offsets_fit(NG_TILE_ROWS, K))
        return NG_ROUTE_PREFILL_LDS;
    return NG_ROUTE_PREFILL_GENERIC;
}

int ng_gated_tiled_fits(int64_t M, int64_t F, int64_t K, int vec)
{
    return vec && M > NG_DECODE_MAX_M && F >= 1 && ng_tile_offsets_fit(F + NG_TILE_ROWS, K);
}

int ng_wide_tiles_fit(int64_t M, int64_t N, int64_t K, int vec)
{
    return vec && M > NG_DECODE_MAX_M && N >= 1 && K >= 64 && K % 64 == 0 &&
           ng_tile_offsets_fit(NG_TILE_ROWS, K);
}

int ng_wide_tiles_pay(int64_t M, int64_t N, int cus)
{
    if (M < 1 || N < 1)
        return 0;
    if (cus < 1)
        cus = 256;
    const int64_t tw = ((M + 255) / 256) * ((N + 191) / 192);
    const int64_t tn = ((M + 127) / 128) * ((N + 255) / 256);
    const int64_t rw = (tw + cus - 1) / cus, rn = (tn + cus - 1) / cus;
    /* bytes per CU: rounds x (256 + 192) rows against rounds x (128 + 256)
     * rows of 64 elements per K step; the wide tile must save at least 10 % */
    return rw * 448 * 10 < rn * 384 * 9;
}

int ng_skip_slice_plan(int64_t M, int64_t N, int64_t K, int cus, int *tails, int *len)
{
    if (M < 1 || N < 1 || K < 1 || cus < 8 || cus % 8 != 0)
        return 0;
    const int64_t tm = (M + 127) / 128, tn = (N + 255) / 256, T = tm * tn;
    if (tn % 8 != 0 || 2 * T <= cus || T >= cus)
        return 0;
    const int64_t tx = T / 8, spare = cus / 8 - tx;
    int64_t e = spare < tx ? spare : tx;
    while (tx % e != 0)
        --e;
    const int64_t slots = tx / e, nkt = (K + 63) / 64;
    /* a spare workgroup's step takes about 1.1 times a main workgroup's
     * (its x steps are shared with fewer workgroups, and each slice starts
     * and drains its own pipeline): (nkt - l) = 1.1 slots l */
    const int64_t l = (100 * nkt) / (100 + 110 * slots);
    if (l < 8)
        return 0;
    if (tails)
        *tails = (int)e;
    if (len)
        *len = (int)l;
    return 1;
}

int ng_gated_split_tiles(int64_t M, int64_t F, int64_t K, int cus)
{
    if (M < 1 || F < 1 || K < 1 || cus < 2)
        return 0;
    const int64_t T = ((M + 127) / 128) * ((F + 127) / 128);
    if (T <= cus || (K + 63) / 64 < 4)
        return 0;
    const int64_t last = T % cus;
    return (last > 0 && 2 * last <= cus) ? (int)last : 0;
}
