/*
 * thd_cp_bench.h -- measurement entry points of libthdcp (MI355X, gfx950).
 *
 * Not part of the layout transform: these calls exist so that a benchmark can
 * sweep the swap's launch shape and set the swap beside the two pure memory
 * streams a row permutation is made of.  Conventions as in thd_cp.h (device
 * pointers, `stream` a hipStream_t passed as void*, stream-ordered, THD_OK or
 * a negative THD_ERR_* code).
 */
#ifndef THD_CP_BENCH_H
#define THD_CP_BENCH_H

#include "thd_cp.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * thd_route_launch_shape -- override the launch shape of later thd_swap calls
 * on `route` (only that route; other routes keep the built-in shape).  For
 * launch-shape sweeps: the results of thd_swap never depend on it.  Setting
 * it while another thread calls thd_swap on the same route is the caller's
 * race, as is rebuilding that route.  A 0 selects the built-in choice for a
 * field.  The built-in shapes, for rows moved in 16-byte units: rows of
 * whole 4 KiB pages (4, 8, 12 KiB, ...) as one 4 KiB slice per 256-thread
 * workgroup, XCD chunks of 256; other rows above 4 KiB in slices of 4-6 KiB
 * on 256 threads, chunks of 64; rows between 1 and 4 KiB that are not powers
 * of two as many whole rows as fit in 6 KiB per 256-thread workgroup, chunks
 * of 64; shorter rows, and 1 KiB and 2 KiB rows, in tiles of about 4 KiB of
 * whole rows (a multiple of 128 bytes where one fits) on 128 threads in
 * natural order.  Rows moved in narrower units: 8 KiB tiles on 256 threads,
 * chunks of 64.  Rows of one unit (1-16 B) whose typical run is shorter than
 * one such tile (4 KiB for 16-byte rows) take an LDS-staged kernel instead.
 * Every workgroup copies exactly one tile.
 *   tile_bytes      output bytes per workgroup tile, rounded up to whole rows;
 *                   with 16-byte units, a value below the row size cuts each
 *                   row into slices of about that size
 *   nontemporal     1: non-temporal loads and stores (built-in), 0: plain
 *   block_threads   128, 256, 512 or 1024; used by the 16-byte path only
 *   tile_order      tiles per XCD chunk: 1 = natural order (tile b to
 *                   workgroup b, so neighbouring tiles go to different
 *                   XCDs); G > 1 = XCD-chunked (tiles cut into chunks of G,
 *                   XCD x streams chunks x, x+8, ...; G >= tiles / 8
 *                   gives each XCD one contiguous eighth)
 * A non-zero tile_bytes or block_threads also sends one-unit rows down the
 * tiled path.  thd_route_launch_shape(route, 0, 1, 0, 0) restores the
 * built-in shape.  THD_ERR_ARG for a null route, a negative field,
 * nontemporal other than 0 or 1, or another block size.  Host only.
 */
int thd_route_launch_shape(thd_route* route, int64_t tile_bytes, int32_t nontemporal, int32_t block_threads,
                           int32_t tile_order);

/*
 * thd_read_stream / thd_write_stream -- the two streams any row permutation
 * is made of, measured on their own: the swap reads each input byte once and
 * writes each output byte once.  HBM carries reads and writes over the same
 * channels, so a stream that mixes them (a copy, a swap) cannot move bytes
 * faster than a pure read or a pure write stream; these two passes measure
 * the pure streams, in the shapes that streamed fastest on MI355X: 16-byte
 * accesses on 128-thread workgroups in XCD-chunked tile order; the read pass
 * non-temporal loads of 4 KiB tiles, the write pass stores of 2 KiB tiles
 * that write through L2 to memory.
 *
 * thd_read_stream reads `bytes` bytes of `in` and adds to *count (device
 * uint32, 4-byte aligned, cleared by the caller) the number of 16-byte words
 * of `in` equal to the 16 bytes at `key` (host).  Only workgroups that find
 * a match touch *count, so with rare matches nothing but reads reach HBM.
 *
 * thd_write_stream writes `bytes` bytes of `out`: 16-byte word w holds four
 * copies of the 32-bit value (uint32)w ^ seed; nothing is read.
 *
 * `bytes` must be a non-negative multiple of 16 and `in` / `out` 16-byte
 * aligned (THD_ERR_ARG otherwise, or for a null pointer with bytes > 0);
 * `count` must not lie inside `in` (THD_ERR_ALIAS).  0 bytes is THD_OK with
 * no launch.  Stream-ordered, one launch each.
 */
int thd_read_stream(const void* in, int64_t bytes, const void* key, uint32_t* count, void* stream);
int thd_write_stream(void* out, int64_t bytes, uint32_t seed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* THD_CP_BENCH_H */
