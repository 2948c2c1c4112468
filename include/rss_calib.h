/*
 * rss_calib.h — bandwidth calibration kernels exported by librss (MI355X, gfx950).
 *
 * Not part of the decode path: a benchmark runs them beside the decode kernels
 * to measure what HBM actually delivers with the decode kernels' own access
 * pattern (16-byte non-temporal loads and stores, fully coalesced: grid-stride
 * streams, and one workgroup per tile as the decode kernels work), so that each
 * kernel's bandwidth can be quoted as a fraction of the achievable read, write
 * or copy rate, or of a traffic-only kernel of its own shape, as well as of the
 * data-sheet peak. The method's premise is
 * that HBM traffic, not arithmetic, bounds the decode (P1, "La fiche qu'on
 * réécrit à chaque token": the eager step reads and writes the whole state for
 * very little arithmetic).
 *
 * Conventions as in rss.h: device pointers owned by the caller, 16-byte
 * aligned; the call only enqueues work on `stream` (a hipStream_t, NULL = the
 * null stream) and returns an rss_status: RSS_E_INVALID for a null or
 * misaligned pointer, a size that is not a multiple of 16, or blocks < 0;
 * RSS_E_HIP if the launch fails. bytes = 0 launches nothing.
 */
#ifndef RSS_CALIB_H_
#define RSS_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#include "rss.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stream-read `bytes` from src (read only; nothing of it is written). sink: a
 * device float the kernel may write (it stores only for one specific sum the
 * inputs are not expected to produce, which keeps the loads from being
 * removed). blocks: workgroups of 256 threads in the grid (0 = 4096). */
int32_t rss_calib_read(const void* src, size_t bytes, float* sink, int32_t blocks, void* stream);

/* Copy `bytes` from src to dst (non-overlapping): reads and writes `bytes`
 * each. blocks as rss_calib_read. */
int32_t rss_calib_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream);

/* Stream-write `bytes` to dst (nothing is read): 16-byte vector i holds the
 * floats (i mod 2^24, 1, 2, 3). blocks as rss_calib_read. The write ceiling
 * bounds the write-heavy baselines (an eager verify that writes one state
 * snapshot per draft token). */
int32_t rss_calib_write(void* dst, size_t bytes, int32_t blocks, void* stream);

/* The decode kernels' shape of work without their arithmetic: one 256-thread
 * workgroup per tile reads a tile of `tile_bytes` (4096, 8192, 16384, 32768
 * or 65536) from src, all of its 16-byte loads issued at once, then writes
 * `write_bytes` (a multiple of 16, at most 4096; 0 = none) per tile to dst.
 * n_tiles tiles, src holding n_tiles * tile_bytes bytes and dst n_tiles *
 * write_bytes. Tile t's 16-byte vector i in dst holds (s, i, t mod 2^24, 1),
 * s = the sum, in fp32, of the floats thread i read (vectors i, i + 256, ...
 * of the tile, added vector by vector, then the four lanes in order). Reading
 * with writes of a decode's bytes per tile, it measures what HBM delivers for
 * a decode's mix of a large streaming read and small writes. write_bytes =
 * tile_bytes instead copies each tile to dst at t * tile_bytes (each thread
 * stores the vectors it read, non-temporal): a read-then-write-back of whole
 * state tiles, as the eager step and the folds do. dst may be NULL when
 * write_bytes = 0. order: 0 = the decode kernels' workgroup-to-tile order (each
 * XCD takes runs of consecutive tiles of up to 512 KiB, the eight XCDs side by
 * side), 1 = one contiguous range of tiles per XCD; which of the two HBM serves
 * faster depends on the traffic. RSS_E_INVALID also for n_tiles < 0, an
 * unsupported tile size or another order. */
int32_t rss_calib_tiles(const void* src, size_t tile_bytes, int32_t n_tiles, void* dst,
                        int32_t write_bytes, int32_t order, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RSS_CALIB_H_ */
