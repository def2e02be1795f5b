/*
 * msda_calib.h - measurement kernels that calibrate the gather ceilings of
 * the MSDA hot path on one MI355X (not part of the operator).
 *
 * The operator's cost is the delivery of 128-byte value rows at random
 * positions ("DEFA: Efficient Deformable Attention Acceleration...",
 * abstract: irregular data access); these calls measure how fast the chip
 * delivers that pattern from each level of the memory hierarchy, so that a
 * kernel's gathered bytes per second can be put against the matching
 * ceiling.  The caller times them (events on `stream`) and divides the bytes
 * moved by the time:
 *   gather kernels: blocks * 256 threads * iters * 16 bytes;
 *   stream kernel: `bytes`.
 *
 * All pointers are DEVICE pointers owned by the caller; nothing is allocated
 * or synchronised; work is enqueued on `stream` (a hipStream_t).  `sink` must
 * hold blocks * 256 * 16 bytes; it is written only in the (practically
 * impossible) case that the loads XOR to a fixed constant, which keeps the
 * compiler from dropping them.  Returns an msda_status (msda.h): NULL
 * pointer, bad size or mode (MSDA_ERR_DIM), or a failed launch.
 */
#ifndef MSDA_CALIB_H
#define MSDA_CALIB_H

#include <stdint.h>

#include "msda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Random 128-byte rows from the first `window_bytes` of `buf` (a power of
 * two, 128 .. 2^31), 8 loads in flight per lane, `iters` loads per lane (a
 * multiple of 8).  lanes_per_row 8: each group of 8 lanes reads a whole row
 * with one 16-byte load per lane; 4: each group of 4 lanes reads a row with
 * two loads per lane (chunks c and c + 4). */
int msda_calib_gather_global(const void* buf, uint64_t window_bytes, int lanes_per_row,
                             int blocks, int iters, void* sink, void* stream);

/* The rows of msda_calib_gather_global with 8 lanes per row, delivered into
 * LDS by the buffer load's LDS mode instead of into registers (window_bytes a
 * power of two, 128 .. 2^30), then read back from LDS, 16 bytes per lane:
 * the rate of the other path from the L1 to a kernel's lanes. */
int msda_calib_gather_global_lds(const void* buf, uint64_t window_bytes, int blocks, int iters,
                                 void* sink, void* stream);

/* 16-byte reads from a 64 KB LDS array (512 rows of 128 bytes plus one spare
 * row) filled from `fill` (at least 65664 bytes), each group of 8 lanes:
 * mode 0 one random row; mode 1 rows in x-adjacent pairs (the groups 2h and
 * 2h + 1 read rows R and R + 1); mode 2 one random 16-byte chunk for all 8
 * lanes (a broadcast); mode 3 half rows on the same banks (lanes 0-3 chunks
 * 0-3 of row R1, lanes 4-7 chunks 0-3 of row R2); mode 4 half rows on opposite
 * banks (lanes 4-7 read chunks 4-7 of R2); mode 5 the four corners of a
 * bilinear sample per 16 lanes (4 lanes per corner row, rows R, R + 1,
 * R + 14, R + 15), half rows swapped in odd rows; mode 6 the same unswapped;
 * mode 7 as mode 6 with rows R + 13, R + 14 for the second pair; mode 8
 * 8-byte reads of a table of 32-byte entries, 4 lanes per word (the slot reads
 * of a corner-per-lane layout). */
int msda_calib_gather_lds(const void* fill, int mode, int blocks, int iters, void* sink,
                          void* stream);

/* A coalesced read of `bytes` (a multiple of 16) of `buf`, grid-strided over
 * `blocks` workgroups of 256 threads, with non-temporal loads. */
int msda_calib_stream(const void* buf, uint64_t bytes, int blocks, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_CALIB_H */
