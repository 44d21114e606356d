/*
 * mgqa_timeline.h - extra C ABI of libmgqa_timeline.so, the attention library
 * built with per-wave timestamps (MGQA_TIMELINE defined).
 *
 * libmgqa_timeline.so exports every entry point of mgqa.h with the same
 * behaviour and the same output bits (the marks move no arithmetic), plus the
 * three calls below.  It is a measurement build: it shows where the time of
 * one launch goes (start-up, first tiles, key loop, merges, per XCD) for the
 * kernels of the library.  The library proper (libmgqa.so) has none of it.
 *
 * Each wave of an attention kernel fills one record of MGQA_TIMELINE_EVENTS
 * + 1 64-bit words in a device array of MGQA_TIMELINE_MAX_WAVES records:
 *   word 0      1 | XCD index << 4 | HW_ID register << 32 (0: no record);
 *   word 1 + e  the 100 MHz real-time counter when the wave passed event e,
 *               0 if it did not.
 * The record of wave w of workgroup g is g * (waves per workgroup) + w; waves
 * past the array's end record nothing.  Every launch rewrites the whole
 * record of each of its waves; the records of other slots keep their
 * contents, so clear before a launch whose grid may be smaller than the last.
 *
 * Events (all kernels: 0 = wave start, 7 = wave end after its last store):
 *   split-KV kernel (decode, short and mid-length sequences):
 *     1 Q and first tile requested, 2 first tile in LDS, 3 key loop done,
 *     4 wave states merged and written (output, or this split's partial),
 *     5 partial stores complete, 6 arrival counted; 7 only on the last
 *     arrival of a row block: all splits merged and written;
 *   short-band kernel (encoder): 1 K and V requested, 2 score products
 *     issued, 3 probabilities done, 4 P.V products issued, 5 wave states in
 *     LDS, 6 merge weights ready;
 *   pipelined head-size-128 prefill: 1 first block's first tiles in LDS,
 *     2 its key loop done, 3 its rows written; 4, 5, 6 the same for a
 *     second block (paired work items only);
 *   other prefill: 1 first tile in LDS, 2 key loop done.
 *
 * Marks are taken between scheduling barriers when the wave's instruction
 * stream reaches them: an event after matrix products marks their issue,
 * not their completion.  Calls overlapping on one GPU write the same array.
 */
#ifndef MGQA_TIMELINE_H
#define MGQA_TIMELINE_H

#include <stddef.h>

#define MGQA_TIMELINE_EVENTS    8
#define MGQA_TIMELINE_MAX_WAVES (1 << 16)

#ifdef __cplusplus
extern "C" {
#endif

/* Records and events per record: *max_waves = MGQA_TIMELINE_MAX_WAVES,
 * *events = MGQA_TIMELINE_EVENTS.  MGQA_ERR_NULL if a pointer is NULL. */
int attn_timeline_layout(int* events, int* max_waves);

/* Queue a fill that zeroes every record of the current device on `stream`
 * (hipStream_t as void*).  MGQA_ERR_HIP if the array or the launch fails. */
int attn_timeline_clear(void* stream);

/* Wait for all work on the current device, then copy the first `words`
 * 64-bit words of its records to host memory `host` (caller-owned, at least
 * `words` * 8 bytes).  MGQA_ERR_NULL for a NULL `host`, MGQA_ERR_RANGE if
 * `words` exceeds the array, MGQA_ERR_HIP if a HIP call fails. */
int attn_timeline_read(unsigned long long* host, size_t words);

#ifdef __cplusplus
}
#endif

#endif /* MGQA_TIMELINE_H */
