/*
 * pa_probe.h - a measurement aid beside the attention library: the HBM read rate a
 * kernel that does nothing but read reaches on this device, reading 4 KiB tiles front
 * to back or in a given order.  4 KiB is the granule a paged K/V pool is read in (one
 * block of 16 tokens of one KV head at head size 128 and 2-byte elements is 4 KiB of
 * K and 4 KiB of V, placed where the block table says: [RK] "什么是 LLM 中的分页注意力
 * (Paged Attention)?它是如何工作的?", 分页注意力是如何工作的), so a shuffled tile
 * order reads memory the way decode over a shuffled pool does.  Not on the attention
 * path: it puts the attention kernels' bandwidth beside what the device delivers.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* bytes per tile, and the bytes of sink one call writes (one word per wave of its
 * 2048 four-wave workgroups) */
#define PA_READ_PROBE_TILE 4096
#define PA_READ_PROBE_SINK_BYTES ((size_t)2048 * 4 * 4)

/*
 * pa_read_probe - read n_tiles tiles of 4096 bytes of src once each, with one 16-byte
 * non-temporal load per thread and tile (eight tiles in flight per 256-thread
 * workgroup, 2048 workgroups), and store an XOR fold of every word read, one uint32
 * per wave, into sink so that no load can be left out.
 *   src        device, 16-byte aligned, src_bytes bytes, a multiple of 4096
 *   tiles      NULL: tiles 0 .. n_tiles-1 in order, n_tiles <= src_bytes / 4096;
 *              else device int32 [n_tiles], tile k of the read is tiles[k] (e.g. a
 *              random permutation).  An index outside [0, src_bytes / 4096) is
 *              skipped, never read (device contract: not checked on the host).
 *   sink       device, 4-byte aligned, sink_bytes >= PA_READ_PROBE_SINK_BYTES; its
 *              first PA_READ_PROBE_SINK_BYTES bytes are overwritten
 *   stream     hipStream_t, or NULL for the default stream
 * Asynchronous: one launch (none for n_tiles = 0).  Errors: PA_ERR_INVALID_ARG for a
 * NULL or misaligned pointer or a bad size; PA_ERR_HIP if the launch fails.
 */
pa_status pa_read_probe(const void* src, size_t src_bytes, const int32_t* tiles,
                        int64_t n_tiles, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
