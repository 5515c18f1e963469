/*
 * tq4_probe.h -- streaming-read bandwidth probe for AMD Instinct MI355X
 * (gfx950), built as its own library (libtq4probe.so) beside libtq4.so.
 *
 * It is measurement support, not part of the attention path: a benchmark
 * times it to report the read rate a plain grid-stride read kernel reaches on
 * this device, beside the vendor's 8 TB/s figure.  It is a reference point,
 * not a ceiling: a kernel with more loads in flight per wavefront (the decode
 * loop) streams faster.
 */
#ifndef TQ4_PROBE_H
#define TQ4_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words (uint32) the sink of tq4_probe_stream_read must hold for a launch of
 * `workgroups` workgroups (one word per thread); 0 for workgroups outside
 * [1, 65535]. */
size_t tq4_probe_sink_words(int32_t workgroups);

/*
 * tq4_probe_stream_read -- read `bytes` bytes of device memory at `src` once
 * (16-byte loads, four in flight per thread, grid-stride), fold the words
 * with XOR so no load can be dropped, and write one word per thread to
 * `sink` (device, tq4_probe_sink_words(workgroups) words).  `src` must be
 * 16-byte aligned and `bytes` a multiple of 64.  Enqueued on `stream`
 * (hipStream_t, NULL = default); returns 0, or -1 for bad arguments (nothing
 * enqueued), or -2 if the launch failed.
 */
int tq4_probe_stream_read(const void *src, size_t bytes, void *sink, int32_t workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ4_PROBE_H */
