/*
 * tq4_probe.h -- streaming-read bandwidth probe for AMD Instinct MI355X
 * (gfx950), built as its own library (libtq4probe.so) beside libtq4.so.
 *
 * It is measurement support, not part of the attention path: a benchmark
 * times it to report the read rate a plain streaming-read kernel reaches on
 * this device, beside the vendor's 8 TB/s figure.
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
 * and fold the words with XOR, one word per thread into `sink` (device,
 * tq4_probe_sink_words(workgroups) words), so no load can be dropped.  The
 * buffer is read in contiguous blocks of 512 x loads_in_flight 16-byte words,
 * block i by workgroup i mod workgroups; each of a workgroup's 512 threads
 * issues loads_in_flight (4, 8 or 16) 16-byte loads per block before using
 * any.  `src` must be 16-byte aligned and `bytes` a multiple of 16.  Enqueued
 * on `stream` (hipStream_t, NULL = default); returns 0, or -1 for bad
 * arguments (nothing enqueued), or -2 if the launch failed.
 */
int tq4_probe_stream_read(const void *src, size_t bytes, void *sink, int32_t workgroups, int32_t loads_in_flight,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ4_PROBE_H */
