/*
 * q8probe.h -- measurement utility shipped beside q8stream: an HBM read probe.
 *
 * Not part of the computation.  The benchmark uses it to measure the device's
 * attainable read bandwidth, the ceiling that the weight-streaming products are
 * compared with [Frigg README, "The machine": the bench vram table quotes a
 * plain read probe and a copy probe beside the GEMV, and ceilings use the
 * measured figure, not the nominal one].
 */
#ifndef Q8PROBE_H
#define Q8PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "q8stream.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes (a positive multiple of 16) from the 16-byte aligned
 * device buffer `src` with 16-byte loads and write one 32-bit checksum per
 * workgroup into `sink` (at least q8_probe_sink_words() words, caller-owned),
 * so that the loads cannot be removed.  Same error conventions as q8stream. */
q8_status q8_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Number of 32-bit words q8_probe_read writes into `sink` on the current device
 * (0 if there is no usable device). */
int64_t q8_probe_sink_words(void);

/* Grid-barrier probe: `workgroups` single-wave workgroups (1 .. number of
 * compute units) pass `rounds` grid-wide barriers one after another, the way a
 * single-launch decode step would have to between two dependent products
 * [Frigg README, Findings 3 and 8: at batch 1 a decode step is bound by launch
 * gaps, not by the products].  Each workgroup publishes its barrier epoch with a
 * write-through store into 8 replicas of a flag array and polls the replica of
 * its XCD with coherent loads until every flag has reached the epoch; no cache
 * write-back or invalidate is involved.  `rounds` = 0 launches an empty kernel
 * (the per-launch cost under graph replay).
 *
 * `flags`: caller-owned device buffer of at least q8_probe_barrier_words()
 * 32-bit words, zero-filled before the first call with a given `workgroups`;
 * consecutive calls continue from the epochs the previous call left.  Every
 * spin is bounded: if a barrier is not complete after about 2^22 polls the
 * kernel sets the last word of `flags` to 1 and every workgroup leaves; the
 * caller reads that word after synchronizing (non-zero = the measurement is
 * void; zero-fill again before the next call).  Q8_ERR_SHAPE for workgroups or
 * rounds out of range. */
q8_status q8_probe_barrier(uint32_t* flags, int workgroups, int rounds, hipStream_t stream);

/* Words q8_probe_barrier needs in `flags`. */
int64_t q8_probe_barrier_words(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8PROBE_H */
