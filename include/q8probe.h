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

#ifdef __cplusplus
}
#endif

#endif /* Q8PROBE_H */
