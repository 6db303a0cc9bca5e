/*
 * q8probe.h -- measurement probes of the benchmark, built as their own library
 * (libq8probe.so) beside q8stream.  Not part of the computation.
 *
 * The benchmark quotes measured ceilings next to the published ones [Frigg
 * README, "The machine": a plain read probe and a copy probe are timed beside
 * the GEMV, and the ceilings use the measured figure, not the nominal one].
 * Error codes and conventions are those of q8stream.h (host-side validation
 * before any HIP call; Q8_ERR_DEVICE without a usable device).
 */
#ifndef Q8PROBE_H
#define Q8PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "q8stream.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes (a positive multiple of 16, at most 2^40) of the 16-byte
 * aligned device buffer `src` once, with the decode product's access pattern:
 * one workgroup of 256 threads per contiguous span of 256 * loads_per_thread *
 * 16 bytes, every thread issuing its loads_per_thread (4, 8, 12 or 16)
 * non-temporal 16-byte loads before using any.  The loaded words are folded
 * into a checksum that is written to sink[0] (a caller-owned 4-byte aligned
 * int32 word) only in a case that never arises for the benchmark's buffers, so
 * the loads cannot be removed and nothing else is written. */
q8_status q8_probe_read(const void* src, int64_t bytes, int loads_per_thread, uint32_t* sink,
                        hipStream_t stream);

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

/* int8 matrix-core probe: `workgroups` workgroups of four waves, each wave
 * running `iters` rounds of eight independent v_mfma_i32_32x32x32_i8 chains
 * (65,536 integer operations per instruction), so workgroups * 4 * iters * 8 *
 * 65,536 operations; the timed rate is the chip's sustained int8 matrix rate.
 * sink: one caller-owned int32 word, written only in a case the probe's
 * operands never produce.  1 <= workgroups <= 2^20, 1 <= iters <= 2^24. */
q8_status q8_probe_mfma_i8(int workgroups, int iters, int32_t* sink, hipStream_t stream);

/* Exact-fold probe: `workgroups` workgroups of four waves, each wave retiring
 * `iters` rounds of four Q8 x Q8 block-tiles with no memory traffic -- per
 * block-tile one v_mfma_i32_32x32x32_i8 (the exact int32 block sums of a
 * 32 x 32 output tile), one v_mfma_f32_32x32x16_f16 (the tile's scale outer
 * product) and the fp32 fold (16 exact int-to-float steps + 16 FMAs per lane),
 * issued as the prefill kernel issues them, on operands that switch like real
 * data [fak
 * MODEL-BASELINE-RESULTS, ACT 4, "How the GEMM was closed": the per-block
 * fold is what bounds the prefill product].  Counted as the int8 product's
 * workgroups * 4 * iters * 4 * 65,536 operations, the timed rate is the
 * ceiling of any prefill kernel that folds exact block sums one block at a
 * time.  sink and limits as q8_probe_mfma_i8. */
q8_status q8_probe_fold(int workgroups, int iters, int32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8PROBE_H */
