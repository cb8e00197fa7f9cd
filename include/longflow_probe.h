/*
 * longflow_probe.h -- measurement helper shipped in liblongflow.so.
 *
 * Not part of the decode step. lf_probe_stream_read reads a device buffer
 * once with the same loads the decode kernel uses for K and V (16-byte buffer
 * loads, non-temporal cache policy) and keeps an XOR of what it read, so a
 * benchmark can report the streaming-read bandwidth this GPU attains next to
 * the decode kernel's; the timing variants record when and where each
 * workgroup of a read or of a decode step ran (and, with
 * lf_probe_decode_phases, when each phase of its step ended);
 * lf_probe_hbm_attributes reports the device's own memory clock and bus
 * width.
 */
#ifndef LONGFLOW_PROBE_H
#define LONGFLOW_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "longflow.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` once: `workgroups` workgroups of 256 threads,
 * each over its own contiguous region of bytes / workgroups bytes.
 *   buf         device, 16-byte aligned; bytes a multiple of 16 * workgroups
 *   sink        device, workgroups * 256 * 16 bytes; receives the XORs
 *   stream      hipStream_t as void* (NULL = default stream); asynchronous
 * Errors: LF_ERR_INVALID_ARG on null pointers, misalignment, a size that is
 * not a multiple of 16 * workgroups, or a region of 2 GiB or more;
 * LF_ERR_HIP if the launch fails. */
lf_status lf_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, void* sink,
                               void* stream);

/* lf_probe_stream_read with a timing record per workgroup: four uint64
 * values, [start, end, XCC id | hardware id << 32, workgroup index]; start
 * and end are thread 0's, on the device's constant 100 MHz clock
 * (s_memrealtime); the XCC id names the accelerator complex die and the
 * hardware id register its shader engine, CU, SIMD and wave slot.
 *   records   device [workgroups][4] uint64
 * Other arguments and errors as lf_probe_stream_read (records NULL is
 * LF_ERR_INVALID_ARG). */
lf_status lf_probe_stream_read_timing(const void* buf, size_t bytes, int32_t workgroups, void* sink,
                                      uint64_t* records, void* stream);

/* One lf_decode_step (the same launch plan, kernels and results) that also
 * writes the timing record above for every workgroup of the launch.
 *   records      device [capacity][4] uint64
 *   workgroups   HOST out: the launch's workgroup count (pairs x splits;
 *                fewer when workgroups take whole pairs in turn; up to twice
 *                the compute units for a stream launch)
 * Errors: those of lf_decode_step, and LF_ERR_INVALID_ARG (nothing queued)
 * on NULL records or workgroups, or capacity below the workgroup count.
 * The records show how one launch spreads over the XCDs and CUs; they cost
 * the decode kernel one uniform branch when not requested. */
lf_status lf_probe_decode_timing(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot,
                                 uint64_t* records, int64_t capacity, int32_t* workgroups,
                                 void* stream);

/* lf_probe_decode_timing that also records when each phase of every
 * workgroup's step ended: thread 0's constant clock at the end of phases 1
 * to 8, eight uint64 values per workgroup (0 where the workgroup did not
 * reach the phase). A workgroup that takes several pairs in turn records its
 * last one.
 *   1  interleaved loop: the first tile processed; phased loop: the K
 *      stream done
 *   2  the K and V stream done
 *   3  split-K part: partial state (and raw logits) published, stores drained
 *   4  split-K part: its arrival ticket back
 *   5  last part of a pair: every part's max and sum in, the pair's formed
 *   6  last part of a pair: the score of every slot done
 *   7  the in-place write of the new token reached
 *   8  unused (0)
 *   records      device [capacity][4] uint64, as lf_probe_decode_timing
 *   phases       device [capacity][8] uint64
 * Caches of float32 leave the phase words 0 (their kernels record no
 * phases). Other arguments and errors as lf_probe_decode_timing (a NULL
 * phases is LF_ERR_INVALID_ARG). The stamps cost the decode kernel one
 * uniform branch each when not requested. */
lf_status lf_probe_decode_phases(lf_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, void* out, int32_t* evicted_slot,
                                 uint64_t* records, uint64_t* phases, int64_t capacity,
                                 int32_t* workgroups, void* stream);

/* The memory attributes the current device reports about itself
 * (hipDeviceAttributeMemoryClockRate in kHz, hipDeviceAttributeMemoryBusWidth
 * in bits), from which a benchmark derives an HBM peak: clock x bus width / 8
 * bytes per transfer per clock, times the transfers per clock of the memory.
 * Host-only query; nothing is launched. Errors: LF_ERR_INVALID_ARG on a NULL
 * pointer; LF_ERR_HIP if the runtime cannot report either attribute. */
lf_status lf_probe_hbm_attributes(int32_t* mem_clock_khz, int32_t* bus_width_bits);

/* The launch plan that lf_decode_step makes for a layer of the evicting
 * main path with no split (lf_cache_set_grid and lf_cache_set_stream,
 * longflow.h), from its inputs alone: host only, no device needed.
 *   pairs          pairs of the layer
 *   n_max          tokens of its longest pair
 *   cus            compute units; resident4: 4-wave workgroups resident
 *                  per compute unit; fits8: an 8-wave workgroup's LDS fits
 *   rows, stride   the layer's workspace rows for cut pairs, and partial
 *                  states per row
 *   forced_stream, forced_grid   the overrides (0: automatic)
 *   plan           HOST out int32[8]: workgroups (0: one per pair), whole
 *                  pairs taken in turn first (pairs [0, sk_first)), cut
 *                  pairs (sk_pairs), tiles per pair, tiles per workgroup
 *                  run, workgroups with a run, partial states per row,
 *                  and waves per workgroup (4 or 8)
 * Errors: LF_ERR_INVALID_ARG on a NULL plan or a count out of range. */
lf_status lf_probe_stream_plan(int64_t pairs, int32_t n_max, int32_t cus, int32_t resident4,
                               int32_t fits8, int32_t rows, int32_t stride, int32_t forced_stream,
                               int32_t forced_grid, int32_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* LONGFLOW_PROBE_H */
