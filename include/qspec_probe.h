/*
 * qspec_probe.h -- ceiling probes of libqspec.so: the rates this GPU sustains
 * for the resources the hot path is bound by, measured with the instruction
 * kinds its kernels use.  A measured fraction of the hot path's kernels is
 * quoted against these next to the published peaks (HBM 8 TB/s; dense int8
 * MFMA 5.0 POPS, bf16 2.5 PFLOPS).  Nothing here is on the hot path.
 *
 * Conventions are those of qspec.h (device pointers owned by the caller,
 * asynchronous on `stream`, host-side validation, nothing allocated).
 */
#ifndef QSPEC_PROBE_H_
#define QSPEC_PROBE_H_

#include "qspec.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every 16-byte unit of buf[0, bytes) once with non-temporal 16-byte
 * loads: `blocks` workgroups of 256 threads stride over the buffer, each
 * thread with `unroll` (1, 2, 4, 8 or 16) loads in flight.  bytes: a
 * positive multiple of 16; buf 16-byte aligned; sink: 256 uint32 of scratch
 * that is written only if the XOR of the data equals a fixed value (it keeps
 * the loads live).  Bytes moved = `bytes`. */
qspec_status qspec_probe_read(const void* buf, int64_t bytes, int blocks, int unroll,
                              uint32_t* sink, qspec_stream stream);

/* `blocks` workgroups of 4 wavefronts, each wavefront running `iters` rounds
 * of 8 independent MFMA accumulators: kind 0 = v_mfma_i32_16x16x64_i8
 * (32768 int8 operations each), kind 1 = v_mfma_f32_16x16x32_bf16 (16384
 * flops each).  Operations per launch = blocks * 4 * iters * 8 * that.
 * sink: 256 floats, written only on an impossible result. */
qspec_status qspec_probe_mfma(int kind, int blocks, int iters, float* sink, qspec_stream stream);

/* One launch of an empty kernel (one wavefront): the cost of a launch. */
qspec_status qspec_probe_empty(qspec_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QSPEC_PROBE_H_ */
