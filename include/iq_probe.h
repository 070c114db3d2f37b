/* iq_probe.h: a measurement helper shipped with libiq.so, not a step of the
 * method.  It streams a device buffer once, so that the decode kernels'
 * HBM rates can be set against a rate this GPU actually reaches for plain
 * reads (the nominal peak is not reachable by any kernel).
 *
 * Every pointer is device memory owned by the caller.  The call is enqueued
 * on `stream` and returns without host synchronization; status codes are
 * those of iq.h (IQ_OK, IQ_ERR_INVALID_ARG, IQ_ERR_MISALIGNED, IQ_ERR_HIP).
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the `bytes` bytes at `buf` once with 16-byte non-temporal loads
 * spread over every compute unit (grid-stride, 8 workgroups of 256 threads
 * per compute unit, each wave's load instruction covering 1 KiB of
 * consecutive bytes, one load in flight per lane).  The data are XOR-folded
 * and written to `sink` (one uint32) only if the fold equals a fixed
 * improbable value, which keeps the loads without adding write traffic.
 *   buf:   16-byte aligned (IQ_ERR_MISALIGNED otherwise), non-null
 *   bytes: > 0 and a multiple of 16 (IQ_ERR_INVALID_ARG otherwise)
 *   sink:  4 bytes, non-null (IQ_ERR_INVALID_ARG otherwise)
 * Launch failures return IQ_ERR_HIP. */
int iq_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
