/*
 * Measurement aids exported by libpagedattn.so beside the public C ABI of
 * include/paged_attention.h, for the benchmark and the tests only: not part
 * of the attention path and not installed with the public header.  Status
 * codes and pa_last_error() are the public ones.
 */
#ifndef PAGED_ATTENTION_MEASURE_H
#define PAGED_ATTENTION_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attention.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_stream_read_probe -- a measurement aid, not part of the attention path:
 * reads `bytes` bytes at `src` once with the same 16-byte non-temporal loads
 * the decode kernels use.  Timed over a buffer far larger than the last-level
 * cache it gives the device's plain read rate, the ceiling the kernels' HBM
 * figures can be compared with.
 *
 * src        device memory, 16-byte aligned; bytes a multiple of 16.
 * run_bytes  0: each workgroup streams one contiguous slice of the buffer.
 *            Otherwise the buffer is read as runs of run_bytes bytes at
 *            scattered positions (a fixed permutation of the runs), each run
 *            by one wave -- with run_bytes the size of one cache tile, the
 *            access pattern of the paged decode.  A power of two >= 1024 such
 *            that bytes / run_bytes is a power of two.
 * sink       device memory of at least pa_stream_read_sink_bytes(bytes) bytes,
 *            16-byte aligned; written only if a lane's XOR of the words it
 *            read has every bit set (keeps the loads live; practically never).
 * Returns PA_OK, PA_ERR_INVALID_ARG, PA_ERR_ALIGNMENT or PA_ERR_LAUNCH.
 */
int pa_stream_read_probe(const void* src, size_t bytes, size_t run_bytes, void* sink,
                         size_t sink_bytes, pa_stream_t stream);
size_t pa_stream_read_sink_bytes(size_t bytes);

/*
 * pa_share_occupancy -- for the equal-share schedule of the decode call with
 * these dims: *table_wgs = workgroups per CU the planner assumes (from the
 * kernel's LDS), *device_wgs = what the runtime's occupancy calculator
 * reports for the compiled kernel on the current device (needs a device),
 * *piece_cost = the stream positions each (kv head, sequence) item takes
 * before its tiles in the call's shares.  Returns PA_OK, PA_ERR_INVALID_ARG
 * (dims without equal shares) or PA_ERR_DEVICE.
 */
int pa_share_occupancy(const pa_dims* dims, int32_t* table_wgs, int32_t* device_wgs,
                       int32_t* piece_cost);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_MEASURE_H */
