/*
 * lora_measure.h - measurement aids, in a library of their own
 * (liblora_measure.so), apart from the multi-LoRA path of lora_mi355x.h.
 *
 * They give the practical HBM ceilings the path's kernels are measured
 * against: a device-to-device copy and an in-place update of one buffer, both
 * with the 16-byte vector accesses the path's kernels use.  Conventions and
 * status codes as in lora_mi355x.h: plain device pointers, one kernel enqueued
 * on the caller's stream, no allocation, no synchronisation; invalid arguments
 * return LORA_ERR_INVALID_ARGUMENT with nothing enqueued.
 */
#ifndef LORA_MEASURE_H
#define LORA_MEASURE_H

#include "lora_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * lora_stream_copy - copy `bytes` bytes from src to dst, giving the practical
 * HBM read+write ceiling next to the nominal 8 TB/s.  bytes must be a positive
 * multiple of 16, both pointers 16-byte aligned, the buffers not overlapping.
 */
lora_status_t lora_stream_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

/*
 * lora_stream_update - read every 16-byte piece of `buf`, change it and write
 * it back in place (the output access pattern of lora_expand), giving the
 * practical in-place update ceiling.  bytes must be a positive multiple of 16,
 * buf 16-byte aligned.  The buffer's contents are scrambled.
 */
lora_status_t lora_stream_update(void *buf, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MEASURE_H */
