/*
 * mnb_probe.h -- C ABI of libmnb_probe, a measurement aid that is not part of
 * the matmul library: the control arm of the benchmark's bandwidth figures.
 *
 * The page "Qwen3 CPU Inference Critical Path" ("INT4 MatMul is first", the
 * kernel-corpus paragraph) asks for effective memory bandwidth next to the
 * weight bytes read; the fraction of the datasheet peak is read against what a
 * plain streaming read of the same memory reaches on the same device in the
 * same run ("achievable" bandwidth).
 */
#ifndef MNB_PROBE_H
#define MNB_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf[0, bytes) once with 16-byte non-temporal loads
 * (bytes a multiple of 16, buf 16-byte aligned, both device memory of the
 * current device) and folds them into a checksum that is written to
 * sink[0, 1024) (uint32, device, written only in the astronomically unlikely
 * case that a lane's checksum equals a fixed constant, so the loads cannot be
 * removed and no store traffic is added).  Enqueued on `stream`.
 * Returns 0, -1 for bad arguments (nothing launched), -5 for a launch error. */
int mnb_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MNB_PROBE_H */
