/* fmha_peaks.h -- attainable-peak probes of one MI355X (measurement aids).
 *
 * Not part of the attention path: the benchmark runs these once to state
 * its roofline fractions against what this GPU actually sustains as well as
 * against the published peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
 * Library: head_attention_fmha_amd/libfmha_peaks.so.  Same conventions as
 * fmha.h: device pointers owned by the caller, work enqueued on `stream`
 * (a hipStream_t; NULL = default) without synchronising, status codes from
 * fmha.h's fmha_status (0 = OK, 1 = invalid argument, 3 = alignment,
 * 4 = launch failure), validation before any HIP call.
 */
#ifndef FMHA_PEAKS_H
#define FMHA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned; bytes a
 * positive multiple of 32 KiB), 16-byte loads spread over the whole chip;
 * nontemporal != 0 sets the non-temporal hint on every load.  The loaded
 * words are folded into one value that is written to *sink only if it
 * equals a constant, so the loads cannot be optimised away.  Time it with
 * stream events: bytes / time is the attainable read bandwidth. */
int fmha_peak_stream_read(const void *buf, int64_t bytes, int nontemporal, unsigned *sink, void *stream);

/* `workgroups` workgroups of four waves, each wave issuing `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 (32768 flop each) on register
 * operands; one float per wave goes to sink[] (workgroups * 4 floats).
 * Flops = workgroups * 4 * iters * 4 * 32768. */
int fmha_peak_mfma_bf16(int workgroups, int iters, float *sink, void *stream);

/* `workgroups` workgroups of four waves running an empty kernel: the time
 * per launch, back to back on one stream, is the launch floor against which
 * the benchmark flags launch-bound workloads. */
int fmha_peak_empty(int workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif
