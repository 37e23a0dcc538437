/*
 * tsa_probe.h - measurement probe beside the TSA library (libtsa_probe.so).
 *
 * Not part of the method: a fixed bf16 MFMA loop whose sustained throughput
 * on the running GPU is the practical ceiling against which the attention
 * kernel's MFMA work is read.  The 2.5 PFLOP/s published bf16 dense peak is
 * reached only when the operands barely toggle; with random bf16 operands
 * the chip holds a lower clock, and this probe measures that rate.
 *
 * Memory and streams follow tsa.h: `sink` is caller-owned device memory,
 * nothing is allocated, and the call returns once the launch is enqueued.
 */
#ifndef TSA_PROBE_H_
#define TSA_PROBE_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device memory the probe's `sink` needs on the current device
 * (one float per thread of its grid); 0 if the device cannot be queried. */
size_t tsa_probe_sink_bytes(void);

/* Enqueues one launch of the probe on `stream`: one 512-thread workgroup per
 * compute unit (two waves per SIMD), each wave issuing `iters` x 16
 * v_mfma_f32_32x32x16_bf16 into four accumulator chains, with operands held
 * in registers: all 1.0 / 0.5 (random_operands = 0) or random bf16 values
 * with random signs and mantissas and magnitudes in [0.25, 2)
 * (random_operands != 0).  The accumulators are written to `sink` so that no
 * work is dropped.  *flops receives the launch's MFMA FLOPs (2*32*32*16 per
 * instruction).  Time the launch with events on `stream`.
 * Returns 0, 1 for a null or small sink, null flops or iters < 1, or 4 when
 * the launch fails. */
int tsa_probe_mfma_bf16(int random_operands, int iters, void* sink, size_t sink_bytes,
                        double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_PROBE_H_ */
