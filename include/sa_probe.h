/*
 * sa_probe.h -- measurement probes shipped beside the attention library
 * (libsa_probe.so; not part of the attention ABI in sa.h).  The benchmark uses
 * them for measured roofline denominators next to the chip's published peaks:
 * the bandwidth of a plain device copy, the bf16 matrix-core rate of a loop of
 * independent MFMAs, and the cost of an empty kernel launch (the floor under
 * microsecond calls such as a decode step).  None comes from the pages; they
 * characterise the machine the attention kernels run on.
 *
 * Pointers are device pointers, `stream` a hipStream_t (NULL: null stream);
 * calls enqueue and return 0, 1 for an invalid argument, 2 for a launch error.
 */
#ifndef SPARSE_CAUSAL_ATTENTION_SA_PROBE_H
#define SPARSE_CAUSAL_ATTENTION_SA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) from src
 * to dst, one 16-byte word per lane per step, four workgroups of 256 lanes
 * per compute unit (grid-stride loop). */
int sa_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* `blocks` workgroups of four wavefronts, each running four independent chains
 * of `iters` v_mfma_f32_32x32x16_bf16; out receives one float per wavefront
 * (4 * blocks floats). */
int sa_probe_mfma(float* out, int blocks, int iters, void* stream);

/* The matrix-core flops one sa_probe_mfma launch performs (host only). */
int sa_probe_mfma_flops(int blocks, int iters, double* flops);

/* One empty kernel (one wavefront). */
int sa_probe_empty(void* stream);

#ifdef __cplusplus
}
#endif
#endif
