/*
 * sa_probe.h -- measurement probes shipped beside the attention library
 * (libsa_probe.so; not part of the attention ABI in sa.h).  The benchmark uses
 * them for measured roofline denominators next to the chip's published peaks:
 * the bandwidth of a plain device copy, the bf16 matrix-core rate of a loop of
 * independent MFMAs, and the cost of an empty kernel launch (the floor under
 * microsecond calls such as a decode step); and issue-rate probes of mixed
 * matrix-core and vector-ALU work (how far one SIMD overlaps them).  None comes from the pages; they
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

/* Issue-rate probes: does the SIMD overlap independent matrix-core and
 * vector-ALU work, and what does each cost?  Variant v (0 <= v <
 * sa_probe_mix_variants()) runs, per round, the counts sa_probe_mix_counts
 * names: MFMAs (v_mfma_f32_32x32x16_bf16, two independent chains), v_fma_f32
 * and v_exp_f32 (sixteen independent chains each), none depending on another.
 * sa_probe_mix launches `blocks` workgroups of four wavefronts running `iters`
 * rounds; out receives four floats per wavefront (16 * blocks floats): the
 * ticks of s_memtime and of s_memrealtime (constant rate, see the device's
 * wall-clock frequency) its rounds took, a value that keeps the work, and 0.
 * With four workgroups per compute unit (blocks = 4 x CUs), time / iters is
 * one SIMD's time for one round of each of its four wavefronts. */
int sa_probe_mix_variants(void);
int sa_probe_mix_counts(int variant, int* n_mfma, int* n_fma, int* n_exp);
int sa_probe_mix(int variant, float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif
