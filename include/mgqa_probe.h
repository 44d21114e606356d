/*
 * mgqa_probe.h - C ABI of libmgqa_probe.so, the throughput probes behind the
 * ceilings the design notes quote for the attention kernels of libmgqa.so.
 *
 * Not part of the attention library: a measurement tool.  Each call queues
 * one probe kernel on `stream` (a hipStream_t passed as void*) and returns
 * at once; the caller times the launch (HIP events on the same stream) and
 * divides the work below by that time.  Every probe writes one 32-bit word
 * per thread to `sink` (device memory the caller owns, at least
 * workgroups * waves * 64 words), so its work cannot be removed by the
 * compiler.
 *
 * Kinds for probe_alu (per wave and iteration):
 *   PROBE_MFMA      8 v_mfma_f32_16x16x32_bf16 on 8 independent accumulators
 *                   (16384 flops each);
 *   PROBE_EXP       8 v_exp_f32 on 8 independent chains per lane;
 *   PROBE_RCP       8 v_rcp_f32 on 8 independent chains per lane;
 *   PROBE_MUL       8 v_mul_f32 on 8 independent chains per lane;
 *   PROBE_MFMA_EXP  the MFMA and the EXP work of one iteration, interleaved;
 *   PROBE_MFMA_MUL  the MFMA and the MUL work of one iteration, interleaved;
 *   PROBE_STEP_MFMA the matrix work of one step of the head-size-128 prefill
 *                   with a softcap (34 MFMAs into 18 accumulators), then a
 *                   workgroup barrier;
 *   PROBE_STEP_VEC  its vector work (16 scores per lane, each
 *                   v_mul, v_exp, v_add, v_rcp, v_fma, v_exp: 48
 *                   transcendental and 48 plain operations), then a barrier;
 *   PROBE_STEP_BOTH both, interleaved, then a barrier.
 * workgroups >= 1, waves per workgroup 1..16, iters >= 1; otherwise
 * MGQA_ERR_SHAPE (-2).  MGQA_ERR_NULL (-1) for a NULL sink, MGQA_ERR_HIP (-8)
 * if the launch fails.
 *
 * probe_read streams `bytes` (a multiple of 16) of device memory at `src`
 * with 16-byte loads, grid-stride over workgroups of 256 threads, and writes
 * the XOR of each thread's 32-bit words to sink[thread] (workgroups * 256
 * words): the XOR of all sink words equals the XOR of all words of src.
 * nontemporal = 1 sets the non-temporal bit of every load (the lines stay in
 * the caches only briefly), 0 reads with the default policy.  Errors as
 * above (bytes not a multiple of 16, nontemporal not 0 or 1:
 * MGQA_ERR_SHAPE).
 */
#ifndef MGQA_PROBE_H
#define MGQA_PROBE_H

#include <stddef.h>

#define PROBE_MFMA      0
#define PROBE_EXP       1
#define PROBE_RCP       2
#define PROBE_MUL       3
#define PROBE_MFMA_EXP  4
#define PROBE_MFMA_MUL  5
#define PROBE_STEP_MFMA 6
#define PROBE_STEP_VEC  7
#define PROBE_STEP_BOTH 8

#ifdef __cplusplus
extern "C" {
#endif

int probe_alu(int kind, int workgroups, int waves, int iters, unsigned* sink, void* stream);

int probe_read(const void* src, size_t bytes, int workgroups, int nontemporal, unsigned* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MGQA_PROBE_H */
