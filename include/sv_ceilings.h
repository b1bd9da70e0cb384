/*
 * sv_ceilings.h -- measured machine ceilings for the roofline figures of the
 * verification step (same library as spec_verify.h).
 *
 * The roofline of the verification step prices each kernel against the HBM
 * read rate (attention streams the KV cache; acceptance streams the logits)
 * and, for the many-row shapes, the MFMA rate; the softmax adds one
 * exponential per score, a third ceiling on the vector units.  The pages state
 * the bound in words only (decode attention is limited by memory traffic, its
 * intensity about 2 G (1 + D) flops per KV element: NVIDIA co-design summary,
 * papanda925.com, guideline 2; "GPU and LLM" ch. 5, section "FlashAttention":
 * the score table never goes to HBM).  These three calls measure the
 * ceilings on the machine at hand, so that a kernel's rate can be given as a
 * fraction of both the published peak and the measured one.
 *
 * Each call enqueues one kernel on `stream` (a hipStream_t, NULL = default
 * stream) and returns at once; the caller times it (e.g. with HIP events on
 * that stream).  The library allocates nothing.  Arguments are checked on the
 * host before any launch (SV_ERR_INVALID with a message in sv_last_error()).
 */
#ifndef SV_CEILINGS_H
#define SV_CEILINGS_H

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every byte of src[0 .. bytes) is read once with 16-byte
 * non-temporal vector loads by a grid of `workgroups` x 256 threads
 * (workgroups in [1, 65536]), each workgroup reading whole 16 KB chunks (the
 * chunks w, w + workgroups, ... for workgroup w; what follows the last whole
 * chunk is read one vector per thread); bytes > 0 and a multiple of 16, src
 * 16-byte aligned.  One float per workgroup (a reduction of the values read, so the
 * loads cannot be dropped) goes to sink[0 .. workgroups).  Rate = bytes /
 * kernel time. */
sv_status sv_ceiling_read(const void* src, size_t bytes, int32_t workgroups, float* sink,
                          void* stream);

/* Dense bf16 matrix-core loop: `workgroups` x 256 threads (4 waves), every wave
 * issuing `iters` x 4 independent v_mfma_f32_32x32x16_bf16 (32768 flops each)
 * on register operands.  workgroups in [1, 65536], iters in [1, 2^20].  Each
 * wave writes its accumulators' sum to sink[0 .. 4 workgroups).  Rate =
 * workgroups * 4 * iters * 4 * 32768 / kernel time. */
sv_status sv_ceiling_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Vector exponential rate: `workgroups` x 256 threads, each running 8
 * independent chains of `iters` base-2 exponentials (v_exp_f32, the
 * instruction the softmax uses).  workgroups in [1, 65536], iters in [1,
 * 2^20].  sink[0 .. 256 workgroups) receives each thread's result.  Rate =
 * workgroups * 256 * iters * 8 / kernel time. */
sv_status sv_ceiling_exp2(int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_CEILINGS_H */
