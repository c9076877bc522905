/*
 * mqa_fp4_probe.h -- measurement library beside the operator (libmqa_fp4_probe.so).
 *
 * Not part of the operator's ABI (include/mqa_fp4_topk.h): these entry points
 * run synthetic loops that measure, on the device the operator runs on and
 * under the clocks it sees, the issue rates its scan kernel is built from:
 * 32x32x64 MXFP4 MFMAs, fp32 VALU operations, the two side by side on one
 * SIMD, and the LDS read pattern of the score-block image. MI355X's published
 * peaks are quoted at 2.4 GHz; these probes give the rates in shader cycles
 * (s_memtime) per SIMD.
 *
 * All pointers are device memory of the stream's device (a gfx950), owned by
 * the caller. Every entry point checks its arguments on the host and returns a
 * negative MQA_ERR_* code (the operator header's values) without launching on
 * a bad one.
 */
#ifndef MQA_FP4_PROBE_H
#define MQA_FP4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of blocks the issue probe launches on the stream's device (one per
 * compute unit); negative on error. */
int32_t mqa_probe_blocks(void* stream);

/*
 * Issue probe: one block per compute unit of 64 * 4 * (n_mfma_waves +
 * n_valu_waves) threads (1 <= n_mfma_waves + n_valu_waves <= 4; its LDS
 * request keeps a second block off the CU), so every SIMD holds n_mfma_waves
 * waves that each issue iters x 4 independent
 * v_mfma_scale_f32_32x32x64_f8f6f4 (MXFP4 x MXFP4, 2*32*32*64 FLOP each) and
 * n_valu_waves waves that each issue iters x 64 independent fp32 FMAs (16
 * chains). Wave w of a block runs the MFMA loop when w / 4 < n_mfma_waves.
 *   rec   uint64 [blocks, 4 * (n_mfma_waves + n_valu_waves), 3]: per wave the
 *         shader-cycle counter at its start and end and its hardware id
 *         (HW_ID | XCC_ID << 32), from which the caller groups waves by SIMD
 *   sink  float [blocks * 64 * 4 * (n_mfma_waves + n_valu_waves)] (keeps the
 *         work live; every element written)
 */
int32_t mqa_probe_issue(int32_t n_mfma_waves, int32_t n_valu_waves, int32_t iters, uint64_t* rec, float* sink,
                        void* stream);

/* The issue probe with the MFMA waves issuing iters x 8 independent
 * v_mfma_scale_f32_16x16x128_f8f6f4 (MXFP4 x MXFP4, 2*16*16*128 FLOP each:
 * the same FLOPs per iteration as mqa_probe_issue); arguments, records and
 * errors as there. */
int32_t mqa_probe_issue16(int32_t n_mfma_waves, int32_t n_valu_waves, int32_t iters, uint64_t* rec, float* sink,
                          void* stream);

/*
 * VALU-waves probe: blocks of 256 threads, waves_per_simd per compute unit
 * (1 <= waves_per_simd <= 6; each block's LDS request, 160 KB / waves_per_simd
 * - 1 KB, keeps one block more off the CU), so every SIMD holds waves_per_simd
 * waves that each issue iters x 64 independent fp32 FMAs (16 chains): the
 * VALU issue rate of one SIMD as a function of its resident waves.
 *   rec   uint64 [blocks * waves_per_simd, 4, 3]: per wave the shader-cycle
 *         counter at its start and end and its hardware id, as in the issue
 *         probe
 *   sink  float [blocks * waves_per_simd * 256] (every element written)
 * blocks = mqa_probe_blocks(stream).
 */
int32_t mqa_probe_valu_waves(int32_t waves_per_simd, int32_t iters, uint64_t* rec, float* sink, void* stream);

/*
 * LDS read probe: blocks x 8 waves x iters x 2 ds_read_b128 over a 16 KB
 * score-block image. pattern 0: the scan's operand reads (chunk swizzle
 * applied), 1: a linear pattern no bank grouping makes conflict, 2: the image
 * without the swizzle. Pattern 0 as fast as pattern 1 means the scan reads the
 * image free of bank conflicts.
 *   out   float [blocks * 512], written once per lane
 */
int32_t mqa_probe_lds(int32_t pattern, float* out, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQA_FP4_PROBE_H */
