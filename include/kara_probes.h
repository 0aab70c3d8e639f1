/*
 * kara_probes.h - achievable-peak probes for MI355X (gfx950), exported by
 * libkara_probes.so.  Measurement tooling beside the Kara library: each call
 * enqueues one kernel on `stream` (a hipStream_t, NULL = default stream) and
 * returns 0, -1 for a bad argument, or the HIP error code of the launch.
 * All pointers are device pointers owned by the caller.
 */
#ifndef KARA_PROBES_H_
#define KARA_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* blocks x 4 waves; each wave issues iters x 4 MFMA 32x32x16 bf16 (32768 FLOP each).
 * out: blocks * 256 floats. */
int kara_probe_mfma(float* out, int blocks, int iters, void* stream);

/* blocks x 256 lanes; each lane issues iters x 8 exp2 (v_exp_f32).  out: blocks * 256 floats. */
int kara_probe_exp(float* out, int blocks, int iters, void* stream);

/* blocks x 256 lanes; each lane issues iters x 8 fp32 FMA.  out: blocks * 256 floats. */
int kara_probe_fma(float* out, int blocks, int iters, void* stream);

/* blocks x threads lanes (threads a multiple of 64, at most 512), iters iterations of:
 * mode 0: 4 independent MFMA 16x16x32 bf16; mode 1: 16 independent fp32 FMA; mode 2: both,
 * interleaved (MFMA, 4 FMA, MFMA, ...); mode 3: the MFMAs interleaved with 16 v_exp_f32;
 * mode 4: the 16 v_exp_f32 alone (modes 3 and 4 multiply each argument first); mode 5: 16
 * bare v_exp_f32 (argument negated by the input modifier); mode 6: the 16 bare v_exp_f32
 * interleaved with 16 independent fp32 FMAs.
 * out: blocks * threads floats.  Comparing the modes' times shows how far the matrix cores
 * and the VALU overlap at a given number of waves per SIMD. */
int kara_probe_coissue(int mode, float* out, int blocks, int threads, int iters, void* stream);

/* Co-issue at a fixed number of waves per SIMD: blocks workgroups of `threads` (256 or 512)
 * lanes, each holding 96 KiB of LDS so that one workgroup runs per compute unit (pass
 * blocks = number of compute units for threads / 256 waves per SIMD).  Per iteration:
 * mode 0: 16 independent 16x16x32 bf16 MFMAs; mode 1: 64 independent fp32 FMAs;
 * modes 2, 3, 4: the 16 MFMAs with 16, 32 or 64 FMAs interleaved (MFMA, 1/2/4 FMAs, ...);
 * mode 5: 32 bare v_exp_f32; mode 6: the 16 MFMAs with the 32 v_exp_f32 interleaved.
 * Modes 7 and 8 (threads = 512 only) split the work between the two waves of each SIMD:
 * waves 0-3 run 16 MFMAs per iteration, waves 4-7 run 64 FMAs (mode 7) or 32 bare
 * v_exp_f32 (mode 8); lane 0 of each wave writes 1000 + 10 * SIMD id + (1 for a vector wave).
 * out: blocks * threads floats. */
int kara_probe_coissue_cu(int mode, float* out, int blocks, int threads, int iters, void* stream);

/* Reads `bytes` (a multiple of 16) of src once.  out: grid * 256 floats. */
int kara_probe_read(const void* src, size_t bytes, float* out, int grid, void* stream);

/* Copies `bytes` (a multiple of 16) from src to dst (each byte read and written once).  grid
 * workgroups of 256 threads stride over the buffer. */
int kara_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream);

/* Reads `bytes` (a multiple of 16) of buf and writes them back in place (each byte read and
 * written once), one workgroup per 16 KiB chunk. */
int kara_probe_rewrite(void* buf, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KARA_PROBES_H_ */
