/* libgdn_calib: measurement aids used by the benchmark; not part of the GDN
 * interface (include/gdn.h).
 *
 * gdn_calib_mfma_bf16 launches `waves` wavefronts on `stream`, each issuing
 * `iters` x 8 independent v_mfma_f32_16x16x32_bf16 instructions (dense bf16
 * matrix-core work, 16384 flop each), and writes one float per lane to
 * `sink` (a device buffer of waves * 64 floats, caller-owned).  Returns 0,
 * -1 for a bad argument, -8 when the launch fails.  Asynchronous: time it
 * with events on `stream`.  gdn_calib_mfma_bf16_flops gives the flop count
 * of one launch.
 */
#ifndef GDN_CALIB_H
#define GDN_CALIB_H

#ifdef __cplusplus
extern "C" {
#endif

int gdn_calib_mfma_bf16(int waves, int iters, float* sink, void* stream);
double gdn_calib_mfma_bf16_flops(int waves, int iters);

#ifdef __cplusplus
}
#endif

#endif
