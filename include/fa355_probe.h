/*
 * fa355_probe.h -- C ABI of libfa355_probe: two measurement kernels that put
 * the attention kernels' rates in context on the machine they run on.  They
 * are not part of the attention path (libfa355); bench.py reports their
 * results beside the roofline fractions, which stay quoted against MI355X's
 * published peaks.
 *
 * Both calls are synchronous: they allocate what they need on the current
 * device, run, wait, free, and return FA_PROBE_OK (0) or FA_PROBE_E_ARG (-1)
 * for an invalid argument (nothing launched) or FA_PROBE_E_HIP (-2) if the
 * HIP runtime fails.
 */
#ifndef FA355_PROBE_H
#define FA355_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { FA_PROBE_OK = 0, FA_PROBE_E_ARG = -1, FA_PROBE_E_HIP = -2 };

/*
 * fa_probe_mfma_bf16 -- attainable dense bf16 matrix-core rate and the
 * engine clock while the matrix cores are saturated.  Every SIMD runs
 * waves_per_simd (1..4) waves, each issuing `iters` (>= 1) rounds of four
 * independent v_mfma_f32_32x32x16_bf16 (32x32x16, 32768 FLOP each) and
 * nothing else.  Outputs: *tflops = FLOP / kernel time (HIP events);
 * *clock_ghz = the mean over waves of (core cycles elapsed) / (constant-rate
 * wall-clock ticks elapsed) times the wall-clock rate; *seconds = the kernel
 * time.  Any output pointer may be NULL.
 */
int fa_probe_mfma_bf16(int iters, int waves_per_simd, double *tflops,
                       double *clock_ghz, double *seconds);

/*
 * fa_probe_read_bw -- streaming read rate of device memory: a buffer of
 * `bytes` (>= 1 MiB, a multiple of 1 MiB) is read `reps` (>= 1) times by a
 * grid-stride kernel of 16-byte non-temporal loads (eight in flight per
 * lane), timed with HIP events after one untimed pass, at 1, 2, 4, 8 and 16
 * workgroups of 256 threads per CU.  *gbs = bytes * reps / time / 1e9 of
 * the fastest shape.
 */
int fa_probe_read_bw(size_t bytes, int reps, double *gbs);

#ifdef __cplusplus
}
#endif

#endif /* FA355_PROBE_H */
