/* Diagnostic probe, separate from the attention library (librra_probe.so).
 *
 * Measures the bf16 matrix-core throughput a kernel can sustain on this GPU
 * when nothing but back-to-back v_mfma_f32_32x32x16_bf16 runs (eight
 * independent accumulators per wave, two waves per SIMD, every CU busy), and
 * the shader clock while it runs.  With real data the multiplier inputs toggle
 * and the part drops its clock to stay within its power limit, so this rate,
 * not the nameplate figure, is the ceiling a bf16 attention kernel meets in
 * practice.
 */
#ifndef RRA_PROBE_H_
#define RRA_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Runs the probe on the current HIP device and blocks until it is done.
 *   operands: 0 = all-zero operands, 1 = operands drawn from N(0, 1) (seeded,
 *             rounded to bf16), alternated between MFMAs so the inputs toggle.
 *   iters:    loop trips per wave (8 MFMAs each); 20000 takes a few ms.
 *   tflops:   out, achieved TFLOP/s from HIP events around the launch.
 *   clock_ghz: out, shader clock = core-clock cycles (s_memtime) over the
 *             100 MHz real-time counter (s_memrealtime), averaged over waves.
 * Allocates and frees its own small device buffers.  Returns 0 or the HIP
 * error code; outputs are untouched on error. */
int rra_probe_mfma_rate(int operands, int iters, double* tflops, double* clock_ghz);

#ifdef __cplusplus
}
#endif

#endif /* RRA_PROBE_H_ */
