/* Measurement aid for the attention kernel's roofline; not part of the method.
 *
 * The data sheet gives MI355X 2.5 PFLOP/s of dense bf16 MFMA at 2.4 GHz.  A
 * long MFMA-bound kernel draws enough power that the chip lowers its shader
 * clock, so the rate it can sustain is lower.  This probe measures that rate
 * directly: every SIMD issues v_mfma_f32_32x32x16_bf16 back to back on varied
 * bf16 operands (four independent accumulator chains per wave), and every
 * workgroup reports how long its product loop ran in clock64 counts and in
 * wall-clock ticks.
 *
 * Built as its own library, libabs_probe.so, next to libabs.so.
 */
#ifndef ABS_PROBE_H
#define ABS_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `workgroups` workgroups of 256 threads (4 waves); each wave runs
 * `iters` rounds of 4 products of 32x32x16, i.e. 4 * 32768 * iters flop.
 *   out    : device, float32 [workgroups * 256], one sum of the accumulators
 *            per thread (keeps the products live);
 *   clocks : device, int64 [workgroups * 2], per workgroup the clock64
 *            counts and the wall-clock ticks (wall_clock64, whose rate is
 *            hipDeviceAttributeWallClockRate) of its product loop.
 * Caller-owned buffers; asynchronous on `stream` (a hipStream_t, NULL for the
 * default stream).  Returns 0, 1 for invalid arguments (no launch) or 4 for
 * a launch error. */
int abs_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out, int64_t* clocks,
                        void* stream);

/* The wall-clock rate of the current device in kHz (the tick rate of the
 * second clocks entry).  Host query; returns 0, 1 for a null pointer, 4 for a
 * HIP error. */
int abs_probe_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* ABS_PROBE_H */
