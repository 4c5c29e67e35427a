/* Measurement aids for the attention kernel's roofline; not part of the method.
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

/* Largest workgroup count either probe accepts (keeps every thread's output
 * index below 2^31). */
#define ABS_PROBE_MAX_WORKGROUPS (1 << 21)

/* Launches `workgroups` workgroups of 256 threads (4 waves); each wave runs
 * `iters` rounds of 4 products of 32x32x16, i.e. 4 * 32768 * iters flop.
 *   out    : device, float32 [workgroups * 256], one sum of the accumulators
 *            per thread (keeps the products live);
 *   clocks : device, int64 [workgroups * 2], per workgroup the clock64
 *            counts and the wall-clock ticks (wall_clock64, whose rate is
 *            hipDeviceAttributeWallClockRate) of its product loop.
 * Caller-owned buffers; asynchronous on `stream` (a hipStream_t, NULL for the
 * default stream).  Returns 0, 1 for invalid arguments (workgroups outside
 * [1, ABS_PROBE_MAX_WORKGROUPS] among them; no launch) or 4 for a launch
 * error. */
int abs_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out, int64_t* clocks,
                        void* stream);

/* The attention kernel's per-subtile arithmetic with nothing around it: no
 * K/V copies, no barrier, no padding, no work items.  Each round of a wave is
 * one 32-key subtile: the softmax of the previous round's scores (exp2, four
 * partial row sums, bf16 conversion), 8 K operand reads from LDS feeding the
 * score products and 8 V operand reads feeding the PV products, each read
 * feeding one product per group of 32 queries the wave holds.
 *   queries_per_wave 32: workgroups of 512 threads (8 waves, two per SIMD, as
 *                        in the attention kernel), 16 products a round;
 *   queries_per_wave 64: workgroups of 256 threads (4 waves, one per SIMD),
 *                        32 products a round.
 * Every round is 4 * 32 * 32 * 128 * 2 flop per 32 queries (the products of
 * one 32-key subtile), i.e. 524288 * queries_per_wave / 32 flop per wave.
 * One workgroup fits a CU (48 KB of LDS and the register budget of its
 * occupancy), so `workgroups` a multiple of the CU count runs whole rounds.
 *   out    : device, float32 [workgroups * (8 or 4) * 64];
 *   clocks : device, int64 [workgroups * 2], as for abs_probe_mfma_bf16.
 * Returns 0, 1 for invalid arguments (queries_per_wave not 32 or 64,
 * workgroups outside [1, ABS_PROBE_MAX_WORKGROUPS]; no launch) or 4 for a
 * launch error. */
int abs_probe_attn_loop(int32_t queries_per_wave, int32_t iters, int32_t workgroups, float* out,
                        int64_t* clocks, void* stream);

/* The wall-clock rate of the current device in kHz (the tick rate of the
 * second clocks entry).  Host query; returns 0, 1 for a null pointer, 4 for a
 * HIP error. */
int abs_probe_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* ABS_PROBE_H */
