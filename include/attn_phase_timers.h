/* Phase timers of the causal attention kernels: a measurement build only.
 *
 * libattn_phase_timers.so is libattn.so compiled with ATTN_PHASE_TIMERS defined: the
 * same entry points (include/attn.h) and the same kernels, plus shader-clock reads
 * (s_memtime) around the two phases of every key tile of the two-group schedule
 * (a matrix phase: P.V of the previous tile and Q.K^T of this one; a softmax phase:
 * mask, max, probabilities, sums; each ends at a workgroup barrier), summed per wave.
 * The reads sit between scheduling barriers, so the timed build's instruction order
 * differs slightly from libattn.so's; it is for finding which phase bounds a kernel,
 * not for timing the product.  libattn.so has none of this.
 *
 * Record of one (workgroup, wave), ATTN_PHASE_TIMER_WORDS unsigned 64-bit words at
 * buf[(workgroup * ATTN_PHASE_TIMER_WAVES + wave) * ATTN_PHASE_TIMER_WORDS]:
 *   [0] tiles counted: the wave's key tiles minus the first two and the last two (the
 *       pipeline's fill and drain), 0 when it has 4 or fewer;
 *   [1] cycles from the start of the counted tiles' matrix phases to their ends,
 *       before the barrier wait, summed;
 *   [2] the same for their softmax phases;
 *   [3] cycles from the start of the first counted tile to the start of the tile after
 *       the last one: the period, summed (so [3] - [1] - [2] is time at barriers);
 *   [4] the device's real-time counter (s_memrealtime, a constant-rate clock shared by
 *       the whole device) when the wave starts;
 *   [5] the same when it enters its first matrix phase (Q loaded, the first two tiles'
 *       copies issued, the first barrier passed: the prologue is [5] - [4]);
 *   [6] the same when it leaves the key loop;
 *   [7] the same once it has issued its O and LSE stores (the epilogue is [7] - [6]; the
 *       stores complete afterwards, and a workgroup's CU takes the next one only then);
 *   [8] the workgroup's key tiles (the loop runs [8] + 1 matrix phases);
 *   [9] the wave's HW_ID register (CU in bits 8-11, shader array bit 12, shader engine
 *       bits 13-15) in the low 32 bits and its XCC_ID register (compute die) in the high.
 * Workgroup index = launch order (the heaviest causal tiles first).  Waves 0-3 are the
 * group that starts with a matrix phase, waves 4-7 the one half a phase behind.
 */
#ifndef ATTN_PHASE_TIMERS_H
#define ATTN_PHASE_TIMERS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_PHASE_TIMER_WAVES 8
#define ATTN_PHASE_TIMER_WORDS 10

/* Record into buf (device memory, 8-byte aligned, owned by the caller, at least
 * bytes long) from every following attention launch of this library, for the
 * workgroups whose index is below bytes / (ATTN_PHASE_TIMER_WAVES *
 * ATTN_PHASE_TIMER_WORDS * 8); buf = NULL stops recording.  Each launch overwrites the
 * records of the workgroups it has.  Returns ATTN_OK, ATTN_E_ALIGN for a misaligned
 * buf, or ATTN_E_INVAL when bytes holds no record.  Not thread-safe: set it before the
 * launches it is meant for. */
int attn_phase_timers_set(void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PHASE_TIMERS_H */
