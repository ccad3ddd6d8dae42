/*
 * dflash_prof.h — measurement hook of libdflash (not part of the drafter's
 * arithmetic).
 *
 * While a timer is running, the library brackets every launch of one kernel
 * class with a pair of HIP events.  The events are recorded on the stream the
 * kernel is launched on.  A benchmark can thus measure one kernel's average
 * duration inside a normal run of the public calls.  One timer exists per
 * process, guarded by a mutex.  The events come from a pool created by
 * dflash_prof_start, which may call hipEventCreate.  While the timer is off,
 * nothing is recorded.
 */
#ifndef DFLASH_PROF_H
#define DFLASH_PROF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* kernel classes (3-7 are launches of the layered round path: batched,
 * paged or windowed rounds; the persistent kernel runs those steps inside
 * its one launch, class 10) */
#define DFLASH_K_GEMM_FC      1   /* fc projection of the taps */
#define DFLASH_K_GEMM_KV      2   /* ingest k|v projection */
#define DFLASH_K_GEMM_QKV     3   /* block q|k|v projection */
#define DFLASH_K_GEMM_O       4   /* o_proj + residual */
#define DFLASH_K_GEMM_GATEUP  5   /* gate|up + SwiGLU */
#define DFLASH_K_GEMM_DOWN    6   /* down + residual */
#define DFLASH_K_ATTN         7   /* attention (splits + merge) */
#define DFLASH_K_ROPE         8   /* head norm + rope + KV stores */
#define DFLASH_K_NORM         9   /* row RMSNorm */
#define DFLASH_K_ROUND       10   /* persistent forward_round kernel (one launch per 8 layers) */

/* Start timing launches of `kernel_class`, for up to `max_launches`
 * launches.  Later launches are not timed.  DFLASH_E_INVAL for a bad class or
 * count; DFLASH_E_HIP if the events cannot be created. */
int dflash_prof_start(int32_t kernel_class, int32_t max_launches);

/* Stop the timer.  Synchronises on the recorded events, then writes the
 * summed duration (ms) and the number of timed launches. */
int dflash_prof_stop(double *total_ms, int32_t *launches);

/* Phase trace of the persistent forward_round kernel.  While enabled, each
 * later launch records GPU wall-clock stamps (100 MHz counter) into a region
 * of its workspace.  Phase p of a launch is 1 + layer * P + i, where i runs
 * over the layer's phases (P = 6: q|k|v, attention, merge, o, gate|up,
 * down; with the DFlash2 wrap P = 8, a coefficient phase before q|k|v and
 * before gate|up).  Words 8p + k, workgroup 0:
 *   k = 0  wave 0 sees the phase's inputs complete
 *   k = 1  wave 0 done with its share
 *   k = 2  the epilogue done and the phase signalled
 *   k = 3  the loader issues the phase's first ring slot
 *   k = 4  the loader has issued the phase's last ring slot
 *   k = 5  the epilogue starts (GEMM phases)
 * Words 512 + 8p + k hold wave 1's stamps in GEMM phases (k = 0 set up,
 * 1 activations loaded, 4 first ring slot available, 2 k steps done,
 * 3 partial sums stored),
 * and word 1024 + 256 (p - 7) + w the time workgroup w signalled phase p,
 * for p in [7, 19).  dflash_prof_trace_read synchronises `stream` and copies
 * the first n stamps (n <= 4096) to host memory. */
int dflash_prof_trace(int32_t enable);
int dflash_prof_trace_read(const struct dflash_model *m, void *ws, size_t ws_bytes, uint64_t *out, int32_t n,
                           void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_PROF_H */
