/*
 * libgdr_debug.h -- race-test hook of libgdr, exported ONLY by the
 * instrumented build libgdr_delay.so (the same kernels compiled with
 * GDR_DEBUG_DELAY); the production libgdr.so does not export it.
 *
 * The method is the one the review of FastVideo PR #1819 ("[kernel] sm_100a
 * CUDA backward for VSA block-sparse attention (blk64)", the reproduction of
 * its cross-warp overlap) uses to confirm a race: delay one side of a
 * suspected race so its window opens, keep the arithmetic unchanged, and
 * compare outputs bitwise, besides many undelayed runs compared bitwise.
 * In the instrumented build every workgroup barrier of every kernel is
 * followed by an optional delay: after a pseudo-random subset of barriers (a
 * hash of the cycle counter, the workgroup index and `salt`, modulo `mod`,
 * equal to zero), the selected wave(s) sleep for `iters` x s_sleep(127)
 * (about 8k cycles each).  A delay changes no arithmetic, so if every LDS
 * hand-off between waves is ordered by a barrier, the outputs with delays
 * are bitwise equal to those without.
 */
#ifndef LIBGDR_DEBUG_H
#define LIBGDR_DEBUG_H

#include "libgdr.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Set the delay of every later launch from this library (all devices share
 * the setting of the current one; set it on the device that will run).
 *   wave   wave index within a workgroup to delay (0..7), or -1 for all
 *   mod    >= 1: a barrier is followed by a delay when the hash % mod == 0
 *          (1: after every barrier)
 *   iters  0..64 sleeps per delay; 0 turns delays off
 *   salt   any value; varies which barriers are chosen
 * The call is synchronous with respect to the host (it copies the settings
 * to device constant memory); do not call it while a launch from this
 * library is in flight.  Returns GDR_ERR_INVALID_ARG for settings out of
 * range, GDR_ERR_HIP if the copy fails. */
gdr_status gdr_debug_set_delay(int wave, int mod, int iters, int salt);

#ifdef __cplusplus
}
#endif

#endif /* LIBGDR_DEBUG_H */
