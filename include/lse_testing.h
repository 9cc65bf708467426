/*
 * lse_testing.h — test hook of liblse.so (include/lse.h is the API).
 *
 * Not for production callers: it exists so that tests can force the paths
 * that keep the cross-workgroup waits of two entry points from depending on
 * scheduling, paths that a normal run almost never takes.
 *
 *   log_softmax_rows / softmax_rows (split rows): a workgroup that runs out of
 *     polls for its siblings' (max, sum) pairs computes the missing ones from
 *     x.  With a limit of 0 no workgroup publishes its own pair, so every
 *     pair comes from that path.  After the call has run, the 32-bit word at
 *     byte offset 4 of the workspace holds the number of pairs computed that
 *     way (rows x chunks at a limit of 0).
 *   fused_conv_gn_act_lse: a workgroup that runs out of polls for its
 *     sample's GroupNorm statistics queues its tile pair and exits; the
 *     launch's last workgroup finishes the queued pairs.  With a limit of 0
 *     every pair is queued.  After the call has run, the 32-bit word at byte
 *     offset align256(8 N groups) + 4 of the workspace holds the number of
 *     pairs finished that way (N x ceil(tiles / 2) at a limit of 0, tiles =
 *     ceil((H - K + 1) / 2) x ceil((W - K + 1) / 128)).
 *
 * The limit is per host thread: it applies to calls that the calling thread
 * enqueues after it returns, and to no other thread's.  The default is 2^24
 * polls; independently of it each wait is bounded in time.
 */
#ifndef LSE_MI355X_TESTING_H
#define LSE_MI355X_TESTING_H

#include <stdint.h>

#include "lse.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Poll limit of the waits described above for the calling thread. */
void lse_testing_set_spin_limit(uint32_t polls);

/* enable != 0: split rows of log_softmax_rows / softmax_rows whose rows are
 * 16-byte aligned (cols a multiple of 4) take the re-read kernel instead of
 * the register-resident one, for calls from the calling thread: each
 * workgroup folds its chunk with the online (max, sum) recurrence in few
 * registers, and after the pairs are merged reads the chunk again (from the
 * caches when it is still there) to write y.  Same results within the usual
 * tolerance (another summation order); the same workspace.  A comparison
 * variant: the default keeps each chunk in registers. */
void lse_testing_set_rows_reread(int enable);

/* Which launches fused_conv_gn_act_lse uses for calls from the calling
 * thread (and which size fused_conv_gn_act_lse_workspace_bytes returns):
 *   0  automatic (the default): one fused launch while a sample's tile pairs
 *      number at most half of what the device holds at once, else the
 *      statistics launch followed by an apply launch that recomputes the conv;
 *   1  one fused launch for any size;
 *   2  statistics launch + recomputing apply launch;
 *   3  statistics launch that also stores each tile pair's conv output (128
 *      KiB per pair) in the workspace + apply launch that reads it back, in
 *      batches of samples of at most 192 MiB of staged output (samples too
 *      large for that take 2).
 * All give the same results.  Returns LSE_OK, or LSE_ERR_SHAPE for another
 * value (the setting is then unchanged).  Query the workspace size after
 * setting the path. */
lse_status_t lse_testing_set_chain_path(int path);

#ifdef __cplusplus
}
#endif

#endif /* LSE_MI355X_TESTING_H */
