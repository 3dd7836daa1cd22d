/*
 * kda_testing.h -- test hooks of the KDA library.  Not part of the
 * computation: they let a test force a failure path from the host so that
 * it can check the failure is visible, with every kernel still exiting
 * normally.
 */
#ifndef KDA_TESTING_H_
#define KDA_TESTING_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The prefill's state pass splits each chunk between a wave that advances
 * the state and a wave that forms the chunk's output; the second waits, a
 * bounded number of polls, for the first to hand over the chunk's write
 * strengths U (the chunked form of section 6 of page "Yanjiu KimiK3 ...",
 * http://www.pwwt.cn/news/3763336/).  If the wait gives up, that chunk's
 * output rows are NaN and the state is unaffected.
 *
 * kda_testing_set_wait_limit sets the number of polls for every later
 * prefill launch in the process (default 1 << 24; 0 makes every wait give up
 * at once).  It returns KDA_OK, or KDA_ERR_INVALID_ARG for a negative value.
 * Process-wide and not synchronised with launches in flight: call it only
 * while no prefill is being enqueued.  kda_testing_wait_limit returns the
 * current value.
 */
KDA_API int kda_testing_set_wait_limit(int polls);
KDA_API int kda_testing_wait_limit(void);

/*
 * The prefill keeps one slot of per-chunk operand tiles for every chunk it
 * has prepared but not yet passed through the state recurrence (section 6:
 * the state moves from chunk to chunk).  When all slots of a call would
 * exceed a budget (512 MiB by default), kda_fwd_chunked cuts the sequence
 * into segments that run one after another through a fixed ring, so its
 * workspace stops growing with T.
 *
 * kda_testing_set_ring_cap sets that budget in bytes for every later
 * kda_fwd_chunked* call and workspace query in the process (0 restores the
 * default); tests use a small budget to run many segments at small sizes.
 * Same threading caveat as above.  kda_testing_ring_cap returns it.
 */
KDA_API int kda_testing_set_ring_cap(size_t bytes);
KDA_API size_t kda_testing_ring_cap(void);

/*
 * kda_testing_check_probe enqueues on `stream` a one-thread kernel that
 * performs one bounds check meant to fail (an index one past the end of a
 * one-element extent) and touches no memory.  In the checked build it
 * returns KDA_ERR_CHECK with bit 11 set in kda_check_sites(); in the normal
 * build the check compiles away and it returns KDA_OK.  KDA_ERR_HIP if the
 * launch fails.
 */
KDA_API int kda_testing_check_probe(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_TESTING_H_ */
