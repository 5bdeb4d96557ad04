/*
 * eagle3_testing.h — fault injection for tests of the library's failure paths
 * (pegainfer PR #707, review: cleanup on failure and abort cases must be
 * covered by tests).
 */
#ifndef EAGLE3_TESTING_H
#define EAGLE3_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Make the n-th device allocation the library attempts from now on (n >= 1;
   counted over all handles and threads) fail as out of memory; n <= 0 disarms.
   The failing call must then return EAGLE3_E_OOM, release everything it had
   allocated and leave its output handle NULL. */
void eagle3_test_fail_allocation(int32_t n);

/* The number of device and pinned host allocations the library holds now, over
   all handles and threads (each load adds its buffers, each free and each failed
   load removes them again). */
int64_t eagle3_test_live_allocations(void);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE3_TESTING_H */
