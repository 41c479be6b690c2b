/*
 * libra_debug.h -- entry points of the counting build of the library
 * (liblibra_debug.so, compiled with LIBRA_COUNT_PAIRS), for tests only.
 *
 * That build's forward kernel counts the (query, key, head) triples it
 * leaves unmasked and adds them to one device counter.  Eq. 8 of the Libra
 * technical review (section 5.3) counts exactly these causal pairs, so after
 * one forward launch over a pack the counter must equal
 * h_q * sum_j l_j (l_j + 1) / 2.  Everything else in the counting build is
 * the regular library; the regular build has neither the counter nor these
 * functions.
 */
#ifndef LIBRA_DEBUG_H
#define LIBRA_DEBUG_H

#include <stdint.h>

#include "libra.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy the counter to *count (synchronises with the device).  LIBRA_EINVAL
 * for a NULL pointer, LIBRA_EHIP if the copy fails. */
libra_status libra_debug_unmasked_pairs(uint64_t *count);

/* Set the counter to 0 (synchronises with the device).  LIBRA_EHIP if the copy
 * fails. */
libra_status libra_debug_reset_unmasked_pairs(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRA_DEBUG_H */
