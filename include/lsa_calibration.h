/*
 * liblsa measurement aid: an access-pattern probe.
 *
 * Not part of the attention method.  It is for callers that report a kernel
 * against the rate its memory access pattern can reach: the routed-block
 * partial kernel reads one 128-byte query row and writes one 128-byte partial
 * row per (query, routed block) pair, both at effectively random places, and
 * no schedule of the key-block-major attention avoids that.  This probe moves
 * 128-byte rows between two tables with the same patterns so the attainable
 * rate can be measured on the machine at hand.
 */
#ifndef LSA_CALIBRATION_H
#define LSA_CALIBRATION_H

#include <stddef.h>
#include <stdint.h>

#include "lsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Row copies dst[w(i)] = src[r(i)] for i in [0, n), each row 128 bytes
 * (8 lanes of 16 bytes each), enqueued on `stream` (a hipStream_t, NULL = the
 * default stream):
 *   mode 0: r(i) = w(i) = i           (sequential copy)
 *   mode 1: r(i) = ridx[i], w(i) = i  (random read, sequential write)
 *   mode 2: r(i) = i, w(i) = widx[i]  (sequential read, random write)
 *   mode 3: r(i) = ridx[i], w(i) = widx[i]
 * src and dst are device tables of table_rows rows; ridx and widx are device
 * arrays of n row numbers, read only by the modes that use them (NULL
 * otherwise).  A copy whose row number is >= table_rows is skipped, so no
 * access leaves the tables whatever the index arrays hold.  The caller owns
 * every buffer; nothing is allocated.
 * Errors: LSA_ERR_NULL (src, dst, or an index array the mode reads is NULL),
 * LSA_ERR_SHAPE (mode outside 0..3, n or table_rows negative, n > table_rows
 * for a mode with a sequential side, or n >= 2^28), LSA_ERR_ALIGN (a pointer
 * not 16-byte aligned), LSA_ERR_DEVICE (the launch failed). */
lsa_status lsa_calibrate_access(const void *src, void *dst, const uint32_t *ridx,
                                const uint32_t *widx, int64_t table_rows, int64_t n,
                                int32_t mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_CALIBRATION_H */
