/*
 * dcn_debug.h -- an entry point that only the debug build of libdcn
 * (libdcn_count.so, compiled with DCN_COUNT_WRITES) exports; libdcn.so does
 * not have it.
 *
 * The forward ops are atomic-free: every output element is written by exactly
 * one store of one thread.  In the debug build every store of an output of
 * dcn_forward, of msda_forward / msda_forward_ref (their vector paths) and of
 * dcn_offset_mask (offsets and mask) also adds one to a per-element counter,
 * so a caller can check that claim after a launch: each of counts[0..n) must
 * read 1, and counts[n] counts the output stores whose address falls outside
 * the registered buffer (0 for a single-output op; for dcn_offset_mask, the
 * elements of its other output).
 */
#ifndef DCN_DEBUG_H
#define DCN_DEBUG_H

#include <stddef.h>

#include "dcn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Register the output buffer that the next forward launches write, on the
 * current device:
 *   counts  device array of n + 1 uint32 counters, zeroed by the caller
 *           (caller-owned; NULL stops counting);
 *   out     device address of the output buffer, n elements of dtype
 *           (DCN_F32, DCN_F16 or DCN_BF16).
 * The counters are added to by device atomics during later launches; the
 * caller reads them back after synchronising.  Only one buffer is
 * registered at a time.  Returns DCN_ERR_INVALID for a bad dtype or a
 * non-NULL counts with a NULL out, DCN_ERR_HIP if the registration fails.
 */
dcn_status dcn_debug_count_writes(unsigned int* counts, const void* out, size_t n, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* DCN_DEBUG_H */
