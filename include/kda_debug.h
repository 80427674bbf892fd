/*
 * kda_debug.h - range-check build of the KDA library (libkda_debug.so).
 *
 * The same sources as libkda.so compiled with -DKDA_DEBUG_RANGE: the chunked prefill
 * kernels (every chunk length, the segment path included) check, as they run, what the
 * -5 log-decay floor guarantees (orkas.ai blog "Kimi K3 architecture", section "A lower
 * bound that deleted a GPU code path"):
 *   bit 1  a diagonal tile's row factor 2^L outside [0, 1], or its column factor 2^-L
 *          outside [1, e^80] (L: a token's log2-decay sum from its 16-token sub-tile's
 *          start);
 *   bit 2  an operand of a matrix product (k 2^L, q 2^L, k 2^-L and the others formed
 *          from them) not finite or beyond the bfloat16 range (the float32 range for
 *          float32 inputs);
 *   bit 4  a kept (unmasked) entry of an A or P tile not finite;
 *   bit 8  a value of the state not finite after a chunk.
 * Each violation ORs its bit into one device word per GPU; results are computed as in
 * libkda.so.  Every entry point of kda.h is exported as well.  For tests, not for
 * production use (the checks cost time).
 */
#ifndef KDA_DEBUG_H_
#define KDA_DEBUG_H_

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the current device's flag word to *flags (synchronous: waits for the device's
 * work to finish), then clears it if `clear` is non-zero.  KDA_ERR_NULL for a NULL
 * `flags`, KDA_ERR_HIP if the runtime fails. */
kda_status_t kda_debug_range_flags(unsigned* flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* KDA_DEBUG_H_ */
