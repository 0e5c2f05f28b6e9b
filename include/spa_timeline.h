/* Per-wave timeline of the decode producer: a diagnostics build only.
 *
 * libspa_timeline.so is libspa.so compiled with SPA_TIMELINE defined: it
 * exports every function of spa.h with the same behaviour, and in addition
 * lane 0 of every wave of the one-token decode producer (decode_kernel)
 * writes the GPU's constant 100 MHz clock (s_memrealtime) at the steps of
 * its chain into a device array of SPA_TIMELINE_WAVES rows of
 * SPA_TIMELINE_SLOTS 64-bit words, row = blockIdx.x * (waves per
 * workgroup) + wave.  The stamps cost a scalar memory round trip each, so
 * times measured with this library are slower than with libspa.so; they
 * show where a wave's time goes, not the kernel's speed.  libspa.so exports
 * none of the functions below.
 *
 * Slots (0 = not reached by the wave):
 *   0  entry                      1  request length known
 *   2  first page id known        3  first page's scores computed
 *   4  all pages done             5  partial states issued (all splits)
 *   6  states in memory (fused)   7  arrival counted (fused)
 *   8  merge done (fused, the last workgroup to arrive)
 *   9  end
 *  10  request | kv head << 16 | first split << 32 (a value, not a time)
 *  11  pages of the workgroup (a value)
 * Rows of waves past SPA_TIMELINE_WAVES are not recorded.  Not thread-safe
 * with respect to concurrent launches: every launch writes the same array.
 */
#ifndef SPA_TIMELINE_H
#define SPA_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPA_TIMELINE_SLOTS 16
#define SPA_TIMELINE_WAVES 65536

/* Zero the current device's timeline (synchronous).  Returns 0 (SPA_OK) or
 * SPA_ERR_HIP. */
int spa_timeline_clear(void);

/* Copy the first `bytes` bytes of the current device's timeline to host
 * memory `dst` (synchronous; bytes <= SPA_TIMELINE_WAVES * SPA_TIMELINE_SLOTS
 * * 8).  Returns 0, SPA_ERR_INVALID_ARGUMENT (null dst, too many bytes) or
 * SPA_ERR_HIP. */
int spa_timeline_read(uint64_t *dst, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* SPA_TIMELINE_H */
