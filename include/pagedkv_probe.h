/*
 * pagedkv_probe.h - a read-bandwidth probe shaped like the decode kernel's K/V
 * traffic, for placing that kernel against what the part delivers (a measuring
 * aid beside libpagedkv, built into libpagedkv_probe.so; not part of the paged
 * attention path).
 *
 * The decode gather reads, per step of a workgroup of eight wavefronts, one
 * 16-token tile slot of one block: the eight KV heads' 4 KiB slices of K (one
 * contiguous 32 KiB run) and the same of V, one 16-byte load per lane per KiB.
 * The probe reads the same pattern from two buffers of num_chunks 32 KiB chunks:
 * workgroup g (eight waves, wave h) visits chunks order[g * chunks_per_group + i]
 * for i < chunks_per_group, each wave reading its 4 KiB of the K and V chunk.
 *
 *   k, v       device, num_chunks * 32 KiB each, 16-B aligned
 *   order      device int32 [num_groups * chunks_per_group], chunk indices in
 *              [0, num_chunks) (identity runs = streaming, a permutation = gather);
 *              out-of-range entries read chunk 0
 *   sink       device uint32 [num_groups * 8]: an XOR of everything read (keeps
 *              the loads alive)
 *   nontemporal  1: loads bypass the caches' allocation (as decode's default)
 *   in_flight    1: a wave waits for its tile before requesting the next (as
 *                decode); 2: the next tile is requested before the current one
 *                is consumed
 * Returns 0 on success, 1 for invalid arguments, 5 for a launch failure.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t pa_probe_gather_read(const void* k, const void* v, int64_t num_chunks,
                             const int32_t* order, int32_t num_groups, int32_t chunks_per_group,
                             uint32_t* sink, int32_t nontemporal, int32_t in_flight,
                             void* stream);

/*
 * The same pattern (one tile in flight) through raw buffer loads whose cache-policy
 * bits are cache_policy: bit 0 sc0, bit 1 nt, bit 4 sc1 (gfx950's load policy
 * bits); one of 0, 1, 2, 3, 16, 17, 18, 19.  Each buffer must be under 2 GiB.
 * Returns 0, or 1 for invalid arguments, 5 for a launch failure.
 */
int32_t pa_probe_gather_read_policy(const void* k, const void* v, int64_t num_chunks,
                                    const int32_t* order, int32_t num_groups,
                                    int32_t chunks_per_group, uint32_t* sink,
                                    int32_t cache_policy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
