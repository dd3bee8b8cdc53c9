/*
 * dopt_vmm.h -- device-memory placement helpers for the arenas of the
 * shard-local AdamW step on AMD Instinct MI355X (gfx950).
 *
 * The step library (dopt.h) never allocates; these calls are the optional
 * allocator a caller may use for the arena arrays.  They are thin wrappers
 * over the HIP virtual-memory API: an arena array is a reserved virtual
 * address range whose pieces ("regions") are each backed by their own
 * physical allocation, so the backing of one region can be replaced without
 * moving the array or touching the others.
 *
 * Why: the second pass of the step reads and writes five arrays at the same
 * index at once, and on MI355X how fast their writes drain depends on where
 * their physical pages sit relative to each other (five plain write streams
 * ran at 5.5 TB/s on ordinary allocations and 7.2 TB/s on others; the step's
 * pass 2 at 5.1 and 6.1 TB/s).  The property cannot be read from user space,
 * but it can be measured: a caller times pass 2 on one region with candidate
 * backings and keeps the fastest, region by region, which needs one spare
 * region of memory instead of a second copy of the whole state.
 *
 * Conventions as in dopt.h: 0 on success or a negative DOPT_ERR_* code with
 * dopt_last_error() set; DOPT_ERR_HIP names the failing HIP call.  Handles are
 * opaque 64-bit values.  Sizes and offsets must be multiples of
 * dopt_vmm_granularity().  Unmapping or releasing memory that queued device
 * work still uses is the caller's error: synchronize first.
 */
#ifndef DOPT_VMM_H
#define DOPT_VMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Allocation granularity (bytes) of physical device memory on `device`. */
int dopt_vmm_granularity(int32_t device, size_t *out);

/* Reserve `bytes` of device virtual address space, aligned to `align`
 * (0: the granularity); *va receives its start.  Nothing is backed yet. */
int dopt_vmm_reserve(size_t bytes, size_t align, uint64_t *va);

/* Return a reservation made by dopt_vmm_reserve (every mapping in it must
 * have been unmapped). */
int dopt_vmm_free(uint64_t va, size_t bytes);

/* Allocate `bytes` of physical memory on `device`; *handle receives it. */
int dopt_vmm_create(int32_t device, size_t bytes, uint64_t *handle);

/* Map the whole of `handle` (of `bytes` bytes) at va. */
int dopt_vmm_map(uint64_t va, size_t bytes, uint64_t handle);

/* Give `device` read-write access to [va, va + bytes), every byte of which is
 * mapped.  Call it once over a whole reservation after its first mappings,
 * and again over a range after mapping other memory there. */
int dopt_vmm_set_access(uint64_t va, size_t bytes, int32_t device);

/* Unmap [va, va + bytes) (a range mapped by dopt_vmm_map). */
int dopt_vmm_unmap(uint64_t va, size_t bytes);

/* Free physical memory made by dopt_vmm_create (unmapped everywhere). */
int dopt_vmm_release(uint64_t handle);

#ifdef __cplusplus
}
#endif
#endif
