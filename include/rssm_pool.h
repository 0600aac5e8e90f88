/*
 * rssm_pool.h -- C ABI of librssm_pool: physically contiguous device memory
 * for the state pools of librssm_materialize (MI355X, gfx950).
 *
 * Not an operation of the pages and not part of the operation's boundary
 * (rssm_materialize.h): a placement helper, built as a library of its own so
 * that librssm_materialize exports nothing that allocates, for the pools that the
 * materialize, commit and decode kernels stream (tens of GiB per layer set),
 * used by the benchmark and the tests to place their pools.  The operation
 * entry points accept any device memory and allocate nothing themselves; only
 * these helpers allocate.
 * Measured on MI355X, a plain hipMalloc of a large pool in the first process
 * on a box can land on physical memory that streams markedly slower than a
 * physically contiguous allocation: a 20 GiB device copy ran at 4.7 TB/s
 * against 5.7 TB/s, and the 48-layer bf16 materialize at 19.4 ms (67-68% of
 * the 8 TB/s HBM peak) against 16.9-17.2 ms (76-78%): the 70% roofline
 * fraction of that workload holds with contiguous pools, not with plain
 * allocations in the first process on such a machine.  These entry points allocate with
 * hipDeviceMallocContiguous and
 * fall back to hipMalloc when the device has no contiguous range that large.
 *
 * Plain C types only.  The memory belongs to the caller until freed with
 * rssm_pool_free; the kernels' entry points themselves still allocate nothing.
 */
#ifndef RSSM_POOL_H
#define RSSM_POOL_H

#include <stdint.h>
#include <sys/types.h>

#include "rssm_materialize.h" /* rssm_status */

#ifdef __cplusplus
extern "C" {
#endif

/* Allocate `bytes` (> 0) of device memory on the current device.  *out gets
 * the address; *contiguous (if not NULL) gets 1 when the memory is physically
 * contiguous, 0 when it came from the plain fallback.  Returns
 * RSSM_ERR_INVALID_ARGUMENT for out == NULL or bytes == 0 (before any HIP
 * call), RSSM_ERR_HIP when both allocations fail.  The memory is not
 * initialised. */
rssm_status rssm_pool_alloc(uint64_t bytes, void **out, int32_t *contiguous);

/* Wait for the device to finish its work, then free memory from
 * rssm_pool_alloc (NULL is a no-op). */
rssm_status rssm_pool_free(void *ptr);

/* The same pair with the signatures of a torch pluggable allocator
 * (torch.cuda.memory.CUDAPluggableAllocator): allocate on `device`
 * (returning NULL on failure), and free.  `stream` is unused: every free
 * waits for the device. */
void *rssm_torch_pool_alloc(ssize_t bytes, int device, void *stream);
void rssm_torch_pool_free(void *ptr, ssize_t bytes, int device, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RSSM_POOL_H */
