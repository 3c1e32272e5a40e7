/*
 * Block-level memory management for the paged KV cache on MI355X (gfx950):
 * a reference-counted pool of physical block ids on the host, and the
 * copy-on-write block copy on the device.
 *
 * "vLLM framework analysis: how PagedAttention achieves a 20x LLM inference
 * speed-up" (intelliparadigm.com), 2.3: requests with the same prefix point
 * at the same physical blocks, a reference count tracks the sharers, a block
 * returns to the free pool when its count reaches zero, and a write into a
 * shared block goes to a private copy first (copy-on-write).  "vLLM memory
 * management and continuous batching from the source" (developer.cloud.
 * tencent.cn), part 2, 2.1-2.2: the physical blocks are a fixed pool handed
 * out on demand as sequences grow.  "vLLM core architecture overview"
 * (5688vip.com), 4.2: preempted requests' KV moves to CPU memory.
 *
 * Return codes are those of paged_attn.h (PA_OK, PA_ERR_*).
 */
#ifndef PAGED_BLOCKS_H
#define PAGED_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- reference-counted block pool (host memory only) ---------------------
 *
 * A pool owns the ids 0 .. num_blocks-1 of one pair of KV caches.  Free ids
 * form a stack: pa_pool_alloc takes the most recently freed id, and at
 * creation the stack holds `order` (a permutation of the ids, or NULL for
 * 0, 1, 2, ...) so that order[0] is taken first.  Every call on one pool is
 * serialised by the pool's own lock, so a pool may be shared by threads.
 * Misuse (an id outside the pool, a reference to a free block) returns
 * PA_ERR_METADATA and changes nothing.
 */
typedef struct pa_block_pool pa_block_pool;

/* Create a pool; *pool receives the handle (release it with
 * pa_pool_destroy).  PA_ERR_SHAPE if num_blocks <= 0 or order is not a
 * permutation of 0 .. num_blocks-1; PA_ERR_NULL if pool is NULL. */
int pa_pool_create(int64_t num_blocks, const int64_t *order, pa_block_pool **pool);
void pa_pool_destroy(pa_block_pool *pool);

int64_t pa_pool_num_blocks(const pa_block_pool *pool);
int64_t pa_pool_num_free(const pa_block_pool *pool);

/* Take a free block with reference count 1.  Returns its id, or -1 when
 * the pool is exhausted (or pool is NULL). */
int64_t pa_pool_alloc(pa_block_pool *pool);

/* One more sharer of an allocated block (a fork of a sequence). */
int pa_pool_incref(pa_block_pool *pool, int64_t block);

/* One sharer fewer; at zero the block goes back on the free stack. */
int pa_pool_decref(pa_block_pool *pool, int64_t block);

/* Reference count of a block (0 when free), or -1 for an id outside the
 * pool. */
int32_t pa_pool_refcount(const pa_block_pool *pool, int64_t block);

/* Copy-on-write decision before a sequence writes into `block`: if the
 * block is shared (count > 1), take a fresh block, drop this sequence's
 * reference to the shared one, and return *dst = the fresh id with
 * *copy = 1; the caller then copies block -> *dst (paged_copy_blocks) and
 * points its table at *dst.  A private block (count 1) gives *dst = block,
 * *copy = 0.  PA_ERR_WORKSPACE when a copy is needed and the pool is empty
 * (nothing changes); PA_ERR_METADATA for a free or out-of-pool block. */
int pa_pool_cow(pa_block_pool *pool, int64_t block, int64_t *dst, int32_t *copy);

/* ---- block copy on the device ---------------------------------------------
 *
 * For every pair i < num_pairs whose two ids are in [0, num_blocks), block
 * pairs[2i+1] of both caches becomes a bit copy of block pairs[2i]: all KV
 * heads, K and V (in the layouts of paged_attn.h a block of either cache is
 * one contiguous run of num_kv_heads * block_size * head_dim elements).
 * Pairs with an id outside the pool (e.g. -1 padding) are skipped.
 *   pairs: device int64 [num_pairs][2] (src, dst), 8-byte aligned.
 *   elem_bytes: 2 for fp16 / bf16 caches, 1 for E4M3 caches.
 *   caches: 16-byte aligned.
 * The copies run concurrently: destinations must be distinct and no
 * destination may be a source in the same call (paged_validate_copy_pairs
 * checks this on a host copy).  Asynchronous on `stream`; PA_OK means
 * enqueued.  num_pairs = 0 is a no-op.
 */
int paged_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t elem_bytes, void *stream);

/* Host check of copy pairs (host pointer): ids in range or negative
 * (skipped), destinations distinct, no destination also a source.
 * PA_OK or PA_ERR_METADATA. */
int paged_validate_copy_pairs(const int64_t *pairs, int64_t num_pairs, int64_t num_blocks);

/* ---- block swap between the device pool and a host pool -------------------
 *
 * "vLLM core architecture overview: PagedAttention, Continuous Batching,
 * distributed inference" (5688vip.com), 4.2: when GPU memory runs short, a
 * low-priority request is preempted and its KV blocks are moved out to CPU
 * memory (and brought back when it resumes).  The host pool has the layouts
 * of the device caches (paged_attn.h) with its own block count; allocate it
 * as pinned memory (hipHostMalloc, or torch's pin_memory=True), which the
 * kernel reads and writes directly through its device mapping.
 *
 * For every pair i < num_pairs with src = pairs[2i] in [0, src_num_blocks)
 * and dst = pairs[2i+1] in [0, dst_num_blocks), block dst of the destination
 * pool (both caches) becomes a bit copy of block src of the source pool.
 * Swap-out: source = device caches, destination = host pool; swap-in: the
 * other way round.  Pairs with an id outside its pool are skipped.
 *   pairs: int64 [num_pairs][2], readable by the device (device or pinned
 *   host memory), 8-byte aligned; caches and pools 16-byte aligned;
 *   elem_bytes 2 (fp16 / bf16) or 1 (E4M3).
 * The two pools must not overlap (within one pool use paged_copy_blocks)
 * and destinations must be distinct (paged_validate_swap_pairs checks a
 * host copy).  Asynchronous on `stream`: the host pool may be read only
 * after the stream has been synchronised.  num_pairs = 0 is a no-op.
 */
int paged_swap_blocks(void *dst_k_cache, void *dst_v_cache, int64_t dst_num_blocks,
                      const void *src_k_cache, const void *src_v_cache, int64_t src_num_blocks,
                      const int64_t *pairs, int64_t num_pairs, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t elem_bytes, void *stream);

/* Host check of swap pairs: ids below their pool's size or negative,
 * destinations distinct.  PA_OK or PA_ERR_METADATA. */
int paged_validate_swap_pairs(const int64_t *pairs, int64_t num_pairs, int64_t src_num_blocks,
                              int64_t dst_num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_BLOCKS_H */
