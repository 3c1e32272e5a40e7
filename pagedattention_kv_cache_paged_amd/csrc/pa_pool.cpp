// Host side of block-level memory management: the reference-counted block
// pool and the argument checks of the block copy (include/paged_blocks.h).
#include <mutex>
#include <vector>

#include "paged_attn.h"
#include "paged_blocks.h"
#include "pa_internal.h"

struct pa_block_pool {
  std::vector<int64_t> free_stack;  // back() is taken next
  std::vector<int32_t> refcount;    // 0: free
  mutable std::mutex mu;
};

namespace {

bool in_pool(const pa_block_pool *p, int64_t b) {
  return b >= 0 && b < (int64_t)p->refcount.size();
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

int pa_pool_create(int64_t num_blocks, const int64_t *order, pa_block_pool **pool) {
  if (!pool) return PA_ERR_NULL;
  *pool = nullptr;
  if (num_blocks <= 0 || num_blocks > ((int64_t)1 << 40)) return PA_ERR_SHAPE;
  auto *p = new pa_block_pool;
  p->refcount.assign((size_t)num_blocks, 0);
  p->free_stack.resize((size_t)num_blocks);
  std::vector<uint8_t> seen((size_t)num_blocks, 0);
  for (int64_t i = 0; i < num_blocks; ++i) {
    const int64_t b = order ? order[i] : i;
    if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
      delete p;
      return PA_ERR_SHAPE;
    }
    seen[(size_t)b] = 1;
    p->free_stack[(size_t)(num_blocks - 1 - i)] = b;  // order[0] on top
  }
  *pool = p;
  return PA_OK;
}

void pa_pool_destroy(pa_block_pool *pool) { delete pool; }

int64_t pa_pool_num_blocks(const pa_block_pool *pool) {
  return pool ? (int64_t)pool->refcount.size() : 0;
}

int64_t pa_pool_num_free(const pa_block_pool *pool) {
  if (!pool) return 0;
  std::lock_guard<std::mutex> g(pool->mu);
  return (int64_t)pool->free_stack.size();
}

int64_t pa_pool_alloc(pa_block_pool *pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> g(pool->mu);
  if (pool->free_stack.empty()) return -1;
  const int64_t b = pool->free_stack.back();
  pool->free_stack.pop_back();
  pool->refcount[(size_t)b] = 1;
  return b;
}

int pa_pool_incref(pa_block_pool *pool, int64_t block) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!in_pool(pool, block) || pool->refcount[(size_t)block] <= 0) return PA_ERR_METADATA;
  if (pool->refcount[(size_t)block] == INT32_MAX) return PA_ERR_METADATA;
  ++pool->refcount[(size_t)block];
  return PA_OK;
}

int pa_pool_decref(pa_block_pool *pool, int64_t block) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!in_pool(pool, block) || pool->refcount[(size_t)block] <= 0) return PA_ERR_METADATA;
  if (--pool->refcount[(size_t)block] == 0) pool->free_stack.push_back(block);
  return PA_OK;
}

int32_t pa_pool_refcount(const pa_block_pool *pool, int64_t block) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> g(pool->mu);
  return in_pool(pool, block) ? pool->refcount[(size_t)block] : -1;
}

int pa_pool_cow(pa_block_pool *pool, int64_t block, int64_t *dst, int32_t *copy) {
  if (!pool || !dst || !copy) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!in_pool(pool, block) || pool->refcount[(size_t)block] <= 0) return PA_ERR_METADATA;
  if (pool->refcount[(size_t)block] == 1) {
    *dst = block;
    *copy = 0;
    return PA_OK;
  }
  if (pool->free_stack.empty()) return PA_ERR_WORKSPACE;
  const int64_t fresh = pool->free_stack.back();
  pool->free_stack.pop_back();
  pool->refcount[(size_t)fresh] = 1;
  --pool->refcount[(size_t)block];  // still >= 1: others keep sharing it
  *dst = fresh;
  *copy = 1;
  return PA_OK;
}

int paged_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t elem_bytes, void *stream) {
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
      (head_dim != 64 && head_dim != 128) ||
      (block_size != 8 && block_size != 16 && block_size != 32) || num_blocks <= 0)
    return PA_ERR_SHAPE;
  const int64_t run = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes;
  if (num_blocks > INT64_MAX / run) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pairs, 8))
    return PA_ERR_ALIGN;
  pa::CopyArgs a{k_cache, v_cache, k_cache, v_cache, pairs, num_pairs, run, num_blocks,
                 num_blocks, stream};
  return pa::launch_copy_blocks(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_swap_blocks(void *dst_k_cache, void *dst_v_cache, int64_t dst_num_blocks,
                      const void *src_k_cache, const void *src_v_cache, int64_t src_num_blocks,
                      const int64_t *pairs, int64_t num_pairs, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t elem_bytes, void *stream) {
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
      (head_dim != 64 && head_dim != 128) ||
      (block_size != 8 && block_size != 16 && block_size != 32) || dst_num_blocks <= 0 ||
      src_num_blocks <= 0)
    return PA_ERR_SHAPE;
  const int64_t run = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes;
  if (dst_num_blocks > INT64_MAX / run || src_num_blocks > INT64_MAX / run) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k_cache || !dst_v_cache || !src_k_cache || !src_v_cache || !pairs) return PA_ERR_NULL;
  if (!aligned(dst_k_cache, 16) || !aligned(dst_v_cache, 16) || !aligned(src_k_cache, 16) ||
      !aligned(src_v_cache, 16) || !aligned(pairs, 8))
    return PA_ERR_ALIGN;
  pa::CopyArgs a{dst_k_cache, dst_v_cache, src_k_cache, src_v_cache, pairs, num_pairs, run,
                 src_num_blocks, dst_num_blocks, stream};
  return pa::launch_copy_blocks(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_validate_swap_pairs(const int64_t *pairs, int64_t num_pairs, int64_t src_num_blocks,
                              int64_t dst_num_blocks) {
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0) return PA_ERR_SHAPE;
  if (num_pairs > 0 && !pairs) return PA_ERR_NULL;
  std::vector<uint8_t> is_dst((size_t)dst_num_blocks, 0);
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s >= src_num_blocks || d >= dst_num_blocks) return PA_ERR_METADATA;
    if (s < 0 || d < 0) continue;
    if (is_dst[(size_t)d]) return PA_ERR_METADATA;
    is_dst[(size_t)d] = 1;
  }
  return PA_OK;
}

int paged_validate_copy_pairs(const int64_t *pairs, int64_t num_pairs, int64_t num_blocks) {
  if (num_pairs < 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (num_pairs > 0 && !pairs) return PA_ERR_NULL;
  std::vector<uint8_t> is_dst((size_t)num_blocks, 0), is_src((size_t)num_blocks, 0);
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s >= num_blocks || d >= num_blocks) return PA_ERR_METADATA;
    if (s < 0 || d < 0) continue;  // skipped pair
    if (is_dst[(size_t)d]) return PA_ERR_METADATA;
    is_dst[(size_t)d] = 1;
    is_src[(size_t)s] = 1;
  }
  for (int64_t b = 0; b < num_blocks; ++b)
    if (is_dst[(size_t)b] && is_src[(size_t)b]) return PA_ERR_METADATA;
  return PA_OK;
}

}  // extern "C"
