// C ABI of the paged attention library: host-side validation, workspace
// sizing and dispatch to the gfx950 kernels.  Declarations and contracts are
// in include/paged_attn.h.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "paged_attn.h"
#include "pa_internal.h"

namespace {

constexpr int64_t kMaxGrid = 65535;  // bound kept for grid y / z

bool supported_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_bs(int32_t b) { return b == 8 || b == 16 || b == 32; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_partition(int32_t pt, int32_t bs) {
  return pt >= pa::kTile && pt % pa::kTile == 0 && pt % bs == 0 && pt <= pa::kWave * bs;
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t max_parts_of(int32_t max_blocks, int32_t bs, int32_t pt) {
  const int64_t cap = (int64_t)max_blocks * bs;
  return (cap + pt - 1) / pt;
}

// Workspace layout: partial outputs fp32 [B][H][P][D], then (m, l) fp32 [B][H][P][2].
size_t ws_bytes(int64_t seqs, int64_t heads, int64_t dim, int64_t parts) {
  if (parts <= 1 || seqs <= 0) return 0;
  const int64_t o = round_up(seqs * heads * parts * dim * 4, pa::kWorkspaceAlign);
  return (size_t)(o + seqs * heads * parts * 2 * 4);
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return 1; }

const char *pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is null";
    case PA_ERR_DTYPE: return "unsupported dtype (expected PA_F16 or PA_BF16)";
    case PA_ERR_SHAPE: return "unsupported or inconsistent size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_METADATA: return "invalid block table, context length or slot";
    case PA_ERR_ALIGN: return "pointer not aligned as required";
  }
  return "unknown error";
}

int32_t paged_attention_default_partition(int32_t max_blocks_per_seq, int32_t block_size) {
  if (!supported_bs(block_size) || max_blocks_per_seq <= 0) return 0;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  const int64_t unit = block_size > pa::kTile ? block_size : pa::kTile;
  if (cap <= 512) return (int32_t)round_up(cap, unit);  // whole context in one partition
  return 256;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_tokens) {
  if (num_seqs <= 0 || num_heads <= 0 || !supported_dim(head_dim) || !supported_bs(block_size) ||
      max_blocks_per_seq <= 0)
    return 0;
  int32_t pt = partition_tokens ? partition_tokens
                                : paged_attention_default_partition(max_blocks_per_seq, block_size);
  if (!valid_partition(pt, block_size)) return 0;
  return ws_bytes(num_seqs, num_heads, head_dim, max_parts_of(max_blocks_per_seq, block_size, pt));
}

int paged_kv_write(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                   void *v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t dtype, void *stream) {
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_tokens > INT32_MAX || num_kv_heads <= 0 || num_kv_heads > kMaxGrid ||
      !supported_dim(head_dim) || !supported_bs(block_size) || num_blocks <= 0 ||
      num_blocks > INT64_MAX / ((int64_t)block_size * num_kv_heads * head_dim))
    return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  pa::WriteArgs a{k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, head_dim,
                  block_size, num_blocks, stream};
  return pa::launch_kv_write(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attention_decode_stages(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, float scale, int32_t block_size,
                                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, int32_t stages,
                                  void *stream) {
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (stages < 1 || stages > 3) return PA_ERR_SHAPE;
  if (num_seqs < 0 || num_seqs > kMaxGrid || num_kv_heads <= 0 || num_kv_heads > kMaxGrid ||
      num_heads <= 0 || num_heads > kMaxGrid || num_heads % num_kv_heads != 0 ||
      num_heads / num_kv_heads > pa::kMaxGroup || !supported_dim(head_dim) ||
      !supported_bs(block_size) || max_blocks_per_seq <= 0 ||
      (int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2 || num_blocks <= 0 ||
      num_blocks > INT32_MAX || !std::isfinite(scale))
    return PA_ERR_SHAPE;
  const int32_t pt = partition_tokens
                         ? partition_tokens
                         : paged_attention_default_partition(max_blocks_per_seq, block_size);
  if (!valid_partition(pt, block_size)) return PA_ERR_SHAPE;
  const int64_t parts = max_parts_of(max_blocks_per_seq, block_size, pt);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 8) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  const size_t need = ws_bytes(num_seqs, num_heads, head_dim, parts);
  float *ws_o = nullptr, *ws_ml = nullptr;
  if (need) {
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
    ws_o = static_cast<float *>(workspace);
    ws_ml = reinterpret_cast<float *>(
        static_cast<char *>(workspace) +
        round_up((int64_t)num_seqs * num_heads * parts * head_dim * 4, pa::kWorkspaceAlign));
  }
  pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                   num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq, num_blocks,
                   dtype, pt, (int32_t)parts, ws_o, ws_ml, stages, stream};
  return pa::launch_decode(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attention_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              float scale, int32_t block_size, int32_t num_kv_heads,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                              int32_t partition_tokens, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return paged_attention_decode_stages(out, q, k_cache, v_cache, block_tables, context_lens,
                                       scale, block_size, num_kv_heads, num_seqs, num_heads,
                                       head_dim, max_blocks_per_seq, num_blocks, dtype,
                                       partition_tokens, workspace, workspace_bytes, 3, stream);
}

int paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                           int32_t num_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int64_t num_blocks, int32_t dtype, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return paged_attention_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                                   max_blocks_per_seq, num_blocks, dtype, 0, workspace,
                                   workspace_bytes, stream);
}

int paged_validate_metadata(const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                            int64_t num_blocks, const int64_t *slot_mapping, int64_t num_tokens) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_NULL;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = context_lens[s];
    if (len < 0 || len > cap) return PA_ERR_METADATA;
    const int64_t used = (len + block_size - 1) / block_size;
    for (int64_t i = 0; i < used; ++i) {
      const int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + i];
      if (b < 0 || b >= num_blocks) return PA_ERR_METADATA;
    }
  }
  if (slot_mapping && num_tokens > 0) {
    const int64_t slots = num_blocks * block_size;
    std::vector<uint8_t> seen((size_t)slots, 0);
    for (int64_t i = 0; i < num_tokens; ++i) {
      const int64_t sl = slot_mapping[i];
      if (sl < 0) continue;
      if (sl >= slots || seen[(size_t)sl]) return PA_ERR_METADATA;
      seen[(size_t)sl] = 1;
    }
  }
  return PA_OK;
}

}  // extern "C"
