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

constexpr int64_t kMaxGrid = 65535;  // bound on head counts and tokens per grid axis

bool supported_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_bs(int32_t b) { return b == 8 || b == 16 || b == 32; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
// A tensor scale of an E4M3 cache: finite, positive, with a finite reciprocal.
bool valid_scale(float s) { return std::isfinite(s) && s > 0.0f && std::isfinite(1.0f / s); }

bool valid_partition(int32_t pt) {
  return pt == 0 || (pt >= pa::kTile && pt % pa::kTile == 0 &&
                     pt <= pa::kMaxTilesPerWave * pa::kTile);
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Upper bound on the 16-token tiles of one KV head over all sequences; with
// `skip` shared tiles, over the tiles past them.
int64_t tiles_cap(int64_t seqs, int64_t max_blocks, int64_t bs, int64_t skip = 0) {
  const int64_t per = (max_blocks * bs + pa::kTile - 1) / pa::kTile - skip;
  return seqs * (per > 0 ? per : 0);
}

// Wavefronts per KV head.  Enough that no wavefront gets more than
// kMaxTilesPerWave tiles even when every sequence is full; by default about
// kTargetWaves in total, otherwise enough that a wavefront holds at most
// partition_tokens tokens.  Never more than there can be tiles.
int64_t split_waves(int64_t seqs, int64_t kv_heads, int64_t max_blocks, int64_t bs,
                    int64_t pt, int64_t skip = 0) {
  const int64_t cap = tiles_cap(seqs, max_blocks, bs, skip);
  if (cap <= 0) return 1;
  const int64_t w_min = (cap + pa::kMaxTilesPerWave - 1) / pa::kMaxTilesPerWave;
  int64_t w = pt ? (cap * pa::kTile + pt - 1) / pt
                 : (pa::kTargetWaves + kv_heads - 1) / kv_heads;
  w = w < w_min ? w_min : w;
  return w < cap ? w : cap;
}

// Workspace layout: partial outputs fp32 [H][slots][D], then (m, l) fp32
// [H][slots][2], then the tile prefix int32 [seqs + 1]; slots = waves + seqs.
// With a shared prefix of `chunks` chunks, then its partials fp32
// [H][seqs][chunks][D] and their (m, l) [H][seqs][chunks][2].
struct WsLayout {
  int64_t o, ml, cu, sh_o, sh_ml, total;
};
WsLayout ws_layout(int64_t seqs, int64_t heads, int64_t dim, int64_t waves,
                   int64_t chunks = 0) {
  const int64_t slots = waves + seqs;
  WsLayout l;
  l.o = 0;
  l.ml = round_up(heads * slots * dim * 4, pa::kWorkspaceAlign);
  l.cu = l.ml + round_up(heads * slots * 2 * 4, pa::kWorkspaceAlign);
  l.sh_o = l.cu + round_up((seqs + 1) * 4, pa::kWorkspaceAlign);
  l.sh_ml = l.sh_o + round_up(heads * seqs * chunks * dim * 4, pa::kWorkspaceAlign);
  l.total = l.sh_ml + (chunks ? round_up(heads * seqs * chunks * 2 * 4, pa::kWorkspaceAlign) : 0);
  return l;
}

// The shared-prefix plan: `shared_blocks` leading table entries, whole
// 16-token tiles of them (a trailing half tile at block size 8 stays with
// the private tiles).  tiles == 0: no shared path.
pa::SharedPrefix shared_plan(int64_t seqs, int64_t heads, int64_t kv_heads,
                             int64_t shared_blocks, int64_t bs) {
  pa::SharedPrefix sh;
  sh.tiles = (int32_t)(shared_blocks * bs / pa::kTile);
  if (sh.tiles == 0 || seqs == 0) {
    sh.tiles = 0;
    return sh;
  }
  const int64_t g = heads / kv_heads;
  sh.chunk_tiles = pa::kSharedChunkTiles;
  sh.chunks = (sh.tiles + sh.chunk_tiles - 1) / sh.chunk_tiles;
  sh.seqs_per_group = (int32_t)(16 / g);
  const int64_t per_set = (int64_t)pa::kSharedGroups * sh.seqs_per_group;
  sh.colsets = (int32_t)((seqs + per_set - 1) / per_set);
  sh.waves = sh.chunks * sh.colsets;
  return sh;
}

bool decode_sizes_ok(int32_t num_seqs, int32_t num_kv_heads, int32_t num_heads,
                     int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size) {
  return num_seqs >= 0 && num_seqs <= pa::kMaxSeqs && num_kv_heads > 0 &&
         num_kv_heads <= kMaxGrid && num_heads > 0 && num_heads <= kMaxGrid &&
         num_heads % num_kv_heads == 0 && num_heads / num_kv_heads <= pa::kMaxGroup &&
         supported_dim(head_dim) && supported_bs(block_size) && max_blocks_per_seq > 0 &&
         (int64_t)max_blocks_per_seq * block_size <= INT32_MAX / 2 &&
         // the split pass keeps its tile prefix over all sequences in int32
         tiles_cap(num_seqs, max_blocks_per_seq, block_size) <= INT32_MAX;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return 9; }

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
    case PA_ERR_SCRATCH:
      return "the call needs more scratch than the library's fixed 16 MiB device array holds";
  }
  return "unknown error";
}

int32_t paged_attention_split_waves(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t partition_tokens) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      !supported_bs(block_size) || !valid_partition(partition_tokens) ||
      tiles_cap(num_seqs, max_blocks_per_seq, block_size) > INT32_MAX)
    return 0;
  const int64_t w = split_waves(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                partition_tokens);
  return w * num_kv_heads > INT32_MAX ? 0 : (int32_t)w;
}

size_t paged_attention_workspace_bytes_shared(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t shared_blocks,
                                              int32_t partition_tokens) {
  if (num_seqs <= 0 ||
      !decode_sizes_ok(num_seqs, num_kv_heads, num_heads, head_dim, max_blocks_per_seq,
                       block_size) ||
      !valid_partition(partition_tokens) || shared_blocks < 0 ||
      shared_blocks > max_blocks_per_seq)
    return 0;
  const pa::SharedPrefix sh = shared_plan(num_seqs, num_heads, num_kv_heads, shared_blocks,
                                          block_size);
  const int64_t w = split_waves(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                partition_tokens, sh.tiles);
  return (size_t)ws_layout(num_seqs, num_heads, head_dim, w, sh.chunks).total;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_tokens) {
  if (num_seqs <= 0 ||
      !decode_sizes_ok(num_seqs, num_kv_heads, num_heads, head_dim, max_blocks_per_seq,
                       block_size) ||
      !valid_partition(partition_tokens))
    return 0;
  const int64_t w = split_waves(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                partition_tokens);
  return (size_t)ws_layout(num_seqs, num_heads, head_dim, w).total;
}

static int kv_write_common(const void *k, const void *v, const int64_t *slot_mapping,
                           void *k_cache, void *v_cache, int64_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, int32_t dtype, int fp8, float k_scale,
                           float v_scale, void *stream) {
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_tokens > INT32_MAX || num_kv_heads <= 0 || num_kv_heads > kMaxGrid ||
      !supported_dim(head_dim) || !supported_bs(block_size) || num_blocks <= 0 ||
      num_blocks > INT64_MAX / ((int64_t)block_size * num_kv_heads * head_dim))
    return PA_ERR_SHAPE;
  if (fp8 && !(valid_scale(k_scale) && valid_scale(v_scale))) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  pa::WriteArgs a{k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, head_dim,
                  block_size, num_blocks, dtype, fp8, 1.0f / k_scale, 1.0f / v_scale, stream};
  return pa::launch_kv_write(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_kv_write(const void *k, const void *v, const int64_t *slot_mapping, void *k_cache,
                   void *v_cache, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t dtype, void *stream) {
  return kv_write_common(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads,
                         head_dim, block_size, num_blocks, dtype, 0, 1.0f, 1.0f, stream);
}

int paged_kv_write_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                       void *k_cache, void *v_cache, int64_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                       float k_scale, float v_scale, void *stream) {
  return kv_write_common(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads,
                         head_dim, block_size, num_blocks, dtype, 1, k_scale, v_scale, stream);
}

static int decode_common(void *out, const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens, float scale,
                         int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                         int32_t num_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int64_t num_blocks, int32_t dtype, int32_t partition_tokens,
                         void *workspace, size_t workspace_bytes, int32_t stages, int fp8,
                         float k_scale, float v_scale, void *stream, int append = 0,
                         const void *k_new = nullptr, const void *v_new = nullptr,
                         bool use_scratch = false, int32_t shared_blocks = 0) {
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (stages < 1 || stages > 3) return PA_ERR_SHAPE;
  if (fp8 && !(valid_scale(k_scale) && valid_scale(v_scale))) return PA_ERR_SHAPE;
  if (!decode_sizes_ok(num_seqs, num_kv_heads, num_heads, head_dim, max_blocks_per_seq,
                       block_size) ||
      num_blocks <= 0 || num_blocks > INT32_MAX || !std::isfinite(scale) ||
      !valid_partition(partition_tokens))
    return PA_ERR_SHAPE;
  if (shared_blocks < 0 || shared_blocks > max_blocks_per_seq) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  pa::SharedPrefix sh = shared_plan(num_seqs, num_heads, num_kv_heads, shared_blocks,
                                    block_size);
  const int64_t waves = split_waves(num_seqs, num_kv_heads, max_blocks_per_seq, block_size,
                                    partition_tokens, sh.tiles);
  if ((waves + sh.waves) * num_kv_heads > INT32_MAX || waves + num_seqs > INT32_MAX)
    return PA_ERR_SHAPE;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (append && (!k_new || !v_new)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 8) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      (append && (!aligned(k_new, 4) || !aligned(v_new, 4))))
    return PA_ERR_ALIGN;
  const WsLayout l = ws_layout(num_seqs, num_heads, head_dim, waves, sh.chunks);
  if (use_scratch) {  // the library's fixed per-GPU array, after every other check
    if ((size_t)l.total > pa::kScratchBytes) return PA_ERR_SCRATCH;
    if (pa::scratch_buffer(&workspace) != 0) return PA_ERR_LAUNCH;
    workspace_bytes = pa::kScratchBytes;
  }
  if (!workspace || workspace_bytes < (size_t)l.total) return PA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  char *ws = static_cast<char *>(workspace);
  pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                   num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq, num_blocks,
                   dtype, fp8, fp8 ? k_scale : 1.0f, fp8 ? v_scale : 1.0f,
                   (int32_t)waves, (int32_t)(waves + num_seqs),
                   reinterpret_cast<float *>(ws + l.o), reinterpret_cast<float *>(ws + l.ml),
                   reinterpret_cast<int32_t *>(ws + l.cu), stages, append, k_new, v_new,
                   fp8 ? 1.0f / k_scale : 1.0f, fp8 ? 1.0f / v_scale : 1.0f, stream};
  if (sh.tiles > 0) {
    sh.o = reinterpret_cast<float *>(ws + l.sh_o);
    sh.ml = reinterpret_cast<float *>(ws + l.sh_ml);
    a.sh = sh;
  }
  return pa::launch_decode(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attention_decode_append_stages(void *out, const void *q, const void *k_new,
                                         const void *v_new, void *k_cache, void *v_cache,
                                         const int32_t *block_tables,
                                         const int32_t *context_lens, float scale,
                                         float k_scale, float v_scale, int32_t block_size,
                                         int32_t num_kv_heads, int32_t num_seqs,
                                         int32_t num_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int64_t num_blocks,
                                         int32_t dtype, int32_t kv_fp8,
                                         int32_t partition_tokens, void *workspace,
                                         size_t workspace_bytes, int32_t stages, void *stream) {
  if (kv_fp8 != 0 && kv_fp8 != 1) return PA_ERR_DTYPE;
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                       num_blocks, dtype, partition_tokens, workspace, workspace_bytes, stages,
                       kv_fp8, k_scale, v_scale, stream, 1, k_new, v_new);
}

int paged_attention_decode_append(void *out, const void *q, const void *k_new,
                                  const void *v_new, void *k_cache, void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, float k_scale, float v_scale, int32_t block_size,
                                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, int32_t kv_fp8,
                                  int32_t partition_tokens, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  return paged_attention_decode_append_stages(out, q, k_new, v_new, k_cache, v_cache,
                                              block_tables, context_lens, scale, k_scale,
                                              v_scale, block_size, num_kv_heads, num_seqs,
                                              num_heads, head_dim, max_blocks_per_seq,
                                              num_blocks, dtype, kv_fp8, partition_tokens,
                                              workspace, workspace_bytes, 3, stream);
}

int paged_attention_decode_append_noalloc(void *out, const void *q, const void *k_new,
                                          const void *v_new, void *k_cache, void *v_cache,
                                          const int32_t *block_tables,
                                          const int32_t *context_lens, float scale,
                                          float k_scale, float v_scale, int32_t block_size,
                                          int32_t num_kv_heads, int32_t num_seqs,
                                          int32_t num_heads, int32_t head_dim,
                                          int32_t max_blocks_per_seq, int64_t num_blocks,
                                          int32_t dtype, int32_t kv_fp8,
                                          int32_t partition_tokens, void *stream) {
  if (kv_fp8 != 0 && kv_fp8 != 1) return PA_ERR_DTYPE;
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                       num_blocks, dtype, partition_tokens, nullptr, 0, 3, kv_fp8, k_scale,
                       v_scale, stream, 1, k_new, v_new, true);
}

int paged_attention_decode_shared(void *out, const void *q, const void *k_new,
                                  const void *v_new, void *k_cache, void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, float k_scale, float v_scale, int32_t block_size,
                                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, int32_t kv_fp8,
                                  int32_t shared_blocks, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, int32_t stages,
                                  void *stream) {
  if (kv_fp8 != 0 && kv_fp8 != 1) return PA_ERR_DTYPE;
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
  const int append = k_new != nullptr;
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                       num_blocks, dtype, partition_tokens, workspace, workspace_bytes, stages,
                       kv_fp8, k_scale, v_scale, stream, append, k_new, v_new, false,
                       shared_blocks);
}

int paged_attention_decode_stages(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, float scale, int32_t block_size,
                                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, int32_t stages,
                                  void *stream) {
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                       num_blocks, dtype, partition_tokens, workspace, workspace_bytes, stages,
                       0, 1.0f, 1.0f, stream);
}

int paged_attention_decode_fp8(void *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, float scale, float k_scale,
                               float v_scale, int32_t block_size, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                               int32_t partition_tokens, void *workspace,
                               size_t workspace_bytes, int32_t stages, void *stream) {
  return decode_common(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                       num_kv_heads, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                       num_blocks, dtype, partition_tokens, workspace, workspace_bytes, stages,
                       1, k_scale, v_scale, stream);
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

static int prefill_common(void *out, const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_tables, const int32_t *context_lens,
                          const int32_t *query_start, float scale, int32_t block_size,
                          int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                          int32_t head_dim, int32_t max_blocks_per_seq, int64_t num_blocks,
                          int32_t dtype, int32_t max_query_len, int kv_fp8, float k_scale,
                          float v_scale, void *stream) {
  if (dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (!decode_sizes_ok(num_seqs, num_kv_heads, num_heads, head_dim, max_blocks_per_seq,
                       block_size) ||
      num_blocks <= 0 || num_blocks > INT32_MAX || !std::isfinite(scale) || !(scale > 0.0f) ||
      max_query_len < 0 || (int64_t)max_query_len > (int64_t)max_blocks_per_seq * block_size ||
      max_blocks_per_seq > pa::kPrefillMaxBlocks)
    return PA_ERR_SHAPE;
  if (kv_fp8 && !(valid_scale(k_scale) && valid_scale(v_scale))) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 8) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  pa::PrefillArgs a{out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                    block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                    max_blocks_per_seq, num_blocks, dtype, max_query_len, kv_fp8,
                    kv_fp8 ? k_scale : 1.0f, kv_fp8 ? v_scale : 1.0f, stream};
  return pa::launch_prefill(a) == 0 ? PA_OK : PA_ERR_LAUNCH;
}

int paged_attention_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start, float scale, int32_t block_size,
                            int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                            int32_t head_dim, int32_t max_blocks_per_seq, int64_t num_blocks,
                            int32_t dtype, int32_t max_query_len, void *stream) {
  return prefill_common(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                        scale, block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                        max_blocks_per_seq, num_blocks, dtype, max_query_len, 0, 1.0f, 1.0f,
                        stream);
}

int paged_attention_prefill_fp8(void *out, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                const int32_t *context_lens, const int32_t *query_start,
                                float scale, float k_scale, float v_scale, int32_t block_size,
                                int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq,
                                int64_t num_blocks, int32_t dtype, int32_t max_query_len,
                                void *stream) {
  return prefill_common(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                        scale, block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                        max_blocks_per_seq, num_blocks, dtype, max_query_len, 1, k_scale,
                        v_scale, stream);
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

int paged_validate_shared_prefix(const int32_t *block_tables, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t shared_blocks, int32_t append) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || shared_blocks < 0 ||
      shared_blocks > max_blocks_per_seq)
    return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_NULL;
  const int64_t prefix = (int64_t)shared_blocks * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = context_lens[s];
    if (len < prefix || (append && shared_blocks > 0 && len <= prefix)) return PA_ERR_METADATA;
    for (int32_t i = 0; i < shared_blocks; ++i)
      if (block_tables[(int64_t)s * max_blocks_per_seq + i] != block_tables[i])
        return PA_ERR_METADATA;
  }
  return PA_OK;
}

int paged_validate_prefill(const int32_t *query_start, const int32_t *context_lens,
                           int32_t num_seqs, int32_t max_query_len, int64_t total_rows) {
  if (num_seqs < 0 || max_query_len < 0 || total_rows < 0) return PA_ERR_SHAPE;
  if (!query_start || (num_seqs > 0 && !context_lens)) return PA_ERR_NULL;
  if (query_start[0] != 0) return PA_ERR_METADATA;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)query_start[s + 1] - query_start[s];
    if (n < 0 || n > max_query_len || n > (int64_t)context_lens[s]) return PA_ERR_METADATA;
  }
  return (int64_t)query_start[num_seqs] <= total_rows ? PA_OK : PA_ERR_METADATA;
}

}  // extern "C"
