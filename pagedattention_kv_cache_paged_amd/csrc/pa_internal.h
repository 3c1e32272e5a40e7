// Internal interface between the C ABI (pa_api.cpp) and the kernel launchers.
// Arguments have been validated by the caller; launchers only enqueue.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kTile = 16;           // tokens per MFMA tile
constexpr int kWave = 64;           // gfx950 wavefront
constexpr int kMaxGroup = 16;       // query heads per KV head served by one wave
constexpr int kWorkspaceAlign = 256;
constexpr int kMaxTilesPerWave = 64; // one tile per lane of the wave's tile map
constexpr int kTargetWaves = 1024;   // default split: one wave per SIMD of 256 CUs
constexpr int kMaxSeqs = 8192;       // tile prefix and lengths live in LDS
constexpr int kPrefillMaxBlocks = 4096;  // prefill keeps a sequence's block ids in LDS
// Device scratch of the no-allocation decode step: a fixed array in the
// library's code object, one per GPU, held until the process ends.
constexpr size_t kScratchBytes = (size_t)16 << 20;

// A prefix shared by every sequence of the batch: the first `tiles` 16-token
// tiles of every sequence are the same blocks (sequence 0's table entries).
// The split pass then gives that prefix to wavefronts of its own, each taking
// `chunk_tiles` tiles of it for the query heads of several sequences at once
// (kSharedGroups groups of 16 MFMA columns: seqs_per_group sequences of G
// heads per group), and splits only the tiles past the prefix the usual way.
constexpr int kSharedGroups = 2;       // 16-column MFMA groups per shared wavefront
constexpr int kSharedChunkTiles = 32;  // prefix tiles per shared wavefront, at most
struct SharedPrefix {
  int32_t tiles = 0;           // shared tiles per sequence (0: no shared path)
  int32_t chunk_tiles = 0;
  int32_t chunks = 0;          // ceil(tiles / chunk_tiles)
  int32_t seqs_per_group = 0;  // 16 / G
  int32_t colsets = 0;         // wavefronts per chunk and KV head
  int32_t waves = 0;           // shared wavefronts per KV head: chunks * colsets
  float *o = nullptr;          // [num_heads][num_seqs][chunks][head_dim]
  float *ml = nullptr;         // [num_heads][num_seqs][chunks][2]
};

struct DecodeArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float scale;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t dtype;
  int32_t kv_fp8;      // 1: caches hold E4M3 codes (k_scale, v_scale apply)
  float k_scale;       // K element = code * k_scale (1 for 16-bit caches)
  float v_scale;       // V element = code * v_scale (1 for 16-bit caches)
  int32_t waves;       // wavefronts per KV head (equal shares of the flat tile list)
  int32_t slots;       // partial-result slots per query head: waves + num_seqs
  float *ws_o;         // [num_heads][slots][head_dim]
  float *ws_ml;        // [num_heads][slots][2]  (running max in log2 units, sum)
  int32_t *ws_cu;      // [num_seqs + 1] tile prefix, written by the split pass
  int32_t stages;      // bit 0: split pass, bit 1: merge pass
  // Fused append: the new token of each sequence (k_new, v_new [num_seqs,
  // num_kv_heads, head_dim], the q dtype) is context position L-1.  The
  // split pass's wavefront holding that position takes the token's K and V
  // from these rows instead of the cache and stores them into its slot.
  int32_t append;
  const void *k_new;
  const void *v_new;
  float k_inv;         // float32(1 / k_scale): E4M3 quantisation of k_new
  float v_inv;
  void *stream;
  SharedPrefix sh;     // tiles == 0: no shared prefix
};

struct WriteArgs {
  const void *k;
  const void *v;
  const int64_t *slot_mapping;
  void *k_cache;
  void *v_cache;
  int64_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
  int32_t dtype;       // k, v element type (PA_F16 / PA_BF16)
  int32_t fp8;         // 1: quantise into E4M3 caches with k_inv / v_inv
  float k_inv;         // float32(1 / k_scale)
  float v_inv;         // float32(1 / v_scale)
  void *stream;
};

struct CopyArgs {
  void *dst_k;
  void *dst_v;
  const void *src_k;
  const void *src_v;
  const int64_t *pairs;  // device-visible [num_pairs][2] (src, dst)
  int64_t num_pairs;
  int64_t run_bytes;     // bytes of one block of one cache (a multiple of 16)
  int64_t src_blocks;
  int64_t dst_blocks;
  void *stream;
};

struct PrefillArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;  // [num_seqs + 1] chunk row offsets
  float scale;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t dtype;
  int32_t max_query_len;        // bound on any sequence's chunk length (grid size)
  int32_t kv_fp8;               // 1: caches hold E4M3 codes (k_scale, v_scale apply)
  float k_scale;
  float v_scale;
  void *stream;
};

// Return 0 on success, a nonzero HIP error code otherwise.
int launch_decode(const DecodeArgs &a);
// Device address of the current GPU's kScratchBytes scratch array (looked
// up once per device, then cached).
int scratch_buffer(void **ptr);
int launch_kv_write(const WriteArgs &a);
int launch_copy_blocks(const CopyArgs &a);
int launch_prefill(const PrefillArgs &a);

}  // namespace pa
