/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged decode attention library.
 *
 * The problem these calls solve is the paged KV cache of PagedAttention:
 *
 *   - "vLLM core architecture overview: PagedAttention, Continuous Batching,
 *     distributed inference" (5688vip.com), 4.1: the KV cache is cut into
 *     fixed-size physical blocks (16 tokens by default, 8 or 32 as options);
 *     a sequence's logically contiguous KV may sit in non-contiguous blocks,
 *     mapped through a block table; requests may share prefix blocks.
 *   - "vLLM memory management and continuous batching from the source"
 *     (developer.cloud.tencent.cn), part 2, 2.1: appending a token writes its
 *     K/V at its block's address plus the offset inside the block; 2.3:
 *     attention takes the list of physical block numbers instead of a
 *     contiguous (batch, seq_len, dim) tensor and gathers K/V through it.
 *
 * All buffers are owned by the caller; the library never allocates or frees
 * memory.  Device pointers are HIP device (or managed) memory of the current
 * device; `stream` is a hipStream_t passed as void* (NULL = null stream).
 * Every call validates its arguments on the host before launching anything;
 * on error nothing is enqueued and no memory is touched.  A return of PA_OK
 * means the work was enqueued on `stream` (the calls are asynchronous).
 * The library may be called from several threads.  Its only state is the
 * fixed per-GPU scratch array of paged_attention_decode_append_noalloc and
 * that array's device address, looked up once per device under a lock.
 *
 * Element type: q, k, v, both caches and out share one 16-bit type, IEEE
 * binary16 (PA_F16) or bfloat16 (PA_BF16); arithmetic is fp32.
 *
 * Layouts (row-major, contiguous):
 *   q, out          [num_seqs][num_heads][head_dim]
 *   k, v (new)      [num_tokens][num_kv_heads][head_dim]
 *   k_cache         [num_blocks][num_kv_heads][block_size][head_dim]  token-major
 *   v_cache         [num_blocks][num_kv_heads][block_size/4][head_dim][4]
 *                   positions in groups of four; within a group the four
 *                   positions of one dimension are adjacent (8 bytes, the
 *                   P.V matrix-core operand of one lane), and one position's
 *                   head_dim values lie in one run of 4 * head_dim elements
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]
 *   context_lens    int32 [num_seqs]   (tokens to attend over, the new one included)
 *   slot_mapping    int64 [num_tokens] slot = block * block_size + offset; < 0 = skip
 * Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Supported: head_dim 64 or 128; block_size 8, 16 or 32;
 * num_heads / num_kv_heads (the GQA group) from 1 to 16.
 * Alignment: q, k, v and caches 16 bytes, out 8 bytes, workspace 16 bytes.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,      /* a required pointer is NULL */
  PA_ERR_DTYPE = -2,     /* dtype is not PA_F16 / PA_BF16 */
  PA_ERR_SHAPE = -3,     /* unsupported or inconsistent size */
  PA_ERR_WORKSPACE = -4, /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -5,    /* the HIP runtime refused a launch */
  PA_ERR_METADATA = -6,  /* (validator) bad block table, length or slot */
  PA_ERR_ALIGN = -7,     /* a pointer is not aligned as required */
  PA_ERR_SCRATCH = -8    /* (no-allocation call) needs more than the fixed scratch */
};

/* Version of this ABI; bumped on any incompatible change (7: the V cache
 * layout became [num_blocks][num_kv_heads][block_size/4][head_dim][4];
 * 8: paged_attention_decode_append_stages; 9: the shared-prefix decode). */
int pa_abi_version(void);

/* Text for a return code (static storage). */
const char *pa_strerror(int code);

/*
 * KV append ("...from the source", part 2, 2.1): for every token i with
 * 0 <= slot_mapping[i] < num_blocks * block_size, copies k[i][j][:] and
 * v[i][j][:] bit for bit into block slot/block_size, offset
 * slot%block_size, of KV head j, for every j.  Slots < 0 are padding and
 * skipped; slots past the pool are skipped too (the kernel never writes
 * outside the caches).  Slots must be distinct (else which copy lands is
 * unspecified), and a block shared by several sequences must be copied
 * before it is written.  k, v are not modified and must not overlap the
 * caches.  num_tokens == 0 is a no-op.
 */
int paged_kv_write(const void *k, const void *v, const int64_t *slot_mapping,
                   void *k_cache, void *v_cache, int64_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, int32_t dtype, void *stream);

/*
 * How paged_attention_decode splits the work.  For each KV head, the
 * 16-token tiles of all sequences are laid end to end (sequence s owns tiles
 * cu[s] .. cu[s+1]-1, cu the prefix sum of ceil(context_lens / 16)) and cut
 * into W equal contiguous ranges, one wavefront each.  A sequence whose
 * tiles fall into several ranges is finished by a log-sum-exp merge of the
 * partial results.  W depends only on the sizes below: at least enough that
 * no range exceeds 64 tiles when every sequence is full, and by default
 * about 1024 wavefronts in total (one per SIMD of a 256-CU MI355X); with
 * partition_tokens = P > 0 (a multiple of 16, at most 1024) instead enough
 * that a range holds at most about P tokens.  Returns W, or 0 for
 * unsupported sizes.
 */
int32_t paged_attention_split_waves(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t partition_tokens);

/*
 * Bytes of device workspace paged_attention_decode_ex needs for these sizes
 * and partition_tokens (0 = default): partial results for W + num_seqs slots
 * per query head plus the tile prefix.  Returns 0 for unsupported sizes
 * (the decode call reports those).
 */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_tokens);

/*
 * Decode attention ("...from the source", part 2, 2.3): for each sequence s
 * and query head h, with L = context_lens[s] and kv head j = h / G,
 *   out[s][h][:] = sum_t softmax_t(scale * q[s][h] . K_t) * V_t,  t < L,
 * where token t's K and V live in block block_tables[s][t / block_size] at
 * offset t % block_size.  L == 0 gives a zero row.  Table entries past
 * ceil(L / block_size) are never read; neither are unused slots of the last
 * block.  Writes `out` (same type as q) and the workspace only.
 * Device-side contract (not checked, results then unspecified, but the
 * kernels stay inside every buffer): block ids in [0, num_blocks),
 * 0 <= L <= max_blocks_per_seq * block_size.  paged_validate_metadata
 * checks these on host copies.  num_seqs is at most 8192.
 * `workspace` (16-byte aligned) must hold paged_attention_workspace_bytes
 * bytes for the default split; out must not overlap any input.  The call
 * is two launches on `stream`: the split pass, then the merge pass.
 */
int paged_attention_decode(void *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, float scale,
                           int32_t block_size, int32_t num_kv_heads,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int64_t num_blocks,
                           int32_t dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * Same as paged_attention_decode with an explicit split (partition_tokens
 * as in paged_attention_split_waves; 0 = default).  The result does not
 * depend on the split beyond floating-point rounding.
 */
int paged_attention_decode_ex(void *out, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              const int32_t *context_lens, float scale,
                              int32_t block_size, int32_t num_kv_heads,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t max_blocks_per_seq, int64_t num_blocks,
                              int32_t dtype, int32_t partition_tokens,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_ex split into its two launches, for callers that
 * schedule or time them separately.  stages: 1 = split pass only (each
 * wavefront reduces its tile range; sequences held by one wavefront get
 * their final row in `out`, the others leave partial results and the tile
 * prefix in the workspace), 2 = merge pass only (log-sum-exp combine of the
 * workspace into `out` for sequences split across wavefronts; the split
 * pass with the same arguments must have run before it on the same
 * stream), 3 = both, which is paged_attention_decode_ex.  Other values give
 * PA_ERR_SHAPE.
 */
int paged_attention_decode_stages(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, float scale,
                                  int32_t block_size, int32_t num_kv_heads,
                                  int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t dtype, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, int32_t stages,
                                  void *stream);

/*
 * FP8 KV cache ("vLLM framework analysis: how PagedAttention speeds up LLM
 * inference 20x" (intelliparadigm.com), 7: FP8 for the attention
 * computation, FP16 for the rest).  The caches hold OCP E4M3 ("e4m3fn")
 * codes, one byte per element, in the layouts above; a K code c stands for
 * c * k_scale and a V code for c * v_scale (one scale per tensor, finite and
 * positive).  q, out, k and v stay 16-bit (dtype).
 *
 * paged_kv_write_fp8: the append of paged_kv_write, quantising: element x
 * of k goes in as the E4M3 code nearest to float32(x) * float32(1/k_scale)
 * (ties to the even code; finite magnitudes from 448 up saturate to +-448;
 * NaN stays NaN), v likewise with v_scale.  Caches 16-byte aligned.
 */
int paged_kv_write_fp8(const void *k, const void *v, const int64_t *slot_mapping,
                       void *k_cache, void *v_cache, int64_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int32_t dtype, float k_scale, float v_scale,
                       void *stream);

/*
 * paged_attention_decode_stages over E4M3 caches: the same attention with
 * K_t = code * k_scale and V_t = code * v_scale.  The codes are converted
 * exactly in registers, K to the q type and V to binary16; P.V then runs
 * with binary16 weights (11 significant bits) whatever the q type.  k_scale
 * joins the score scale and v_scale the output.  Workspace as for the
 * 16-bit caches.
 */
int paged_attention_decode_fp8(void *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, float scale, float k_scale,
                               float v_scale, int32_t block_size, int32_t num_kv_heads,
                               int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                               int32_t partition_tokens, void *workspace,
                               size_t workspace_bytes, int32_t stages, void *stream);

/*
 * One decode step with the append fused in ("vLLM memory management and
 * continuous batching from the source" (developer.cloud.tencent.cn), part 2:
 * 2.1, the new token's K/V written at its block's address plus offset; 2.3,
 * attention reading K/V through the block table).  For every sequence s with
 * L = context_lens[s] >= 1 the new token is context position L-1: its rows
 * k_new[s], v_new[s] ([num_seqs, num_kv_heads, head_dim], dtype) are stored
 * at block block_tables[s][(L-1) / block_size], offset (L-1) % block_size,
 * of both caches, and out[s] is the attention of q[s] over all L tokens, the
 * new one included.  That is paged_kv_write with slot_mapping[s] = that slot,
 * followed by paged_attention_decode, in two launches instead of three, with
 * the same arithmetic (the outputs and caches are bit-identical to those two
 * calls): the split pass's wavefront that holds position L-1 takes its K/V
 * from k_new / v_new rather than the cache and stores them into the slot.
 * L = 0: out[s] = 0 and no store; a table entry outside [0, num_blocks) for
 * position L-1: no store (the token still enters the attention).
 *
 * kv_fp8 = 0: 16-bit caches, k_scale / v_scale ignored.  kv_fp8 = 1: E4M3
 * caches as for paged_kv_write_fp8 / paged_attention_decode_fp8; the new
 * token is quantised with the scales and enters the attention as its codes'
 * values.  k_new, v_new: 4-byte aligned.  The workspace is that of
 * paged_attention_decode for the same sizes.  The caller owns all buffers;
 * out, the new token's cache slots and the workspace are written.  In the V
 * cache the new token's group of four positions is written whole for each KV
 * head, its other three positions with the bytes they held, so the caller
 * must not modify that block during the call (it owns it alone anyway: a
 * shared block is copied before a write into it).
 */
int paged_attention_decode_append(void *out, const void *q, const void *k_new,
                                  const void *v_new, void *k_cache, void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, float k_scale, float v_scale,
                                  int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                                  int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t dtype, int32_t kv_fp8, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_append split into its two launches, as
 * paged_attention_decode_stages splits paged_attention_decode: stages 1 =
 * the split pass with the new tokens' stores (sequences held by one
 * wavefront get their final row), 2 = the merge pass (the same launch as
 * paged_attention_decode_stages' stage 2; the split pass with the same
 * arguments must have run before it on the same stream), 3 = both, which is
 * paged_attention_decode_append.  Other values give PA_ERR_SHAPE.  Running
 * stage 1 again with the same arguments stores the same bytes again.
 */
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
                                         size_t workspace_bytes, int32_t stages, void *stream);

/*
 * Decode with a prefix shared by the whole batch ("vLLM framework analysis:
 * how PagedAttention speeds up LLM inference 20x" (intelliparadigm.com), 2.3:
 * requests with a common system prompt hold its blocks by reference;
 * "vLLM core architecture overview" (5688vip.com), 4.1: prefix blocks
 * shared across requests).  The caller states that every sequence's first
 * shared_blocks table entries are the same physical blocks and that every
 * context_lens[s] >= shared_blocks * block_size (paged_validate_shared_prefix
 * checks both on host copies; a violation gives unspecified values, the
 * kernels staying inside every buffer).  The result is the attention of
 * paged_attention_decode (k_new == v_new == NULL) or of
 * paged_attention_decode_append (both non-NULL; then every context length
 * must exceed the prefix, so that each new token lands in a private block),
 * up to floating-point rounding; only the work is arranged differently: the
 * prefix's K/V tiles are streamed once per group of sequences (as many as
 * fill 32 matrix-core columns with their query heads) instead of once per
 * sequence, and merged with each sequence's own tiles by log-sum-exp.  Only
 * whole 16-token tiles of the prefix are shared (at block size 8 an odd
 * shared_blocks leaves its last block with the private tokens);
 * shared_blocks = 0 is the call without a prefix.  0 <= shared_blocks <=
 * max_blocks_per_seq, else PA_ERR_SHAPE.  kv_fp8, scales, partition_tokens
 * and stages as for paged_attention_decode_append_stages.  The workspace
 * must hold paged_attention_workspace_bytes_shared bytes (the partials of
 * the prefix come on top of those of paged_attention_workspace_bytes).
 */
size_t paged_attention_workspace_bytes_shared(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int32_t shared_blocks, int32_t partition_tokens);
int paged_attention_decode_shared(void *out, const void *q, const void *k_new,
                                  const void *v_new, void *k_cache, void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  float scale, float k_scale, float v_scale, int32_t block_size,
                                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, int32_t kv_fp8,
                                  int32_t shared_blocks, int32_t partition_tokens,
                                  void *workspace, size_t workspace_bytes, int32_t stages,
                                  void *stream);

/*
 * Host-side check of the shared-prefix contract (host pointers): every
 * sequence's first shared_blocks table entries equal sequence 0's, every
 * context length is at least shared_blocks * block_size, and with append != 0
 * (the fused step) greater than it.  Returns PA_OK, PA_ERR_METADATA on a
 * violation, PA_ERR_NULL / PA_ERR_SHAPE for bad arguments.
 */
int paged_validate_shared_prefix(const int32_t *block_tables, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int32_t block_size, int32_t shared_blocks, int32_t append);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the step
 * of paged_attention_decode_append with no workspace argument.  Its partial
 * results and tile prefix go to a fixed 16 MiB array inside the library
 * (PA_SCRATCH_BYTES), one per GPU, held until the process ends; the call
 * allocates nothing.  Every other argument, result and error is that of
 * paged_attention_decode_append.  Sizes whose workspace
 * (paged_attention_workspace_bytes) exceeds PA_SCRATCH_BYTES are refused
 * with PA_ERR_SCRATCH before anything is enqueued; the five workloads this
 * library is measured on need at most about 9 MiB (8 x 32768 tokens, 64
 * query heads).  Every call on one GPU shares that GPU's array and leaves
 * its contents behind (nothing in it needs clearing between calls): calls
 * that overlap on one GPU -- on other streams, or from other threads before
 * the first has finished on the device -- race and give unspecified results.
 */
#define PA_SCRATCH_BYTES ((size_t)16 << 20)
int paged_attention_decode_append_noalloc(void *out, const void *q, const void *k_new,
                                          const void *v_new, void *k_cache, void *v_cache,
                                          const int32_t *block_tables,
                                          const int32_t *context_lens, float scale,
                                          float k_scale, float v_scale, int32_t block_size,
                                          int32_t num_kv_heads, int32_t num_seqs,
                                          int32_t num_heads, int32_t head_dim,
                                          int32_t max_blocks_per_seq, int64_t num_blocks,
                                          int32_t dtype, int32_t kv_fp8,
                                          int32_t partition_tokens, void *stream);

/*
 * Paged (chunked) prefill attention ("vLLM core architecture overview"
 * (5688vip.com), 4.3, and "vLLM framework analysis: how PagedAttention
 * achieves a 20x LLM inference speed-up" (intelliparadigm.com), 4.2: a long
 * prompt is processed in chunks).  Sequence s contributes the query rows
 * query_start[s] .. query_start[s+1]-1 of q and out ([total_rows, num_heads,
 * head_dim], dtype): its last n_s context positions L-n_s .. L-1, with
 * L = context_lens[s] counting the chunk, whose K/V are already in the caches
 * (appended with paged_kv_write).  Row i (position p = L-n_s+i), query head h:
 *   out[i,h] = softmax(scale * q[i,h] K[0..p]^T) V[0..p]
 * over KV head h / (num_heads / num_kv_heads), reached through the block
 * table as in paged_attention_decode (same cache layouts, 16-bit caches).
 * query_start: device int32 [num_seqs + 1], non-decreasing from 0.
 * max_query_len: host bound on every n_s (it sizes the grid; rows of a
 * longer chunk are not computed); 0 is a no-op.  A sequence with n_s > L
 * gets no rows written.  scale > 0 and max_blocks_per_seq <= 4096 (a
 * workgroup keeps its sequence's block ids on chip), else PA_ERR_SHAPE.
 * Numerics: scores and the softmax in fp32; P.V in binary16 weights times
 * binary16 V with fp32 accumulation.  With bfloat16 caches, V is converted
 * to binary16 on chip: exact for magnitudes 2^-17 .. 65280, rounded by less
 * than 2^-24 below.  A workgroup (64 rows of one sequence, up to 4 heads of
 * one KV head) that meets a bfloat16 V of magnitude 65536 or more instead
 * recomputes its rows with bfloat16 V (scaled by 2^-40 on chip, exact down
 * to 2^-86) and the weights split into bfloat16 hi + lo parts: no finite V
 * is clamped, at about twice that workgroup's time.  Infinite V and NaN in
 * q, K or V give unspecified values in the rows that see them.  No
 * workspace; out rows of the chunks are the only writes.  Asynchronous on
 * `stream`.
 */
int paged_attention_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            const int32_t *query_start, float scale, int32_t block_size,
                            int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                            int32_t head_dim, int32_t max_blocks_per_seq, int64_t num_blocks,
                            int32_t dtype, int32_t max_query_len, void *stream);

/*
 * paged_attention_prefill over E4M3 caches (the FP8 reading of
 * paged_kv_write_fp8: uint8 codes in the same layouts, a code c standing for
 * c * k_scale in K and c * v_scale in V; "vLLM framework analysis: how
 * PagedAttention speeds up LLM inference 20x", 7).  q and out stay in
 * `dtype`.  The codes are converted exactly (K to q's type, V to binary16)
 * as the kernel stores them to its tiles; k_scale joins the score scale and
 * v_scale multiplies the output.  k_scale, v_scale: finite, normal, > 0,
 * else PA_ERR_SHAPE.  Every other argument, check and limit is that of
 * paged_attention_prefill.
 */
int paged_attention_prefill_fp8(void *out, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                const int32_t *context_lens, const int32_t *query_start,
                                float scale, float k_scale, float v_scale, int32_t block_size,
                                int32_t num_kv_heads, int32_t num_seqs, int32_t num_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq,
                                int64_t num_blocks, int32_t dtype, int32_t max_query_len,
                                void *stream);

/*
 * Host-side check of metadata (host pointers): every context length in
 * [0, max_blocks_per_seq * block_size]; every table entry a sequence reads,
 * i.e. the first ceil(L / block_size) of its row, in [0, num_blocks); every
 * non-negative slot below num_blocks * block_size and no slot repeated.
 * slot_mapping may be NULL (num_tokens ignored).  Returns PA_OK or
 * PA_ERR_METADATA.  Meant for tests and debugging, not the hot path.
 */
int paged_validate_metadata(const int32_t *block_tables, const int32_t *context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq,
                            int32_t block_size, int64_t num_blocks,
                            const int64_t *slot_mapping, int64_t num_tokens);

/*
 * Host-side check of chunked-prefill metadata (host pointers), the device
 * contract paged_attention_prefill does not check: query_start[0] == 0,
 * non-decreasing, query_start[num_seqs] <= total_rows (the rows of q and
 * out); every chunk length n_s at most max_query_len and at most its context
 * length context_lens[s].  Returns PA_OK, PA_ERR_METADATA on a violation,
 * PA_ERR_NULL / PA_ERR_SHAPE for bad arguments.
 */
int paged_validate_prefill(const int32_t *query_start, const int32_t *context_lens,
                           int32_t num_seqs, int32_t max_query_len, int64_t total_rows);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
