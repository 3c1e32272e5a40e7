// Whole-block copies between two pools of the same layout: within one
// device pool for copy-on-write ("vLLM framework analysis: how PagedAttention
// achieves a 20x LLM inference speed-up" (intelliparadigm.com), 2.3: a write
// into a shared block goes to a private copy), and between the device pool
// and a pinned host pool for swapping ("vLLM core architecture overview"
// (5688vip.com), 4.2: under memory pressure a request's KV is moved out to
// CPU memory).  A block of either cache is one contiguous run of
// num_kv_heads * block_size * head_dim elements, so a copy is a plain move of
// two runs: HBM-bound within the device, host-link-bound across it.  The
// kernel reads and writes pinned host memory directly through its device
// mapping, so a batch of small blocks costs one launch, not one DMA each.
//
// One workgroup per (pair, cache, part of the run): 256 lanes move 16 bytes
// each, four times, with all four loads issued before the stores.  K/V are
// touched once, so both directions bypass the caches' normal replacement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte chunks per lane per workgroup
constexpr int64_t kChunksPerPart = (int64_t)kCopyThreads * kCopyUnroll;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4 *__restrict__ dst_k, u32x4 *__restrict__ dst_v, const u32x4 *__restrict__ src_k,
    const u32x4 *__restrict__ src_v, const int64_t *__restrict__ pairs, int64_t src_blocks,
    int64_t dst_blocks, int64_t run16, int64_t parts) {
  const int64_t wg = blockIdx.x;
  const int64_t part = wg % parts;
  const int64_t rest = wg / parts;
  const int64_t i = rest >> 1;
  const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks) return;
  const u32x4 *s = ((rest & 1) ? src_v : src_k) + src * run16;
  u32x4 *d = ((rest & 1) ? dst_v : dst_k) + dst * run16;
  const int64_t c0 = part * kChunksPerPart + threadIdx.x;
  u32x4 x[kCopyUnroll];
#pragma unroll
  for (int j = 0; j < kCopyUnroll; ++j) {
    const int64_t c = c0 + (int64_t)j * kCopyThreads;
    if (c < run16) x[j] = __builtin_nontemporal_load(s + c);
  }
#pragma unroll
  for (int j = 0; j < kCopyUnroll; ++j) {
    const int64_t c = c0 + (int64_t)j * kCopyThreads;
    if (c < run16) __builtin_nontemporal_store(x[j], d + c);
  }
}

}  // namespace

int launch_copy_blocks(const CopyArgs &a) {
  const int64_t run16 = a.run_bytes / 16;
  const int64_t parts = (run16 + kChunksPerPart - 1) / kChunksPerPart;
  const int64_t groups = a.num_pairs * 2 * parts;
  if (groups > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
  copy_blocks_kernel<<<dim3((unsigned)groups), kCopyThreads, 0, (hipStream_t)a.stream>>>(
      (u32x4 *)a.dst_k, (u32x4 *)a.dst_v, (const u32x4 *)a.src_k, (const u32x4 *)a.src_v,
      a.pairs, a.src_blocks, a.dst_blocks, run16, parts);
  return (int)hipGetLastError();
}

}  // namespace pa
