// Paged KV append for gfx950: the write step of "vLLM memory management and
// continuous batching from the source" (developer.cloud.tencent.cn), part 2,
// 2.1 -- each new token's K and V go to its block's address plus the offset
// inside the block.  The slot (block * block_size + offset) is chosen by the
// caller's block manager; this is a pure bit copy.
//
// The FP8 variant quantises while it scatters (see kv_write_fp8_kernel).
//
// One workgroup per token.  A K row (head_dim contiguous elements) lands
// contiguously in the token-major K cache, moved as 16-byte vectors.  The V
// cache holds each (block, head) slice as block_size/4 groups of [head_dim][4]
// (four positions of one dimension adjacent), so a V row lands with a stride
// of 4 elements inside its position group: read as 16-byte vectors, stored
// as single elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int D, int BS>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int64_t *__restrict__ slot_mapping, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int num_kv_heads, int64_t num_slots) {
  constexpr int CH = D / 8;  // 16-byte chunks per head row
  const int64_t tok = blockIdx.x;
  const int nch = num_kv_heads * CH;
  // The first chunk's k/v loads go out together with the slot load (they do
  // not depend on it), so the launch costs one memory round trip, not two.
  const int c0 = threadIdx.x;
  u32x4 kx0 = {0, 0, 0, 0}, vx0 = {0, 0, 0, 0};
  if (c0 < nch) {
    const int64_t src = (tok * num_kv_heads + c0 / CH) * D + (c0 % CH) * 8;
    kx0 = *(const u32x4 *)(k + src);
    vx0 = *(const u32x4 *)(v + src);
  }
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  for (int c = c0; c < nch; c += blockDim.x) {
    const int h = c / CH;
    const int d0 = (c % CH) * 8;
    const int64_t src = (tok * num_kv_heads + h) * D + d0;
    const u32x4 kx = c == c0 ? kx0 : *(const u32x4 *)(k + src);
    const u32x4 vx = c == c0 ? vx0 : *(const u32x4 *)(v + src);
    const int64_t bh = blk * num_kv_heads + h;
    *(u32x4 *)(k_cache + (bh * BS + off) * D + d0) = kx;
    uint16_t *vd = v_cache + bh * BS * D + ((off >> 2) * D + d0) * 4 + (off & 3);
    vd[0 * 4] = (uint16_t)(vx.x & 0xffffu);
    vd[1 * 4] = (uint16_t)(vx.x >> 16);
    vd[2 * 4] = (uint16_t)(vx.y & 0xffffu);
    vd[3 * 4] = (uint16_t)(vx.y >> 16);
    vd[4 * 4] = (uint16_t)(vx.z & 0xffffu);
    vd[5 * 4] = (uint16_t)(vx.z >> 16);
    vd[6 * 4] = (uint16_t)(vx.w & 0xffffu);
    vd[7 * 4] = (uint16_t)(vx.w >> 16);
  }
}

// Quantising append into E4M3 caches: element x goes in as the code of
// float32(x) * inv (inv = float32(1 / scale) from the host).  Layouts as for
// the 16-bit caches, one byte per element.
template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int64_t *__restrict__ slot_mapping, uint8_t *__restrict__ k_cache,
    uint8_t *__restrict__ v_cache, int num_kv_heads, int64_t num_slots, float k_inv,
    float v_inv) {
  constexpr int CH = D / 8;  // 8-element chunks per head row
  const int64_t tok = blockIdx.x;
  const int nch = num_kv_heads * CH;
  const int c0 = threadIdx.x;
  u32x4 kx0 = {0, 0, 0, 0}, vx0 = {0, 0, 0, 0};
  if (c0 < nch) {
    const int64_t src = (tok * num_kv_heads + c0 / CH) * D + (c0 % CH) * 8;
    kx0 = *(const u32x4 *)(k + src);
    vx0 = *(const u32x4 *)(v + src);
  }
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  for (int c = c0; c < nch; c += blockDim.x) {
    const int h = c / CH;
    const int d0 = (c % CH) * 8;
    const int64_t src = (tok * num_kv_heads + h) * D + d0;
    const u32x4 kx = c == c0 ? kx0 : *(const u32x4 *)(k + src);
    const u32x4 vx = c == c0 ? vx0 : *(const u32x4 *)(v + src);
    uint32_t kc[8], vc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kc[2 * i] = e4m3_code(elem_to_float<DT>(kx[i] & 0xffffu) * k_inv);
      kc[2 * i + 1] = e4m3_code(elem_to_float<DT>(kx[i] >> 16) * k_inv);
      vc[2 * i] = e4m3_code(elem_to_float<DT>(vx[i] & 0xffffu) * v_inv);
      vc[2 * i + 1] = e4m3_code(elem_to_float<DT>(vx[i] >> 16) * v_inv);
    }
    const int64_t bh = blk * num_kv_heads + h;
    u32x2 kw;
    kw.x = kc[0] | (kc[1] << 8) | (kc[2] << 16) | (kc[3] << 24);
    kw.y = kc[4] | (kc[5] << 8) | (kc[6] << 16) | (kc[7] << 24);
    *(u32x2 *)(k_cache + (bh * BS + off) * D + d0) = kw;  // 8-byte aligned: d0 % 8 == 0
    uint8_t *vd = v_cache + bh * BS * D + ((off >> 2) * D + d0) * 4 + (off & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) vd[i * 4] = (uint8_t)vc[i];
  }
}

template <int D, int BS>
int launch_typed(const WriteArgs &a) {
  const int nch = a.num_kv_heads * (D / 8);
  int threads = (nch + kWave - 1) / kWave * kWave;
  threads = threads < kWave ? kWave : (threads > 256 ? 256 : threads);
  const dim3 grid((unsigned)a.num_tokens);
  hipStream_t st = (hipStream_t)a.stream;
  if (!a.fp8) {
    kv_write_kernel<D, BS><<<grid, threads, 0, st>>>(
        (const uint16_t *)a.k, (const uint16_t *)a.v, a.slot_mapping, (uint16_t *)a.k_cache,
        (uint16_t *)a.v_cache, a.num_kv_heads, a.num_blocks * BS);
  } else if (a.dtype == 1) {
    kv_write_fp8_kernel<1, D, BS><<<grid, threads, 0, st>>>(
        (const uint16_t *)a.k, (const uint16_t *)a.v, a.slot_mapping, (uint8_t *)a.k_cache,
        (uint8_t *)a.v_cache, a.num_kv_heads, a.num_blocks * BS, a.k_inv, a.v_inv);
  } else {
    kv_write_fp8_kernel<0, D, BS><<<grid, threads, 0, st>>>(
        (const uint16_t *)a.k, (const uint16_t *)a.v, a.slot_mapping, (uint8_t *)a.k_cache,
        (uint8_t *)a.v_cache, a.num_kv_heads, a.num_blocks * BS, a.k_inv, a.v_inv);
  }
  return (int)hipGetLastError();
}

template <int D>
int launch_bs(const WriteArgs &a) {
  switch (a.block_size) {
    case 8: return launch_typed<D, 8>(a);
    case 16: return launch_typed<D, 16>(a);
    case 32: return launch_typed<D, 32>(a);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_kv_write(const WriteArgs &a) {
  switch (a.head_dim) {
    case 64: return launch_bs<64>(a);
    case 128: return launch_bs<128>(a);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
