// Paged decode attention for gfx950 (CDNA4): one wavefront per
// (sequence, KV head, context partition), serving every query head of the
// KV head's GQA group so each K/V block is read from HBM once.
//
// Method: "vLLM memory management and continuous batching from the source"
// (developer.cloud.tencent.cn), part 2, 2.3 -- attention receives block
// tables instead of a contiguous (batch, seq_len, dim) tensor and gathers
// K/V through them; 2.1 -- a token lives in block table[t / block_size] at
// offset t % block_size.  The math is plain softmax(scale * q K^T) V,
// computed with a running max and sum over 16-token tiles and, for contexts
// longer than one partition, merged across partitions by log-sum-exp.
//
// Per 16-token tile, with G <= 16 query heads padded to 16:
//   S^T[16 tok x 16 head] = K[16 tok x D] * Q^T[D x 16 head]
//        -> D/32 MFMA 16x16x32; A = K rows as stored (token-major cache),
//           each lane loading 16 contiguous bytes of one token's row.
//   O^T[D x 16 head]     += V^T[D x 16 tok] * P^T[16 tok x 16 head]
//        -> D/16 MFMA 16x16x16; A = V^T read straight from the dim-major
//           V cache (8 contiguous bytes = 4 tokens of one dim per lane),
//           B = P exactly as the QK MFMA left it in registers (lane l holds
//           head l%16, tokens 4*(l/16)+0..3), so no shuffle is needed.
//           For bfloat16, P goes in as a hi and a lo bfloat16 part (two
//           MFMAs) so the weights keep ~16 significant bits.
// Every lane's softmax state and accumulators belong to head l%16, so the
// rescale by exp(m_old - m_new) is lane-local; only the tile max and the
// final sum cross the wave's four 16-lane rows (permlane16/32 swaps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kF16 = 0;
constexpr int kBF16 = 1;

template <int DT>
struct Elem;

// kSplitP: the weights P enter the PV MFMA as hi + lo halves (two MFMAs),
// giving ~16 significant bits instead of bfloat16's 8.
template <>
struct Elem<kBF16> {
  static constexpr bool kSplitP = true;
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  // two floats -> packed pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

template <>
struct Elem<kF16> {
  static constexpr bool kSplitP = false;  // binary16 weights already carry 11 bits
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[0];
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(f16x2, w)[1];
  }
};

// Reductions over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows
// of the wave) with the gfx950 row-swap permutes; no LDS round trip.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// K and V registers of one 16-token tile.
template <int D>
struct Frag {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

template <int DT, int D, int BS>
__global__ __launch_bounds__(kWave) void decode_partition_kernel(
    uint16_t *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, float scale_log2, int num_kv_heads,
    int num_heads, int group, int max_blocks, int64_t num_blocks, int max_parts,
    int part_tokens) {
  using E = Elem<DT>;
  constexpr int KSTEPS = D / 32;  // 16x16x32 MFMAs per QK tile
  constexpr int DTILES = D / 16;  // 16x16x16 MFMAs per PV tile

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int lane = threadIdx.x;
  const int row = lane & 15;  // A-row / B-column / head index inside a tile
  const int grp = lane >> 4;  // quarter of the wave: k-slice and 4-row group

  int len = context_lens[seq];
  len = len < 0 ? 0 : (len > max_blocks * BS ? max_blocks * BS : len);
  const int nparts = (len + part_tokens - 1) / part_tokens;
  const int head = kvh * group + row;
  const bool head_ok = row < group;

  if (len == 0) {
    if (part == 0 && head_ok) {
      uint16_t *op = out + ((int64_t)seq * num_heads + head) * D + grp * (D / 4);
#pragma unroll
      for (int i = 0; i < D / 4; i += 4) *(u32x2 *)(op + i) = u32x2{0, 0};  // out: 8-byte aligned
    }
    return;
  }
  if (part >= nparts) return;

  const int t_begin = part * part_tokens;
  const int ntok = min(len - t_begin, part_tokens);
  const int nblk = (ntok + BS - 1) / BS;

  // Block numbers of this partition, one per lane (never past the sequence's
  // last block; ids outside the pool are replaced so no access leaves it).
  int bid = 0;
  if (lane < nblk) {
    const int b = block_tables[(int64_t)seq * max_blocks + t_begin / BS + lane];
    bid = (b >= 0 && b < num_blocks) ? b : 0;
  }

  // Query fragment: lane (row, grp) holds q[head row][32*ks + 8*grp .. +8].
  u32x4 qf[KSTEPS];
  {
    const uint16_t *qp = q + ((int64_t)seq * num_heads + head) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = head_ok ? *(const u32x4 *)(qp + ks * 32) : u32x4{0, 0, 0, 0};
  }

  const int64_t blk_stride = (int64_t)num_kv_heads * BS * D;  // elements per block
  const uint16_t *kbase = k_cache + (int64_t)kvh * BS * D;
  const uint16_t *vbase = v_cache + (int64_t)kvh * D * BS;

  // Loads of one tile, straight-line (no branch around them, so the wait for
  // the current tile does not also wait for the prefetched one).  Token
  // indices are clamped into the partition; what a clamped lane reads is
  // masked away in the last tile.
  auto load = [&](Frag<D> &f, int tile) {
    const int ktok = min(tile * kTile + row, ntok - 1);
    const int vtok = min(tile * kTile + grp * 4, (ntok - 1) & ~3);
    int kb, vb;
    if constexpr (BS == 8) {  // two blocks per tile
      kb = __builtin_amdgcn_ds_bpermute((ktok / BS) << 2, bid);
      vb = __builtin_amdgcn_ds_bpermute((vtok / BS) << 2, bid);
    } else {
      kb = vb = __builtin_amdgcn_readlane(bid, tile * kTile / BS);
    }
    const uint16_t *kp = kbase + (int64_t)kb * blk_stride + (ktok % BS) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) f.k[ks] = *(const u32x4 *)(kp + ks * 32);
    const uint16_t *vp = vbase + (int64_t)vb * blk_stride + row * BS + (vtok % BS);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) f.v[dt] = *(const u32x2 *)(vp + dt * 16 * BS);
  };

  // Running max per head in log2 units.  The accumulators are rescaled only
  // when some head's max has grown by more than 2^kSlack; in between, the
  // weights exp2(s - m_ref) may exceed one by at most that factor, which
  // fp32 sums and the 16-bit weights carry without loss of relative
  // precision.
  constexpr float kSlack = 8.0f;
  float m_ref = -INFINITY;
  float l_run = 0.f;  // this lane's share of the running sum
  f32x4 acc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](Frag<D> &f, int tile, auto last_tag) {
    constexpr bool kLast = decltype(last_tag)::value;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) sc = E::qk(f.k[ks], qf[ks], sc);
    const int tb = tile * kTile + grp * 4;  // this lane's first token of the four
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = sc[r] * scale_log2;
      if constexpr (kLast) s[r] = (tb + r < ntok) ? s[r] : -INFINITY;
    }
    const float mx = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kSlack) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) acc[dt] *= alpha;
      m_ref = m_new;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - m_ref);
    u32x2 ph, pl;
    ph.x = E::pack(p[0], p[1]);
    ph.y = E::pack(p[2], p[3]);
    if constexpr (E::kSplitP) {
      // residuals are exact in fp32; the sum is taken over the full weights
      pl.x = E::pack(p[0] - E::lo(ph.x), p[1] - E::hi(ph.x));
      pl.y = E::pack(p[2] - E::lo(ph.y), p[3] - E::hi(ph.y));
      l_run += (p[0] + p[1]) + (p[2] + p[3]);
    } else {
      // the sum uses the rounded weights the MFMA multiplies with
      l_run += (E::lo(ph.x) + E::hi(ph.x)) + (E::lo(ph.y) + E::hi(ph.y));
    }
    if constexpr (kLast) {  // ragged tail: zero V of tokens past the end (may hold NaN)
      const int c = ntok - tb;
      if (c < 4) {
        const uint32_t w0 = c >= 2 ? 0xffffffffu : (c == 1 ? 0x0000ffffu : 0u);
        const uint32_t w1 = c == 3 ? 0x0000ffffu : 0u;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) {
          f.v[dt].x &= w0;
          f.v[dt].y &= w1;
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      acc[dt] = E::pv(f.v[dt], ph, acc[dt]);
      if constexpr (E::kSplitP) acc[dt] = E::pv(f.v[dt], pl, acc[dt]);
    }
  };

  // Ping-pong over two register sets: the next tile's loads are in flight
  // while the current one is computed, and no register copy waits on them.
  const int ntiles = (ntok + kTile - 1) / kTile;
  Frag<D> fa, fb;
  load(fa, 0);
  int tile = 0;
  for (; tile + 2 < ntiles; tile += 2) {
    load(fb, tile + 1);
    step(fa, tile, std::false_type{});
    load(fa, tile + 2);
    step(fb, tile + 1, std::false_type{});
  }
  if (tile + 1 < ntiles) {
    load(fb, tile + 1);
    step(fa, tile, std::false_type{});
    step(fb, tile + 1, std::true_type{});
  } else {
    step(fa, tile, std::true_type{});
  }
  const float m_run = m_ref;

  const float l_tot = rows_sum(l_run);
  if (!head_ok) return;
  const float inv = 1.0f / l_tot;

  if (nparts == 1) {
    // lane (row, grp) holds dims 16*dt + 4*grp + 0..3 of head row
    uint16_t *op = out + ((int64_t)seq * num_heads + head) * D + grp * 4;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      u32x2 w;
      w.x = E::pack(acc[dt][0] * inv, acc[dt][1] * inv);
      w.y = E::pack(acc[dt][2] * inv, acc[dt][3] * inv);
      *(u32x2 *)(op + dt * 16) = w;
    }
  } else {
    const int64_t slot = ((int64_t)seq * num_heads + head) * max_parts + part;
    float *op = ws_o + slot * D + grp * 4;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) *(f32x4 *)(op + dt * 16) = acc[dt] * inv;
    if (grp == 0) *(f32x2 *)(ws_ml + slot * 2) = f32x2{m_run, l_tot};
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
//   M = max_p m_p,  c_p = l_p * 2^(m_p - M),  out = sum_p c_p o_p / sum_p c_p.
template <int DT, int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(
    uint16_t *__restrict__ out, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml, const int32_t *__restrict__ context_lens,
    int num_heads, int max_len, int max_parts, int part_tokens) {
  using E = Elem<DT>;
  constexpr int PER = D / kWave;  // dims per lane
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  int len = context_lens[seq];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const int nparts = (len + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;

  const int64_t base = ((int64_t)seq * num_heads + head) * max_parts;
  const f32x2 *ml = (const f32x2 *)(ws_ml + base * 2);
  float big = -INFINITY;
  for (int p = lane; p < nparts; p += kWave) big = fmaxf(big, ml[p].x);
  big = wave_max(big);

  float num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  float den = 0.f;
  const float *o = ws_o + base * D + lane * PER;
#pragma unroll 4
  for (int p = 0; p < nparts; ++p) {
    const f32x2 v = ml[p];
    const float c = v.y * __builtin_amdgcn_exp2f(v.x - big);
    den += c;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] += c * o[(int64_t)p * D + i];
  }
  const float inv = 1.0f / den;
  uint16_t *op = out + ((int64_t)seq * num_heads + head) * D + lane * PER;
  if constexpr (PER == 2) {
    *(uint32_t *)op = E::pack(num[0] * inv, num[1] * inv);
  } else {
    op[0] = (uint16_t)(E::pack(num[0] * inv, 0.f) & 0xffffu);
  }
}

template <int DT, int D, int BS>
int launch_typed(const DecodeArgs &a) {
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  hipStream_t st = (hipStream_t)a.stream;
  const int group = a.num_heads / a.num_kv_heads;
  hipError_t e = hipSuccess;
  if (a.stages & 1) {
    dim3 grid((unsigned)a.max_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    decode_partition_kernel<DT, D, BS><<<grid, kWave, 0, st>>>(
        (uint16_t *)a.out, a.ws_o, a.ws_ml, (const uint16_t *)a.q,
        (const uint16_t *)a.k_cache, (const uint16_t *)a.v_cache, a.block_tables,
        a.context_lens, scale_log2, a.num_kv_heads, a.num_heads, group,
        a.max_blocks_per_seq, a.num_blocks, a.max_parts, a.partition_tokens);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  if ((a.stages & 2) && a.max_parts > 1) {
    dim3 g2((unsigned)a.num_heads, (unsigned)a.num_seqs);
    decode_merge_kernel<DT, D><<<g2, kWave, 0, st>>>(
        (uint16_t *)a.out, a.ws_o, a.ws_ml, a.context_lens, a.num_heads,
        a.max_blocks_per_seq * BS, a.max_parts, a.partition_tokens);
    e = hipGetLastError();
  }
  return (int)e;
}

template <int DT, int D>
int launch_bs(const DecodeArgs &a) {
  switch (a.block_size) {
    case 8: return launch_typed<DT, D, 8>(a);
    case 16: return launch_typed<DT, D, 16>(a);
    case 32: return launch_typed<DT, D, 32>(a);
  }
  return (int)hipErrorInvalidValue;
}

template <int DT>
int launch_dim(const DecodeArgs &a) {
  switch (a.head_dim) {
    case 64: return launch_bs<DT, 64>(a);
    case 128: return launch_bs<DT, 128>(a);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_decode(const DecodeArgs &a) {
  return a.dtype == kBF16 ? launch_dim<kBF16>(a) : launch_dim<kF16>(a);
}

}  // namespace pa
