// Paged (chunked) prefill attention for gfx950.
//
// "vLLM core architecture overview" (5688vip.com), 4.3, and "vLLM framework
// analysis: how PagedAttention achieves a 20x LLM inference speed-up"
// (intelliparadigm.com), 4.2: a long prompt is processed in chunks.  Each
// chunk token (context position p) attends over positions 0 .. p of its
// sequence, reached through the block table as in decode ("vLLM memory
// management and continuous batching from the source", part 2, 2.3); the
// chunk's own K/V are already in the caches (appended before the call).
//
// Unlike decode this is a dense contraction: every K/V tile meets many query
// rows, so the bound is the MFMA rate, not HBM.  Work split:
//   workgroup = (64 query tokens of one sequence) x (up to 4 query heads of
//   one KV head); waves of 16 tokens x up to 2 heads (at most 32 query rows,
//   under 256 registers, two waves per SIMD).
//   The workgroup walks the keys 0 .. its last position in tiles of 64 (one
//   barrier, one max reduction and one round of staging per 64 keys): K and
//   V tiles go through double-buffered LDS (the lanes move 16-byte pieces),
//   so a tile is read from memory once per 64 tokens x 4 heads.
//   Workgroups run heaviest-first (last query block first) and the blocks of
//   one (sequence, KV head) land on one XCD, sharing its L2.
// Per wave and 64-key tile, with q held in registers as the B operand:
//   S^T[64 keys x 16 tokens] per head = K[keys x D] q^T  (16x16x32 MFMAs, A =
//     K rows from LDS, four 16-key row blocks), so lane (token l%16, quarter
//     l/16) holds the scores of keys 16*rb + 4*(l/16) + r;
//   O^T[D x 16 tokens] += V^T[D x 32 keys] P^T for each 32-key half (16x16x32
//     MFMAs, A = the dim-major V tile from LDS, B = P in the registers the QK
//     MFMA wrote: the k index of both operands runs over the same eight keys
//     per lane, so no shuffle is needed).
// Online softmax per (head, token) with a lazily raised reference max, as in
// decode; P.V runs in binary16 (see Elem below, and the exact mode for
// bfloat16 V beyond binary16's range); the causal mask runs only
// on tiles that reach past a wave's first position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kQT = 16;          // query tokens per wave
constexpr int kTG = 4;           // token groups per workgroup
constexpr int kQB = kQT * kTG;   // query tokens per workgroup
constexpr int kKT = 64;          // keys per tile
constexpr int kRB = kKT / 16;    // 16-key row blocks per tile (QK)
constexpr int kNH = kKT / 32;    // 32-key halves per tile (PV)

// QK runs in the caches' own 16-bit type; P.V runs in binary16: the weights
// lie in [0, 2^8] (the reference max lags by at most kSlack), where binary16
// keeps 11 significant bits, and a bfloat16 V tile is converted to binary16
// as it is stored to LDS.  That conversion is exact for every bfloat16 value
// of magnitude 2^-17 .. 65280 (8 significant bits fit in 11) and rounds
// smaller ones by less than 2^-24.  Larger ones (65536 and up) would
// saturate: a workgroup that stages one recomputes its rows in an exact mode
// (bfloat16 V, weights split into bfloat16 hi + lo), so no V is clamped.
// Elem<DT>: the QK product and the output in the caches' type.
template <int DT>
struct Elem;
template <>
struct Elem<1> {
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
};
template <>
struct Elem<0> {
  static __device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
};

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {  // round to nearest even
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
// two bfloat16 values -> two binary16 values (toward zero: exact in range,
// saturating beyond it)
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                 __uint_as_float(w & 0xffff0000u)));
}

// four E4M3 codes (bytes 0..3) -> four values of the caller's 16-bit type
// (DT 0 binary16, DT 1 bfloat16), exact: every E4M3 value fits both
template <int DT>
__device__ __forceinline__ u32x2 e4m3x4_to(uint32_t c) {
  if constexpr (DT == 1)
    return u32x2{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true))};
  else
    return u32x2{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, true))};
}
// eight E4M3 codes -> eight 16-bit values
template <int DT>
__device__ __forceinline__ u32x4 e4m3x8_to(u32x2 c) {
  const u32x2 a = e4m3x4_to<DT>(c.x), b = e4m3x4_to<DT>(c.y);
  return u32x4{a.x, a.y, b.x, b.y};
}

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

// LDS tile layouts (16-bit elements), rows padded so that the 16 rows one
// MFMA operand reads spread over the banks:
//   K tile [64 keys][D + 8]  (token-major, as in the cache)
//   V tile [D][64 + 4]       (dim-major: the cache's groups of four keys
//                             laid end to end per dimension; a 34-dword row,
//                             the fastest measured of a few 8-byte-aligned ones)
template <int D>
struct Tile {
  static constexpr int kRow = D + 8;        // K row, in elements
  static constexpr int vRow = kKT + 4;      // V row, in elements
  static constexpr int kElems = kKT * kRow;
  static constexpr int vElems = D * vRow;
  static constexpr int elems = kElems + vElems;
};

// HW query heads per wave (1 or 2) and NWH head groups per workgroup (1 or
// 2): a workgroup is 4 * NWH waves serving 64 tokens x HW * NWH heads, and a
// wave stays under 256 registers, so two waves share each SIMD.  q rows
// beyond the chunk and padded heads compute on clamped inputs and are never
// stored.  KV8: the caches hold E4M3 codes, converted exactly to q's type
// (K) and binary16 (V) as they are stored to LDS; scale_log2 then carries
// k_scale and out_scale is v_scale.
template <int DT, int D, int HW, int NWH, bool KV8>
__global__ __launch_bounds__(kWave * kTG * NWH) void prefill_kernel(
    uint16_t *__restrict__ out, const uint16_t *__restrict__ q,
    const void *__restrict__ k_cache, const void *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const int32_t *__restrict__ query_start, float scale_log2, float out_scale, int log2_bs,
    int num_seqs, int num_kv_heads, int num_heads, int group, int chunks, int max_blocks,
    int64_t num_blocks, int nqb) {
  using E = Elem<DT>;
  constexpr int HC = HW * NWH;     // query heads per workgroup
  constexpr int kThreads = kWave * kTG * NWH;
  constexpr int KSTEPS = D / 32;   // 16x16x32 MFMAs per QK product
  constexpr int DTILES = D / 16;   // 16-dim output tiles
  using T = Tile<D>;
  // LDS: two K/V tile buffers, then the sequence's block ids (clamped into
  // the pool), so that tile addresses never wait on a global load.
  extern __shared__ __align__(16) uint16_t lds[];
  int32_t *tbl_lds = reinterpret_cast<int32_t *>(lds + 2 * T::elems);

  // workgroup -> (query block, sequence, KV head, head chunk); heaviest first
  const int per_qb = num_seqs * num_kv_heads * chunks;
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);
  const int rest = blockIdx.x % per_qb;
  const int chunk = rest % chunks;
  const int kvh = (rest / chunks) % num_kv_heads;
  const int seq = rest / (chunks * num_kv_heads);
  const int q0 = query_start[seq];
  const int n = query_start[seq + 1] - q0;
  const int bs = 1 << log2_bs;
  const int len = min(context_lens[seq], max_blocks * bs);
  if (qb * kQB >= n || n > len) return;  // no rows here (or an invalid chunk)

  const int tid = threadIdx.x;
  const int wave = (tid / kWave) % kTG;   // token group
  const int hgrp = tid / (kWave * kTG);   // head group
  const int lane = tid % kWave;
  const int col = lane & 15;   // token within the wave's 16 (B column / C column)
  const int grp = lane >> 4;   // quarter: k slice of the operands, 4-row group of C
  const int first_pos = len - n;                      // position of chunk row 0
  const int wt0 = qb * kQB + wave * kQT;              // wave's first chunk row
  const int tok = min(wt0 + col, n - 1);              // this lane's chunk row (clamped)
  const int pos = first_pos + tok;                    // its context position
  const int wave_lo = first_pos + min(wt0, n - 1);    // wave's first / last positions
  const int wave_hi = first_pos + min(wt0 + kQT - 1, n - 1);
  // (workgroup-uniform: read back as scalars, so the address and mask
  // arithmetic built on them stays on the scalar unit)
  const int wg_hi = __builtin_amdgcn_readfirstlane(first_pos + min(qb * kQB + kQB - 1, n - 1));
  const int ntiles = __builtin_amdgcn_readfirstlane(wg_hi / kKT + 1);  // keys 0 .. wg_hi
  const int32_t *tbl = block_tables + (int64_t)seq * max_blocks;
  const int nent = (wg_hi >> log2_bs) + 1;  // table entries of keys 0 .. wg_hi
  for (int i = tid; i < nent; i += kThreads) {
    const int b = tbl[i];
    tbl_lds[i] = (b >= 0 && b < num_blocks) ? b : 0;
  }
  __syncthreads();
  constexpr int EB = KV8 ? 1 : 2;  // bytes per cache element
  const int64_t blk_bytes = (int64_t)num_kv_heads * bs * D * EB;  // one block of one cache
  const char *kbase = (const char *)k_cache + (int64_t)kvh * bs * D * EB;
  const char *vbase = (const char *)v_cache + (int64_t)kvh * D * bs * EB;

  // q of this lane's token for the wave's HW heads, as B operands (dims
  // 32ks+8grp..+8)
  u32x4 qf[HW][KSTEPS];
#pragma unroll
  for (int c = 0; c < HW; ++c) {
    const int h = kvh * group + min(chunk * HC + hgrp * HW + c, group - 1);
    const uint16_t *qp = q + ((int64_t)(q0 + tok) * num_heads + h) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[c][ks] = *(const u32x4 *)(qp + ks * 32);
  }

  // Tile loads: a tile is 8*D pieces of 8 elements (16 bytes, or 8 with E4M3
  // codes) of K (piece p: key p / (D/8), dims 8*(p % (D/8)) ..) and 8*D of V
  // (piece p: keys 8*(p / D) .. +7 of dim p % D, two runs of 4 adjacent
  // elements, since the V cache keeps positions in groups of [D][4]).  Wave w's load j moves pieces w*64 + j*threads .. +63 of each:
  // 64 / (D/8) whole K rows, or 64 dims of one key octet, so every piece of
  // one load lies in one cache block (blocks hold at least 8 tokens).  The
  // block base is then a scalar and each lane adds a fixed offset.
  constexpr int KPR = D / 8;  // 16-byte pieces per K row
  constexpr int PIECES = kKT * D / 8;  // 8-element pieces of one cache per tile
  constexpr int NP = (PIECES + kThreads - 1) / kThreads;  // pieces of each cache per lane
  constexpr bool kAllLoad = NP * kThreads == PIECES;      // every lane has NP pieces
  constexpr int KPL = kWave / KPR;  // keys per K load (4 at D = 128, 8 at D = 64)
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const uint32_t koff = (uint32_t)((lane / KPR) * D + (lane % KPR) * 8) * EB;  // bytes
  const uint32_t voff = (uint32_t)(lane * 4) * EB;
  using Piece = std::conditional_t<KV8, u32x2, u32x4>;
  // A ring of kStages register stages: a tile's loads are issued
  // kStages - 1 tiles before they go into LDS, so the wait for them is
  // covered by that many tiles of compute.
  constexpr int kStages = 3;
  Piece st_k[kStages][NP], st_v[kStages][NP];
  auto fetch = [&](int stage, int tile) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int pw = min(wv * kWave + j * kThreads, PIECES - kWave);  // first piece (uniform)
      // the load's keys; past the rows' reach it rereads the group of the
      // last key seen (same block, in bounds)
      const int key0 =
          __builtin_amdgcn_readfirstlane(min(tile * kKT + pw / KPR, wg_hi & ~(KPL - 1)));
      const int blk = __builtin_amdgcn_readfirstlane(tbl_lds[key0 >> log2_bs]);
      const char *src = kbase + blk * blk_bytes + (int64_t)((key0 & (bs - 1)) * D * EB);
      st_k[stage][j] = __builtin_nontemporal_load((const Piece *)(src + koff));
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int pw = min(wv * kWave + j * kThreads, PIECES - kWave);
      // the load's key octet
      const int key0 = __builtin_amdgcn_readfirstlane(min(tile * kKT + (pw / D) * 8, wg_hi & ~7));
      const int blk = __builtin_amdgcn_readfirstlane(tbl_lds[key0 >> log2_bs]);
      const char *src = vbase + blk * blk_bytes +
                        (int64_t)((((key0 & (bs - 1)) >> 2) * D + pw % D) * 4 * EB) + voff;
      using Half = std::conditional_t<KV8, uint32_t, u32x2>;  // 4 keys of one dim
      const Half lo = __builtin_nontemporal_load((const Half *)src);
      const Half hi = __builtin_nontemporal_load((const Half *)(src + D * 4 * EB));
      if constexpr (KV8) st_v[stage][j] = Piece{lo, hi};
      else st_v[stage][j] = Piece{lo.x, lo.y, hi.x, hi.y};
    }
  };
  // bfloat16 V beyond binary16's range (magnitude 65536 and up: the largest
  // bfloat16 value below it is 65280) would saturate in the conversion, so
  // the conversion keeps the largest magnitude it met in vmax; a workgroup
  // that met one reruns its keys in the exact mode (see below).
  constexpr bool kCheckV = DT == 1 && !KV8;
  float vmax = 0.f;
  // Into LDS; V of keys past the workgroup's last position is zeroed there
  // (those keys are not loaded, or lie past the context, and meet weight 0).
  // exact (bfloat16 caches only, for the exact mode below): V stays
  // bfloat16, scaled by 2^-40 (exact down to magnitude 2^-86), so that the
  // fp32 accumulators of up to 2^17 keys times weights up to 2^8 stay finite
  // for every finite bfloat16 V.
  auto stash = [&](auto exact, int stage, int buf, int tile) {
    constexpr bool EXACT = decltype(exact)::value;
    uint16_t *kl = lds + buf * T::elems;
    uint16_t *vl = kl + T::kElems;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int pw = wv * kWave + j * kThreads;
      if (!kAllLoad && pw >= PIECES) break;
      const int p = pw + lane;
      u32x4 kv;
      if constexpr (KV8) kv = e4m3x8_to<DT>(st_k[stage][j]);
      else kv = st_k[stage][j];
      *(u32x4 *)(kl + (p / KPR) * T::kRow + (p % KPR) * 8) = kv;
      const int k8 = (pw / D) * 8;
      // keys the rows can see
      const int valid = __builtin_amdgcn_readfirstlane(wg_hi + 1 - (tile * kKT + k8));
      u32x4 v;
      if constexpr (KV8) {
        v = e4m3x8_to<0>(st_v[stage][j]);  // binary16, exact
      } else {
        v = st_v[stage][j];
      }
      // (zeroing before or after the conversion gives the same bits)
      if (valid < 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = valid - 2 * e;
          v[e] &= c >= 2 ? 0xffffffffu : (c == 1 ? 0x0000ffffu : 0u);
        }
      }
      if constexpr (kCheckV) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xffff0000u);
          if constexpr (EXACT) {
            v[e] = Elem<1>::pack(lo * 0x1p-40f, hi * 0x1p-40f);
          } else {
            vmax = fmaxf(vmax, fmaxf(fabsf(lo), fabsf(hi)));
            v[e] = bf16x2_to_f16x2(v[e]);
          }
        }
      }
      uint16_t *vd = vl + (p % D) * T::vRow + k8;
      if constexpr ((T::vRow * 2) % 16 == 0) {
        *(u32x4 *)vd = v;
      } else {  // V rows are 8-byte aligned only
        *(u32x2 *)vd = u32x2{v.x, v.y};
        *(u32x2 *)(vd + 4) = u32x2{v.z, v.w};
      }
    }
  };

  constexpr float kSlack = 8.f;
  float m_ref[HW], l_run[HW];
  f32x4 acc[HW][DTILES];

  float out_mul = out_scale;  // multiplies the normalised rows
  float thr[HW];  // m_ref + kSlack in units of raw scores
  const float inv_scale = 1.0f / scale_log2;
#pragma unroll
  for (int c = 0; c < HW; ++c) {
    m_ref[c] = -INFINITY;
    thr[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) acc[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Tiles go LDS buffer (tile % 2); tile t's registers sit in stage t % kStages.
#pragma unroll
  for (int b = 0; b < kStages - 1; ++b) fetch(b, min(b, ntiles - 1));
  stash(std::false_type{}, 0, 0, 0);
  __syncthreads();
  for (int tb = 0; tb < ntiles; tb += kStages) {
#pragma unroll
    for (int b = 0; b < kStages; ++b) {
      const int tile = tb + b;
      // past the last tile the ring reloads the last tile (cache hits), so
      // no load sits behind a branch and every wait stays exact
      fetch((b + kStages - 1) % kStages, min(tile + kStages - 1, ntiles - 1));
      if (tile < ntiles) {
        const int buf = tile & 1;
        const int t0 = tile * kKT;
        if (t0 <= wave_hi) {  // the wave sees at least one key of this tile
          const uint16_t *kl = lds + buf * T::elems;
          const uint16_t *vl = kl + T::kElems;
          // raw scores q.k: kRB 16-key row blocks x HW heads; the scale (> 0,
          // in log2 units) joins in the exponent's FMA (the max check below
          // runs on raw scores)
          // k-step outer: the four row blocks' fragments of one k-step are
          // read together, then feed kRB * HW independent accumulations, so
          // no MFMA waits on the one before it or on a read just issued.
          f32x4 sc[kRB][HW];
    #pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
    #pragma unroll
            for (int c = 0; c < HW; ++c) sc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
          // Raised wave priority over the QK MFMAs: when both waves of a
          // SIMD can issue, the one with matrix work goes first and the
          // other fills the vector ALU.
          __builtin_amdgcn_s_setprio(1);
    #pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 ka[kRB];
    #pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              ka[rb] = *(const u32x4 *)(kl + (rb * 16 + col) * T::kRow + ks * 32 + grp * 8);
    #pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
    #pragma unroll
              for (int c = 0; c < HW; ++c) sc[rb][c] = E::mfma(ka[rb], qf[c][ks], sc[rb][c]);
          }
          __builtin_amdgcn_s_setprio(0);
          if (t0 + kKT - 1 > wave_lo) {  // causal edge: keys past a row's position
    #pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
    #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const bool ok = t0 + rb * 16 + grp * 4 + r <= pos;
    #pragma unroll
                for (int c = 0; c < HW; ++c) sc[rb][c][r] = ok ? sc[rb][c][r] : -INFINITY;
              }
          }
          // P^T as B operands, one per 32-key half h: keys 32h+4grp..+3, then
          // 32h+16+4grp..+3 (row blocks 2h and 2h+1)
          u32x4 pb[kNH][HW];
    #pragma unroll
          for (int c = 0; c < HW; ++c) {
            // The reference max moves only when a score passes m_ref + kSlack:
            // each lane checks its own 16 raw scores against that bound (thr,
            // in raw units), and only then is the row max reduced over the
            // row's four lanes (a row whose keys all lie past it gives -inf).
            float lm = -INFINITY;
    #pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              lm = fmaxf(lm, fmaxf(fmaxf(sc[rb][c][0], sc[rb][c][1]), fmaxf(sc[rb][c][2], sc[rb][c][3])));
            if (__ballot(lm > thr[c])) {
              const float mx = rows_max(lm) * scale_log2;
              const float m_new = fmaxf(m_ref[c], mx);
              const float alpha = __builtin_amdgcn_exp2f(m_ref[c] - m_new);
              l_run[c] *= alpha;
    #pragma unroll
              for (int dt = 0; dt < DTILES; ++dt) acc[c][dt] *= alpha;
              m_ref[c] = m_new;
              thr[c] = (m_new + kSlack) * inv_scale;
            }
            float lsum = 0.f;
    #pragma unroll
            for (int h = 0; h < kNH; ++h) {
              float p[8];
    #pragma unroll
              for (int r = 0; r < 4; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * h][c][r], scale_log2, -m_ref[c]));
                p[4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * h + 1][c][r], scale_log2, -m_ref[c]));
              }
              const u32x4 w = {pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]),
                               pack_f16(p[6], p[7])};
              pb[h][c] = w;
              // the row sum takes the fp32 weights; the MFMA multiplies their
              // binary16 roundings (relative error <= 2^-11 each), so an
              // output row is off a convex combination of V rows by at most
              // 2^-11 * max |V|
              lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            }
            l_run[c] += lsum;
          }
          // O^T += V^T P^T over each 32-key half, in the key order of pb
    #pragma unroll
          for (int h = 0; h < kNH; ++h)
    #pragma unroll
            for (int dt = 0; dt < DTILES; ++dt) {
              const uint16_t *vr = vl + (dt * 16 + col) * T::vRow + 32 * h + grp * 4;
              const u32x2 lo = *(const u32x2 *)vr;          // keys 32h+4grp .. +3
              const u32x2 hi = *(const u32x2 *)(vr + 16);   // keys 32h+16+4grp .. +3
              const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
    #pragma unroll
              for (int c = 0; c < HW; ++c) acc[c][dt] = mfma_f16(va, pb[h][c], acc[c][dt]);
            }
        }
        if (tile + 1 < ntiles) {
          // The other buffer was last read in the previous tile, before its
          // barrier, so it can be filled now; the barrier after makes the
          // fill visible before anyone reads it (and keeps any wave from
          // refilling this buffer while another still reads it).
          stash(std::false_type{}, (b + 1) % kStages, buf ^ 1, tile + 1);
          __syncthreads();
        }
      }
    }
  }
  if constexpr (kCheckV) {
    // Exact mode, for the rare workgroup that staged a bfloat16 V beyond
    // binary16's range: the walk again from the first key, one tile at a
    // time (no load ring: this path is short of registers, not of time).
    // The reduction is a barrier, so every wave has left the walk above.
    if (__syncthreads_or(vmax >= 65536.f)) {
      out_mul = 0x1p40f;  // undoes the scaling of V
#pragma unroll
      for (int c = 0; c < HW; ++c) {
        m_ref[c] = -INFINITY;
        l_run[c] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) acc[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int tile = 0; tile < ntiles; ++tile) {
        fetch(0, tile);
        stash(std::true_type{}, 0, 0, tile);
        __syncthreads();
        const int t0 = tile * kKT;
        if (t0 <= wave_hi) {
          const uint16_t *kl = lds;
          const uint16_t *vl = kl + T::kElems;
          f32x4 sc[kRB][HW];
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int c = 0; c < HW; ++c) sc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              const u32x4 ka = *(const u32x4 *)(kl + (rb * 16 + col) * T::kRow + ks * 32 + grp * 8);
#pragma unroll
              for (int c = 0; c < HW; ++c) sc[rb][c] = E::mfma(ka, qf[c][ks], sc[rb][c]);
            }
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool ok = t0 + rb * 16 + grp * 4 + r <= pos;
#pragma unroll
              for (int c = 0; c < HW; ++c) sc[rb][c][r] = ok ? sc[rb][c][r] : -INFINITY;
            }
#pragma unroll
          for (int c = 0; c < HW; ++c) {
            float mx = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              mx = fmaxf(mx, fmaxf(fmaxf(sc[rb][c][0], sc[rb][c][1]), fmaxf(sc[rb][c][2], sc[rb][c][3])));
            mx = rows_max(mx) * scale_log2;
            if (__ballot(mx > m_ref[c] + kSlack)) {
              const float m_new = fmaxf(m_ref[c], mx);
              const float alpha = __builtin_amdgcn_exp2f(m_ref[c] - m_new);
              l_run[c] *= alpha;
#pragma unroll
              for (int dt = 0; dt < DTILES; ++dt) acc[c][dt] *= alpha;
              m_ref[c] = m_new;
            }
            float lsum = 0.f;
#pragma unroll
            for (int h = 0; h < kNH; ++h) {
              // weights of keys 32h+4grp..+3 and 32h+16+4grp..+3 as
              // bfloat16 hi + lo (16 significant bits)
              float p[8];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * h][c][r], scale_log2, -m_ref[c]));
                p[4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[2 * h + 1][c][r], scale_log2, -m_ref[c]));
              }
              u32x4 w, lo;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                w[e] = Elem<1>::pack(p[2 * e], p[2 * e + 1]);
                lo[e] = Elem<1>::pack(p[2 * e] - __uint_as_float(w[e] << 16),
                                      p[2 * e + 1] - __uint_as_float(w[e] & 0xffff0000u));
              }
              lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
              for (int dt = 0; dt < DTILES; ++dt) {
                const uint16_t *vr = vl + (dt * 16 + col) * T::vRow + 32 * h + grp * 4;
                const u32x2 a = *(const u32x2 *)vr;
                const u32x2 b = *(const u32x2 *)(vr + 16);
                const u32x4 va = {a.x, a.y, b.x, b.y};
                acc[c][dt] = Elem<1>::mfma(va, w, acc[c][dt]);
                acc[c][dt] = Elem<1>::mfma(va, lo, acc[c][dt]);
              }
            }
            l_run[c] += lsum;
          }
        }
        __syncthreads();  // before the next tile overwrites the buffer
      }
    }
  }
  // rows of this lane: token col of the wave, heads c; lane holds dims
  // 16*dt + 4*grp + 0..3
  float inv[HW];
#pragma unroll
  for (int c = 0; c < HW; ++c) inv[c] = out_mul / rows_sum(l_run[c]);  // whole wave
  const int row = wt0 + col;
  if (row < n) {
#pragma unroll
    for (int c = 0; c < HW; ++c) {
      const int hg = chunk * HC + hgrp * HW + c;
      if (hg >= group) continue;
      uint16_t *op = out + ((int64_t)(q0 + row) * num_heads + kvh * group + hg) * D + grp * 4;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        u32x2 w;
        w.x = E::pack(acc[c][dt][0] * inv[c], acc[c][dt][1] * inv[c]);
        w.y = E::pack(acc[c][dt][2] * inv[c], acc[c][dt][3] * inv[c]);
        *(u32x2 *)(op + dt * 16) = w;
      }
    }
  }
}

template <int DT, int D, int HW, int NWH, bool KV8>
int launch_hc(const PrefillArgs &a) {
  constexpr int HC = HW * NWH;
  const int group = a.num_heads / a.num_kv_heads;
  const int chunks = (group + HC - 1) / HC;
  const int nqb = (a.max_query_len + kQB - 1) / kQB;
  const int64_t groups = (int64_t)nqb * a.num_seqs * a.num_kv_heads * chunks;
  if (groups == 0) return 0;
  if (groups > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  // log2(e) folds the exponential's base into the score scale; an E4M3
  // cache's k_scale multiplies every score and its v_scale every output.
  const float scale_log2 =
      (float)((double)a.scale * (KV8 ? (double)a.k_scale : 1.0) * 1.4426950408889634);
  const float out_scale = KV8 ? a.v_scale : 1.0f;
  const size_t lds = 2 * sizeof(uint16_t) * Tile<D>::elems + sizeof(int32_t) * a.max_blocks_per_seq;
  prefill_kernel<DT, D, HW, NWH, KV8>
      <<<dim3((unsigned)groups), kWave * kTG * NWH, lds, (hipStream_t)a.stream>>>(
          (uint16_t *)a.out, (const uint16_t *)a.q, a.k_cache, a.v_cache, a.block_tables,
          a.context_lens, a.query_start, scale_log2, out_scale, log2_bs, a.num_seqs,
          a.num_kv_heads, a.num_heads, group, chunks, a.max_blocks_per_seq, a.num_blocks, nqb);
  return (int)hipGetLastError();
}

template <int DT, int D, bool KV8>
int launch_d(const PrefillArgs &a) {
  const int group = a.num_heads / a.num_kv_heads;
  if (group == 1) return launch_hc<DT, D, 1, 1, KV8>(a);
  if (group == 2) return launch_hc<DT, D, 2, 1, KV8>(a);
  return launch_hc<DT, D, 2, 2, KV8>(a);
}

template <int DT, bool KV8>
int launch_dt(const PrefillArgs &a) {
  return a.head_dim == 64 ? launch_d<DT, 64, KV8>(a) : launch_d<DT, 128, KV8>(a);
}

}  // namespace

int launch_prefill(const PrefillArgs &a) {
  if (a.kv_fp8) return a.dtype == 1 ? launch_dt<1, true>(a) : launch_dt<0, true>(a);
  return a.dtype == 1 ? launch_dt<1, false>(a) : launch_dt<0, false>(a);
}

}  // namespace pa
