// Paged decode attention for gfx950 (CDNA4).
//
// Method: "vLLM memory management and continuous batching from the source"
// (developer.cloud.tencent.cn), part 2, 2.3 -- attention receives block
// tables instead of a contiguous (batch, seq_len, dim) tensor and gathers
// K/V through them; 2.1 -- a token lives in block table[t / block_size] at
// offset t % block_size.  The math is plain softmax(scale * q K^T) V per
// query head, computed with a running max and sum over 16-token tiles; a
// sequence split across several wavefronts is merged by log-sum-exp.
//
// Work split ("flat split-K").  For one KV head, the 16-token tiles of all
// sequences are laid end to end (sequence s owns tiles cu[s] .. cu[s+1]-1)
// and cut into `waves` equal contiguous ranges, one wavefront each, so every
// wavefront streams the same number of bytes whatever the length mix.  A
// range may end inside one sequence and start inside another: the wavefront
// then produces one partial result (m, l, o) per sequence segment, in slot
// (wave + sequence) of the workspace, and the merge pass combines the
// partials of each sequence.  A sequence held entirely by one wavefront is
// written to `out` directly.  Wavefront (kv head h, range j) is workgroup
// j * num_kv_heads + h: workgroups go to the eight XCDs round-robin in
// launch order, so with kv head fastest each XCD streams an equal share.
//
// Per 16-token tile, with G <= 16 query heads padded to 16:
//   S^T[16 tok x 16 head] = K[16 tok x D] * Q^T[D x 16 head]
//        -> D/32 MFMA 16x16x32; A = K rows as stored (token-major cache),
//           each lane loading 16 contiguous bytes of one token's row (E4M3
//           at D = 128: loaded as whole lines and rearranged through LDS).
//   O^T[D x 16 head]     += V^T[D x 16 tok] * P^T[16 tok x 16 head]
//        -> D/16 MFMA 16x16x16; A = V^T read straight from the V cache,
//           whose (block, head) slice is block_size/4 groups of [D][4]
//           (4 tokens of one dim adjacent; each lane loads 16 bytes, the
//           4 tokens of VG adjacent dims, see VLayout),
//           B = P exactly as the QK MFMA left it in registers (lane l holds
//           head l%16, tokens 4*(l/16)+0..3), so no shuffle is needed.
//           For bfloat16 caches, P goes in as a hi and a lo bfloat16 part
//           (two MFMAs) so the weights keep ~16 significant bits; over
//           binary16 and E4M3 caches it is one binary16 MFMA.
// Every lane's softmax state and accumulators belong to head l%16, so the
// rescale by exp(m_old - m_new) is lane-local; only the tile max (when a
// lane's own scores pass the current reference by the slack) and the
// final sum cross the wave's four 16-lane rows (permlane16/32 swaps).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "pa_device.h"
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
  // four E4M3 codes (bytes 0..3) -> four bfloat16 values, exact
  static __device__ __forceinline__ u32x2 from_e4m3(uint32_t c) {
    return u32x2{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true))};
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
  // four E4M3 codes (bytes 0..3) -> four binary16 values, exact
  static __device__ __forceinline__ u32x2 from_e4m3(uint32_t c) {
    return u32x2{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, true))};
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



// Inclusive prefix sum over the wave's 64 lanes, by DPP: shifts by 1, 2, 4
// and 8 within each row of 16 lanes (sources outside the row read 0), then
// row 0's total joins row 1 and row 2's joins row 3 (broadcast of lanes 15
// and 47), then lane 31's (rows 0-1) joins rows 2 and 3.  Rows that a
// broadcast does not enable keep their value.  No LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Wavefront whose range [j*n/w, (j+1)*n/w) holds flat tile tau (0 <= tau < n,
// 1 <= w <= n, so that no range is empty).
__device__ __forceinline__ int wave_of(int tau, int n, int w) {
  return (int)((((int64_t)tau + 1) * w - 1) / n);
}

// K and V registers of one 16-token tile as loaded: 16-bit values, or E4M3
// codes (KV8) that step() converts to the q type before the MFMAs.
template <int D, bool KV8>
struct Frag;
template <int D>
struct Frag<D, false> {
  u32x4 k[D / 32];  // one 16x16x32 A fragment per k-step
  u32x2 v[D / 16];  // 4 tokens of one dimension per fragment (see vdim)
};
template <int D>
struct Frag<D, true> {
  u32x4 k[D / 64];     // 16 codes = two k-steps
  uint32_t v[D / 16];  // 4 token codes of one dimension per fragment (see vdim)
};

// V fragment layout.  Each lane loads 16 bytes of one 4-token group per
// load, VG adjacent dimensions (VG = 16 / (4 tokens x element bytes): 4
// for E4M3 codes, 2 for 16-bit values), so that the 16 lanes of a quarter
// read one contiguous 256-byte run of the cache's [D][4] group.  V^T
// fragment dt (one 16x16 MFMA A operand, rows i = 0..15) then holds dims
// 16*VG*(dt/VG) + VG*i + dt%VG, and the output lanes hold 4*VG adjacent
// dims per group of VG fragments (see vdim).
template <bool KV8>
struct VLayout {
  static constexpr int VG = KV8 ? 4 : 2;
};
// dimension of row i of V fragment dt
template <bool KV8>
__device__ __forceinline__ constexpr int vdim(int dt, int i) {
  constexpr int VG = VLayout<KV8>::VG;
  return 16 * VG * (dt / VG) + VG * i + dt % VG;
}

// Tiles in flight per wave (register ring depth).
constexpr int kBuf = 2;

// V registers of one tile from 16-byte loads: group g (fragments VG*g ..
// VG*g + VG-1) at element offset 64*VG*g from vp, which points at this
// lane's first dimension (VG*row) of its 4-token group.
template <int D, bool KV8, bool NT, typename CT>
__device__ __forceinline__ void load_v(Frag<D, KV8> &f, const CT *vp) {
  constexpr int VG = VLayout<KV8>::VG;
#pragma unroll
  for (int g = 0; g < D / 16 / VG; ++g) {
    const u32x4 *src = (const u32x4 *)(vp + 64 * VG * g);
    const u32x4 w = NT ? __builtin_nontemporal_load(src) : *src;
    if constexpr (KV8) {
      f.v[4 * g] = w.x; f.v[4 * g + 1] = w.y; f.v[4 * g + 2] = w.z; f.v[4 * g + 3] = w.w;
    } else {
      f.v[2 * g] = u32x2{w.x, w.y}; f.v[2 * g + 1] = u32x2{w.z, w.w};
    }
  }
}

// One (sequence, head) row of results, scaled: acc[dt][r] holds the
// fragment layout's dim vdim(dt, 4*grp + r); lane (., grp) writes its 4*VG
// adjacent dims of each group g, at 16*VG*g + 4*VG*grp.
template <int D, bool KV8, typename F>
__device__ __forceinline__ void row_values(const f32x4 (&acc)[D / 16], int g, F &&emit) {
  constexpr int VG = VLayout<KV8>::VG;
#pragma unroll
  for (int c = 0; c < VG; ++c) {  // f32x4 chunk c: elements 4c .. 4c+3
    f32x4 v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = 4 * c + t;  // element e = VG*r + j
      v[t] = acc[VG * g + e % VG][e / VG];
    }
    emit(c, v);
  }
}

// Lazy rescale slack (log2 units): the reference max is raised only when a
// tile's max exceeds it by more than this.
constexpr float kSlack = 8.f;

// Tiles in flight per shared-prefix wavefront.
constexpr int kSharedBuf = 2;

// One wavefront of a shared prefix ("vLLM framework analysis: how
// PagedAttention speeds up LLM inference 20x" (intelliparadigm.com), 2.3:
// sequences hold a common prompt's blocks by reference).  Every sequence's
// first sh.tiles tiles are the same blocks, so one wavefront streams a chunk
// of them once for the query heads of kSharedGroups * seqs_per_group
// sequences: per tile, the K and V fragments are the A operands of the MFMAs
// of every 16-column group (column c of group gi: sequence
// (colset * kSharedGroups + gi) * seqs_per_group + c / G, head c % G).  Each
// (sequence, query head) leaves one partial (o, m, l) per chunk for the
// merge.  The prefix is read through the caches (other column sets read the
// same chunk), and every tile is full.
template <int DT, int D, int BS, bool KV8>
__device__ __forceinline__ void shared_prefix_wave(
    const SharedPrefix &sh, int sw, int kvh, const uint16_t *__restrict__ q,
    const void *__restrict__ k_cache, const void *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, float scale_log2, float out_scale,
    int num_seqs, int num_kv_heads, int num_heads, int group, int64_t num_blocks) {
  using E = Elem<DT>;
  // P.V over E4M3 caches in binary16 (every code value is one; weights
  // keep 11 significant bits), otherwise in the caches' type
  using PE = std::conditional_t<KV8, Elem<kF16>, E>;
  using CT = std::conditional_t<KV8, uint8_t, uint16_t>;
  constexpr int KSTEPS = D / 32;
  constexpr int DTILES = D / 16;
  constexpr int NG = kSharedGroups;
  const int lane = threadIdx.x;
  const int row = lane & 15;
  const int grp = lane >> 4;
  // the column sets of one chunk are adjacent in launch order, so they run
  // together and share the chunk in the caches
  const int ch = sw / sh.colsets;
  const int cs = sw - ch * sh.colsets;
  const int tbeg = ch * sh.chunk_tiles;
  const int cnt = min(sh.chunk_tiles, sh.tiles - tbeg);  // >= 1

  // Lane l describes prefix tile tbeg + l (lanes past the chunk repeat its
  // last tile): its block ids, from sequence 0's row of the table.
  const int it = tbeg + min(lane, cnt - 1);
  int b0, b1 = 0, boff = 0;
  if constexpr (BS == 8) {
    b0 = block_tables[2 * it];
    b1 = block_tables[2 * it + 1];
  } else if constexpr (BS == 16) {
    b0 = block_tables[it];
  } else {
    b0 = block_tables[it >> 1];
    boff = (it & 1) * kTile;
  }
  b0 = (b0 >= 0 && b0 < num_blocks) ? b0 : 0;  // ids outside the pool: stay inside it
  b1 = (b1 >= 0 && b1 < num_blocks) ? b1 : 0;

  // Query fragments of both column groups, held for the whole chunk (the
  // dimension order of the private path: E4M3 codes come 16 to a lane).
  int seq[NG], head[NG];
  bool valid[NG];
  u32x4 qf[NG][KSTEPS];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int s0 = (cs * NG + gi) * sh.seqs_per_group;
    const int sq = s0 + row / group;
    valid[gi] = row < sh.seqs_per_group * group && sq < num_seqs;
    seq[gi] = valid[gi] ? sq : min(s0, num_seqs - 1);
    head[gi] = kvh * group + (valid[gi] ? row % group : 0);
    const uint16_t *qp = q + ((int64_t)seq[gi] * num_heads + head[gi]) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d0 = KV8 ? 64 * (ks / 2) + 16 * grp + 8 * (ks % 2) : 32 * ks + 8 * grp;
      qf[gi][ks] = *(const u32x4 *)(qp + d0);
    }
  }

  const int64_t blk_stride = (int64_t)num_kv_heads * BS * D;
  const CT *kbase = static_cast<const CT *>(k_cache) + (int64_t)kvh * BS * D;
  const CT *vbase = static_cast<const CT *>(v_cache) + (int64_t)kvh * D * BS;
  // Loads of one full tile: lane (row, grp) reads token row's K dims and the
  // four tokens 4 * grp .. +3 of V dimensions vdim(dt, row).
  auto load = [&](Frag<D, KV8> &f, int idx) {
    const int ka = __builtin_amdgcn_readlane(b0, idx);
    const CT *kp, *vp;
    if constexpr (BS == 8) {
      const int kz = __builtin_amdgcn_readlane(b1, idx);
      kp = kbase + (int64_t)(row < 8 ? ka : kz) * blk_stride + (row & 7) * D + grp * (KV8 ? 16 : 8);
      vp = vbase + (int64_t)(grp < 2 ? ka : kz) * blk_stride +
           ((grp & 1) * D + VLayout<KV8>::VG * row) * 4;
    } else {
      const int o = BS == 16 ? 0 : __builtin_amdgcn_readlane(boff, idx);
      const CT *kblk = kbase + (int64_t)ka * blk_stride + o * D;
      const CT *vblk = vbase + (int64_t)ka * blk_stride;
      kp = kblk + (uint32_t)(row * D + grp * (KV8 ? 16 : 8));
      vp = vblk + (uint32_t)((((o >> 2) + grp) * D + VLayout<KV8>::VG * row) * 4);
    }
    if constexpr (KV8) {
#pragma unroll
      for (int h = 0; h < D / 64; ++h) f.k[h] = *(const u32x4 *)(kp + h * 64);
    } else {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) f.k[ks] = *(const u32x4 *)(kp + ks * 32);
    }
    load_v<D, KV8, false>(f, vp);
  };

  float m_ref[NG], l_run[NG];
  float thr[NG];  // m_ref + kSlack in units of raw scores
  const float inv_scale = 1.0f / scale_log2;
  f32x4 acc[NG][DTILES];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m_ref[gi] = -INFINITY;
    thr[gi] = -INFINITY;
    l_run[gi] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) acc[gi][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile for both column groups: scores, lazy online softmax, P.V.
  auto step = [&](Frag<D, KV8> &f) {
    u32x4 kf[KSTEPS];
    u32x2 vv[DTILES];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (KV8) {
        const u32x4 c = f.k[ks / 2];
        const u32x2 a = E::from_e4m3(ks % 2 ? c.z : c.x);
        const u32x2 b = E::from_e4m3(ks % 2 ? c.w : c.y);
        kf[ks] = u32x4{a.x, a.y, b.x, b.y};
      } else {
        kf[ks] = f.k[ks];
      }
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      if constexpr (KV8) vv[dt] = PE::from_e4m3(f.v[dt]);
      else vv[dt] = f.v[dt];
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) sc = E::qk(kf[ks], qf[gi][ks], sc);
      // raw scores, checked lane by lane against thr before any reduction
      // (as in the split pass); the scale joins in the exponent's FMA
      const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__ballot(lm > thr[gi])) {
        const float mx = rows_max(lm) * scale_log2;
        const float m_new = fmaxf(m_ref[gi], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_ref[gi] - m_new);
        l_run[gi] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) acc[gi][dt] *= alpha;
        m_ref[gi] = m_new;
        thr[gi] = (m_new + kSlack) * inv_scale;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -m_ref[gi]));
      u32x2 ph, pl;
      ph.x = PE::pack(p[0], p[1]);
      ph.y = PE::pack(p[2], p[3]);
      if constexpr (PE::kSplitP) {
        pl.x = PE::pack(p[0] - PE::lo(ph.x), p[1] - PE::hi(ph.x));
        pl.y = PE::pack(p[2] - PE::lo(ph.y), p[3] - PE::hi(ph.y));
        l_run[gi] += (p[0] + p[1]) + (p[2] + p[3]);
      } else {
        l_run[gi] += (PE::lo(ph.x) + PE::hi(ph.x)) + (PE::lo(ph.y) + PE::hi(ph.y));
      }
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        acc[gi][dt] = PE::pv(vv[dt], ph, acc[gi][dt]);
        if constexpr (PE::kSplitP) acc[gi][dt] = PE::pv(vv[dt], pl, acc[gi][dt]);
      }
    }
  };

  Frag<D, KV8> f[kSharedBuf];
#pragma unroll
  for (int b = 0; b < kSharedBuf - 1; ++b) load(f[b], min(b, cnt - 1));
  __builtin_amdgcn_sched_barrier(0);
  for (int t = 0; t < cnt; t += kSharedBuf) {
#pragma unroll
    for (int b = 0; b < kSharedBuf; ++b) {
      load(f[(b + kSharedBuf - 1) % kSharedBuf], min(t + b + kSharedBuf - 1, cnt - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (t + b < cnt) step(f[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The chunk's partial of each (sequence, query head): lane (row, grp)
  // holds dims vdim(dt, 4 * grp + 0..3) of column row.
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l_tot = rows_sum(l_run[gi]);
    if (valid[gi]) {
      const int64_t slot = ((int64_t)head[gi] * num_seqs + seq[gi]) * sh.chunks + ch;
      const float inv = out_scale / l_tot;
      constexpr int VG = VLayout<KV8>::VG;
      float *op = sh.o + slot * D + grp * 4 * VG;
#pragma unroll
      for (int g = 0; g < DTILES / VG; ++g)
        row_values<D, KV8>(acc[gi], g, [&](int c, f32x4 v) {
          *(f32x4 *)(op + 16 * VG * g + 4 * c) = v * inv;
        });
      if (grp == 0) *(f32x2 *)(sh.ml + slot * 2) = f32x2{m_ref[gi], l_tot};
    }
  }
}

// KV8: the caches hold E4M3 codes; scale_log2 then carries k_scale and
// out_scale is v_scale (1 for 16-bit caches).  APPEND: the fused decode
// step, whose new tokens come from k_new / v_new (position L - 1).
// SHARED: every sequence's first sh.tiles tiles are one shared prefix; the
// first sh.waves * num_kv_heads workgroups stream it (shared_prefix_wave),
// the others split only the tiles past it, and every sequence segment
// leaves a partial for the merge.
template <int DT, int D, int BS, bool KV8, bool APPEND, bool SHARED>
__global__ __launch_bounds__(kWave) void decode_split_kernel(
    uint16_t *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int32_t *__restrict__ ws_cu, const uint16_t *__restrict__ q,
    void *__restrict__ k_cache, void *__restrict__ v_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    float scale_log2, float out_scale, float k_inv, float v_inv, int num_seqs,
    int num_kv_heads, int num_heads, int group, int max_blocks, int waves, int slots,
    int64_t num_blocks, SharedPrefix sh) {
  // (waves sits next to the other sizes, in the argument line that the first
  // scalar loads fetch: it is needed right after the length scan)
  using E = Elem<DT>;
  // P.V over E4M3 caches in binary16 (every code value is one; weights
  // keep 11 significant bits), otherwise in the caches' type
  using PE = std::conditional_t<KV8, Elem<kF16>, E>;
  using CT = std::conditional_t<KV8, uint8_t, uint16_t>;  // cache element
  constexpr int KSTEPS = D / 32;  // 16x16x32 MFMAs per QK tile
  constexpr int DTILES = D / 16;  // 16x16x16 MFMAs per PV tile
  constexpr int PER = D / kWave;  // elements of a K or V row per lane
  // LDS: cu[num_seqs + 1], lens[num_seqs], then (16-byte aligned) the
  // current segment's query fragments, lane-major per k-step; with APPEND
  // also the new token's K and V rows of the current segment's sequence
  // (16-bit), and for KV8 their E4M3 codes; for KV8 at D = 128 one tile's K
  // codes; last, the first segment's partial result.
  extern __shared__ __align__(16) int lds[];
  int *cu = lds;
  int *lens = lds + num_seqs + 1;
  u32x4 *q_lds = reinterpret_cast<u32x4 *>(lds + ((2 * num_seqs + 1 + 3) & ~3));
  uint16_t *kn_raw = reinterpret_cast<uint16_t *>(q_lds + KSTEPS * kWave);
  uint16_t *vn_raw = kn_raw + D;
  CT *kn_lds = KV8 ? reinterpret_cast<CT *>(vn_raw + D) : reinterpret_cast<CT *>(kn_raw);
  CT *vn_lds = KV8 ? kn_lds + D : reinterpret_cast<CT *>(vn_raw);
  // E4M3 at D = 128: one tile's K codes, 16 token rows of 144 bytes (128
  // + 16 of padding, so that the fragment reads spread over the banks)
  constexpr bool kKT = KV8 && D == 128;
  constexpr int kKTRow = 144;
  uint8_t *kt_lds = reinterpret_cast<uint8_t *>(q_lds + KSTEPS * kWave) + (APPEND ? 6 * D : 0);
  // The partial result of the wavefront's first segment (group rows of D
  // floats, then group (m, l) pairs), kept here until the tile loop is done.
  float *stg = reinterpret_cast<float *>(kt_lds + (kKT ? 16 * kKTRow : 0));

  int bid = blockIdx.x;
  if constexpr (SHARED) {
    const int nsh = sh.waves * num_kv_heads;
    if (bid < nsh) {
      shared_prefix_wave<DT, D, BS, KV8>(sh, bid / num_kv_heads, bid % num_kv_heads, q,
                                         k_cache, v_cache, block_tables, scale_log2,
                                         out_scale, num_seqs, num_kv_heads, num_heads, group,
                                         num_blocks);
      return;
    }
    bid -= nsh;
  }
  const int kvh = bid % num_kv_heads;
  const int j = bid / num_kv_heads;
  const int lane = threadIdx.x;
  const int row = lane & 15;  // A-row / B-column / head index inside a tile
  const int grp = lane >> 4;  // quarter of the wave: k-slice and 4-row group
  const int max_len = max_blocks * BS;

  // Tile prefix over all sequences (the same in every wavefront); with a
  // shared prefix, over the tiles past it.  Range-0 wavefronts also write the
  // zero rows of sequences with nothing to attend.
  // With a fused append the last position L - 1 is the new token: the
  // wavefront holding that tile takes its K and V from k_new / v_new
  // instead of the cache and stores them into the cache slot.
  // The lengths of kScanChunks chunks of 64 sequences are loaded together,
  // so that they cost one round trip, and their scans are independent until
  // the chunks' totals are added in.  The loads take no branch: lanes past
  // the last sequence read its length again and drop it (a branch around
  // each load made each one wait for its own data).
  constexpr int kScanChunks = 4;
  int carry = 0;
  int c0 = 0;
  do {  // num_seqs >= 1: no test before the first group's loads
    int len[kScanChunks], incl[kScanChunks];
#pragma unroll
    for (int b = 0; b < kScanChunks; ++b)
      len[b] = context_lens[min(c0 + b * kWave + lane, num_seqs - 1)];
#pragma unroll
    for (int b = 0; b < kScanChunks; ++b) {
      len[b] = c0 + b * kWave + lane < num_seqs ? min(max(len[b], 0), max_len) : 0;
      const int own = SHARED ? max((len[b] + kTile - 1) / kTile - sh.tiles, 0)
                             : (len[b] + kTile - 1) / kTile;
      incl[b] = wave_incl_scan(own);
    }
#pragma unroll
    for (int b = 0; b < kScanChunks; ++b) {
      const int c = c0 + b * kWave;
      const int s = c + lane;
      const int total = __builtin_amdgcn_readlane(incl[b], kWave - 1);
      if (s < num_seqs) {
        cu[s + 1] = incl[b] + carry;
        lens[s] = len[b];
      }
      carry += total;
      if (!SHARED && j == 0) {
        uint64_t zero = __ballot(s < num_seqs && len[b] == 0);
        while (zero) {
          const int zs = c + __builtin_ctzll(zero);
          zero &= zero - 1;
          uint16_t *op = out + ((int64_t)zs * num_heads + kvh * group) * D;
          for (int e = lane * 4; e < group * D; e += kWave * 4) *(u32x2 *)(op + e) = u32x2{0, 0};
        }
      }
    }
    c0 += kScanChunks * kWave;
  } while (c0 < num_seqs);
  if (lane == 0) cu[0] = 0;
  __syncthreads();
  const int n_tiles = __builtin_amdgcn_readfirstlane(carry);  // uniform: scalar loop control
  if (kvh == 0 && j == 0)  // for the merge pass
    for (int s = lane; s <= num_seqs; s += kWave) ws_cu[s] = cu[s];

  // With fewer tiles than wavefronts only the first n_tiles take part, so
  // that every range is non-empty (the merge pass relies on it).
  const int wv = min(waves, n_tiles);
  if (j >= wv) return;
  const int t0 = (int)((int64_t)j * n_tiles / wv);
  const int t1 = (int)((int64_t)(j + 1) * n_tiles / wv);
  const int cnt = t1 - t0;  // 1 .. 64: the host makes waves >= tiles / 64

  // Lane l describes flat tile t0 + l (lanes past the range repeat the last
  // one and are never read): its sequence, tile index in that sequence,
  // valid tokens, block ids, and whether a sequence segment ends there.
  const int tau = t0 + min(lane, cnt - 1);
  int lo = 0, hi = num_seqs - 1;  // the largest s with cu[s] <= tau
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tau) lo = mid;
    else hi = mid - 1;
  }
  const int sq = lo;
  const int first = cu[sq];
  const int ntiles_sq = cu[sq + 1] - first;
  const int rel = tau - first;                  // among the sequence's split tiles
  const int it = rel + (SHARED ? sh.tiles : 0);  // tile index in the sequence
  const int nvalid = min(kTile, lens[sq] - it * kTile);  // >= 1
  const int32_t *tbl = block_tables + (int64_t)sq * max_blocks;
  int b0, b1 = 0, boff = 0;
  if constexpr (BS == 8) {  // two blocks per tile
    b0 = tbl[2 * it];
    b1 = nvalid > 8 ? tbl[2 * it + 1] : b0;
  } else if constexpr (BS == 16) {
    b0 = tbl[it];
  } else {  // half a block per tile
    b0 = tbl[it >> 1];
    boff = (it & 1) * kTile;
  }
  // Fused append: the sequence's last tile holds the new token at row
  // nvalid - 1; nblk is its block (-1 if the id is outside the pool: the
  // token then enters the attention but is not stored).
  const bool is_new = APPEND && rel == ntiles_sq - 1;
  const int nraw = (BS == 8 && nvalid > 8) ? b1 : b0;
  const int nblk = (is_new && nraw >= 0 && nraw < num_blocks) ? nraw : -1;
  b0 = (b0 >= 0 && b0 < num_blocks) ? b0 : 0;  // ids outside the pool: stay inside it
  b1 = (b1 >= 0 && b1 < num_blocks) ? b1 : 0;
  const int seg_end = (rel == ntiles_sq - 1 || tau == t1 - 1) ? 1 : 0;
  // (with a shared prefix no wavefront holds a whole sequence)
  const int whole = (!SHARED && first >= t0 && first + ntiles_sq <= t1) ? 1 : 0;
  const uint64_t ends = __ballot(seg_end && lane < cnt);  // bit i: a segment ends at tile i
  // The flags of tile t0 + lane in one word, so that one readlane per tile
  // fetches them: bits 0-4 valid tokens, 5 segment end, 6 whole sequence,
  // 7 the sequence's new token (fused append).
  constexpr int kEnd = 1 << 5, kWhole = 1 << 6, kNew = 1 << 7;
  const int meta = nvalid | (seg_end ? kEnd : 0) | (whole ? kWhole : 0) | (is_new ? kNew : 0);

  // Query fragment of the current segment and, one segment ahead, of the
  // next.  Lane (row, grp) holds 8 dims of head row per k-step: dims
  // 32*ks + 8*grp .. +8 for 16-bit caches; for E4M3 caches, whose lanes
  // load 16 codes at once, dims 64*(ks/2) + 16*grp + 8*(ks%2) .. +8 (the
  // same permutation of the dimensions on both operands of the dot product).
  // Padded head lanes (row >= group) read a real query row and compute
  // values that are never stored.
  const int qh = kvh * group + min(row, group - 1);
  auto load_q = [&](u32x4 (&dst)[KSTEPS], int idx) {
    const int s = __builtin_amdgcn_readlane(sq, idx);
    const uint16_t *qp = q + ((int64_t)s * num_heads + qh) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d0 = KV8 ? 64 * (ks / 2) + 16 * grp + 8 * (ks % 2) : 32 * ks + 8 * grp;
      dst[ks] = *(const u32x4 *)(qp + d0);
    }
  };
  // first tile of the segment after the one ending at tile `e` (cnt - 1 if none)
  auto next_first = [&](int e) {
    return e + 1 < cnt ? e + 1 : cnt - 1;
  };
  // The current fragment lives in LDS and is read there each tile; only the
  // next segment's, prefetched one segment ahead, is held in registers.
  // (Two register sets swapped at segment ends make the compiler copy a
  // fresh load, which waits for it and drains the ring.)
  // With APPEND the new token's K and V rows go the same way, PER elements
  // per lane.
  uint32_t knx[PER], vnx[PER];
  int first_sq = -1;  // sequence of a first-segment partial waiting in LDS
  auto load_new = [&](int idx) {
    if constexpr (APPEND) {
      const int s = __builtin_amdgcn_readlane(sq, idx);
      const int64_t src = ((int64_t)s * num_kv_heads + kvh) * D + lane * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        knx[i] = k_new[src + i];
        vnx[i] = v_new[src + i];
      }
    }
  };
  auto publish_new = [&]() {
    if constexpr (APPEND) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        kn_raw[lane * PER + i] = (uint16_t)knx[i];
        vn_raw[lane * PER + i] = (uint16_t)vnx[i];
      }
    }
  };
  u32x4 qnext[KSTEPS];
  load_q(qnext, 0);
  load_new(0);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) q_lds[ks * kWave + lane] = qnext[ks];
  publish_new();
  __builtin_amdgcn_sched_barrier(0);
  load_q(qnext, next_first(__builtin_ctzll(ends)));
  load_new(next_first(__builtin_ctzll(ends)));
  const int64_t blk_stride = (int64_t)num_kv_heads * BS * D;  // elements per block
  const CT *kbase = static_cast<const CT *>(k_cache) + (int64_t)kvh * BS * D;
  const CT *vbase = static_cast<const CT *>(v_cache) + (int64_t)kvh * D * BS;

  // Loads of one tile (idx = position in the range, < cnt), straight-line:
  // no branch around them, so the wait for one tile never waits for the
  // prefetched ones.  Token indices are clamped to the tile's valid tokens;
  // what a clamped lane reads is masked away by step().  K and V are read
  // once per launch, so they bypass the caches' normal replacement.
  auto load = [&](Frag<D, KV8> &f, int idx) {
    const int mt = __builtin_amdgcn_readlane(meta, idx);
    const int n = mt & 31;
    const int ka = __builtin_amdgcn_readlane(b0, idx);
    const int ktok = min(row, n - 1);
    const int vtok = min(grp * 4, (n - 1) & ~3);  // this lane's 4-token group
    const CT *kp, *vp;
    if constexpr (BS == 8) {  // the tile's two blocks: per-lane choice
      const int kz = __builtin_amdgcn_readlane(b1, idx);
      kp = kbase + (int64_t)(ktok < 8 ? ka : kz) * blk_stride + (ktok & 7) * D + grp * (KV8 ? 16 : 8);
      vp = vbase + (int64_t)(vtok < 8 ? ka : kz) * blk_stride +
           (((vtok & 7) >> 2) * D + VLayout<KV8>::VG * row) * 4;
    } else {
      // block base in scalar registers, 32-bit lane offsets
      const int o = BS == 16 ? 0 : __builtin_amdgcn_readlane(boff, idx);
      const CT *kblk = kbase + (int64_t)ka * blk_stride + o * D;
      const CT *vblk = vbase + (int64_t)ka * blk_stride;
      kp = kblk + (uint32_t)(ktok * D + grp * (KV8 ? 16 : 8));
      vp = vblk + (uint32_t)((((o + vtok) >> 2) * D + VLayout<KV8>::VG * row) * 4);
    }
    if constexpr (kKT) {
      // whole lines: load h reads tokens 8h .. 8h+7, lane l 16 codes of
      // token 8h + l/8 (clamped to the valid ones) at 16 * (l % 8)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = min(8 * h + (lane >> 3), n - 1);
        const CT *src;
        if constexpr (BS == 8) {
          const int kz = __builtin_amdgcn_readlane(b1, idx);
          src = kbase + (int64_t)(t < 8 ? ka : kz) * blk_stride + (t & 7) * D + (lane & 7) * 16;
        } else {
          const int o = BS == 16 ? 0 : __builtin_amdgcn_readlane(boff, idx);
          src = kbase + (int64_t)ka * blk_stride + o * D + (uint32_t)(t * D + (lane & 7) * 16);
        }
        f.k[h] = __builtin_nontemporal_load((const u32x4 *)src);
      }
    } else if constexpr (KV8) {
#pragma unroll
      for (int h = 0; h < D / 64; ++h)
        f.k[h] = __builtin_nontemporal_load((const u32x4 *)(kp + h * 64));
    } else {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        f.k[ks] = __builtin_nontemporal_load((const u32x4 *)(kp + ks * 32));
    }
    load_v<D, KV8, true>(f, vp);
  };

  // Reference max per head in log2 units, reset at each sequence segment.
  // It is raised only when a tile's max exceeds it by more than kSlack, so
  // most tiles skip the rescale of the accumulators; the weights
  // 2^(s - m_ref) then stay below 2^kSlack, far inside the range of every
  // weight type (bfloat16, binary16).  The softmax is the same for any
  // reference.
  float m_ref = -INFINITY;
  float thr = -INFINITY;  // m_ref + kSlack in units of raw scores
  const float inv_scale = 1.0f / scale_log2;
  float l_run = 0.f;  // this lane's share of the running sum
  f32x4 acc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One tile of scores, softmax update and P.V; at the end of a sequence
  // segment, the segment's result goes out and the state is reset.  In the
  // last tile of a sequence, tokens at or past its valid count get weight
  // zero and their V entries are zeroed (unused slots may hold anything,
  // NaN included).  Both branches here are wave-uniform and hold no loads.
  auto step = [&](Frag<D, KV8> &f, int idx) {
    const int mt = __builtin_amdgcn_readlane(meta, idx);
    const int n = mt & 31;
    if constexpr (kKT) {  // K as loaded -> LDS -> the MFMA layout (token row, codes 64h + 16grp)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(u32x4 *)(kt_lds + (8 * h + (lane >> 3)) * kKTRow + (lane & 7) * 16) = f.k[h];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.k[h] = *(const u32x4 *)(kt_lds + row * kKTRow + (4 * h + grp) * 16);
    }
    if (APPEND && (mt & kNew)) {
      // The new token (row r of the tile) comes from k_new / v_new, not
      // from its cache slot, which this wavefront now fills.  Lanes of A-row
      // r hold the token's K pieces (its V follows after the QK MFMAs).
      // E4M3 caches: the wave first quantises the rows, PER elements per lane
      // (the lane's own LDS writes).
      const int r = n - 1;
      if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int d = lane * PER + i;
          kn_lds[d] = (uint8_t)e4m3_code(elem_to_float<DT>(kn_raw[d]) * k_inv);
          vn_lds[d] = (uint8_t)e4m3_code(elem_to_float<DT>(vn_raw[d]) * v_inv);
        }
        __syncthreads();  // the codes of every lane before the reads below
      }
      if (row == r) {
#pragma unroll
        for (int h = 0; h < (KV8 ? D / 64 : KSTEPS); ++h)
          f.k[h] = *(const u32x4 *)(kn_lds + (KV8 ? 64 * h + 16 * grp : 32 * h + 8 * grp));
      }
    }
    u32x4 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = q_lds[ks * kWave + lane];
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 kf;
      if constexpr (KV8) {  // codes 8*(ks%2) .. +8 of the 16 loaded for ks/2
        const u32x4 c = f.k[ks / 2];
        const u32x2 a = E::from_e4m3(ks % 2 ? c.z : c.x);
        const u32x2 b = E::from_e4m3(ks % 2 ? c.w : c.y);
        kf = u32x4{a.x, a.y, b.x, b.y};
      } else {
        kf = f.k[ks];
      }
      sc = E::qk(kf, qf[ks], sc);
    }
    if (APPEND && (mt & kNew)) {
      // V of the new token, and the stores, after the QK MFMAs are issued (as
      // in any tile, V is first waited for here) and before the mask below
      // zeroes the group's later positions, which go back as they were.
      // Lanes of quarter r / 4 hold element r % 4 of each V^T fragment.
      const int r = n - 1;
      const int e = r & 3;
      if (grp == (r >> 2)) {
        // all reads first, then selects: a branch per fragment on the
        // (uniform) position e made each read wait for its own LDS round trip
        uint32_t x[DTILES];
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) x[dt] = vn_lds[vdim<KV8>(dt, row)];
        if constexpr (KV8) {
          const uint32_t keep = ~(0xffu << (8 * e));
#pragma unroll
          for (int dt = 0; dt < DTILES; ++dt) f.v[dt] = (f.v[dt] & keep) | (x[dt] << (8 * e));
        } else {
          const int sh = 16 * (e & 1);
          const uint32_t keep = ~(0xffffu << sh);
          const bool upper = (e >> 1) != 0;  // token in the second dword of the fragment
#pragma unroll
          for (int dt = 0; dt < DTILES; ++dt) {
            const uint32_t w = ((upper ? f.v[dt].y : f.v[dt].x) & keep) | (x[dt] << sh);
            f.v[dt].x = upper ? f.v[dt].x : w;
            f.v[dt].y = upper ? w : f.v[dt].y;
          }
        }
      }
      // Store the token: its K row, and its V as part of its whole 4-token
      // group (the lanes of quarter r / 4 hold that group's [D][4] run, the
      // other three positions with the bytes they held), so that both
      // stores write whole cache lines rather than a few bytes of each.
      const int nb = __builtin_amdgcn_readlane(nblk, idx);
      if (nb >= 0) {
        const int bo = BS == 32 ? __builtin_amdgcn_readlane(boff, idx) : 0;
        const int off = BS == 8 ? (r & 7) : bo + r;
        const int64_t bh = (int64_t)nb * num_kv_heads + kvh;
        CT *kd = static_cast<CT *>(k_cache) + (bh * BS + off) * D;
        CT *vd = static_cast<CT *>(v_cache) + bh * D * BS;
        // the K row from LDS, where it sits in dimension order: 16 bytes per
        // lane, so that one store instruction writes the whole row
        constexpr int KL = D * (int)sizeof(CT) / 16;  // lanes that store
        if (lane < KL) *(u32x4 *)(kd + lane * (16 / (int)sizeof(CT))) =
            *(const u32x4 *)(kn_lds + lane * (16 / (int)sizeof(CT)));
        if (grp == (r >> 2)) {
          const int g4 = ((BS == 8 ? (grp * 4) & 7 : bo + grp * 4) >> 2);  // group in the block
          constexpr int VG = VLayout<KV8>::VG;
#pragma unroll
          for (int g = 0; g < DTILES / VG; ++g) {
            CT *vp = vd + (g4 * D + 16 * VG * g + VG * row) * 4;
            if constexpr (KV8)
              *(u32x4 *)vp = u32x4{f.v[4 * g], f.v[4 * g + 1], f.v[4 * g + 2], f.v[4 * g + 3]};
            else
              *(u32x4 *)vp = u32x4{f.v[2 * g].x, f.v[2 * g].y, f.v[2 * g + 1].x, f.v[2 * g + 1].y};
          }
        }
      }
    }
    // raw scores; the scale (> 0, log2 units) joins in the exponent's FMA
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = sc[r];
    if (n < kTile) {
      const int c = n - grp * 4;  // valid tokens among this lane's four
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = r < c ? s[r] : -INFINITY;
      if constexpr (KV8) {  // one code byte per token
        const uint32_t w = c >= 4 ? 0xffffffffu : (c <= 0 ? 0u : (1u << (8 * c)) - 1u);
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) f.v[dt] &= w;
      } else {  // two 16-bit tokens per word
        const uint32_t w0 = c >= 2 ? 0xffffffffu : (c == 1 ? 0x0000ffffu : 0u);
        const uint32_t w1 = c >= 4 ? 0xffffffffu : (c == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) {
          f.v[dt].x &= w0;
          f.v[dt].y &= w1;
        }
      }
    }
    // The reference moves only when a score passes m_ref + kSlack: each
    // lane checks its own four raw scores against that bound (thr, in raw
    // units), and only then is the max reduced over the column's lanes.
    const float lm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__ballot(lm > thr)) {  // always on a segment's first tile
      const float mx = rows_max(lm) * scale_log2;
      const float m_new = fmaxf(m_ref, mx);  // finite: every tile has a valid token
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) acc[dt] *= alpha;
      m_ref = m_new;
      thr = (m_new + kSlack) * inv_scale;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -m_ref));
    u32x2 ph, pl;
    ph.x = PE::pack(p[0], p[1]);
    ph.y = PE::pack(p[2], p[3]);
    if constexpr (PE::kSplitP) {
      // residuals are exact in fp32; the sum is taken over the full weights
      pl.x = PE::pack(p[0] - PE::lo(ph.x), p[1] - PE::hi(ph.x));
      pl.y = PE::pack(p[2] - PE::lo(ph.y), p[3] - PE::hi(ph.y));
      l_run += (p[0] + p[1]) + (p[2] + p[3]);
    } else {
      // the sum uses the rounded weights the MFMA multiplies with
      l_run += (PE::lo(ph.x) + PE::hi(ph.x)) + (PE::lo(ph.y) + PE::hi(ph.y));
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      u32x2 vv;
      if constexpr (KV8) vv = PE::from_e4m3(f.v[dt]);
      else vv = f.v[dt];
      acc[dt] = PE::pv(vv, ph, acc[dt]);
      if constexpr (PE::kSplitP) acc[dt] = PE::pv(vv, pl, acc[dt]);
    }
    if (mt & kEnd) {
      const float l_tot = rows_sum(l_run);
      const int sqn = __builtin_amdgcn_readlane(sq, idx);
      if (row < group) {
        const int head = kvh * group + row;
        const float inv = out_scale / l_tot;
        constexpr int VG = VLayout<KV8>::VG;
        if (mt & kWhole) {
          // lane (row, grp) holds dims 16*VG*g + 4*VG*grp .. +4*VG of head row
          uint16_t *op = out + ((int64_t)sqn * num_heads + head) * D + grp * 4 * VG;
#pragma unroll
          for (int g = 0; g < DTILES / VG; ++g)
            row_values<D, KV8>(acc, g, [&](int c, f32x4 v) {
              const u32x2 w = {E::pack(v[0] * inv, v[1] * inv), E::pack(v[2] * inv, v[3] * inv)};
              *(u32x2 *)(op + 16 * VG * g + 4 * c) = w;
            });
        } else if ((ends & ((1ull << idx) - 1)) == 0) {  // no earlier segment end
          // The first segment continues a sequence from the previous
          // wavefront.  Its partial waits in LDS and is stored after the tile
          // loop: stored here, it would hold up this wavefront's next waits.
          float *sp = stg + row * D + grp * 4 * VG;
#pragma unroll
          for (int g = 0; g < DTILES / VG; ++g)
            row_values<D, KV8>(acc, g, [&](int c, f32x4 v) {
              *(f32x4 *)(sp + 16 * VG * g + 4 * c) = v * inv;
            });
          if (grp == 0) *(f32x2 *)(stg + group * D + row * 2) = f32x2{m_ref, l_tot};
        } else {
          const int64_t slot = (int64_t)head * slots + j + sqn;
          float *op = ws_o + slot * D + grp * 4 * VG;
#pragma unroll
          for (int g = 0; g < DTILES / VG; ++g)
            row_values<D, KV8>(acc, g, [&](int c, f32x4 v) {
              *(f32x4 *)(op + 16 * VG * g + 4 * c) = v * inv;
            });
          if (grp == 0) *(f32x2 *)(ws_ml + slot * 2) = f32x2{m_ref, l_tot};
        }
      }
      if (!(mt & kWhole) && (ends & ((1ull << idx) - 1)) == 0) first_sq = sqn;
      m_ref = -INFINITY;
      thr = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Publish the next segment's query (prefetched a segment ago, so this
      // does not wait on recent loads), then prefetch the one after it,
      // which starts after the next segment end following tile idx.
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) q_lds[ks * kWave + lane] = qnext[ks];
      publish_new();
      __builtin_amdgcn_sched_barrier(0);
      const uint64_t later = idx + 1 < kWave ? ends & (~0ull << (idx + 1)) : 0ull;
      const int nf = later ? next_first(__builtin_ctzll(later)) : cnt - 1;
      load_q(qnext, nf);
      load_new(nf);
    }
  };

  // Ring of kBuf register sets: while tile t is computed, tiles t+1 ..
  // t+kBuf-1 are in flight.  The ring is indexed by compile-time constants
  // (the inner loop is unrolled) so it stays in registers.  Past the last
  // tile the ring reloads the last tile (cache hits); those steps are
  // skipped.  sched_barrier keeps the scheduler from sinking a load down to
  // its use, which would trade the prefetch for fewer registers.
  Frag<D, KV8> f[kBuf];
#pragma unroll
  for (int b = 0; b < kBuf - 1; ++b) load(f[b], min(b, cnt - 1));
  __builtin_amdgcn_sched_barrier(0);
  for (int t = 0; t < cnt; t += kBuf) {
#pragma unroll
    for (int b = 0; b < kBuf; ++b) {
      load(f[(b + kBuf - 1) % kBuf], min(t + b + kBuf - 1, cnt - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (t + b < cnt) step(f[b], t + b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (first_sq >= 0) {  // the deferred partial, 16 bytes per lane and store
    for (int e = lane * 4; e < group * D; e += kWave * 4) {
      const int r = e / D;
      *(f32x4 *)(ws_o + ((int64_t)(kvh * group + r) * slots + j + first_sq) * D + (e - r * D)) =
          *(const f32x4 *)(stg + e);
    }
    if (lane < group)
      *(f32x2 *)(ws_ml + ((int64_t)(kvh * group + lane) * slots + j + first_sq) * 2) =
          *(const f32x2 *)(stg + group * D + lane * 2);
  }
}

// Query heads per merge workgroup (one wavefront each), at most: when each
// sequence has few partials, workgroups of four wavefronts dispatch faster
// than four single-wavefront ones, which shortens this latency-bound launch
// by about 1 us at 2048 (sequence, head) rows (eight or sixteen are slower
// again); with many partials per sequence the four heavier wavefronts of a
// workgroup compete on one CU, and the launcher uses one.
constexpr int kMergeHeads = 4;

// Log-sum-exp merge of the partial results of one (sequence, query head):
//   M = max_p m_p,  c_p = l_p * 2^(m_p - M),  out = sum_p c_p o_p / sum_p c_p.
// The partials of sequence s come from wavefronts wave_of(cu[s]) ..
// wave_of(cu[s+1] - 1), in consecutive slots starting at that first
// wavefront + s.  SHARED: also the sh.chunks partials of the shared prefix,
// and a sequence held by one wavefront is merged too.
template <int DT, int D, bool SHARED>
__global__ __launch_bounds__(kMergeHeads * kWave) void decode_merge_kernel(
    uint16_t *__restrict__ out, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml, const int32_t *__restrict__ ws_cu, int num_seqs,
    int num_heads, int waves, int slots, SharedPrefix sh) {
  using E = Elem<DT>;
  constexpr int PER = D / kWave;  // dims per lane
  const int head = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int seq = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  // The three tile-prefix entries go out together, before any branch: each
  // is a round trip to memory that the split pass wrote, and a test that
  // needs all three (c1 <= n_tiles always holds) keeps the compiler from
  // moving one of them behind the wait for the others.
  const int n_tiles = ws_cu[num_seqs];
  const int c0 = ws_cu[seq], c1 = ws_cu[seq + 1];
  if (head >= num_heads || c1 > n_tiles) return;
  int np = 0, jf = 0;
  if (c1 > c0) {
    const int wv = min(waves, n_tiles);  // as in the split pass: all ranges non-empty
    jf = wave_of(c0, n_tiles, wv);
    const int jl = wave_of(c1 - 1, n_tiles, wv);
    if (!SHARED && jf == jl) return;  // one wavefront held the sequence and wrote its row
    np = jl - jf + 1;
  } else if (!SHARED) {
    return;  // nothing to attend: the split pass wrote zeros
  }

  // One pass with a running maximum, so each partial's (m, l) and o are
  // loaded together: c_p = l_p * 2^(m_p - M) rescaled as M grows.
  float big = -INFINITY, den = 0.f;
  float num[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  auto absorb = [&](const f32x2 *ml, const float *o, int n) {
#pragma unroll 4
    for (int p = 0; p < n; ++p) {
      const f32x2 v = ml[p];
      float op[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) op[i] = o[(int64_t)p * D + i];
      const float m_new = fmaxf(big, v.x);
      const float a = __builtin_amdgcn_exp2f(big - m_new);  // 0 on the first partial
      const float c = v.y * __builtin_amdgcn_exp2f(v.x - m_new);
      den = den * a + c;
#pragma unroll
      for (int i = 0; i < PER; ++i) num[i] = num[i] * a + c * op[i];
      big = m_new;
    }
  };
  if constexpr (SHARED) {
    const int64_t sb = ((int64_t)head * num_seqs + seq) * sh.chunks;
    absorb((const f32x2 *)(sh.ml + sb * 2), sh.o + sb * D + lane * PER, sh.chunks);
  }
  if (np > 0) {
    const int64_t base = (int64_t)head * slots + jf + seq;
    absorb((const f32x2 *)(ws_ml + base * 2), ws_o + base * D + lane * PER, np);
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
  // log2(e) folds the exponential's base into the score scale; an E4M3
  // cache's k_scale multiplies every score and its v_scale every output.
  const float scale_log2 = (float)((double)a.scale * (double)a.k_scale * 1.4426950408889634);
  hipStream_t st = (hipStream_t)a.stream;
  const int group = a.num_heads / a.num_kv_heads;
  const bool shared = a.sh.tiles > 0;
  hipError_t e = hipSuccess;
  if (a.num_seqs < 1) return (int)hipErrorInvalidValue;  // the split pass reads lengths[0]
  if (a.stages & 1) {
    dim3 grid((unsigned)a.num_kv_heads * (unsigned)(a.waves + (shared ? a.sh.waves : 0)));
    // LDS: tile prefix and lengths, query fragments, for the fused append
    // the new rows (16-bit, plus E4M3 codes), for E4M3 at D = 128 one K
    // tile, and the first segment's partial (group x (D + 2) floats).
    const size_t lds = (size_t)((2 * a.num_seqs + 1 + 3) & ~3) * sizeof(int) +
                       (size_t)(D / 32) * kWave * 16 + (a.append ? 6 * D : 0) +
                       (a.kv_fp8 && D == 128 ? 16 * 144 : 0) +
                       (size_t)group * (D + 2) * sizeof(float);
#define PA_SPLIT(KV8, APPEND, SHARED, OUT_SCALE)                                               \
  decode_split_kernel<DT, D, BS, KV8, APPEND, SHARED><<<grid, kWave, lds, st>>>(               \
      (uint16_t *)a.out, a.ws_o, a.ws_ml, a.ws_cu, (const uint16_t *)a.q, (void *)a.k_cache,  \
      (void *)a.v_cache, a.block_tables, a.context_lens, (const uint16_t *)a.k_new,           \
      (const uint16_t *)a.v_new, scale_log2, OUT_SCALE, a.k_inv, a.v_inv, a.num_seqs,         \
      a.num_kv_heads, a.num_heads, group, a.max_blocks_per_seq, a.waves, a.slots,             \
      a.num_blocks, a.sh)
#define PA_SPLIT_SH(KV8, APPEND, OUT_SCALE)                                                   \
  do {                                                                                        \
    if (shared) PA_SPLIT(KV8, APPEND, true, OUT_SCALE);                                       \
    else PA_SPLIT(KV8, APPEND, false, OUT_SCALE);                                             \
  } while (0)
    if (a.kv_fp8) {
      if (a.append) PA_SPLIT_SH(true, true, a.v_scale);
      else PA_SPLIT_SH(true, false, a.v_scale);
    } else {
      if (a.append) PA_SPLIT_SH(false, true, 1.0f);
      else PA_SPLIT_SH(false, false, 1.0f);
    }
#undef PA_SPLIT_SH
#undef PA_SPLIT
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  if (a.stages & 2) {
    // about waves / num_seqs partials per sequence
    const int mh = a.waves <= 4 * a.num_seqs ? kMergeHeads : 1;
    dim3 g2((unsigned)((a.num_heads + mh - 1) / mh), (unsigned)a.num_seqs);
    if (shared)
      decode_merge_kernel<DT, D, true><<<g2, mh * kWave, 0, st>>>(
          (uint16_t *)a.out, a.ws_o, a.ws_ml, a.ws_cu, a.num_seqs, a.num_heads, a.waves,
          a.slots, a.sh);
    else
      decode_merge_kernel<DT, D, false><<<g2, mh * kWave, 0, st>>>(
          (uint16_t *)a.out, a.ws_o, a.ws_ml, a.ws_cu, a.num_seqs, a.num_heads, a.waves,
          a.slots, a.sh);
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

// Workspace of the no-allocation decode step.  Each GPU the library runs on
// holds its own copy of this array at its own address.  In host code its name
// is only a host-side stand-in, so kernels and copies take the device address
// that hipGetSymbolAddress returns for the current device, looked up once
// per device and cached.  Every call on one GPU shares the array: calls that
// overlap on one GPU (other streams, other threads) race.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];
}  // namespace

int scratch_buffer(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return 0;
}

}  // namespace pa
