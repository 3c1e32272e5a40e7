/*
 * Paged-attention CPU oracle (fp64).  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, plainly written reference that the GPU path is
 * checked against.  Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library under pagedattention_kv_cache_paged_amd/csrc.
 *
 * Sources (titles of the pages this follows; sections as numbered there):
 *   [P1] "vLLM core architecture overview: PagedAttention, Continuous
 *        Batching, distributed inference" (5688vip.com), 4.1.
 *   [P3] "vLLM memory management and continuous batching from the source"
 *        (developer.cloud.tencent.cn), part 2, 2.1 (BlockTable and
 *        append_token) and 2.3 (attention forward over block tables).
 *   [P4] "vLLM framework analysis: how PagedAttention speeds up LLM
 *        inference 20x" (intelliparadigm.com), 2.3 (shared blocks), 7
 *        (mixed precision).
 *
 * The pages never write the attention formula down.  The oracle computes the
 * standard scaled-dot-product softmax attention of one decode query per
 * (sequence, query head) over that sequence's context tokens, reaching each
 * token's K and V through the sequence's block table exactly as [P3] 2.3
 * describes (a list of physical block numbers replaces the contiguous
 * (batch, seq_len, dim) tensor).  Everything is accumulated in double
 * precision, tokens are visited in increasing logical position, and no
 * blocking, fusion or reordering is applied.
 *
 * Storage (shared by the oracle and the library only as a documented
 * convention; each side has its own code for it):
 *   K cache  [num_blocks][num_kv_heads][block_size][head_dim]   token-major
 *   V cache  [num_blocks][num_kv_heads][block_size/4][head_dim][4]
 *            positions in groups of four; inside a group the four positions
 *            of one dimension are adjacent (block_size a multiple of 4)
 *   q        [num_seqs][num_heads][head_dim]
 *   k, v     [num_tokens][num_kv_heads][head_dim]   (new tokens to append)
 *   slot     int64 [num_tokens]; slot = physical_block * block_size + offset,
 *            negative = padding, skipped.
 *   Elements are raw IEEE binary16 (dtype 0) or bfloat16 (dtype 1) bit
 *   patterns, decoded here by hand; an FP8 cache holds OCP E4M3 codes, one
 *   byte per element in the same layouts, standing for code * tensor scale
 *   ([P4] 7: FP8 for attention, FP16 elsewhere).
 *
 * Parity pins: every function below is pinned by tests under tests/ that do
 * not retype its formula (see the test module docstrings).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F16 0
#define ORACLE_BF16 1
#define ORACLE_FP8 2 /* cache element type only: E4M3 codes with a tensor scale */

#define ORACLE_OK 0
#define ORACLE_EARG -1    /* bad sizes or dtype */
#define ORACLE_ESLOT -2   /* slot out of range or used twice */
#define ORACLE_EBLOCK -3  /* block table names a block outside the pool */
#define ORACLE_ELEN -4    /* context length exceeds the table's capacity */
#define ORACLE_ENORM -5   /* normalised weights do not sum to one */
#define ORACLE_ENOMEM -6

/* ---- element decoding --------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exact conversion, subnormals, infinities and NaN included. */
double oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* 0.frac * 2^-14 */
  } else if (expo == 0x1f) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac + 1024), expo - 25); /* 1.frac * 2^(expo-15) */
  }
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 7) & 0xff;
  int frac = bits & 0x7f;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -133); /* 0.frac * 2^-126 */
  } else if (expo == 0xff) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac + 128), expo - 134); /* 1.frac * 2^(expo-127) */
  }
  return sign ? -mag : mag;
}

static double decode(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 fraction
 * bits, no infinities; S.1111.111 is NaN, the largest finite magnitude is
 * 1.75 * 2^8 = 448 and subnormals are m * 2^-9.  Exact conversion. */
double oracle_e4m3_to_f64(uint8_t code) {
  int sign = code >> 7;
  int expo = (code >> 3) & 0xf;
  int frac = code & 7;
  double mag;
  if (expo == 0xf && frac == 7) {
    mag = NAN;
  } else if (expo == 0) {
    mag = ldexp((double)frac, -9); /* 0.frac * 2^-6 */
  } else {
    mag = ldexp((double)(frac + 8), expo - 10); /* 1.frac * 2^(expo-7) */
  }
  return sign ? -mag : mag;
}

/* The E4M3 code nearest to y, ties to the code with an even fraction (the
 * representable magnitudes are the integers n * u with u the spacing, and
 * the fraction's last bit is the parity of n); finite magnitudes beyond 448
 * saturate to +-448; NaN gives NaN.  All candidates are dyadic rationals, so
 * the comparisons below are exact in double precision. */
uint8_t oracle_f64_to_e4m3(double y) {
  if (isnan(y)) return 0x7f;
  int sign = signbit(y) ? 1 : 0;
  double a = fabs(y);
  if (a >= 448.0) return (uint8_t)((sign << 7) | 0x7e);
  double u; /* spacing of representable magnitudes at a */
  if (a < ldexp(1.0, -6)) {
    u = ldexp(1.0, -9);
  } else {
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
    u = ldexp(1.0, e - 1 - 3);
  }
  double n = floor(a / u); /* a / u is exact: u is a power of two */
  double below = a - n * u, above = (n + 1) * u - a;
  if (above < below || (above == below && fmod(n, 2.0) != 0.0)) n += 1.0;
  double pick = n * u; /* <= 448 because a < 448 */
  int code;
  if (pick < ldexp(1.0, -6)) {
    code = (int)(pick / ldexp(1.0, -9)); /* subnormal (or zero) */
  } else {
    int e;
    double f = frexp(pick, &e); /* pick = f * 2^e */
    code = ((e - 1 + 7) << 3) | (int)(f * 16.0 - 8.0);
  }
  return (uint8_t)((sign << 7) | code);
}

/* One cache element as a real number: a 16-bit value, or an E4M3 code
 * times its tensor scale. */
static double cache_value(const void *cache, int64_t index, int cache_dtype,
                          double scale) {
  if (cache_dtype == ORACLE_FP8)
    return oracle_e4m3_to_f64(((const uint8_t *)cache)[index]) * scale;
  return decode(((const uint16_t *)cache)[index], cache_dtype) * scale;
}

/* ---- cache accessors ---------------------------------------------------- */

static const uint16_t *k_row(const uint16_t *k_cache, int64_t block, int kv_head,
                             int offset, int num_kv_heads, int block_size,
                             int head_dim) {
  int64_t row = (block * num_kv_heads + kv_head) * (int64_t)block_size + offset;
  return k_cache + row * head_dim;
}

/* Index of V element (block, kv_head, position offset, dimension dim): the
 * (block, head) slice holds block_size * head_dim elements, as block_size/4
 * groups of [head_dim][4]. */
static int64_t v_index(int64_t block, int kv_head, int offset, int dim, int num_kv_heads,
                       int block_size, int head_dim) {
  int64_t slice = (block * num_kv_heads + kv_head) * (int64_t)block_size * head_dim;
  return slice + ((int64_t)(offset / 4) * head_dim + dim) * 4 + offset % 4;
}

static uint16_t v_elem(const uint16_t *v_cache, int64_t block, int kv_head,
                       int offset, int dim, int num_kv_heads, int block_size,
                       int head_dim) {
  return v_cache[v_index(block, kv_head, offset, dim, num_kv_heads, block_size, head_dim)];
}

/* ---- KV append ---------------------------------------------------------- */

/* Append step of [P3] 2.1: a token's K and V are written at its physical
 * block's address plus its offset within that block.  The caller has already chosen the slot
 * (block allocated when the sequence's fill count is a multiple of the block
 * size); here every token with a non-negative slot is copied bit for bit into
 * block slot/block_size at offset slot%block_size, for every KV head.
 * All slots are checked first (in range, none repeated); on error nothing is
 * written. */
int oracle_kv_write(const uint16_t *k, const uint16_t *v,
                    const int64_t *slot_mapping, uint16_t *k_cache,
                    uint16_t *v_cache, int64_t num_tokens, int num_kv_heads,
                    int head_dim, int block_size, int64_t num_blocks) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 ||
      num_blocks <= 0)
    return ORACLE_EARG;
  int64_t num_slots = num_blocks * block_size;
  unsigned char *seen = calloc((size_t)num_slots, 1);
  if (!seen) return ORACLE_ENOMEM;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= num_slots || seen[slot]) {
      free(seen);
      return ORACLE_ESLOT;
    }
    seen[slot] = 1;
  }
  free(seen);

  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t block = slot / block_size;
    int offset = (int)(slot % block_size);
    for (int j = 0; j < num_kv_heads; ++j) {
      const uint16_t *src_k = k + (i * num_kv_heads + j) * (int64_t)head_dim;
      const uint16_t *src_v = v + (i * num_kv_heads + j) * (int64_t)head_dim;
      uint16_t *dst_k =
          (uint16_t *)k_row(k_cache, block, j, offset, num_kv_heads, block_size, head_dim);
      for (int d = 0; d < head_dim; ++d) {
        dst_k[d] = src_k[d];
        v_cache[v_index(block, j, offset, d, num_kv_heads, block_size, head_dim)] = src_v[d];
      }
    }
  }
  return ORACLE_OK;
}

/* ---- decode attention --------------------------------------------------- */

/* One (sequence s, query head h) row of decode attention.
 *
 * Query head h reads KV head h / G with G = num_heads / num_kv_heads
 * (consecutive query heads share one KV head).  For each logical position
 * t < L = context_lens[s], the physical block is block_tables[s][t / bs]
 * and the offset inside it is t % bs ([P3] 2.1 and 2.3):
 *     x[t]   = scale * sum_d q[s,h,d] * K[t,d]
 *     w[t]   = exp(x[t] - max_t x[t])
 *     out[d] = sum_t w[t] * V[t,d] / sum_t w[t]
 * L == 0 gives an all-zero row.  The normalised weights are checked to sum
 * to one within 1e-12.  K and V elements are 16-bit values of the q type,
 * or E4M3 codes times k_scale / v_scale (cache_dtype ORACLE_FP8). */
static int decode_row_any(double *out_row, const uint16_t *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, double scale, int block_size,
                          int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                          int max_blocks_per_seq, int64_t num_blocks, int q_dtype,
                          int cache_dtype, double k_scale, double v_scale, int s, int h) {
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || s < 0 ||
      s >= num_seqs || h < 0 || h >= num_heads || block_size <= 0 ||
      block_size % 4 != 0 || head_dim <= 0 || (q_dtype != ORACLE_F16 && q_dtype != ORACLE_BF16) ||
      (cache_dtype != ORACLE_F16 && cache_dtype != ORACLE_BF16 &&
       cache_dtype != ORACLE_FP8))
    return ORACLE_EARG;
  int group = num_heads / num_kv_heads;
  int kv_head = h / group;
  int64_t len = context_lens[s];
  for (int d = 0; d < head_dim; ++d) out_row[d] = 0.0;
  if (len <= 0) return ORACLE_OK;
  if (len > (int64_t)max_blocks_per_seq * block_size) return ORACLE_ELEN;

  const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
  const uint16_t *qrow = q + ((int64_t)s * num_heads + h) * head_dim;
  double *x = malloc((size_t)len * sizeof(double));
  if (!x) return ORACLE_ENOMEM;

  for (int64_t t = 0; t < len; ++t) {
    int64_t block = table[t / block_size];
    if (block < 0 || block >= num_blocks) {
      free(x);
      return ORACLE_EBLOCK;
    }
    /* K row of token t: [block][kv_head][offset][:] */
    int64_t krow = ((block * num_kv_heads + kv_head) * (int64_t)block_size +
                    (int)(t % block_size)) * head_dim;
    double dot = 0.0;
    for (int d = 0; d < head_dim; ++d)
      dot += decode(qrow[d], q_dtype) * cache_value(k_cache, krow + d, cache_dtype, k_scale);
    x[t] = scale * dot;
  }

  double m = x[0];
  for (int64_t t = 1; t < len; ++t)
    if (x[t] > m) m = x[t];
  double z = 0.0;
  for (int64_t t = 0; t < len; ++t) {
    x[t] = exp(x[t] - m); /* x now holds the unnormalised weight w[t] */
    z += x[t];
  }
  double wsum = 0.0;
  for (int64_t t = 0; t < len; ++t) wsum += x[t] / z;
  if (!(fabs(wsum - 1.0) <= 1e-12)) {
    free(x);
    return ORACLE_ENORM;
  }
  for (int64_t t = 0; t < len; ++t) {
    int64_t block = table[t / block_size];
    int offset = (int)(t % block_size);
    for (int d = 0; d < head_dim; ++d) {
      int64_t vi = v_index(block, kv_head, offset, d, num_kv_heads, block_size, head_dim);
      out_row[d] += x[t] * cache_value(v_cache, vi, cache_dtype, v_scale);
    }
  }
  for (int d = 0; d < head_dim; ++d) out_row[d] /= z;
  free(x);
  return ORACLE_OK;
}

/* 16-bit caches: K and V elements are values of the q type (scale 1, exact). */
int oracle_decode_row(double *out_row, const uint16_t *q, const uint16_t *k_cache,
                      const uint16_t *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, double scale, int block_size,
                      int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                      int max_blocks_per_seq, int64_t num_blocks, int dtype, int s,
                      int h) {
  return decode_row_any(out_row, q, k_cache, v_cache, block_tables, context_lens, scale,
                        block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                        max_blocks_per_seq, num_blocks, dtype, dtype, 1.0, 1.0, s, h);
}

/* Every (sequence, query head) row; out is [num_seqs][num_heads][head_dim]. */
int oracle_decode(double *out, const uint16_t *q, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, double scale, int block_size,
                  int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                  int max_blocks_per_seq, int64_t num_blocks, int dtype) {
  for (int s = 0; s < num_seqs; ++s)
    for (int h = 0; h < num_heads; ++h) {
      int rc = oracle_decode_row(out + ((int64_t)s * num_heads + h) * head_dim, q,
                                 k_cache, v_cache, block_tables, context_lens, scale,
                                 block_size, num_kv_heads, num_seqs, num_heads,
                                 head_dim, max_blocks_per_seq, num_blocks, dtype, s, h);
      if (rc != ORACLE_OK) return rc;
    }
  return ORACLE_OK;
}

/* Selected rows only: rows[2*i] = sequence, rows[2*i+1] = query head;
 * out is [num_rows][head_dim].  Used to check sampled outputs of large
 * workloads. */
int oracle_decode_rows(double *out, const int32_t *rows, int num_rows,
                       const uint16_t *q, const uint16_t *k_cache,
                       const uint16_t *v_cache, const int32_t *block_tables,
                       const int32_t *context_lens, double scale, int block_size,
                       int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                       int max_blocks_per_seq, int64_t num_blocks, int dtype) {
  for (int i = 0; i < num_rows; ++i) {
    int rc = oracle_decode_row(out + (int64_t)i * head_dim, q, k_cache, v_cache,
                               block_tables, context_lens, scale, block_size,
                               num_kv_heads, num_seqs, num_heads, head_dim,
                               max_blocks_per_seq, num_blocks, dtype, rows[2 * i],
                               rows[2 * i + 1]);
    if (rc != ORACLE_OK) return rc;
  }
  return ORACLE_OK;
}

/* Split-context form of the same row.  The context is cut into partitions
 * of part_tokens consecutive positions; each partition p is reduced on its
 * own to (m_p = max x, l_p = sum exp(x - m_p), o_p = sum exp(x - m_p) V / l_p)
 * and the partitions are then merged by the log-sum-exp rule
 *     M = max_p m_p,  c_p = l_p * exp(m_p - M),
 *     out = sum_p c_p * o_p / sum_p c_p.
 * Mathematically equal to oracle_decode_row; used to pin the merge rule. */
int oracle_decode_row_partitioned(double *out_row, const uint16_t *q,
                                  const uint16_t *k_cache, const uint16_t *v_cache,
                                  const int32_t *block_tables,
                                  const int32_t *context_lens, double scale,
                                  int block_size, int num_kv_heads, int num_seqs,
                                  int num_heads, int head_dim,
                                  int max_blocks_per_seq, int64_t num_blocks,
                                  int dtype, int s, int h, int part_tokens) {
  if (part_tokens <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      s < 0 || s >= num_seqs || h < 0 || h >= num_heads || block_size <= 0 ||
      block_size % 4 != 0 ||
      head_dim <= 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return ORACLE_EARG;
  int group = num_heads / num_kv_heads;
  int kv_head = h / group;
  int64_t len = context_lens[s];
  for (int d = 0; d < head_dim; ++d) out_row[d] = 0.0;
  if (len <= 0) return ORACLE_OK;
  if (len > (int64_t)max_blocks_per_seq * block_size) return ORACLE_ELEN;

  const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
  const uint16_t *qrow = q + ((int64_t)s * num_heads + h) * head_dim;
  int64_t nparts = (len + part_tokens - 1) / part_tokens;
  double *pm = malloc((size_t)nparts * sizeof(double));
  double *pl = malloc((size_t)nparts * sizeof(double));
  double *po = calloc((size_t)(nparts * head_dim), sizeof(double));
  double *x = malloc((size_t)part_tokens * sizeof(double));
  if (!pm || !pl || !po || !x) {
    free(pm); free(pl); free(po); free(x);
    return ORACLE_ENOMEM;
  }
  int rc = ORACLE_OK;
  for (int64_t p = 0; p < nparts && rc == ORACLE_OK; ++p) {
    int64_t t0 = p * part_tokens;
    int64_t t1 = t0 + part_tokens < len ? t0 + part_tokens : len;
    for (int64_t t = t0; t < t1; ++t) {
      int64_t block = table[t / block_size];
      if (block < 0 || block >= num_blocks) {
        rc = ORACLE_EBLOCK;
        break;
      }
      const uint16_t *krow = k_row(k_cache, block, kv_head, (int)(t % block_size),
                                   num_kv_heads, block_size, head_dim);
      double dot = 0.0;
      for (int d = 0; d < head_dim; ++d) dot += decode(qrow[d], dtype) * decode(krow[d], dtype);
      x[t - t0] = scale * dot;
    }
    if (rc != ORACLE_OK) break;
    double m = x[0];
    for (int64_t t = t0 + 1; t < t1; ++t)
      if (x[t - t0] > m) m = x[t - t0];
    double l = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      x[t - t0] = exp(x[t - t0] - m);
      l += x[t - t0];
    }
    double *o = po + p * head_dim;
    for (int64_t t = t0; t < t1; ++t) {
      int64_t block = table[t / block_size];
      int offset = (int)(t % block_size);
      for (int d = 0; d < head_dim; ++d)
        o[d] += x[t - t0] *
                decode(v_elem(v_cache, block, kv_head, offset, d, num_kv_heads,
                              block_size, head_dim),
                       dtype);
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= l;
    pm[p] = m;
    pl[p] = l;
  }
  if (rc == ORACLE_OK) {
    double big = pm[0];
    for (int64_t p = 1; p < nparts; ++p)
      if (pm[p] > big) big = pm[p];
    double csum = 0.0;
    for (int64_t p = 0; p < nparts; ++p) {
      double c = pl[p] * exp(pm[p] - big);
      csum += c;
      for (int d = 0; d < head_dim; ++d) out_row[d] += c * po[p * head_dim + d];
    }
    for (int d = 0; d < head_dim; ++d) out_row[d] /= csum;
  }
  free(pm); free(pl); free(po); free(x);
  return rc;
}

/* ---- FP8 (E4M3) KV cache ------------------------------------------------- */

/* "Advanced optimisation directions" of the PagedAttention 20x page,
 * mixed precision: attention in FP8, the rest in FP16.  Read here as an E4M3
 * KV cache with one scale per tensor: an element x of the new token's K (or
 * V) is stored as the code nearest to float32(x) * float32(1 / k_scale),
 * the product rounded to float32 as written; it stands for code * k_scale.
 * Same slots, checks and layouts as oracle_kv_write, one byte per element. */
int oracle_kv_write_fp8(const uint16_t *k, const uint16_t *v,
                        const int64_t *slot_mapping, uint8_t *k_cache, uint8_t *v_cache,
                        int64_t num_tokens, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int dtype, float k_scale,
                        float v_scale) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 ||
      num_blocks <= 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
      !(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
    return ORACLE_EARG;
  int64_t num_slots = num_blocks * block_size;
  unsigned char *seen = calloc((size_t)num_slots, 1);
  if (!seen) return ORACLE_ENOMEM;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= num_slots || seen[slot]) {
      free(seen);
      return ORACLE_ESLOT;
    }
    seen[slot] = 1;
  }
  free(seen);

  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t block = slot / block_size;
    int offset = (int)(slot % block_size);
    for (int j = 0; j < num_kv_heads; ++j) {
      for (int d = 0; d < head_dim; ++d) {
        int64_t src = (i * num_kv_heads + j) * (int64_t)head_dim + d;
        float kx = (float)decode(k[src], dtype) * k_inv;
        float vx = (float)decode(v[src], dtype) * v_inv;
        k_cache[((block * num_kv_heads + j) * (int64_t)block_size + offset) * head_dim + d] =
            oracle_f64_to_e4m3((double)kx);
        v_cache[v_index(block, j, offset, d, num_kv_heads, block_size, head_dim)] =
            oracle_f64_to_e4m3((double)vx);
      }
    }
  }
  return ORACLE_OK;
}

/* Decode attention over an E4M3 cache: K = code * k_scale, V = code *
 * v_scale (exact in double), q and the result as for the 16-bit caches. */
int oracle_decode_fp8(double *out, const uint16_t *q, const uint8_t *k_cache,
                      const uint8_t *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, double scale, int block_size,
                      int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                      int max_blocks_per_seq, int64_t num_blocks, int q_dtype,
                      double k_scale, double v_scale) {
  for (int s = 0; s < num_seqs; ++s)
    for (int h = 0; h < num_heads; ++h) {
      int rc = decode_row_any(out + ((int64_t)s * num_heads + h) * head_dim, q, k_cache,
                              v_cache, block_tables, context_lens, scale, block_size,
                              num_kv_heads, num_seqs, num_heads, head_dim,
                              max_blocks_per_seq, num_blocks, q_dtype, ORACLE_FP8,
                              k_scale, v_scale, s, h);
      if (rc != ORACLE_OK) return rc;
    }
  return ORACLE_OK;
}

/* Selected rows of oracle_decode_fp8 (rows as in oracle_decode_rows). */
int oracle_decode_fp8_rows(double *out, const int32_t *rows, int num_rows,
                           const uint16_t *q, const uint8_t *k_cache,
                           const uint8_t *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, double scale, int block_size,
                           int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                           int max_blocks_per_seq, int64_t num_blocks, int q_dtype,
                           double k_scale, double v_scale) {
  for (int i = 0; i < num_rows; ++i) {
    int rc = decode_row_any(out + (int64_t)i * head_dim, q, k_cache, v_cache, block_tables,
                            context_lens, scale, block_size, num_kv_heads, num_seqs,
                            num_heads, head_dim, max_blocks_per_seq, num_blocks, q_dtype,
                            ORACLE_FP8, k_scale, v_scale, rows[2 * i], rows[2 * i + 1]);
    if (rc != ORACLE_OK) return rc;
  }
  return ORACLE_OK;
}


/* ---- block copy for copy-on-write ------------------------------------------ */

/* [P4] 2.3: a sequence about to write into a block it shares with others
 * gets a private copy first.  For each pair i in order (src = pairs[2i],
 * dst = pairs[2i+1]), every element of block dst in both caches becomes the
 * element of block src at the same (kv head, offset, dim): K[dst][j][o][d] =
 * K[src][j][o][d] and V[dst][j][d][o] = V[src][j][d][o].  Elements are
 * elem_bytes wide (2: binary16 / bfloat16 bits, 1: E4M3 codes) and copied
 * as raw bytes.  A pair with a negative id is skipped.  The pairs must have
 * distinct destinations, none of them also a source, so that the order of
 * the copies cannot matter; otherwise, or for an id >= num_blocks, nothing
 * is copied and ORACLE_EBLOCK is returned. */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t num_pairs,
                       int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                       int elem_bytes) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 ||
      num_blocks <= 0 || (elem_bytes != 1 && elem_bytes != 2))
    return ORACLE_EARG;
  unsigned char *role = calloc((size_t)num_blocks, 1); /* bit 0: source, bit 1: destination */
  if (!role) return ORACLE_ENOMEM;
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src >= num_blocks || dst >= num_blocks) {
      free(role);
      return ORACLE_EBLOCK;
    }
    if (src < 0 || dst < 0) continue;
    if (role[dst] & 2) {
      free(role);
      return ORACLE_EBLOCK;
    }
    role[dst] |= 2;
    role[src] |= 1;
  }
  for (int64_t b = 0; b < num_blocks; ++b)
    if (role[b] == 3) {
      free(role);
      return ORACLE_EBLOCK;
    }
  free(role);

  unsigned char *kc = (unsigned char *)k_cache, *vc = (unsigned char *)v_cache;
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0) continue;
    for (int j = 0; j < num_kv_heads; ++j)
      for (int o = 0; o < block_size; ++o)
        for (int d = 0; d < head_dim; ++d) {
          int64_t ks = (((src * num_kv_heads + j) * (int64_t)block_size + o) * head_dim + d);
          int64_t kd = (((dst * num_kv_heads + j) * (int64_t)block_size + o) * head_dim + d);
          int64_t vs = v_index(src, j, o, d, num_kv_heads, block_size, head_dim);
          int64_t vd = v_index(dst, j, o, d, num_kv_heads, block_size, head_dim);
          memcpy(kc + kd * elem_bytes, kc + ks * elem_bytes, (size_t)elem_bytes);
          memcpy(vc + vd * elem_bytes, vc + vs * elem_bytes, (size_t)elem_bytes);
        }
  }
  return ORACLE_OK;
}

/* ---- block swap between two pools ------------------------------------------- */

/* [P1] 4.2: a preempted request's KV blocks move to CPU memory and back.
 * For each pair i (src = pairs[2i] of the source pool, dst = pairs[2i+1] of
 * the destination pool; both pools in the cache layouts above, with their
 * own block counts), every element of destination block dst in both caches
 * becomes the source element at the same (kv head, offset, dim), copied as
 * raw bytes of elem_bytes.  A pair with a negative id is skipped.
 * Destinations must be distinct; otherwise, or for an id past its pool,
 * nothing is copied and ORACLE_EBLOCK is returned.  The pools are distinct
 * objects, so no copy can read another's destination. */
int oracle_swap_blocks(void *dst_k, void *dst_v, int64_t dst_num_blocks, const void *src_k,
                       const void *src_v, int64_t src_num_blocks, const int64_t *pairs,
                       int64_t num_pairs, int num_kv_heads, int head_dim, int block_size,
                       int elem_bytes) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 ||
      dst_num_blocks <= 0 || src_num_blocks <= 0 || (elem_bytes != 1 && elem_bytes != 2))
    return ORACLE_EARG;
  unsigned char *taken = calloc((size_t)dst_num_blocks, 1);
  if (!taken) return ORACLE_ENOMEM;
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src >= src_num_blocks || dst >= dst_num_blocks) {
      free(taken);
      return ORACLE_EBLOCK;
    }
    if (src < 0 || dst < 0) continue;
    if (taken[dst]) {
      free(taken);
      return ORACLE_EBLOCK;
    }
    taken[dst] = 1;
  }
  free(taken);
  unsigned char *dk = (unsigned char *)dst_k, *dv = (unsigned char *)dst_v;
  const unsigned char *sk = (const unsigned char *)src_k, *sv = (const unsigned char *)src_v;
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0) continue;
    for (int j = 0; j < num_kv_heads; ++j)
      for (int o = 0; o < block_size; ++o)
        for (int d = 0; d < head_dim; ++d) {
          int64_t ks = (((src * num_kv_heads + j) * (int64_t)block_size + o) * head_dim + d);
          int64_t kd = (((dst * num_kv_heads + j) * (int64_t)block_size + o) * head_dim + d);
          int64_t vs = v_index(src, j, o, d, num_kv_heads, block_size, head_dim);
          int64_t vd = v_index(dst, j, o, d, num_kv_heads, block_size, head_dim);
          memcpy(dk + kd * elem_bytes, sk + ks * elem_bytes, (size_t)elem_bytes);
          memcpy(dv + vd * elem_bytes, sv + vs * elem_bytes, (size_t)elem_bytes);
        }
  }
  return ORACLE_OK;
}

/* ---- paged prefill (chunked prefill) ------------------------------------------ */

/* [P1] 4.3 (a long prompt is split into chunks so that its prefill does not
 * hold up decoding) and [P4] 4.2 (chunked prefill, a prefill chunk size):
 * each chunk's tokens attend over the sequence's cached KV and, causally,
 * over the chunk itself.  Sequence s contributes n_s = query_start[s+1] -
 * query_start[s] query rows (rows query_start[s] .. query_start[s+1]-1 of q
 * and out, layout [row][num_heads][head_dim]); they are its context
 * positions L-n_s .. L-1, where L = context_lens[s] counts the chunk too, so
 * their K and V are in the caches already (appended before the call).  Row
 * i of the chunk (position p = L-n_s+i), query head h:
 *     x[t]   = scale * sum_d q[i,h,d] * K[t,d]        for t = 0 .. p
 *     out[d] = sum_t exp(x[t] - max x) V[t,d] / sum_t exp(x[t] - max x)
 * reaching token t through block_tables[s][t / bs] at offset t % bs, with
 * KV head h / (num_heads / num_kv_heads).  n_s > L is an error
 * (ORACLE_ELEN); n_s = 0 contributes nothing.  The cache elements are 16-bit
 * values of q's type, or E4M3 codes times k_scale / v_scale (cache_dtype
 * ORACLE_FP8, as in oracle_decode_fp8). */
static int prefill_any(double *out, const uint16_t *q, const void *k_cache,
                       const void *v_cache, const int32_t *block_tables,
                       const int32_t *context_lens, const int32_t *query_start, double scale,
                       int block_size, int num_kv_heads, int num_seqs, int num_heads,
                       int head_dim, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                       int cache_dtype, double k_scale, double v_scale) {
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || num_seqs < 0 ||
      block_size <= 0 || block_size % 4 != 0 || head_dim <= 0 ||
      (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
      (cache_dtype != dtype && cache_dtype != ORACLE_FP8))
    return ORACLE_EARG;
  int group = num_heads / num_kv_heads;
  for (int s = 0; s < num_seqs; ++s) {
    int64_t row0 = query_start[s], n = (int64_t)query_start[s + 1] - query_start[s];
    int64_t len = context_lens[s];
    if (n < 0) return ORACLE_EARG;
    if (n == 0) continue;
    if (n > len || len > (int64_t)max_blocks_per_seq * block_size) return ORACLE_ELEN;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t t = 0; t < len; ++t)
      if (table[t / block_size] < 0 || table[t / block_size] >= num_blocks) return ORACLE_EBLOCK;
    double *x = malloc((size_t)len * sizeof(double));
    if (!x) return ORACLE_ENOMEM;
    for (int64_t i = 0; i < n; ++i) {
      int64_t p = len - n + i; /* the row's own position: it sees tokens 0 .. p */
      for (int h = 0; h < num_heads; ++h) {
        int kv_head = h / group;
        const uint16_t *qrow = q + ((row0 + i) * num_heads + h) * (int64_t)head_dim;
        double *orow = out + ((row0 + i) * num_heads + h) * (int64_t)head_dim;
        for (int64_t t = 0; t <= p; ++t) {
          int64_t block = table[t / block_size];
          int64_t krow = ((block * num_kv_heads + kv_head) * (int64_t)block_size +
                          (int)(t % block_size)) * head_dim;
          double dot = 0.0;
          for (int d = 0; d < head_dim; ++d)
            dot += decode(qrow[d], dtype) * cache_value(k_cache, krow + d, cache_dtype, k_scale);
          x[t] = scale * dot;
        }
        double m = x[0];
        for (int64_t t = 1; t <= p; ++t)
          if (x[t] > m) m = x[t];
        double z = 0.0;
        for (int64_t t = 0; t <= p; ++t) {
          x[t] = exp(x[t] - m);
          z += x[t];
        }
        for (int d = 0; d < head_dim; ++d) orow[d] = 0.0;
        for (int64_t t = 0; t <= p; ++t) {
          int64_t block = table[t / block_size];
          int offset = (int)(t % block_size);
          for (int d = 0; d < head_dim; ++d) {
            int64_t vi = v_index(block, kv_head, offset, d, num_kv_heads, block_size, head_dim);
            orow[d] += x[t] * cache_value(v_cache, vi, cache_dtype, v_scale);
          }
        }
        for (int d = 0; d < head_dim; ++d) orow[d] /= z;
      }
    }
    free(x);
  }
  return ORACLE_OK;
}

/* Chunked prefill over 16-bit caches of q's type. */
int oracle_prefill(double *out, const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *block_tables,
                   const int32_t *context_lens, const int32_t *query_start, double scale,
                   int block_size, int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                   int max_blocks_per_seq, int64_t num_blocks, int dtype) {
  return prefill_any(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                     block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                     max_blocks_per_seq, num_blocks, dtype, dtype, 1.0, 1.0);
}

/* Chunked prefill over E4M3 caches (the FP8 reading of oracle_kv_write_fp8):
 * K = code * k_scale, V = code * v_scale, exact in double; q (type q_dtype)
 * and the result as for the 16-bit caches. */
int oracle_prefill_fp8(double *out, const uint16_t *q, const uint8_t *k_cache,
                       const uint8_t *v_cache, const int32_t *block_tables,
                       const int32_t *context_lens, const int32_t *query_start, double scale,
                       int block_size, int num_kv_heads, int num_seqs, int num_heads,
                       int head_dim, int max_blocks_per_seq, int64_t num_blocks, int q_dtype,
                       double k_scale, double v_scale) {
  return prefill_any(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                     block_size, num_kv_heads, num_seqs, num_heads, head_dim,
                     max_blocks_per_seq, num_blocks, q_dtype, ORACLE_FP8, k_scale, v_scale);
}
