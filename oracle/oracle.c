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
 *        inference 20x" (intelliparadigm.com), 2.3 (shared blocks).
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
 *   V cache  [num_blocks][num_kv_heads][head_dim][block_size]   dim-major
 *   q        [num_seqs][num_heads][head_dim]
 *   k, v     [num_tokens][num_kv_heads][head_dim]   (new tokens to append)
 *   slot     int64 [num_tokens]; slot = physical_block * block_size + offset,
 *            negative = padding, skipped.
 *   Elements are raw IEEE binary16 (dtype 0) or bfloat16 (dtype 1) bit
 *   patterns, decoded here by hand.
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

/* ---- cache accessors ---------------------------------------------------- */

static const uint16_t *k_row(const uint16_t *k_cache, int64_t block, int kv_head,
                             int offset, int num_kv_heads, int block_size,
                             int head_dim) {
  int64_t row = (block * num_kv_heads + kv_head) * (int64_t)block_size + offset;
  return k_cache + row * head_dim;
}

static uint16_t v_elem(const uint16_t *v_cache, int64_t block, int kv_head,
                       int offset, int dim, int num_kv_heads, int block_size,
                       int head_dim) {
  int64_t base = (block * num_kv_heads + kv_head) * (int64_t)head_dim + dim;
  return v_cache[base * block_size + offset];
}

/* ---- KV append ---------------------------------------------------------- */

/* Append step of [P3] 2.1: a token's K and V go to "physical block address
 * plus offset inside the block".  The caller has already chosen the slot
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
        int64_t vbase = (block * num_kv_heads + j) * (int64_t)head_dim + d;
        v_cache[vbase * block_size + offset] = src_v[d];
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
 * to one within 1e-12. */
int oracle_decode_row(double *out_row, const uint16_t *q, const uint16_t *k_cache,
                      const uint16_t *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, double scale, int block_size,
                      int num_kv_heads, int num_seqs, int num_heads, int head_dim,
                      int max_blocks_per_seq, int64_t num_blocks, int dtype, int s,
                      int h) {
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || s < 0 ||
      s >= num_seqs || h < 0 || h >= num_heads || block_size <= 0 ||
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
  double *x = malloc((size_t)len * sizeof(double));
  if (!x) return ORACLE_ENOMEM;

  for (int64_t t = 0; t < len; ++t) {
    int64_t block = table[t / block_size];
    if (block < 0 || block >= num_blocks) {
      free(x);
      return ORACLE_EBLOCK;
    }
    const uint16_t *krow = k_row(k_cache, block, kv_head, (int)(t % block_size),
                                 num_kv_heads, block_size, head_dim);
    double dot = 0.0;
    for (int d = 0; d < head_dim; ++d) dot += decode(qrow[d], dtype) * decode(krow[d], dtype);
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
    for (int d = 0; d < head_dim; ++d)
      out_row[d] += x[t] *
                    decode(v_elem(v_cache, block, kv_head, offset, d, num_kv_heads,
                                  block_size, head_dim),
                           dtype);
  }
  for (int d = 0; d < head_dim; ++d) out_row[d] /= z;
  free(x);
  return ORACLE_OK;
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
