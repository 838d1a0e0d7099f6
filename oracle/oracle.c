/*
 * oracle.c — plain, slow CPU oracle for paged KV-cache attention.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke entry
 * point and the benchmark's CPU-baseline leg, never by the product library.
 * Scalar loops, IEEE double arithmetic on exactly-decoded inputs, OpenMP over
 * independent (sequence, query head) pairs so that every output element is
 * produced by one thread in a fixed order (deterministic for any thread count).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* threads the OpenMP loops use from now on (n >= 1); a timing knob only */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- [P2 "Page-table addressing"] ------------------------------------------
 * The page's reference: reject a non-positive block size or a negative position
 * (ValueError); split the position into (logical block, offset); a logical
 * block at or past the table's length is not allocated (IndexError); a negative
 * physical id is invalid (ValueError); else slot = physical * B + offset. */
int orc_physical_slot(const int32_t* table, int64_t table_len, int64_t block_size,
                      int64_t token_pos, int64_t* slot) {
  if (block_size <= 0 || token_pos < 0) return ORC_EVALUE;
  int64_t logical_block = token_pos / block_size;
  int64_t offset = token_pos % block_size;
  if (logical_block >= table_len) return ORC_EINDEX;
  int64_t physical_block = table[logical_block];
  if (physical_block < 0) return ORC_EVALUE;
  *slot = physical_block * block_size + offset;
  return ORC_OK;
}

/* ---- [P1 §4.1] write path: one slot per new token ------------------------- */
void orc_slot_mapping(const int32_t* block_table, int64_t num_seqs, int64_t max_blocks_per_seq,
                      const int32_t* seq_idx, const int32_t* positions, int64_t num_tokens,
                      int64_t block_size, int64_t* slot_mapping) {
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t s = seq_idx[i];
    int64_t slot = -1;
    if (s >= 0 && s < num_seqs && positions[i] >= 0) {
      int64_t out;
      if (orc_physical_slot(block_table + s * max_blocks_per_seq, max_blocks_per_seq, block_size,
                            positions[i], &out) == ORC_OK)
        slot = out;
    }
    slot_mapping[i] = slot;
  }
}

/* ---- storage decoders ------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_decode(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24); /* subnormal: f/1024 * 2^-14 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp(1.0 + f / 1024.0, e - 15);
  return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
double orc_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return (double)x;
}

/* OCP 8-bit floating point, E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xf;
  int m = c & 7;
  double mag;
  if (e == 15 && m == 7)
    mag = NAN;
  else if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Nearest E4M3 value to x by exhaustive search over the 127 non-negative finite
 * codes; on a tie the even code wins (even code <=> even mantissa LSB, which is
 * round-half-to-even).  |x| above the largest finite value saturates to it. */
uint8_t orc_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7f);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e); /* saturate (covers infinities) */
  int best = 0;
  double best_err = a; /* distance to code 0 (value 0) */
  for (int c = 1; c <= 0x7e; ++c) {
    double err = fabs(a - orc_e4m3_decode((uint8_t)c));
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* symmetric int8 of x (already divided by the scale): nearest integer, ties to
 * even (rint under the default rounding mode), saturated to [-127, 127]; NaN -> 0 */
int8_t orc_int8_encode(float x) {
  if (isnan(x)) return 0;
  double r = rint((double)x);
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (int8_t)r;
}

static size_t elem_size(int t) {
  switch (t) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8_E4M3: return 1;
    case ORC_INT8: return 1;
    default: return 0;
  }
}

static int quantised(int t) { return t == ORC_FP8_E4M3 || t == ORC_INT8; }

/* index of the scale of element (blk, kvh, off) */
static int64_t scale_index(int mode, int64_t blk, int64_t kvh, int64_t off, int64_t num_kv_heads,
                           int64_t block_size) {
  if (mode == ORC_SCALE_TENSOR) return 0;
  if (mode == ORC_SCALE_TOKEN) return (blk * num_kv_heads + kvh) * block_size + off;
  return blk * num_kv_heads + kvh;
}

/* exact value of element i of an array of storage type t */
static double load_value(const void* p, int t, size_t i) {
  switch (t) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_F16: return orc_f16_decode(((const uint16_t*)p)[i]);
    case ORC_BF16: return orc_bf16_decode(((const uint16_t*)p)[i]);
    case ORC_FP8_E4M3: return orc_e4m3_decode(((const uint8_t*)p)[i]);
    case ORC_INT8: return (double)((const int8_t*)p)[i];
    default: return NAN;
  }
}

void orc_decode_n(const void* p, int dtype, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = load_value(p, dtype, (size_t)i);
}

void orc_int8_encode_n(const float* x, int64_t n, int8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_int8_encode(x[i]);
}

void orc_e4m3_encode_n(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

/* ---- [P1 §4.1, §8.1] scatter write ---------------------------------------- */
int orc_kv_cache_write(const int64_t* slot_mapping, int64_t num_tokens, const void* k,
                       const void* v, int src_dtype, int64_t num_blocks, int64_t block_size,
                       int64_t num_kv_heads, int64_t head_dim, int kv_dtype, void* k_pool,
                       void* v_pool, const float* k_scale, const float* v_scale,
                       int scale_mode) {
  if (elem_size(src_dtype) == 0 || elem_size(kv_dtype) == 0) return -1;
  if (!quantised(kv_dtype) && src_dtype != kv_dtype) return -1;
  if (quantised(kv_dtype) && (quantised(src_dtype) || !k_scale || !v_scale)) return -1;
  if (scale_mode < ORC_SCALE_BLOCK || scale_mode > ORC_SCALE_TOKEN) return -1;
  size_t es = elem_size(kv_dtype);
  size_t ss = elem_size(src_dtype);
  const void* src[2] = {k, v};
  void* dst[2] = {k_pool, v_pool};
  const float* scl[2] = {k_scale, v_scale};
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= num_blocks * block_size) continue; /* padding / out of pool */
    int64_t blk = slot / block_size, off = slot % block_size;
    for (int which = 0; which < 2; ++which) {
      for (int64_t h = 0; h < num_kv_heads; ++h) {
        size_t src_row = ((size_t)i * num_kv_heads + h) * head_dim;
        size_t dst_row = (((size_t)blk * num_kv_heads + h) * block_size + off) * head_dim;
        if (!quantised(kv_dtype)) {
          memcpy((char*)dst[which] + dst_row * es, (const char*)src[which] + src_row * ss,
                 head_dim * es);
        } else {
          float s = scl[which][scale_index(scale_mode, blk, h, off, num_kv_heads, block_size)];
          for (int64_t d = 0; d < head_dim; ++d) {
            float x = (float)load_value(src[which], src_dtype, src_row + d); /* exact */
            float y = x / s; /* IEEE fp32 division, round to nearest even */
            if (kv_dtype == ORC_FP8_E4M3)
              ((uint8_t*)dst[which])[dst_row + d] = orc_e4m3_encode(y);
            else
              ((int8_t*)dst[which])[dst_row + d] = orc_int8_encode(y);
          }
        }
      }
    }
  }
  return 0;
}

/* ---- [P1 §3, §4] gather one token's K or V row through the table ---------- */

/* exact value of pool[blk][kvh][off][:] (times its scale for a quantised pool) */
static void load_row(const orc_pool* pool, int which, int64_t blk, int64_t kvh, int64_t off,
                     double* row) {
  const void* base = which == 0 ? pool->k_pool : pool->v_pool;
  size_t r = (((size_t)blk * pool->num_kv_heads + kvh) * pool->block_size + off) * pool->head_dim;
  double s = 1.0;
  if (quantised(pool->kv_dtype)) {
    const float* sc = which == 0 ? pool->k_scale : pool->v_scale;
    s = (double)sc[scale_index(pool->scale_mode, blk, kvh, off, pool->num_kv_heads,
                               pool->block_size)];
  }
  for (int64_t d = 0; d < pool->head_dim; ++d)
    row[d] = load_value(base, pool->kv_dtype, r + d) * s;
}

/* Attention of one query vector over keys [t0, t1) of one sequence, given as
 * the state (m, l, acc): m = max z, l = sum exp(z - m), acc = sum exp(z - m) V.
 * A range with no key gives (-inf, 0, 0). */
static void attend_range(const double* qv, const orc_pool* pool, const int32_t* table,
                         int64_t kvh, int64_t t0, int64_t t1, double scale, double* m_out,
                         double* l_out, double* acc, double* z, double* krow, double* vrow) {
  int64_t D = pool->head_dim, B = pool->block_size;
  for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
  if (t1 <= t0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  /* scores, then their maximum */
  double m = -INFINITY;
  for (int64_t t = t0; t < t1; ++t) {
    int64_t blk = table[t / B];
    load_row(pool, 0, blk, kvh, t % B, krow);
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qv[d] * krow[d];
    z[t - t0] = scale * dot;
    if (z[t - t0] > m) m = z[t - t0];
  }
  /* exponentials and the weighted sum of values */
  double l = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    double w = exp(z[t - t0] - m);
    l += w;
    int64_t blk = table[t / B];
    load_row(pool, 1, blk, kvh, t % B, vrow);
    for (int64_t d = 0; d < D; ++d) acc[d] += w * vrow[d];
  }
  *m_out = m;
  *l_out = l;
}

static int check_pool(const orc_pool* pool, int64_t num_q_heads) {
  if (!pool || elem_size(pool->kv_dtype) == 0 || pool->block_size <= 0 || pool->head_dim <= 0 ||
      pool->num_kv_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return -1;
  if (quantised(pool->kv_dtype) && (!pool->k_scale || !pool->v_scale)) return -1;
  return 0;
}

/* ---- [P1 §4], [P3 §5] decode: one-shot softmax over the gathered context ---
 * [P1 §1.1, §7] with a window w > 0 the query at position p = ctx - 1 sees only
 * the keys of [p - w + 1, p], i.e. t in [max(0, ctx - w), ctx). */
int orc_paged_decode(const void* q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                     const orc_pool* pool, const int32_t* block_table,
                     int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                     int64_t window, const int32_t* seqs, int64_t n_sel, double* out,
                     double* lse) {
  if (window < 0) return -1;
  if (check_pool(pool, num_q_heads) || elem_size(q_dtype) == 0 || quantised(q_dtype))
    return -1;
  if (!seqs) n_sel = num_seqs;
  int64_t D = pool->head_dim, G = num_q_heads / pool->num_kv_heads;
  int64_t max_ctx = 0;
  for (int64_t i = 0; i < n_sel; ++i) {
    int64_t s = seqs ? seqs[i] : i;
    if (context_lens[s] > max_ctx) max_ctx = context_lens[s];
  }
  int64_t npairs = n_sel * num_q_heads;
#pragma omp parallel
  {
    double* qv = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    double* krow = (double*)malloc(sizeof(double) * D);
    double* vrow = (double*)malloc(sizeof(double) * D);
    double* z = (double*)malloc(sizeof(double) * (max_ctx > 0 ? max_ctx : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < npairs; ++pi) {
      int64_t i = pi / num_q_heads, h = pi % num_q_heads;
      int64_t s = seqs ? seqs[i] : i;
      for (int64_t d = 0; d < D; ++d) qv[d] = load_value(q, q_dtype, (s * num_q_heads + h) * D + d);
      double m, l;
      int64_t first = 0;  /* the oldest visible key */
      if (window > 0 && context_lens[s] > window) first = context_lens[s] - window;
      attend_range(qv, pool, block_table + s * max_blocks_per_seq, h / G, first,
                   context_lens[s], scale, &m, &l, acc, z, krow, vrow);
      double* o = out + (i * num_q_heads + h) * D;
      for (int64_t d = 0; d < D; ++d) o[d] = l > 0 ? acc[d] / l : 0.0;
      if (lse) lse[i * num_q_heads + h] = l > 0 ? m + log(l) : -INFINITY;
    }
    free(qv); free(acc); free(krow); free(vrow); free(z);
  }
  return 0;
}

/* ---- [P1 §4] split-KV partitions ------------------------------------------ */
int orc_decode_partials(const void* q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                        const orc_pool* pool, const int32_t* block_table,
                        int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                        int64_t partition_size, int64_t max_partitions, double* part_out,
                        double* part_max, double* part_sum) {
  if (check_pool(pool, num_q_heads) || elem_size(q_dtype) == 0 || quantised(q_dtype) ||
      partition_size <= 0)
    return -1;
  int64_t D = pool->head_dim, G = num_q_heads / pool->num_kv_heads;
  int64_t npairs = num_seqs * num_q_heads;
#pragma omp parallel
  {
    double* qv = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    double* krow = (double*)malloc(sizeof(double) * D);
    double* vrow = (double*)malloc(sizeof(double) * D);
    double* z = (double*)malloc(sizeof(double) * partition_size);
#pragma omp for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < npairs; ++pi) {
      int64_t s = pi / num_q_heads, h = pi % num_q_heads;
      for (int64_t d = 0; d < D; ++d) qv[d] = load_value(q, q_dtype, (s * num_q_heads + h) * D + d);
      for (int64_t p = 0; p < max_partitions; ++p) {
        int64_t t0 = p * partition_size;
        int64_t t1 = t0 + partition_size;
        if (t1 > context_lens[s]) t1 = context_lens[s];
        double m, l;
        attend_range(qv, pool, block_table + s * max_blocks_per_seq, h / G, t0, t1, scale, &m,
                     &l, acc, z, krow, vrow);
        size_t idx = (size_t)pi * max_partitions + p;
        part_max[idx] = m;
        part_sum[idx] = l;
        for (int64_t d = 0; d < D; ++d) part_out[idx * D + d] = l > 0 ? acc[d] / l : 0.0;
      }
    }
    free(qv); free(acc); free(krow); free(vrow); free(z);
  }
  return 0;
}

/* ---- [P1 §4] merge of (max, exp_sum, weighted_value) ---------------------- */
void orc_state_merge(double m1, double l1, const double* acc1, double m2, double l2,
                     const double* acc2, int64_t head_dim, double* m, double* l, double* acc) {
  double mm = m1 > m2 ? m1 : m2;
  if (mm == -INFINITY) { /* both empty */
    *m = -INFINITY;
    *l = 0.0;
    for (int64_t d = 0; d < head_dim; ++d) acc[d] = 0.0;
    return;
  }
  double a1 = m1 == -INFINITY ? 0.0 : exp(m1 - mm);
  double a2 = m2 == -INFINITY ? 0.0 : exp(m2 - mm);
  *m = mm;
  *l = a1 * l1 + a2 * l2;
  for (int64_t d = 0; d < head_dim; ++d) acc[d] = a1 * acc1[d] + a2 * acc2[d];
}

void orc_split_reduce(const double* part_out, const double* part_max, const double* part_sum,
                      const int32_t* context_lens, int64_t num_seqs, int64_t num_q_heads,
                      int64_t head_dim, int64_t partition_size, int64_t max_partitions,
                      double* out) {
  int64_t D = head_dim;
  int64_t npairs = num_seqs * num_q_heads;
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * D);
    double* pacc = (double*)malloc(sizeof(double) * D);
    double* nacc = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < npairs; ++pi) {
      int64_t s = pi / num_q_heads;
      int64_t np = (context_lens[s] + partition_size - 1) / partition_size;
      if (np > max_partitions) np = max_partitions;
      double m = -INFINITY, l = 0.0;
      for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
      for (int64_t p = 0; p < np; ++p) {
        size_t idx = (size_t)pi * max_partitions + p;
        /* back to the unnormalised weighted sum of this partition */
        for (int64_t d = 0; d < D; ++d) pacc[d] = part_out[idx * D + d] * part_sum[idx];
        double nm, nl;
        orc_state_merge(m, l, acc, part_max[idx], part_sum[idx], pacc, D, &nm, &nl, nacc);
        m = nm;
        l = nl;
        memcpy(acc, nacc, sizeof(double) * D);
      }
      for (int64_t d = 0; d < D; ++d) out[pi * D + d] = l > 0 ? acc[d] / l : 0.0;
    }
    free(acc); free(pacc); free(nacc);
  }
}

/* ---- [P1 §4] chunked prefill over the paged cache ------------------------- */
int orc_paged_prefill(const void* q, int q_dtype, const int32_t* cu_seqlens_q, int64_t num_seqs,
                      int64_t num_q_heads, const orc_pool* pool, const int32_t* block_table,
                      int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                      int causal, const int64_t* rows, int64_t n_rows, double* out) {
  if (check_pool(pool, num_q_heads) || elem_size(q_dtype) == 0 || quantised(q_dtype))
    return -1;
  int64_t total_q = cu_seqlens_q[num_seqs];
  if (!rows) n_rows = total_q;
  int64_t D = pool->head_dim, G = num_q_heads / pool->num_kv_heads;
  int64_t max_ctx = 1;
  for (int64_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_ctx) max_ctx = context_lens[s];
  int64_t npairs = n_rows * num_q_heads;
#pragma omp parallel
  {
    double* qv = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    double* krow = (double*)malloc(sizeof(double) * D);
    double* vrow = (double*)malloc(sizeof(double) * D);
    double* z = (double*)malloc(sizeof(double) * max_ctx);
#pragma omp for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < npairs; ++pi) {
      int64_t i = pi / num_q_heads, h = pi % num_q_heads;
      int64_t row = rows ? rows[i] : i;
      int64_t s = 0; /* owning sequence: cu[s] <= row < cu[s+1] */
      while (s + 1 < num_seqs && cu_seqlens_q[s + 1] <= row) ++s;
      int64_t n = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
      int64_t a = context_lens[s] - n + (row - cu_seqlens_q[s]); /* absolute position */
      int64_t t1 = causal ? a + 1 : context_lens[s];
      if (t1 > context_lens[s]) t1 = context_lens[s];
      for (int64_t d = 0; d < D; ++d)
        qv[d] = load_value(q, q_dtype, (row * num_q_heads + h) * D + d);
      double m, l;
      attend_range(qv, pool, block_table + s * max_blocks_per_seq, h / G, 0, t1, scale, &m, &l,
                   acc, z, krow, vrow);
      double* o = out + (i * num_q_heads + h) * D;
      for (int64_t d = 0; d < D; ++d) o[d] = l > 0 ? acc[d] / l : 0.0;
    }
    free(qv); free(acc); free(krow); free(vrow); free(z);
  }
  return 0;
}
