/*
 * oracle.h — plain, slow CPU oracle for paged KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test-suite, the smoke entry point and the CPU
 * baseline leg of the benchmark do.  It shares no source with the HIP library
 * (no headers, helpers, tables or constants): it is written from the pages'
 * statement of the method, in the most direct form that statement allows.
 *
 * Sources (web pages, by title and section):
 *   [P1] "03 | PagedAttention and the KV-cache memory system"
 *        (llm-infra-atlas): §1 per-token size, §3 block table and slot
 *        formula, §3.1 page bytes, §4 paged kernel loop and online-softmax
 *        triple, §4.1 write path via slot_mapping, §8.1 FP8 with FP32 scales.
 *   [P2] "KV Cache: capacity, layout, lifecycle" (wineandchord):
 *        "Page-table addressing" (physical_slot reference and its errors),
 *        "Physical layout", "Validation" checklist.
 *   [P3] "What is the principle of PagedAttention?" (aigcbaba): §5, paging
 *        does not change the attention result.
 *   [P4] "vLLM notes: PagedAttention memory management" (amentiraz): the
 *        contiguous static cache [max_batch][max_seq][kv_heads][head_dim].
 *
 * Conventions fixed by this oracle (readings where the pages are silent):
 *   - Logical pool layout: pool[num_blocks][num_kv_heads][block_size][head_dim]
 *     of the KV storage type (one page per (block, kv head)), for K and V.
 *   - Query head h reads kv head h / (H_q / H_kv)  (consecutive grouping).
 *   - Decode: context_lens[s] counts every cached token including the one
 *     just written; no mask inside [0, ctx).
 *   - fp8 is OCP E4M3 (bias 7, no infinity, S.1111.111 = NaN, max 448);
 *     dequantised value = decode(code) * scale; encoding takes x / scale in IEEE
 *     fp32 and rounds to nearest, ties to even, saturating finite overflow (and
 *     infinities) to +-448; NaN -> 0x7F with the sign of x.
 *   - int8 ([P1 §8.1] names per-token-head INT8 and nothing more): symmetric,
 *     dequantised value = code * scale; encoding rounds x / scale (IEEE fp32) to
 *     the nearest integer, ties to even, saturating to [-127, 127]; NaN -> 0.
 *   - The scale of element (block, kv head, offset) ([P1 §8.1]: per-tensor
 *     FP8, per-token-head INT8/FP8, the scales counted in the page size):
 *       ORC_SCALE_BLOCK  scale[block * num_kv_heads + head]
 *       ORC_SCALE_TENSOR scale[0]
 *       ORC_SCALE_TOKEN  scale[(block * num_kv_heads + head) * block_size + offset]
 *   - A slot or slot-mapping entry that is negative is padding: skipped.
 *   - ctx = 0 gives an all-zero output and lse = -inf.
 *   - All arithmetic on decoded values is in IEEE double.
 *
 * Parity pins (which test pins which function) are listed at each function.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage type codes (oracle's own numbering) */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_FP8_E4M3 3
#define ORC_INT8 4

/* where the scale of a quantised element lives (see the conventions above) */
#define ORC_SCALE_BLOCK 0
#define ORC_SCALE_TENSOR 1
#define ORC_SCALE_TOKEN 2

/* results of orc_physical_slot, mirroring the page's exceptions */
#define ORC_OK 0
#define ORC_EVALUE 1 /* "invalid block size or token position", or negative physical id */
#define ORC_EINDEX 2 /* "logical block is not allocated" */

/* [P2 "Page-table addressing"]: slot of token_pos through one sequence's table.
 * Pinned by the printed asserts (table [9,2,17], B=4) and by brute force. */
int orc_physical_slot(const int32_t* table, int64_t table_len, int64_t block_size,
                      int64_t token_pos, int64_t* slot);

/* [P1 §4.1]: slot_mapping[i] = table[seq_idx[i]][positions[i] / B] * B + positions[i] % B.
 * Entries whose seq index or position is negative, or for which orc_physical_slot
 * fails, are -1 (padding).  block_table is [num_seqs][max_blocks_per_seq]. */
void orc_slot_mapping(const int32_t* block_table, int64_t num_seqs, int64_t max_blocks_per_seq,
                      const int32_t* seq_idx, const int32_t* positions, int64_t num_tokens,
                      int64_t block_size, int64_t* slot_mapping);

/* storage decoders: exact values of the stored codes */
double orc_f16_decode(uint16_t h);   /* IEEE 754 binary16 */
double orc_bf16_decode(uint16_t b);  /* upper half of an IEEE binary32 */
double orc_e4m3_decode(uint8_t c);   /* OCP 8-bit floating point, E4M3 */
/* nearest E4M3 code to x (ties to even code), saturating; see conventions */
uint8_t orc_e4m3_encode(float x);

/* array forms of the codecs above (for the tests' exhaustive sweeps) */
void orc_decode_n(const void* p, int dtype, int64_t n, double* out);
void orc_e4m3_encode_n(const float* x, int64_t n, uint8_t* out);
/* symmetric int8 code of x (already divided by its scale); pinned against numpy's
 * rint (ties to even) and clip on ties, saturation and random values */
int8_t orc_int8_encode(float x);
void orc_int8_encode_n(const float* x, int64_t n, int8_t* out);

/* [P1 §4.1, §8.1]: scatter the new tokens' K/V into the logical pools.
 * k, v: [num_tokens][num_kv_heads][head_dim] in src_dtype (f32/f16/bf16 bits).
 * For kv_dtype != FP8 the source type must equal kv_dtype and the copy is bitwise;
 * for FP8 each element is encoded as e4m3(x / scale[block][head]).
 * Slots that are negative or >= num_blocks*block_size are skipped.
 * Returns 0, or -1 on an unsupported type combination. */
int orc_kv_cache_write(const int64_t* slot_mapping, int64_t num_tokens, const void* k,
                       const void* v, int src_dtype, int64_t num_blocks, int64_t block_size,
                       int64_t num_kv_heads, int64_t head_dim, int kv_dtype, void* k_pool,
                       void* v_pool, const float* k_scale, const float* v_scale,
                       int scale_mode);

/* Common description of a paged pool, as the oracle reads it. */
typedef struct orc_pool {
  const void* k_pool;    /* logical layout [num_blocks][num_kv_heads][block_size][head_dim] */
  const void* v_pool;
  const float* k_scale;  /* quantised pools only (else NULL), indexed per scale_mode */
  const float* v_scale;
  int64_t num_blocks, block_size, num_kv_heads, head_dim;
  int kv_dtype;
  int scale_mode;        /* ORC_SCALE_*, quantised pools only */
} orc_pool;

/* [P1 §4], [P3 §5]: decode attention.  For each selected sequence s and query
 * head h: gather K_t, V_t for t < ctx_s through block_table, z_t = scale * q.K_t,
 * out = sum_t exp(z_t - max z) V_t / sum_t exp(z_t - max z).
 * q: [num_seqs][num_q_heads][head_dim] of q_dtype.  seqs: indices of the sequences
 * to compute (NULL: all, n_sel ignored).  out: [n_sel][num_q_heads][head_dim];
 * lse (optional): [n_sel][num_q_heads] natural-log sum-exp of z.
 * Pinned by dense contiguous attention (brute force and a library routine), by the
 * closed forms ctx=1 and q=0, and by block-id permutation invariance.
 * window > 0: [P1 §1.1 table, §7] sliding/local attention, only the keys
 * t in [max(0, ctx_s - window), ctx_s) are gathered; 0 = the whole context.
 * Pinned by masked dense attention, window = 1 (out = the newest V row) and by
 * NaN written into every key before the window. */
int orc_paged_decode(const void* q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                     const orc_pool* pool, const int32_t* block_table,
                     int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                     int64_t window, const int32_t* seqs, int64_t n_sel, double* out,
                     double* lse);

/* [P1 §4] split-KV: partition i of sequence s covers tokens
 * [i*P, min((i+1)*P, ctx_s)).  For each non-empty partition:
 * part_max = max z, part_sum = sum exp(z - part_max),
 * part_out = sum exp(z - part_max) V / part_sum.  Empty partitions get
 * (-inf, 0, 0).  Arrays: part_out [num_seqs][num_q_heads][max_partitions][head_dim],
 * part_max/part_sum [num_seqs][num_q_heads][max_partitions]. */
int orc_decode_partials(const void* q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                        const orc_pool* pool, const int32_t* block_table,
                        int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                        int64_t partition_size, int64_t max_partitions, double* part_out,
                        double* part_max, double* part_sum);

/* [P1 §4] merge of two online-softmax states (max, exp_sum, weighted_value),
 * where weighted_value is the UNnormalised sum exp(z - max) V.  An empty state is
 * (-inf, 0, 0); merging with it returns the other state. */
void orc_state_merge(double m1, double l1, const double* acc1, double m2, double l2,
                     const double* acc2, int64_t head_dim, double* m, double* l, double* acc);

/* Log-sum-exp reduction of partitions written in orc_decode_partials' format
 * (normalised part_out): the first ceil(ctx_s / P) partitions of sequence s are
 * folded with orc_state_merge in order; ctx 0 gives zeros.
 * out: [num_seqs][num_q_heads][head_dim]. */
void orc_split_reduce(const double* part_out, const double* part_max, const double* part_sum,
                      const int32_t* context_lens, int64_t num_seqs, int64_t num_q_heads,
                      int64_t head_dim, int64_t partition_size, int64_t max_partitions,
                      double* out);

/* [P1 §4] chunked prefill over the paged cache.  Sequence s owns query rows
 * [cu_seqlens_q[s], cu_seqlens_q[s+1]); with n_s rows, row i sits at absolute
 * position a = ctx_s - n_s + i and (causal) sees keys t <= a, or (non-causal)
 * every t < ctx_s.  A row that sees no key gets zeros.
 * q: [total_q][num_q_heads][head_dim].  rows: global row indices to compute
 * (NULL: all rows, n_rows = total_q).  out: [n_rows][num_q_heads][head_dim]. */
int orc_paged_prefill(const void* q, int q_dtype, const int32_t* cu_seqlens_q, int64_t num_seqs,
                      int64_t num_q_heads, const orc_pool* pool, const int32_t* block_table,
                      int64_t max_blocks_per_seq, const int32_t* context_lens, double scale,
                      int causal, const int64_t* rows, int64_t n_rows, double* out);

/* number of OpenMP threads the oracle uses (for reporting) */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
