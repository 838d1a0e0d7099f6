/*
 * pagedkv.h — C ABI of libpagedkv.so: paged KV-cache attention for AMD MI355X
 * (gfx950).
 *
 * The method (web pages, by title and section):
 *   [P1] "03 | PagedAttention and the KV-cache memory system" (llm-infra-atlas)
 *        §3 block table, slot formula; §3.1 page bytes; §4 paged kernel loop,
 *        online-softmax triple, split-KV decode, tiled prefill given the table;
 *        §4.1 write path through slot_mapping; §4.2 stable buffers, free only
 *        after consumers finish; §8.1 quantised KV (FP8 / INT8 codes with FP32
 *        scales per block and head, per tensor, or per token and head).
 *   [P2] "KV Cache: capacity, layout, lifecycle" (wineandchord)
 *        "Page-table addressing" (physical_slot and its errors), "Physical
 *        layout", "Correctness contract" (reject a mismatched descriptor),
 *        "Lifecycle and ownership" and "Reference counting and tail-block
 *        COW" (the block allocator).
 *
 * General conventions
 *   - Every pointer named *device* is device memory the CALLER owns.  The
 *     library never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and is complete only
 *     when that stream is.  Nothing is copied host<->device on any call.
 *   - Blocks must not be freed or reused until the stream work that reads or
 *     writes them has completed ([P1 §4.2]); that is the caller's job.
 *   - Device pointers must be 16-byte aligned; tensors are dense, row-major.
 *   - Outputs never alias inputs.
 *   - Return value: PKV_OK (0) or a negative status (pkv_strerror explains it).
 *     Argument errors are detected on the host before anything is enqueued.
 *     Contents of device arrays (block tables, context lengths, slots) cannot
 *     be checked without a copy; kernels treat them defensively instead (see
 *     each call) so that a bad entry can corrupt results but never memory
 *     outside the caller's buffers.
 *   - All entry points are thread-safe.  The only process-wide state is a
 *     per-device cache of device properties, an atomic call counter that tags
 *     balanced-mode calls, and the scratch array of
 *     pkv_paged_attention_decode_noalloc (one per device) with its resolved
 *     addresses.  The block allocator (pkv_alloc_*) is host bookkeeping with one
 *     lock per allocator.
 *
 * Physical pool layout (owned by this library; one pool for K, one for V, per
 * layer).  With E = bytes per element and X = 16 / E elements per 16 bytes:
 *   K pool: [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *   V pool: [num_blocks][num_kv_heads][block_size / TG][head_dim][TG],
 *           TG = min(X, block_size) consecutive tokens of a dim per run
 *   scales of a quantised pool (K and V separately): float arrays whose shape
 *   the descriptor's scale_mode sets (pkv_scale_mode below)
 * (block strides other than the dense one: see pkv_pool_desc.block_stride).
 * One (block, kv head) page is contiguous in each pool.  The logical element
 * K[block][head][t][d] lives at K pool index
 *   (((block*num_kv_heads + head)*(head_dim/X) + d/X)*block_size + t)*X + d%X
 * and V[block][head][t][d] at V pool index
 *   (block*num_kv_heads + head)*block_size*head_dim + (t/TG)*TG*head_dim + d*TG + t%TG.
 * Both are the operand layouts of the matrix-core products: 16 bytes of one K
 * row (X consecutive dims of a token) and a run of one V column (consecutive
 * tokens of a dim) are a lane's loads.  A token's V row lies in one run group:
 * its head_dim elements are TG elements apart, so storing a new token touches
 * head_dim * TG * E / 64 lines of 64 bytes rather than head_dim.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_VERSION 100

/* element types; fp8 is OCP E4M3 (bias 7, max 448, no infinity); int8 is a
 * symmetric code (value = code * scale).  fp8 and int8 pools are "quantised":
 * each element has an fp32 scale, placed as the descriptor's scale_mode says. */
typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3,
  PKV_INT8 = 4
} pkv_dtype;

/* [P1 §8.1] where the scale of a quantised element (block, kv head, token offset)
 * lives; k_scale and v_scale are separate device float arrays of this shape:
 *   PKV_SCALE_BLOCK  [num_blocks][num_kv_heads]               (one per page)
 *   PKV_SCALE_TENSOR [1]                                      (one per pool)
 *   PKV_SCALE_TOKEN  [num_blocks][num_kv_heads][block_size]   (per token and head) */
typedef enum pkv_scale_mode {
  PKV_SCALE_BLOCK = 0,
  PKV_SCALE_TENSOR = 1,
  PKV_SCALE_TOKEN = 2
} pkv_scale_mode;

/* status codes */
enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,       /* invalid argument (null/misaligned pointer, size, mismatch) */
  PKV_ERANGE = -2,       /* position / block id outside the table or the pool */
  PKV_EUNSUPPORTED = -3, /* valid request with no kernel instantiation here */
  PKV_EWORKSPACE = -4,   /* workspace too small */
  PKV_EHIP = -5,         /* HIP runtime reported an error while launching */
  PKV_ENOBLOCKS = -6     /* block allocator: no free block (nothing was changed) */
};

/* Descriptor of one layer's paged pool ([P1 §3.1]; [P2 "Correctness contract"]:
 * every call validates it and rejects a mismatch instead of reinterpreting).
 * Supported: block_size a power of two in [1, 64]; head_dim 64 or 128;
 * num_kv_heads >= 1; num_blocks >= 1. */
typedef struct pkv_pool_desc {
  int32_t num_blocks;
  int32_t block_size;   /* tokens per block (B) */
  int32_t num_kv_heads; /* H_kv */
  int32_t head_dim;     /* D */
  int32_t kv_dtype;     /* pkv_dtype */
  int32_t scale_mode;   /* pkv_scale_mode: quantised pools; 0 for the others */
  /* [P1 §3.1] bytes from block b to block b + 1 in each pool; 0 = dense
   * (num_kv_heads pages of block_size * head_dim elements).  A larger stride,
   * a multiple of 16, lets one allocation hold every layer's K and V of a block
   * together ("cross-layer" blocks, [block][layer][K|V][kv head][page]): layer
   * l's k_pool / v_pool point at its K / V pages of block 0 and the stride is
   * the whole block.  All layers share the block ids (and a block table). */
  int64_t block_stride;
} pkv_pool_desc;

/* Human-readable text of a status code (static storage). */
const char* pkv_strerror(int status);

/* PKV_VERSION of the built library. */
int pkv_version(void);

/* [P1 §3.1] Bytes of the K pool and the V pool:
 *   num_blocks * num_kv_heads * block_size * head_dim * E  each,
 * i.e. the per-layer page size 2*block_size*num_kv_heads*head_dim*E split
 * into K and V; with a block_stride, the span one pool pointer addresses,
 * (num_blocks - 1) * block_stride + num_kv_heads * block_size * head_dim * E;
 * for quantised pools also the bytes of ONE scale array in the
 * descriptor's scale mode ([P1 §8.1]: the scales count in the page size), else
 * 0.  Any output pointer may be NULL.
 * Errors: PKV_EINVAL for a NULL/invalid descriptor, PKV_EUNSUPPORTED for a
 * valid one this library has no kernels for. */
int pkv_pool_bytes(const pkv_pool_desc* pool, size_t* k_bytes, size_t* v_bytes,
                   size_t* scale_bytes_each);

/* [P2 "Page-table addressing"] Host-side slot of one position, with the page's
 * error rules: block_size <= 0 or token_pos < 0 -> PKV_EINVAL;
 * token_pos / block_size >= table_len -> PKV_ERANGE ("logical block is not
 * allocated"); a negative physical id -> PKV_EINVAL.  Otherwise
 * *slot = table[token_pos / B] * B + token_pos % B.  `table` is HOST memory. */
int pkv_physical_slot(const int32_t* table, int32_t table_len, int32_t block_size,
                      int64_t token_pos, int64_t* slot);

/* Host-side check of block tables before they are uploaded: for each sequence
 * s, entries [0, ceil(context_lens[s] / block_size)) of its row must lie in
 * [0, num_blocks), and ceil(ctx/B) <= max_blocks_per_seq.  HOST arrays.
 * Returns PKV_OK, PKV_ERANGE (bad entry or length) or PKV_EINVAL. */
int pkv_validate_block_table(const int32_t* block_table, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t block_size, int32_t num_blocks);

/* [P1 §3, §4.1] Slot of every new token, on the device:
 *   slot_mapping[i] = block_table[seq_idx[i]][positions[i] / B] * B + positions[i] % B.
 * Device arrays: block_table int32 [num_seqs][max_blocks_per_seq],
 * seq_idx and positions int32 [num_tokens], slot_mapping int64 [num_tokens] (out).
 * Token i gets -1 (padding, skipped by pkv_kv_cache_write) wherever the host
 * reference would raise: seq_idx outside [0, num_seqs), positions[i] < 0,
 * logical block >= max_blocks_per_seq, or a negative table entry.
 * num_tokens == 0 enqueues nothing.  Errors: PKV_EINVAL, PKV_EHIP. */
int pkv_slot_mapping(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                     const int32_t* seq_idx, const int32_t* positions, int32_t num_tokens,
                     int32_t block_size, int64_t* slot_mapping, void* stream);

/* [P1 §4.1, §8.1] Scatter the new tokens' K and V into the pools
 * ("reshape_and_cache"): for i < num_tokens (the length of slot_mapping, not of
 * any padded K/V), if 0 <= slot_mapping[i] < num_blocks*block_size, token i's
 * K/V rows k[i][h][:], v[i][h][:] are stored at block slot/B, offset slot%B.
 *   k, v: device [num_tokens][num_kv_heads][head_dim] of src_dtype.
 *   Unquantised pools: src_dtype must equal pool->kv_dtype; the copy is bitwise.
 *   Quantised pools: src_dtype in {F32, F16, BF16}.  With s the element's scale
 *     (the one for its block and head, for the pool, or for its token and head,
 *     as scale_mode says) and x / s an IEEE fp32 division, fp8 stores
 *     e4m3(x / s) rounded to nearest (ties to even), saturating finite overflow
 *     and infinities to +-448, NaN staying NaN; int8 stores x / s rounded to
 *     the nearest integer (ties to even) and clamped to [-127, 127], infinities
 *     giving +-127 and NaN 0.  k_scale, v_scale: device float arrays of the
 *     scale mode's shape, read only: the caller owns and chooses the scales
 *     (in token mode, those of the tokens being written).
 * Negative or out-of-pool slots are skipped.  Two tokens with the same slot
 * race (the caller's slot mapping should be injective).
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP. */
int pkv_kv_cache_write(const int64_t* slot_mapping, int32_t num_tokens, const void* k,
                       const void* v, int32_t src_dtype, const pkv_pool_desc* pool,
                       void* k_pool, void* v_pool, const float* k_scale, const float* v_scale,
                       void* stream);

/* [P1 §3, §4.1] Slot mapping and scatter in one launch: token i is written as by
 * pkv_kv_cache_write at the slot pkv_slot_mapping computes for
 * (seq_idx[i], positions[i]) through block_table (-1 cases skipped).  Same
 * arguments and rules as those two calls; slot_mapping_out (device int64
 * [num_tokens]) receives the slots when non-NULL.  For a decode step, where the
 * one new token of each sequence needs no separate slot array.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP. */
int pkv_kv_cache_append(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* seq_idx, const int32_t* positions, int32_t num_tokens,
                        const void* k, const void* v, int32_t src_dtype,
                        const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                        const float* k_scale, const float* v_scale, int64_t* slot_mapping_out,
                        void* stream);

/* partition_size value selecting balanced split-KV (see pkv_paged_attention_decode) */
#define PKV_PARTITION_BALANCED (-1)
/* upper bound on the wavefront workers of the balanced mode */
#define PKV_MAX_WORKERS 4096

/* Workspace bytes pkv_paged_attention_decode needs for a given partition size:
 *   partition_size == 0 (unsplit): 0.
 *   partition_size > 0 (fixed partitions of P tokens):
 *     num_seqs * num_q_heads * P_max * (head_dim + 2) * 4,  P_max = ceil(max_context_len / P),
 *     laid out as part_out float [S][H_q][P_max][D], then part_max float [S][H_q][P_max],
 *     then part_sum float [S][H_q][P_max] (the arrays pkv_split_kv_reduce takes).
 *   partition_size == PKV_PARTITION_BALANCED: enough for PKV_MAX_WORKERS workers,
 *     C + 2 * PKV_MAX_WORKERS * (num_q_heads / num_kv_heads) * (head_dim + 2) * 4 with
 *     C = num_seqs * num_kv_heads * 8 rounded up to a multiple of 256; the layout is
 *     internal (a counter per (sequence, kv head), then the partial states of the
 *     pairs that workers share).  It needs no initialisation: counters written by
 *     another call are recognised as stale, and every call leaves its counters at
 *     rest, so the same workspace serves any number of calls (and graph replays);
 *     calls that share one workspace must not overlap in time.
 * Errors: PKV_EINVAL (negative sizes, num_q_heads % num_kv_heads != 0, any other
 * partition_size that is not a positive multiple of 64). */
int pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                               size_t* bytes);

/* [P1 §4] Partition size for a decode step, from the context lengths as the host
 * holds them (a serving loop knows them before it launches).  The unsplit and
 * fixed-partition decodes run one workgroup per CU, handed out in launch order,
 * so the step is fastest when the workgroups fill the CUs in few rounds of even
 * work:
 *   - 0 (unsplit, longest contexts first) when the (sequence, kv head) pairs with a
 *     token already number at least num_cus, or when no split would cut anything;
 *   - else the smallest multiple of 64, P >= 256 (a 64-token chunk for each of a
 *     workgroup's four wavefronts), with num_kv_heads * sum_s ceil(ctx_s / P) <=
 *     num_cus (one round of workgroups); 0 if that P cuts no context.
 *   context_lens: HOST int32 [num_seqs], clamped to [0, max_context_len] as the
 *     decode clamps them.
 *   num_cus: compute units of the device the step runs on; <= 0 asks the current
 *     HIP device.
 *   partition_size: out, 0 or a positive multiple of 64, for
 *     pkv_paged_attention_decode / pkv_decode_append.
 * Errors: PKV_EINVAL (negative sizes, num_kv_heads < 1, null pointers), PKV_EHIP
 * (no current device to ask). */
int pkv_decode_partition_size(const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_kv_heads, int32_t max_context_len, int32_t num_cus,
                              int32_t* partition_size);

/* [P1 §4] Paged decode attention, one query token per sequence.
 * For sequence s and query head h (kv head h / (num_q_heads / num_kv_heads)):
 *   z_t = scale * <q[s][h], K_t>,  t < ctx_s, K_t/V_t found through
 *   block_table[s][t / B] at offset t % B (a quantised code times its scale),
 *   out[s][h] = sum_t exp(z_t - max z) V_t / sum_t exp(z_t - max z)
 * with fp32 accumulation; ctx_s = 0 gives zeros.  The newest token's K/V
 * must already have been written (context_lens counts it).
 *   q: device [num_seqs][num_q_heads][head_dim] of q_dtype;
 *      (pool f32, q f32), (f16, f16), (bf16, bf16), (fp8 or int8, bf16|f16)
 *      supported, each scale mode for the quantised pools.  Quantised pools:
 *      the softmax weights (at most 1) times V's scale enter the P.V product
 *      as f16 values, so v_scale must stay below 65504.
 *   k_pool, v_pool: device, layout above; k_scale, v_scale: quantised pools
 *      only, else NULL.  Scales of slots past a sequence's context are never
 *      used (in token mode they may hold anything, NaN included).
 *   block_table: device int32 [num_seqs][max_blocks_per_seq].
 *   context_lens: device int32 [num_seqs]; each is clamped to
 *      [0, min(max_context_len, max_blocks_per_seq * block_size)].
 *   max_context_len: host-known upper bound on context_lens (sizes the grid).
 *   partition_size: 0 = one pass per (sequence, kv head); a positive multiple
 *      of 64 = the context is split into partitions of that many tokens,
 *      scanned in parallel and merged by log-sum-exp (split-KV, [P1 §4]; at most
 *      8192 partitions of max_context_len, else PKV_EUNSUPPORTED);
 *      PKV_PARTITION_BALANCED = the 64-token chunks of all (sequence, kv head)
 *      pairs are cut into equal contiguous shares, one per resident wavefront,
 *      and the pairs that shares split are merged by log-sum-exp (same
 *      algebra; evenly loaded whatever the length mix; num_seqs <= 16384).
 *   workspace: device scratch of pkv_decode_workspace_bytes (NULL if 0 bytes);
 *      in balanced mode a smaller workspace just means fewer workers (it must
 *      hold the counters and one worker: C + 2 * G * (head_dim + 2) * 4 bytes).
 *      In balanced mode the pairs that several workers share are merged by the
 *      last of them to finish, inside the same kernel launch.
 *   out: device [num_seqs][num_q_heads][head_dim] of q_dtype (rounded to nearest).
 * Table entries outside [0, num_blocks) are clamped into range (wrong results,
 * never a fault); pkv_validate_block_table checks tables on the host.
 * Errors: PKV_EINVAL (incl. num_q_heads % num_kv_heads != 0), PKV_EUNSUPPORTED
 * (e.g. group size > 16 or a dtype pair above not listed), PKV_EWORKSPACE, PKV_EHIP. */
int pkv_paged_attention_decode(const void* q, int32_t q_dtype, int32_t num_seqs,
                               int32_t num_q_heads, const pkv_pool_desc* pool,
                               const void* k_pool, const void* v_pool, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, float scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, void* out, void* stream);

/* [P1 §4.1, §4] One decode step in one launch: the write path's append of each
 * sequence's newest token followed by decode, i.e. the same pool bytes and output
 * as pkv_kv_cache_append (positions ctx_s - 1) then pkv_paged_attention_decode
 * with the same partition_size (PKV_PARTITION_BALANCED, 0, or a positive multiple
 * of 64: fixed partitions add the reduce launch).  The wavefront that reads the
 * newest token's chunk first stores its K and V rows (from k_new / v_new) into slot
 * block_table[s][(ctx_s - 1) / B] * B + (ctx_s - 1) % B and then reads them back
 * from the pool like any other key; a table entry outside the pool skips the
 * store (slot -1).
 *   k_new, v_new: device [num_seqs][num_kv_heads][head_dim] of the pool's type.
 *   Supported: f16 or bf16 pools with q of the same type (else PKV_EUNSUPPORTED).
 *   context_lens count the new token (ctx_s >= 1 for a sequence that has one;
 *   ctx_s = 0 stores nothing, leaves slot_mapping_out[s] as it was and gives
 *   zeros); their clamping, the workspace (pkv_decode_workspace_bytes with the
 *   same partition_size; none for 0) and
 *   the errors are those of pkv_paged_attention_decode.
 *   slot_mapping_out: optional device int64 [num_seqs], the slots written. */
int pkv_decode_append(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                      const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len, const void* k_new,
                      const void* v_new, float scale, int32_t partition_size, void* workspace,
                      size_t workspace_bytes, void* out, int64_t* slot_mapping_out,
                      void* stream);

/* [P1 §1.1 table, §7] Sliding-window (local) decode: as pkv_paged_attention_decode,
 * but the query of sequence s (at position p = ctx_s - 1) sees only the keys of
 * its window [p - window + 1, p], i.e. t in [max(0, ctx_s - window), ctx_s).
 * Blocks entirely older than the window are never read and their table entries
 * may hold anything (the allocator may have released them): with block_size >=
 * 16 the kernels start at the window's first 16-token tile, which lies in that
 * key's own block; with smaller blocks every token below the window is replaced
 * by the window's first key before its block is looked up.  window = 0 is the
 * whole context (pkv_paged_attention_decode is this call with window 0).  Same
 * arguments, partition modes, workspace sizes and errors otherwise; window < 0
 * is PKV_EINVAL. */
int pkv_paged_attention_decode_window(const void* q, int32_t q_dtype, int32_t num_seqs,
                                      int32_t num_q_heads, const pkv_pool_desc* pool,
                                      const void* k_pool, const void* v_pool,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      float scale, int32_t window, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* out,
                                      void* stream);

/* Decode for a batch whose sequences share a prefix of blocks ([P1] §5: two
 * requests that hit the same prefix pages point their block tables at the same
 * physical blocks, with reference counts; [P3] section 4, block-level sharing:
 * sequences with the same prompt share read-only physical blocks).  Computes
 * exactly what pkv_paged_attention_decode computes (up to rounding order), but
 * reads each shared block once per kv head for the whole batch instead of once
 * per sequence:
 *   1. the prefix tokens [0, shared_len): one pass per (kv head, slice of the
 *      prefix) over row 0's blocks, the queries of 16/G sequences x G heads in
 *      the 16 columns of each matrix-core tile.  For the type pairs, block
 *      sizes and groups that pkv_paged_prefill takes, the pass is that
 *      kernel's: each K/V chunk is staged once in LDS for 128/G sequences, and
 *      a sequence's rows see the prefix keys below min(ctx_s, shared_len);
 *      prefix slots past every sequence's context are never read;
 *   2. every sequence's own tokens [shared_len, ctx_s): the balanced decode,
 *      started shared_len / block_size entries into each table row;
 *   3. the log-sum-exp merge of the prefix slices and the tail (as
 *      pkv_split_kv_reduce).
 *   shared_len: a multiple of block_size, at most max_blocks_per_seq *
 *      block_size.  The caller guarantees block_table[s][j] == block_table[0][j]
 *      for every s and every j < shared_len / block_size (the kernel reads row
 *      0 there; a row that differs is not detected and gets row 0's keys).  A
 *      sequence with ctx_s < shared_len sees only its first ctx_s keys.
 *   workspace: device, at least pkv_decode_shared_workspace_bytes bytes,
 *      16-byte aligned, no initialisation needed; calls that share it must
 *      not overlap in time.
 *   Everything else as pkv_paged_attention_decode (same dtypes, scale modes,
 *   block sizes and head-group limits); shared_len = 0 is the balanced decode.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP. */
int pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t shared_len,
                                      size_t* bytes);
int pkv_paged_attention_decode_shared(const void* q, int32_t q_dtype, int32_t num_seqs,
                                      int32_t num_q_heads, const pkv_pool_desc* pool,
                                      const void* k_pool, const void* v_pool,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t shared_len, float scale, void* workspace,
                                      size_t workspace_bytes, void* out, void* stream);

/* Bytes of the device array behind pkv_paged_attention_decode_noalloc (one per
 * device, held until the process ends). */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): pkv_paged_attention_decode
 * without the workspace argument.  The split-KV scratch is a device array owned by
 * the library, PKV_NOALLOC_SCRATCH_BYTES bytes on each device the call runs on;
 * its address is resolved on the first call made with that device current
 * (a caller that captures makes one call before capturing).  No call allocates or
 * frees anything.  Every argument and partition mode as in
 * pkv_paged_attention_decode: 0 uses no scratch; fixed partitions need
 * pkv_decode_workspace_bytes(...) bytes, and a call that needs more than the array
 * returns PKV_EWORKSPACE before touching the device; the balanced mode runs as
 * many wavefront workers as the array holds.  All calls on one device share the
 * array, which keeps the last call's contents (no call needs it cleared): calls
 * that overlap in time on one device race, so issue them on one stream or order
 * their streams.  Errors as pkv_paged_attention_decode, plus PKV_EWORKSPACE. */
int pkv_paged_attention_decode_noalloc(const void* q, int32_t q_dtype, int32_t num_seqs,
                                       int32_t num_q_heads, const pkv_pool_desc* pool,
                                       const void* k_pool, const void* v_pool,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len,
                                       float scale, int32_t partition_size, void* out,
                                       void* stream);

/* [P1 §4] Log-sum-exp merge of split-KV partitions.  For sequence s, head h,
 * partitions i < min(ceil(ctx_s / partition_size), max_partitions) with state
 * (m_i = part_max, l_i = part_sum, o_i = part_out normalised by l_i):
 *   M = max_i m_i,  w_i = exp(m_i - M) * l_i,  out = sum_i w_i o_i / sum_i w_i.
 * m is in natural-log units of the scaled logits z.  Partitions with l_i = 0
 * contribute nothing; ctx_s = 0 gives zeros.
 *   part_out: device float [num_seqs][num_q_heads][max_partitions][head_dim];
 *   part_max, part_sum: device float [num_seqs][num_q_heads][max_partitions];
 *   context_lens: device int32 [num_seqs] (clamped to [0, max_partitions*P]);
 *   out: device [num_seqs][num_q_heads][head_dim] of out_dtype (F32/F16/BF16).
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP. */
int pkv_split_kv_reduce(const float* part_out, const float* part_max, const float* part_sum,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t head_dim, int32_t partition_size, int32_t max_partitions,
                        void* out, int32_t out_dtype, void* stream);

/* [P1 §4] Chunked prefill over the paged cache (tiled, matrix cores).
 * Sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]); with n_s
 * rows, row i sits at absolute position a = ctx_s - n_s + i and attends to
 * keys t <= a (causal != 0) or to every t < ctx_s (causal == 0), read through
 * the block table; those tokens' K/V must already be in the pool.  Rows that
 * see no key (n_s > ctx_s) get zeros.
 *   q: device [total_q][num_q_heads][head_dim] of q_dtype; out likewise.
 *   cu_seqlens_q: device int32 [num_seqs + 1], non-decreasing, last = total_q.
 *   max_q_len: host-known upper bound on n_s (sizes the grid).
 *   Supported: q bf16 with a bf16 pool or an fp8 pool in PKV_SCALE_BLOCK mode,
 *   q f16 with an f16 pool (other pairs: PKV_EUNSUPPORTED); out has q's
 *   dtype; head_dim 64 or 128; block_size 16..64 (a 16-token tile must lie
 *   in one block); group size G = H_q/H_kv in {1, 2, 4, 8, 16}.  fp8 keys
 *   widen exactly to bf16 for QK^T and K's scale multiplies the scores; fp8
 *   values widen exactly to f16 and are multiplied in f16 by V's scale
 *   (rounded to f16), so the scaled values must lie in f16's range.  The
 *   probabilities (taken against a reference that trails the running max by
 *   less than a factor 16) enter P.V as f16 for fp8 and f16 pools, and their
 *   sum adds those same f16 values; with a bf16 pool they enter as a hi + lo
 *   pair of bf16 values.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP. */
int pkv_paged_prefill(const void* q, int32_t q_dtype, const int32_t* cu_seqlens_q,
                      int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                      const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t causal, void* out,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Block allocator (host) and block copies.  [P2] "Lifecycle and ownership",
 * "Reference counting and tail-block COW"; [P1] §5 (free queue, reference
 * counts, fork of shared prefixes).
 *
 * A physical block is free, exclusive (refcount 1) or shared read-only
 * (refcount > 1); a block's refcount is the number of live sequences whose
 * table holds it.  The allocator keeps each sequence's block table and its
 * committed length.  Free blocks form a stack: the block pushed last is handed
 * out first.
 *   fork: the child starts with a copy of the parent's table and length; every
 *     block gains a reference.  Full blocks stay shared: nobody writes them.
 *   append: claims the slot of the sequence's next token and commits it (table
 *     and length change together).  A token that opens a block takes a fresh
 *     block.  A token that lands in a partly filled tail shared with another
 *     sequence first moves this sequence onto a fresh block (copy on write):
 *     the old block loses one reference and the call reports the pair
 *     (cow_src, cow_dst), whose committed K/V and scales the caller copies with
 *     pkv_copy_blocks on the stream BEFORE any kernel reads the new table or
 *     writes the slot.  No copy: both are -1.
 *   free: releases each block of the sequence once.  A block whose refcount
 *     drops to 0 goes back on the free stack right away, or, given an event
 *     recorded after the last GPU work that touches the sequence, only once
 *     that event has completed (checked whenever a fresh block is needed and by
 *     pkv_alloc_free_blocks), so queued GPU work never sees a block reused.
 *     Released blocks are pushed in reverse table order: the sequence's first
 *     block is handed out next.
 * Device block tables are the caller's to upload (pkv_alloc_block_table
 * exports one sequence's row).  Errors: PKV_EINVAL (bad argument, unknown or
 * already released sequence), PKV_ERANGE (capacity too small, block id out of
 * range), PKV_ENOBLOCKS (no free block; the allocator is unchanged).
 * -------------------------------------------------------------------------*/
typedef struct pkv_alloc pkv_alloc;

/* free_order: HOST int32 [num_free], the initial free stack bottom to top (its
 * last entry is handed out first); ids must be distinct and in [0, num_blocks);
 * blocks left out are never handed out (a padding block, say).  NULL: every
 * block, handed out as 0, 1, 2, ...  *out receives the allocator. */
int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                     int32_t num_free, pkv_alloc** out);
void pkv_alloc_destroy(pkv_alloc* alloc);
/* a new empty sequence; *seq receives its id */
int pkv_alloc_add_seq(pkv_alloc* alloc, int32_t* seq);
int pkv_alloc_fork(pkv_alloc* alloc, int32_t parent, int32_t* child);
/* *slot = table[length / B] * B + length % B for the token being committed */
int pkv_alloc_append(pkv_alloc* alloc, int32_t seq, int64_t* slot, int32_t* cow_src,
                     int32_t* cow_dst);
/* event: a hipEvent_t recorded after the sequence's last GPU use, or NULL; it
 * must stay valid until its blocks are back on the free stack (or the allocator
 * is destroyed) */
int pkv_alloc_free_seq(pkv_alloc* alloc, int32_t seq, void* event);
/* table: HOST int32 [capacity] (may be NULL to query the sizes only) */
int pkv_alloc_block_table(pkv_alloc* alloc, int32_t seq, int32_t* table, int32_t capacity,
                          int32_t* num_blocks, int64_t* length);
int pkv_alloc_refcount(pkv_alloc* alloc, int32_t block, int32_t* refcount);
/* the free stack bottom to top (after reclaiming blocks whose events completed) */
int pkv_alloc_free_blocks(pkv_alloc* alloc, int32_t* free_order, int32_t capacity,
                          int32_t* num_free);

/* [P2] "Reference counting and tail-block COW": copy whole blocks.
 *   pairs: device int32 [num_pairs][2] of (src, dst) block ids.  For each pair,
 *   every byte of block src in both pools (all kv heads) and, for quantised
 *   pools in block or token mode, its scales (k_scale[src] and v_scale[src]:
 *   every head, and every offset in token mode) are copied to dst; a
 *   PKV_SCALE_TENSOR scale belongs to no block and is left as it is.  Pairs with
 *   an id outside [0, num_blocks), or src == dst, are skipped; destinations
 *   must be distinct and must not be the source of another pair (else the
 *   copies race).  k_scale, v_scale: device float arrays of the scale mode's
 *   shape, quantised pools only (else ignored).  Errors: PKV_EINVAL, PKV_EUNSUPPORTED,
 *   PKV_EHIP. */
int pkv_copy_blocks(const int32_t* pairs, int32_t num_pairs, const pkv_pool_desc* pool,
                    void* k_pool, void* v_pool, float* k_scale, float* v_scale, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
