// api.cpp — C-ABI front end of libpagedkv.so: argument validation on the host,
// then dispatch to the kernel launchers.  Stateless and allocation-free.
#include "../../include/pagedkv.h"

#include <hip/hip_runtime_api.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "internal.hpp"
#include "prefill.hpp"
#include "slot.hpp"

namespace {

constexpr int kMaxHeadsGroup = 16;
constexpr int kMaxBalancedSeqs = 16384;  // unit prefix lives in LDS

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_INT8: return 1;
    default: return 0;
  }
}

bool quantised(int dt) { return dt == PKV_FP8_E4M3 || dt == PKV_INT8; }

// floats in one scale array of a quantised pool
size_t scale_count(const pkv_pool_desc* d) {
  switch (d->scale_mode) {
    case PKV_SCALE_TENSOR: return 1;
    case PKV_SCALE_TOKEN: return (size_t)d->num_blocks * d->num_kv_heads * d->block_size;
    default: return (size_t)d->num_blocks * d->num_kv_heads;
  }
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// 16-byte units from one block to the next in each pool (of a validated descriptor)
long long block_units(const pkv_pool_desc* d) {
  const int64_t bytes = d->block_stride ? d->block_stride
                                        : (int64_t)d->num_kv_heads * d->block_size *
                                              d->head_dim * elem_bytes(d->kv_dtype);
  return (long long)(bytes / 16);
}

// Descriptor validation ("KV Cache: capacity, layout, lifecycle", correctness
// contract: a mismatched descriptor is rejected, never reinterpreted).
int check_desc(const pkv_pool_desc* d) {
  if (!d) return PKV_EINVAL;
  if (d->num_blocks < 1 || d->block_size < 1 || d->num_kv_heads < 1 || d->head_dim < 1)
    return PKV_EINVAL;
  if (elem_bytes(d->kv_dtype) == 0) return PKV_EINVAL;
  if (quantised(d->kv_dtype) ? (d->scale_mode < PKV_SCALE_BLOCK || d->scale_mode > PKV_SCALE_TOKEN)
                             : d->scale_mode != 0)
    return PKV_EINVAL;
  if ((d->head_dim * elem_bytes(d->kv_dtype)) % 16 != 0) return PKV_EINVAL;
  if (!pow2(d->block_size) || d->block_size > 64) return PKV_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_EUNSUPPORTED;
  // a block stride leaves room for at least the block's own pages, in 16-byte steps
  const int64_t dense = (int64_t)d->num_kv_heads * d->block_size * d->head_dim *
                        elem_bytes(d->kv_dtype);
  if (d->block_stride != 0 && (d->block_stride < dense || d->block_stride % 16 != 0))
    return PKV_EINVAL;
  // page-aligned pools: total element count must fit the kernels' index math
  const double rows = (double)d->num_blocks * d->num_kv_heads * d->block_size;
  if (rows >= 4294967296.0) return PKV_EUNSUPPORTED;
  return PKV_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// balanced mode: one 8-byte counter per (sequence, kv head), rounded to 256 bytes
size_t balanced_counter_bytes(int num_seqs, int num_kv_heads) {
  const size_t b = (size_t)num_seqs * num_kv_heads * 8;
  return (b + 255) / 256 * 256;
}

// a fresh nonzero tag per balanced call (see the counter scheme in decode.hip)
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0x9e3779b9u};
  uint32_t e;
  do {
    e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  } while (e == 0);
  return e;
}

}  // namespace

extern "C" {

const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_ERANGE: return "position or block id outside the table or the pool";
    case PKV_EUNSUPPORTED: return "no kernel for this configuration";
    case PKV_EWORKSPACE: return "workspace too small";
    case PKV_EHIP: return "HIP runtime error while launching";
    case PKV_ENOBLOCKS: return "no free block";
    default: return "unknown status";
  }
}

int pkv_version(void) { return PKV_VERSION; }

int pkv_pool_bytes(const pkv_pool_desc* pool, size_t* k_bytes, size_t* v_bytes,
                   size_t* scale_bytes_each) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  const size_t block = (size_t)pool->num_kv_heads * pool->block_size * pool->head_dim *
                       elem_bytes(pool->kv_dtype);
  const size_t e = pool->block_stride
                       ? (size_t)(pool->num_blocks - 1) * pool->block_stride + block
                       : (size_t)pool->num_blocks * block;
  if (k_bytes) *k_bytes = e;
  if (v_bytes) *v_bytes = e;
  if (scale_bytes_each)
    *scale_bytes_each = quantised(pool->kv_dtype) ? scale_count(pool) * sizeof(float) : 0;
  return PKV_OK;
}

// The slot rule the write kernels use (slot.hpp), on one host-side table row:
// a bad argument is PKV_EINVAL and an unmapped logical block PKV_ERANGE.
int pkv_physical_slot(const int32_t* table, int32_t table_len, int32_t block_size,
                      int64_t token_pos, int64_t* slot) {
  if (!slot || table_len < 0 || (table_len > 0 && !table)) return PKV_EINVAL;
  const pkv::SlotLookup r = pkv::lookup_slot(table, table_len, block_size, token_pos);
  if (r.fault == pkv::kSlotUnmapped) return PKV_ERANGE;
  if (r.fault != pkv::kSlotOk) return PKV_EINVAL;
  *slot = r.slot;
  return PKV_OK;
}

int pkv_validate_block_table(const int32_t* block_table, int32_t num_seqs,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t block_size, int32_t num_blocks) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_table)))
    return PKV_EINVAL;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t ctx = context_lens[s];
    if (ctx < 0) return PKV_ERANGE;
    const int64_t nb = (ctx + block_size - 1) / block_size;
    if (nb > max_blocks_per_seq) return PKV_ERANGE;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = block_table[(int64_t)s * max_blocks_per_seq + j];
      if (id < 0 || id >= num_blocks) return PKV_ERANGE;
    }
  }
  return PKV_OK;
}

int pkv_slot_mapping(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                     const int32_t* seq_idx, const int32_t* positions, int32_t num_tokens,
                     int32_t block_size, int64_t* slot_mapping, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0)
    return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!seq_idx || !positions || !slot_mapping) return PKV_EINVAL;
  if (num_seqs > 0 && max_blocks_per_seq > 0 && !block_table) return PKV_EINVAL;
  if (num_seqs == 0 || max_blocks_per_seq == 0) block_table = nullptr;
  int rc = pkv::launch_slot_mapping(block_table, block_table ? num_seqs : 0, max_blocks_per_seq,
                                    seq_idx, positions, num_tokens, block_size, slot_mapping,
                                    as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

namespace {

// argument checks shared by the write and the append
int check_write(int32_t num_tokens, const void* k, const void* v, int32_t src_dtype,
                const pkv_pool_desc* pool, void* k_pool, void* v_pool, const float* k_scale,
                const float* v_scale) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  if (num_tokens < 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_pool || !v_pool) return PKV_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_EINVAL;
  if (elem_bytes(src_dtype) == 0 || quantised(src_dtype)) return PKV_EINVAL;
  if (quantised(pool->kv_dtype)) {
    if (!k_scale || !v_scale) return PKV_EINVAL;
  } else if (src_dtype != pool->kv_dtype) {
    return PKV_EINVAL;  // descriptor/dtype mismatch: no silent conversion
  }
  return PKV_OK;
}

pkv::WriteLaunch write_launch(int32_t num_tokens, const void* k, const void* v, int32_t src_dtype,
                              const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                              const float* k_scale, const float* v_scale) {
  pkv::WriteLaunch p{};
  p.num_tokens = num_tokens;
  p.k = k;
  p.v = v;
  p.src_dtype = src_dtype;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_blocks = pool->num_blocks;
  p.block_size = pool->block_size;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.kv_dtype = pool->kv_dtype;
  p.scale_mode = pool->scale_mode;
  p.bstride = block_units(pool);
  return p;
}

}  // namespace

int pkv_kv_cache_write(const int64_t* slot_mapping, int32_t num_tokens, const void* k,
                       const void* v, int32_t src_dtype, const pkv_pool_desc* pool,
                       void* k_pool, void* v_pool, const float* k_scale, const float* v_scale,
                       void* stream) {
  int rc = check_write(num_tokens, k, v, src_dtype, pool, k_pool, v_pool, k_scale, v_scale);
  if (rc != PKV_OK || num_tokens == 0) return rc;
  if (!slot_mapping) return PKV_EINVAL;
  pkv::WriteLaunch p = write_launch(num_tokens, k, v, src_dtype, pool, k_pool, v_pool, k_scale,
                                    v_scale);
  p.slot_mapping = slot_mapping;
  rc = pkv::launch_kv_cache_write(p, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_kv_cache_append(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* seq_idx, const int32_t* positions, int32_t num_tokens,
                        const void* k, const void* v, int32_t src_dtype,
                        const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                        const float* k_scale, const float* v_scale, int64_t* slot_mapping_out,
                        void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0) return PKV_EINVAL;
  int rc = check_write(num_tokens, k, v, src_dtype, pool, k_pool, v_pool, k_scale, v_scale);
  if (rc != PKV_OK || num_tokens == 0) return rc;
  if (!seq_idx || !positions) return PKV_EINVAL;
  if (num_seqs > 0 && max_blocks_per_seq > 0 && !block_table) return PKV_EINVAL;
  pkv::WriteLaunch p = write_launch(num_tokens, k, v, src_dtype, pool, k_pool, v_pool, k_scale,
                                    v_scale);
  p.slot_mapping = nullptr;
  const bool table = num_seqs > 0 && max_blocks_per_seq > 0;
  p.block_table = table ? block_table : nullptr;
  p.num_seqs = table ? num_seqs : 0;  // no table: every token is padding
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.seq_idx = seq_idx;
  p.positions = positions;
  p.slot_out = slot_mapping_out;
  rc = pkv::launch_kv_cache_write(p, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_copy_blocks(const int32_t* pairs, int32_t num_pairs, const pkv_pool_desc* pool,
                    void* k_pool, void* v_pool, float* k_scale, float* v_scale, void* stream) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (num_pairs > 0x7fffffff / 2) return PKV_EINVAL;
  if (!pairs || !k_pool || !v_pool || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_EINVAL;
  if (quantised(pool->kv_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  rc = pkv::launch_copy_blocks(pairs, num_pairs, k_pool, v_pool, k_scale, v_scale,
                               pool->num_blocks, pool->block_size, pool->num_kv_heads,
                               pool->head_dim, pool->kv_dtype, pool->scale_mode,
                               block_units(pool), as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

namespace {

// The balanced decode on a prepared launch (p.ctx_cap = the per-sequence token
// cap of the stream): one stream of 64-token chunks over every (sequence, kv
// head) pair, cut evenly across the resident wavefronts.
int launch_balanced(pkv::DecodeLaunch& p, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const int64_t units = (int64_t)p.num_seqs * ((p.ctx_cap + 63) / 64) * p.num_kv_heads;
  if (p.num_seqs > kMaxBalancedSeqs || units >= ((int64_t)1 << 31)) return PKV_EUNSUPPORTED;
  const int group = p.num_q_heads / p.num_kv_heads;
  const size_t slot_bytes = (size_t)group * ((size_t)p.head_dim + 2) * sizeof(float);
  const size_t cnt_bytes = balanced_counter_bytes(p.num_seqs, p.num_kv_heads);
  if (!workspace || workspace_bytes < cnt_bytes + 2 * slot_bytes) return PKV_EWORKSPACE;
  if (!aligned16(workspace)) return PKV_EINVAL;
  int nw = pkv::balanced_worker_capacity(p.kv_dtype, p.q_dtype, p.head_dim, p.block_size);
  if (nw > PKV_MAX_WORKERS) nw = PKV_MAX_WORKERS;
  const size_t fit = (workspace_bytes - cnt_bytes) / (2 * slot_bytes);
  if ((size_t)nw > fit) nw = (int)fit;
  char* base = static_cast<char*>(workspace);
  float* ws = reinterpret_cast<float*>(base + cnt_bytes);
  p.balanced = 1;
  p.split = 1;
  p.num_workers = nw;
  p.counters = reinterpret_cast<unsigned long long*>(base);         // [S][H_kv]
  p.epoch = next_epoch();
  p.part_out = ws;                                                  // [2*nw][G][D]
  p.part_max = ws + (size_t)2 * nw * group * p.head_dim;            // [2*nw][G][2]
  const int rc = pkv::launch_decode(p, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

size_t balanced_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim) {
  const size_t group = (size_t)(num_q_heads / num_kv_heads);
  return balanced_counter_bytes(num_seqs, num_kv_heads) +
         2 * (size_t)PKV_MAX_WORKERS * group * ((size_t)head_dim + 2) * sizeof(float);
}

// Type pairs of the matrix-core prefill kernel: bf16 q over bf16 or fp8 (one scale
// per block and kv head) pools, f16 q over f16 pools.
bool prefill_types_ok(int q_dtype, const pkv_pool_desc* pool) {
  switch (pool->kv_dtype) {
    case PKV_BF16: return q_dtype == PKV_BF16;
    case PKV_F16: return q_dtype == PKV_F16;
    case PKV_FP8_E4M3: return q_dtype == PKV_BF16 && pool->scale_mode == PKV_SCALE_BLOCK;
    default: return false;
  }
}

// How a shared-prefix decode cuts the prefix: slices of whole 64-token chunks,
// enough of them that (kv heads x column tiles x slices) reaches about 2048
// wavefronts; the partial slots are the slices plus one for the tails.
struct SharedPlan {
  int n_slices, slice_chunks, max_parts;
  size_t part_bytes;  // partial arrays, rounded up to 256 bytes
};

SharedPlan shared_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int shared_len) {
  SharedPlan sp = {};
  const int nch = (shared_len + 63) / 64;
  if (nch > 0) {
    const int G = num_q_heads / num_kv_heads;
    const int64_t tiles = (num_seqs + 16 / G - 1) / (16 / G);
    const int64_t per_slice = (int64_t)num_kv_heads * (tiles > 0 ? tiles : 1);
    int64_t want = (2048 + per_slice - 1) / per_slice;
    if (want > nch) want = nch;
    sp.slice_chunks = (int)((nch + want - 1) / want);
    sp.n_slices = (nch + sp.slice_chunks - 1) / sp.slice_chunks;
  }
  sp.max_parts = sp.n_slices + 1;
  const size_t n = (size_t)num_seqs * num_q_heads * sp.max_parts;
  sp.part_bytes = (n * ((size_t)head_dim + 2) * sizeof(float) + 255) / 256 * 256;
  return sp;
}

}  // namespace

int pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                               size_t* bytes) {
  if (!bytes || num_seqs < 0 || num_q_heads < 0 || num_kv_heads < 1 || head_dim < 0 ||
      max_context_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (partition_size == 0) {
    *bytes = 0;
    return PKV_OK;
  }
  if (partition_size == PKV_PARTITION_BALANCED) {
    *bytes = balanced_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
    return PKV_OK;
  }
  if (partition_size < 0 || partition_size % 64 != 0) return PKV_EINVAL;
  const size_t pmax = ((size_t)max_context_len + partition_size - 1) / partition_size;
  *bytes = (size_t)num_seqs * num_q_heads * pmax * ((size_t)head_dim + 2) * sizeof(float);
  return PKV_OK;
}

int pkv_paged_attention_decode(const void* q, int32_t q_dtype, int32_t num_seqs,
                               int32_t num_q_heads, const pkv_pool_desc* pool,
                               const void* k_pool, const void* v_pool, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, float scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, void* out,
                               void* stream) {
  return pkv_paged_attention_decode_window(q, q_dtype, num_seqs, num_q_heads, pool, k_pool,
                                           v_pool, k_scale, v_scale, block_table,
                                           max_blocks_per_seq, context_lens, max_context_len,
                                           scale, 0, partition_size, workspace, workspace_bytes,
                                           out, stream);
}

int pkv_decode_partition_size(const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_kv_heads, int32_t max_context_len, int32_t num_cus,
                              int32_t* partition_size) {
  if (!partition_size || num_seqs < 0 || num_kv_heads < 1 || max_context_len < 0)
    return PKV_EINVAL;
  if (num_seqs > 0 && !context_lens) return PKV_EINVAL;
  if (num_cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        num_cus < 1)
      return PKV_EHIP;
  }
  int64_t live = 0, longest = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t c = std::min<int64_t>(std::max<int32_t>(context_lens[s], 0), max_context_len);
    live += c > 0;
    longest = std::max(longest, c);
  }
  *partition_size = 0;
  if (live * num_kv_heads >= num_cus) return PKV_OK;  // the pairs fill the CUs already
  // workgroups at P = 64 k tokens; non-increasing in k, and at most num_cus once
  // every sequence is one partition (k = ceil(longest / 64)).  At least 4 chunks
  // (k >= 4), one for each wavefront of a workgroup.
  auto groups = [&](int64_t k) {
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int64_t c = std::min<int64_t>(std::max<int32_t>(context_lens[s], 0), max_context_len);
      n += (c + 64 * k - 1) / (64 * k);
    }
    return n * num_kv_heads;
  };
  int64_t lo = 4, hi = std::max<int64_t>(4, (longest + 63) / 64);
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (groups(mid) <= num_cus)
      hi = mid;
    else
      lo = mid + 1;
  }
  if (64 * lo < longest) *partition_size = (int32_t)(64 * lo);  // else nothing is cut
  return PKV_OK;
}

// Fixed partitions of partition_size tokens: the decode writes each partition's
// (normalised output, log-sum-exp) into the workspace, then the reduce merges them
// into p.out.  The workspace layout follows max_context_len (the documented P_max).
static int launch_partitioned(pkv::DecodeLaunch& p, int32_t partition_size,
                              int32_t max_context_len, void* workspace, size_t workspace_bytes,
                              void* stream) {
  size_t need = 0;
  int rc = pkv_decode_workspace_bytes(p.num_seqs, p.num_q_heads, p.num_kv_heads, p.head_dim,
                                      max_context_len, partition_size, &need);
  if (rc != PKV_OK) return rc;
  const int max_parts = (int)(((int64_t)max_context_len + partition_size - 1) / partition_size);
  if (max_parts > pkv::kMaxPartitions) return PKV_EUNSUPPORTED;  // the reduce's limit
  p.max_parts = max_parts;
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_EWORKSPACE;
  if (need > 0 && !aligned16(workspace)) return PKV_EINVAL;
  const size_t n_part = (size_t)p.num_seqs * p.num_q_heads * max_parts;
  float* ws = static_cast<float*>(workspace);
  p.split = 1;
  p.part_size = partition_size;
  p.part_out = ws;
  p.part_max = ws ? ws + n_part * p.head_dim : nullptr;
  p.part_sum = ws ? p.part_max + n_part : nullptr;
  if (max_parts > 0 || p.fuse) {
    // (fused with the append and max_context_len == 0: one empty partition slice
    // appends the new tokens and writes no partial)
    if (max_parts == 0) p.max_parts = 1;
    rc = pkv::launch_decode(p, as_stream(stream));
    p.max_parts = max_parts;
    if (rc != 0) return rc;
  }
  pkv::ReduceLaunch r;
  r.part_out = p.part_out;
  r.part_max = p.part_max;
  r.part_sum = p.part_sum;
  r.context_lens = p.context_lens;
  r.out = p.out;
  r.out_dtype = p.q_dtype;
  r.num_seqs = p.num_seqs;
  r.num_q_heads = p.num_q_heads;
  r.head_dim = p.head_dim;
  r.part_size = partition_size;
  r.max_parts = max_parts;
  r.ctx_cap = p.ctx_cap;  // no partition past the decode's clamp was written
  rc = pkv::launch_split_reduce(r, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_paged_attention_decode_window(const void* q, int32_t q_dtype, int32_t num_seqs,
                                      int32_t num_q_heads, const pkv_pool_desc* pool,
                                      const void* k_pool, const void* v_pool,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      float scale, int32_t window, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* out,
                                      void* stream) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  if (window < 0) return PKV_EINVAL;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_EINVAL;
  if (num_q_heads / pool->num_kv_heads > kMaxHeadsGroup) return PKV_EUNSUPPORTED;
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  if (!balanced && (partition_size < 0 || partition_size % 64 != 0)) return PKV_EINVAL;
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_EINVAL;
  if (max_context_len > (1 << 30)) return PKV_EUNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PKV_EINVAL;
  if (quantised(pool->kv_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (num_seqs > 65535 || pool->num_kv_heads > 65535) return PKV_EUNSUPPORTED;

  int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
  if (cap > max_context_len) cap = max_context_len;

  pkv::DecodeLaunch p = {};
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.kv_dtype = pool->kv_dtype;
  p.scale_mode = pool->scale_mode;
  p.bstride = block_units(pool);
  p.block_size = pool->block_size;
  p.num_blocks = pool->num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.ctx_cap = (int)cap;
  p.scale = scale;
  p.window = window;

  if (balanced) return launch_balanced(p, workspace, workspace_bytes, stream);

  if (partition_size == 0) {
    p.split = 0;
    p.max_parts = 1;
    p.part_size = (int)((cap + 63) / 64 * 64);
    if (p.part_size == 0) p.part_size = 64;
    rc = pkv::launch_decode(p, as_stream(stream));
    return rc == 0 ? PKV_OK : rc;
  }

  return launch_partitioned(p, partition_size, max_context_len, workspace, workspace_bytes,
                            stream);
}

int pkv_decode_append(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                      const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len, const void* k_new,
                      const void* v_new, float scale, int32_t partition_size, void* workspace,
                      size_t workspace_bytes, void* out, int64_t* slot_mapping_out,
                      void* stream) {
  int rc = check_desc(pool);
  if (partition_size != PKV_PARTITION_BALANCED &&
      (partition_size < 0 || partition_size % 64 != 0))
    return PKV_EINVAL;
  if (rc != PKV_OK) return rc;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_EINVAL;
  if (num_q_heads / pool->num_kv_heads > kMaxHeadsGroup) return PKV_EUNSUPPORTED;
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_EINVAL;
  // the new rows are stored as they are: a 16-bit pool of the query's type
  if ((pool->kv_dtype != PKV_F16 && pool->kv_dtype != PKV_BF16) || q_dtype != pool->kv_dtype)
    return PKV_EUNSUPPORTED;
  if (max_context_len > (1 << 30)) return PKV_EUNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out || !k_new || !v_new)
    return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned16(k_new) || !aligned16(v_new))
    return PKV_EINVAL;
  if (num_seqs > 65535 || pool->num_kv_heads > 65535) return PKV_EUNSUPPORTED;
  int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
  if (cap > max_context_len) cap = max_context_len;

  pkv::DecodeLaunch p = {};
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.kv_dtype = pool->kv_dtype;
  p.scale_mode = pool->scale_mode;
  p.bstride = block_units(pool);
  p.block_size = pool->block_size;
  p.num_blocks = pool->num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.ctx_cap = (int)cap;
  p.scale = scale;
  p.fuse = 1;
  p.k_new = k_new;
  p.v_new = v_new;
  p.slot_out = slot_mapping_out;
  if (partition_size == PKV_PARTITION_BALANCED)
    return launch_balanced(p, workspace, workspace_bytes, stream);
  if (partition_size > 0)  // the store goes with the partition holding the newest token
    return launch_partitioned(p, partition_size, max_context_len, workspace, workspace_bytes,
                              stream);
  p.split = 0;  // unsplit: one workgroup per (sequence, kv head)
  p.max_parts = 1;
  p.part_size = (int)((cap + 63) / 64 * 64);
  if (p.part_size == 0) p.part_size = 64;
  rc = pkv::launch_decode(p, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t shared_len,
                                      size_t* bytes) {
  if (!bytes || num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 0 ||
      shared_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (num_q_heads / num_kv_heads > kMaxHeadsGroup) return PKV_EUNSUPPORTED;
  const SharedPlan sp = shared_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, shared_len);
  *bytes = sp.part_bytes + balanced_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
  return PKV_OK;
}

int pkv_paged_attention_decode_shared(const void* q, int32_t q_dtype, int32_t num_seqs,
                                      int32_t num_q_heads, const pkv_pool_desc* pool,
                                      const void* k_pool, const void* v_pool,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t shared_len, float scale, void* workspace,
                                      size_t workspace_bytes, void* out, void* stream) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  if (num_seqs < 0 || num_q_heads < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_EINVAL;
  if (num_q_heads / pool->num_kv_heads > kMaxHeadsGroup) return PKV_EUNSUPPORTED;
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16) return PKV_EINVAL;
  if (shared_len < 0 || shared_len % pool->block_size != 0 ||
      (int64_t)shared_len > (int64_t)max_blocks_per_seq * pool->block_size)
    return PKV_EINVAL;
  if (max_context_len > (1 << 30)) return PKV_EUNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PKV_EINVAL;
  if (quantised(pool->kv_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (num_seqs > 65535 || pool->num_kv_heads > 65535) return PKV_EUNSUPPORTED;
  size_t need = 0;
  rc = pkv_decode_shared_workspace_bytes(num_seqs, num_q_heads, pool->num_kv_heads,
                                         pool->head_dim, shared_len, &need);
  if (rc != PKV_OK) return rc;
  if (!workspace || workspace_bytes < need) return PKV_EWORKSPACE;
  if (!aligned16(workspace)) return PKV_EINVAL;
  if (shared_len == 0)  // nothing shared: the plain balanced decode
    return pkv_paged_attention_decode(q, q_dtype, num_seqs, num_q_heads, pool, k_pool, v_pool,
                                      k_scale, v_scale, block_table, max_blocks_per_seq,
                                      context_lens, max_context_len, scale,
                                      PKV_PARTITION_BALANCED, workspace, workspace_bytes, out,
                                      stream);

  int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
  if (cap > max_context_len) cap = max_context_len;
  const SharedPlan sp =
      shared_plan(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim, shared_len);
  const size_t n_part = (size_t)num_seqs * num_q_heads * sp.max_parts;
  float* part_out = static_cast<float*>(workspace);
  float* part_max = part_out + n_part * pool->head_dim;
  float* part_sum = part_max + n_part;
  char* bal = static_cast<char*>(workspace) + sp.part_bytes;

  pkv::DecodeLaunch p = {};
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.kv_dtype = pool->kv_dtype;
  p.scale_mode = pool->scale_mode;
  p.bstride = block_units(pool);
  p.block_size = pool->block_size;
  p.num_blocks = pool->num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.scale = scale;
  p.max_parts = sp.max_parts;

  // 1. the prefix, read once per kv head: partial slots 0 .. n_slices-1.  On the
  // matrix-core prefill kernel (its K/V chunks staged once in LDS for 128/G
  // sequences) where it takes the types and shapes, else on the decode tiles.
  const int group = num_q_heads / pool->num_kv_heads;
  if (prefill_types_ok(q_dtype, pool) && pool->block_size >= 16 && 16 % group == 0) {
    pkv::PrefillLaunch pl;
    pl.q = q;
    pl.q_dtype = q_dtype;
    pl.cu_seqlens_q = nullptr;
    pl.num_seqs = num_seqs;
    pl.total_q = num_seqs;
    pl.max_q_len = 1;
    pl.num_q_heads = num_q_heads;
    pl.k_pool = k_pool;
    pl.v_pool = v_pool;
    pl.k_scale = k_scale;
    pl.v_scale = v_scale;
    pl.num_blocks = pool->num_blocks;
    pl.block_size = pool->block_size;
    pl.num_kv_heads = pool->num_kv_heads;
    pl.head_dim = pool->head_dim;
    pl.kv_dtype = pool->kv_dtype;
    pl.bstride = block_units(pool);
    pl.block_table = block_table;
    pl.max_blocks_per_seq = max_blocks_per_seq;
    pl.context_lens = context_lens;
    pl.ctx_cap = (int)cap;
    pl.scale = scale;
    pl.causal = 0;
    pl.out = nullptr;
    pl.prefix = 1;
    pl.shared_len = shared_len;
    pl.n_slices = sp.n_slices;
    pl.slice_chunks = sp.slice_chunks;
    pl.max_parts = sp.max_parts;
    pl.part_out = part_out;
    pl.part_max = part_max;
    pl.part_sum = part_sum;
    rc = pkv::launch_prefill(pl, as_stream(stream));
  } else {
    pkv::DecodeLaunch pre = p;
    pre.prefix = 1;
    pre.ctx_cap = (int)cap;
    pre.shared_len = shared_len;
    pre.n_slices = sp.n_slices;
    pre.slice_chunks = sp.slice_chunks;
    pre.part_out = part_out;
    pre.part_max = part_max;
    pre.part_sum = part_sum;
    rc = pkv::launch_decode(pre, as_stream(stream));
  }
  if (rc != 0) return rc;

  // 2. the private tails, balanced: partial slot n_slices
  pkv::DecodeLaunch tail = p;
  const int64_t tail_cap = cap - shared_len;
  const int64_t tail_rows = ((int64_t)max_blocks_per_seq * pool->block_size - shared_len);
  tail.ctx_off = shared_len;
  tail.tbl_off = shared_len / pool->block_size;
  tail.ctx_cap = (int)(tail_cap < 0 ? 0 : (tail_cap < tail_rows ? tail_cap : tail_rows));
  tail.tail_part = sp.n_slices;
  tail.tail_out = part_out;
  tail.tail_max = part_max;
  tail.tail_sum = part_sum;
  rc = launch_balanced(tail, bal, workspace_bytes - sp.part_bytes, stream);
  if (rc != PKV_OK) return rc;

  // 3. the log-sum-exp merge of every slot
  pkv::ReduceLaunch r;
  r.part_out = part_out;
  r.part_max = part_max;
  r.part_sum = part_sum;
  r.context_lens = nullptr;  // all max_parts slots
  r.out = out;
  r.out_dtype = q_dtype;
  r.num_seqs = num_seqs;
  r.num_q_heads = num_q_heads;
  r.head_dim = pool->head_dim;
  r.part_size = 1;
  r.max_parts = sp.max_parts;
  r.ctx_cap = 0x7fffffff;
  rc = pkv::launch_split_reduce(r, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_split_kv_reduce(const float* part_out, const float* part_max, const float* part_sum,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t head_dim, int32_t partition_size, int32_t max_partitions,
                        void* out, int32_t out_dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads < 1 || partition_size < 1 || max_partitions < 0)
    return PKV_EINVAL;
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16 && out_dtype != PKV_BF16) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !out || (max_partitions > 0 && (!part_out || !part_max || !part_sum)))
    return PKV_EINVAL;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_EUNSUPPORTED;
  pkv::ReduceLaunch r;
  r.part_out = part_out;
  r.part_max = part_max;
  r.part_sum = part_sum;
  r.context_lens = context_lens;
  r.out = out;
  r.out_dtype = out_dtype;
  r.num_seqs = num_seqs;
  r.num_q_heads = num_q_heads;
  r.head_dim = head_dim;
  r.part_size = partition_size;
  r.max_parts = max_partitions;
  r.ctx_cap = 0x7fffffff;  // only max_partitions * partition_size clamps here
  int rc = pkv::launch_split_reduce(r, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

int pkv_paged_prefill(const void* q, int32_t q_dtype, const int32_t* cu_seqlens_q,
                      int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                      const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, float scale, int32_t causal, void* out,
                      void* stream) {
  int rc = check_desc(pool);
  if (rc != PKV_OK) return rc;
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_q_heads < 1 ||
      max_blocks_per_seq < 1 || max_context_len < 0)
    return PKV_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_EINVAL;
  if (!prefill_types_ok(q_dtype, pool)) return PKV_EUNSUPPORTED;
  if (pool->head_dim != 128 && pool->head_dim != 64) return PKV_EUNSUPPORTED;
  if (pool->block_size < 16) return PKV_EUNSUPPORTED;  // a 16-token tile sits in one block
  {
    const int group = num_q_heads / pool->num_kv_heads;
    if (group > 16 || 16 % group != 0) return PKV_EUNSUPPORTED;
  }
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (!q || !cu_seqlens_q || !k_pool || !v_pool || !block_table || !context_lens || !out)
    return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PKV_EINVAL;
  if (quantised(pool->kv_dtype) && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_EUNSUPPORTED;
  int64_t cap = (int64_t)max_blocks_per_seq * pool->block_size;
  if (cap > max_context_len) cap = max_context_len;
  if (cap > (int64_t)1 << 30) return PKV_EUNSUPPORTED;
  pkv::PrefillLaunch p;
  p.q = q;
  p.q_dtype = q_dtype;
  p.cu_seqlens_q = cu_seqlens_q;
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.max_q_len = max_q_len;
  p.num_q_heads = num_q_heads;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_blocks = pool->num_blocks;
  p.block_size = pool->block_size;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.kv_dtype = pool->kv_dtype;
  p.bstride = block_units(pool);
  p.block_table = block_table;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.context_lens = context_lens;
  p.ctx_cap = (int)cap;
  p.scale = scale;
  p.causal = causal != 0;
  p.out = out;
  rc = pkv::launch_prefill(p, as_stream(stream));
  return rc == 0 ? PKV_OK : rc;
}

}  // extern "C"
