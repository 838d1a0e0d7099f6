// internal.hpp — host-side declarations shared by the C-ABI front end (api.cpp)
// and the kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// most partitions per sequence the split-KV reduce takes (its weights sit in LDS)
constexpr int kMaxPartitions = 8192;

struct DecodeLaunch {
  const void* q;
  int q_dtype;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  float* part_out;
  float* part_max;
  float* part_sum;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, kv_dtype;
  int scale_mode;     // quantised pools: where an element's scale lives
  long long bstride;  // 16-byte units from one block to the next in each pool
  int block_size, num_blocks, max_blocks_per_seq;
  int ctx_cap;        // min(max_context_len, max_blocks_per_seq * block_size)
  int part_size;      // > 0: tokens per partition (multiple of 64)
  int max_parts;      // partitions per sequence covered by the grid
  int split;          // write partials (1) or the final output (0)
  int balanced;       // balanced wavefront workers (part_out/part_max hold the slots)
  int num_workers;    // balanced: wavefront workers
  unsigned long long* counters;  // balanced: one per (sequence, kv head)
  uint32_t epoch;     // balanced: tag of this call for the counters
  float scale;
  // balanced over the private tails of a shared-prefix batch: start ctx_off
  // tokens / tbl_off table entries in, result to partial slot tail_part (< 0: off)
  int ctx_off = 0, tbl_off = 0, tail_part = -1;
  float* tail_out = nullptr;
  float* tail_max = nullptr;
  float* tail_sum = nullptr;
  // the shared-prefix kernel (part_out/part_max/part_sum: partial slots 0 ..
  // n_slices-1 of stride max_parts)
  int prefix = 0;
  int shared_len = 0, n_slices = 0, slice_chunks = 0;
  int window = 0;  // > 0: sliding-window decode (keys [ctx - window, ctx))
  // balanced decode fused with the append of each sequence's newest token
  int fuse = 0;
  const void* k_new = nullptr;  // [S][H_kv][D], the pool's 16-bit type
  const void* v_new = nullptr;
  int64_t* slot_out = nullptr;  // optional [S]: the slots written
};

// Wavefront workers the balanced decode can keep resident on the current device
// for this instantiation (CUs x resident waves per CU), computed once per device.
int balanced_worker_capacity(int kv_dtype, int q_dtype, int head_dim, int block_size);

// returns a PKV_* status
int launch_decode(const DecodeLaunch& p, hipStream_t stream);

struct ReduceLaunch {
  const float* part_out;
  const float* part_max;
  const float* part_sum;
  const int32_t* context_lens;
  void* out;
  int out_dtype;
  int num_seqs, num_q_heads, head_dim, part_size, max_parts;
  int ctx_cap;  // contexts are clamped to this many tokens (the decode's clamp)
};
int launch_split_reduce(const ReduceLaunch& p, hipStream_t stream);

int launch_slot_mapping(const int32_t* block_table, int num_seqs, int max_blocks_per_seq,
                        const int32_t* seq_idx, const int32_t* positions, int num_tokens,
                        int block_size, int64_t* slot_mapping, hipStream_t stream);

struct WriteLaunch {
  const int64_t* slot_mapping;  // given slots, or null: computed from the fields below
  const int32_t* block_table;
  const int32_t* seq_idx;
  const int32_t* positions;
  int num_seqs, max_blocks_per_seq;
  int64_t* slot_out;            // optional copy of the computed slots
  int num_tokens;
  const void* k;
  const void* v;
  int src_dtype;
  void* k_pool;
  void* v_pool;
  const float* k_scale;
  const float* v_scale;
  int num_blocks, block_size, num_kv_heads, head_dim, kv_dtype;
  int scale_mode;
  long long bstride;            // 16-byte units from one block to the next
};
int launch_kv_cache_write(const WriteLaunch& p, hipStream_t stream);

int launch_copy_blocks(const int32_t* pairs, int num_pairs, void* k_pool, void* v_pool,
                       float* k_scale, float* v_scale, int num_blocks, int block_size, int Hkv,
                       int head_dim, int kv_dtype, int scale_mode, long long bstride,
                       hipStream_t stream);

}  // namespace pkv
