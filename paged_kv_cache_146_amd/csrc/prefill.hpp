// prefill.hpp — host-side declaration of the chunked-prefill launch, shared by the
// C-ABI front end (api.cpp) and prefill.hip.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct PrefillLaunch {
  const void* q;
  int q_dtype;
  const int32_t* cu_seqlens_q;
  int num_seqs, total_q, max_q_len, num_q_heads;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  int num_blocks, block_size, num_kv_heads, head_dim, kv_dtype;
  long long bstride;  // 16-byte units from one block to the next
  const int32_t* block_table;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int ctx_cap;
  float scale;
  int causal;
  void* out;
  // prefix mode (a shared-prefix decode's prefix on the matrix cores): the rows are
  // the num_seqs sequences, the keys the first shared_len tokens of table row 0 in
  // n_slices slices of slice_chunks 64-token chunks; slice i's state goes to partial
  // slot i of max_parts
  int prefix = 0;
  int shared_len = 0, n_slices = 0, slice_chunks = 0, max_parts = 0;
  float* part_out = nullptr;
  float* part_max = nullptr;
  float* part_sum = nullptr;
};
int launch_prefill(const PrefillLaunch& p, hipStream_t stream);

}  // namespace pkv
