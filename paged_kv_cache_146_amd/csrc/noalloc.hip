// noalloc.hip — paged decode whose split-KV scratch is a device array owned by the
// library, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives for the whole process on every device the entry point runs on.
// Its device address is resolved once per device, on the first call made with that
// device current, and kept; host code never uses the array's own name except to
// resolve it (in host code that name is a host-side stand-in, not a device
// address).  All calls on one device share the array, so calls that overlap in
// time on one device race.  Nothing in it needs clearing between calls: the
// fixed-partition decode writes every partial it later merges, and the balanced
// decode tags its counters with a fresh call epoch (see decode.hip).
#include "../../include/pagedkv.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // each device's copy of the array, once resolved

// The current device's copy of the array (resolved on the first call per device).
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PKV_EHIP;
  if (dev >= kMaxDevices) return PKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attention_decode_noalloc(
    const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
    const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, const float* k_scale,
    const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, float scale, int32_t partition_size,
    void* out, void* stream) {
  if (!pool || pool->num_kv_heads < 1 || num_q_heads < 1 || num_seqs < 0 ||
      max_context_len < 0 || pool->head_dim < 1)
    return PKV_EINVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PKV_EINVAL;
  // the scratch this call needs, checked against the array before anything else
  size_t need = 0;
  if (partition_size == PKV_PARTITION_BALANCED) {
    // the counters and one worker's two partial states; more space, more workers
    const size_t counters = ((size_t)num_seqs * pool->num_kv_heads * 8 + 255) / 256 * 256;
    need = counters + 2 * (size_t)(num_q_heads / pool->num_kv_heads) *
                          ((size_t)pool->head_dim + 2) * sizeof(float);
  } else {
    const int rc = pkv_decode_workspace_bytes(num_seqs, num_q_heads, pool->num_kv_heads,
                                              pool->head_dim, max_context_len, partition_size,
                                              &need);
    if (rc != PKV_OK) return rc;
  }
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_EWORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (partition_size != 0 && num_seqs > 0) {
    const int rc = device_scratch(&ws);
    if (rc != PKV_OK) return rc;
    ws_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  }
  return pkv_paged_attention_decode(q, q_dtype, num_seqs, num_q_heads, pool, k_pool, v_pool,
                                    k_scale, v_scale, block_table, max_blocks_per_seq,
                                    context_lens, max_context_len, scale, partition_size, ws,
                                    ws_bytes, out, stream);
}
