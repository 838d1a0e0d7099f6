// cache_write.hip — the write path: slot mapping and the scatter of new K/V.
//
// Method: "03 | PagedAttention and the KV-cache memory system", §3 (slot =
// physical_id * B + position mod B, physical_id = block_table[position / B])
// and §4.1 (the model runner scatters each new token's K/V to its slot; the
// number of tokens written is the length of slot_mapping); §8.1 (quantised
// pages: fp8 or int8 codes with fp32 scales, one per block and head, per
// tensor, or per token and head).  "KV Cache: capacity, layout, lifecycle", "Page-table
// addressing": the cases where the reference raises become padding (-1) here.
//
// The fused append computes each token's slot in the scatter itself (one launch
// for both steps).  The scatter works in 16-byte source pieces: one thread moves one piece of
// one (token, kv head) row.  In the K pool ([block][head][D/X][B][X]) the piece
// lands as one 16-byte store; in the V pool ([block][head][B/TG][D][TG], runs of
// TG = min(X, B) tokens per dim) its elements go TG elements apart, one store
// each.  Bit
// copies for f32/f16/bf16 pools; for quantised pools the thread divides 16
// source elements by their scale (IEEE fp32 division) and encodes them as OCP
// E4M3 (nearest, ties to even, saturating) or as symmetric int8 (nearest, ties
// to even, clamped to +-127).
#include "device.hpp"
#include "internal.hpp"
#include "slot.hpp"

namespace pkv {

constexpr int kWriteThreads = 256;

// slot of token i by the pool's address rule (slot.hpp) on its sequence's table
// row, or -1 (padding) for a sequence out of range and wherever the rule faults
__device__ __forceinline__ long long token_slot(const int32_t* __restrict__ block_table,
                                                int num_seqs, int W,
                                                const int32_t* __restrict__ seq_idx,
                                                const int32_t* __restrict__ positions,
                                                long long i, int B) {
  const int s = seq_idx[i];
  if (s < 0 || s >= num_seqs) return -1;
  const SlotLookup r = lookup_slot(block_table + (size_t)s * W, W, B, positions[i]);
  return r.fault == kSlotOk ? r.slot : -1;
}

__global__ __launch_bounds__(kWriteThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ block_table, int num_seqs, int W,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ positions, int num_tokens,
    int B, int64_t* __restrict__ slot_mapping) {
  const int i = blockIdx.x * kWriteThreads + threadIdx.x;
  if (i >= num_tokens) return;
  slot_mapping[i] = token_slot(block_table, num_seqs, W, seq_idx, positions, i, B);
}

// Where the write kernels take each token's slot: a given slot mapping, or (the
// fused append) computed from the block table, optionally written out too by the
// thread that moves the token's first K piece.
struct SlotSource {
  const int64_t* slot_mapping;  // non-null: given slots
  const int32_t* block_table;
  const int32_t* seq_idx;
  const int32_t* positions;
  int num_seqs, W;
  int64_t* slot_out;            // optional, computed slots only
};

__device__ __forceinline__ long long source_slot(const SlotSource& ss, long long i, int c, int h,
                                                 int B) {
  if (ss.slot_mapping) return ss.slot_mapping[i];
  const long long slot =
      token_slot(ss.block_table, ss.num_seqs, ss.W, ss.seq_idx, ss.positions, i, B);
  if (ss.slot_out && c == 0 && h == 0 && blockIdx.y == 0) ss.slot_out[i] = slot;
  return slot;
}

// log2 of a power of two
__device__ __forceinline__ int log2_of(int x) { return 31 - __builtin_clz(x); }

// Bit copy of one 16-byte piece (non-fp8 pools); ES = bytes per element.
template <int ES>
__global__ __launch_bounds__(kWriteThreads) void kv_write_copy_kernel(
    const SlotSource ss, int num_tokens, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    int num_blocks, int B, int Hkv, int D, long long bstride) {
  const int NC = D * ES / 16;  // pieces per row
  const long long total = (long long)num_tokens * Hkv * NC;
  const long long idx = (long long)blockIdx.x * kWriteThreads + threadIdx.x;
  if (idx >= total) return;
  // token fastest: consecutive slots (a prefill chunk, a pool fill) give
  // consecutive destinations in both pools
  const long long i = idx % num_tokens;
  const int c = (int)((idx / num_tokens) % NC);
  const int h = (int)(idx / ((long long)num_tokens * NC));
  const long long slot = source_slot(ss, i, c, h, B);
  if (slot < 0 || slot >= (long long)num_blocks * B) return;
  const long long blk = slot / B, off = slot % B;
  const size_t src = ((size_t)i * Hkv + h) * NC + c;  // in 16-byte pieces
  constexpr int E = 16 / ES;
  const size_t blk16 = (size_t)blk * (size_t)bstride;  // where the block starts, 16-byte units
  if (blockIdx.y == 0) {
    reinterpret_cast<u32x4*>(k_pool)[blk16 + ((size_t)h * NC + c) * B + off] =
        reinterpret_cast<const u32x4*>(k)[src];
  } else {
    const u32x4 x = reinterpret_cast<const u32x4*>(v)[src];
    // V page [B/TG][D][TG], TG = min(E, B): element (dim c E, token off), then the
    // next dims TG elements apart
    const int tgl = min(E == 4 ? 2 : 3, log2_of(B));
    const size_t d0 = blk16 * E + (size_t)h * D * B +
                      (((size_t)(off >> tgl) * D + (size_t)c * E) << tgl) + (off & ((1 << tgl) - 1));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t w = x[e * ES / 4];
      if constexpr (ES == 4)
        reinterpret_cast<uint32_t*>(v_pool)[d0 + ((size_t)e << tgl)] = w;
      else
        reinterpret_cast<uint16_t*>(v_pool)[d0 + ((size_t)e << tgl)] =
            (uint16_t)(w >> (16 * (e & 1)));
    }
  }
}

// symmetric int8 code of y (already divided by the scale): nearest integer, ties to
// even, saturated to [-127, 127]; NaN -> 0
__device__ __forceinline__ uint32_t f32_to_i8(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(y == y ? (int)r : 0);
}

// index of the scale of (block, head, token offset) in the pool's scale mode
__device__ __forceinline__ size_t scale_index(int mode, size_t page, long long off, int B) {
  return mode == SCALE_TENSOR ? 0 : (mode == SCALE_TOKEN ? page * B + off : page);
}

// quantised pools: 16 source elements of SRC type -> one 16-byte piece of KVT codes
// (E4M3 or int8), each divided by its scale first.
template <int SRC, int KVT>
__global__ __launch_bounds__(kWriteThreads) void kv_write_quant_kernel(
    const SlotSource ss, int num_tokens, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int scale_mode,
    int num_blocks, int B, int Hkv, int D, long long bstride) {
  constexpr int SES = Elem<SRC>::bytes;
  const int NC = D / 16;
  const long long total = (long long)num_tokens * Hkv * NC;
  const long long idx = (long long)blockIdx.x * kWriteThreads + threadIdx.x;
  if (idx >= total) return;
  const long long i = idx % num_tokens;  // token fastest, as above
  const int c = (int)((idx / num_tokens) % NC);
  const int h = (int)(idx / ((long long)num_tokens * NC));
  const long long slot = source_slot(ss, i, c, h, B);
  if (slot < 0 || slot >= (long long)num_blocks * B) return;
  const long long blk = slot / B, off = slot % B;
  const bool isv = blockIdx.y != 0;
  const uint8_t* src = (isv ? v : k) + (((size_t)i * Hkv + h) * D + (size_t)c * 16) * SES;
  const size_t page = (size_t)blk * Hkv + h;
  const float scale = (isv ? v_scale : k_scale)[scale_index(scale_mode, page, off, B)];

  float x[16];
  const u32x4* sp = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int part = 0; part < SES; ++part) unpack16<SRC>(sp[part], x + part * (16 / SES));
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float y = __fdiv_rn(x[e], scale);
    w[e >> 2] |= (KVT == DT_FP8 ? f32_to_e4m3(y) : f32_to_i8(y)) << (8 * (e & 3));
  }
  const size_t blk16 = (size_t)blk * (size_t)bstride;  // where the block starts, 16-byte units
  if (!isv) {
    const u32x4 packed = {w[0], w[1], w[2], w[3]};
    reinterpret_cast<u32x4*>(k_pool)[blk16 + ((size_t)h * NC + c) * B + off] = packed;
  } else {
    // one-byte codes, 16 per 16-byte unit; V page [B/TG][D][TG], TG = min(16, B):
    // element (dim 16 c, token off), then the next dims TG elements apart
    const int tgl = min(4, log2_of(B));
    const size_t d0 = blk16 * 16 + (size_t)h * D * B +
                      (((size_t)(off >> tgl) * D + (size_t)c * 16) << tgl) + (off & ((1 << tgl) - 1));
#pragma unroll
    for (int e = 0; e < 16; ++e)
      v_pool[d0 + ((size_t)e << tgl)] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  }
}

// Whole-block copies for copy on write ("KV Cache: capacity, layout,
// lifecycle", "Reference counting and tail-block COW": the committed K/V and
// the quantisation scales of the old tail block are copied before the new table
// is published).  One block is contiguous in each pool ([block][head][...]), so
// a copy is one run of H_kv pages per pool; workgroup (pair, pool, part) moves
// a slice of it in 16-byte pieces, and part 0 of each pool also copies the fp8
// scales of the block.
__global__ __launch_bounds__(kWriteThreads) void copy_blocks_kernel(
    const int32_t* __restrict__ pairs, int num_pairs, uint8_t* k_pool, uint8_t* v_pool,
    float* k_scale, float* v_scale, int num_blocks, int scales_per_block,
    long long block_pieces, long long bstride) {
  const int pr = blockIdx.x;
  const int src = pairs[2 * pr], dst = pairs[2 * pr + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const bool isv = blockIdx.y != 0;
  u32x4* pool = reinterpret_cast<u32x4*>(isv ? v_pool : k_pool);
  const u32x4* from = pool + (size_t)src * (size_t)bstride;
  u32x4* to = pool + (size_t)dst * (size_t)bstride;
  for (long long i = (long long)blockIdx.z * kWriteThreads + threadIdx.x; i < block_pieces;
       i += (long long)gridDim.z * kWriteThreads)
    to[i] = from[i];
  float* sc = isv ? v_scale : k_scale;
  if (sc && blockIdx.z == 0)  // the block's scales: one per kv head, or per (head, token)
    for (int i = threadIdx.x; i < scales_per_block; i += kWriteThreads)
      sc[(size_t)dst * scales_per_block + i] = sc[(size_t)src * scales_per_block + i];
}

int launch_copy_blocks(const int32_t* pairs, int num_pairs, void* k_pool, void* v_pool,
                       float* k_scale, float* v_scale, int num_blocks, int block_size, int Hkv,
                       int head_dim, int kv_dtype, int scale_mode, long long bstride,
                       hipStream_t st) {
  if (num_pairs == 0) return 0;
  const bool quant = kv_dtype == DT_FP8 || kv_dtype == DT_I8;
  const int ES = kv_dtype == DT_F32 ? 4 : (quant ? 1 : 2);
  // a per-tensor scale belongs to no block; the others move with their block
  const int spb = !quant || scale_mode == SCALE_TENSOR
                      ? 0
                      : (scale_mode == SCALE_TOKEN ? Hkv * block_size : Hkv);
  const long long pieces = (long long)Hkv * head_dim * block_size * ES / 16;  // per pool
  const long long parts = (pieces + 4 * kWriteThreads - 1) / (4 * kWriteThreads);
  dim3 grid((unsigned)num_pairs, 2, (unsigned)(parts < 1 ? 1 : (parts > 64 ? 64 : parts)));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kWriteThreads), 0, st, pairs, num_pairs,
                     (uint8_t*)k_pool, (uint8_t*)v_pool, spb ? k_scale : nullptr,
                     spb ? v_scale : nullptr, num_blocks, spb, pieces, bstride);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_slot_mapping(const int32_t* block_table, int num_seqs, int W, const int32_t* seq_idx,
                        const int32_t* positions, int num_tokens, int B, int64_t* slot_mapping,
                        hipStream_t st) {
  if (num_tokens == 0) return 0;
  dim3 grid((num_tokens + kWriteThreads - 1) / kWriteThreads);
  hipLaunchKernelGGL(slot_mapping_kernel, grid, dim3(kWriteThreads), 0, st, block_table,
                     num_seqs, W, seq_idx, positions, num_tokens, B, slot_mapping);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_kv_cache_write(const WriteLaunch& p, hipStream_t st) {
  if (p.num_tokens == 0) return 0;
  const bool quant = p.kv_dtype == DT_FP8 || p.kv_dtype == DT_I8;
  const int ES = p.kv_dtype == DT_F32 ? 4 : (quant ? 1 : 2);
  const long long pieces = (long long)p.num_tokens * p.num_kv_heads * (p.head_dim * ES / 16);
  const long long blocks = (pieces + kWriteThreads - 1) / kWriteThreads;
  if (blocks > 0x7fffffffLL) return -3;
  dim3 grid((unsigned)blocks, 2);
  SlotSource ss;
  ss.slot_mapping = p.slot_mapping;
  ss.block_table = p.block_table;
  ss.seq_idx = p.seq_idx;
  ss.positions = p.positions;
  ss.num_seqs = p.num_seqs;
  ss.W = p.max_blocks_per_seq;
  ss.slot_out = p.slot_out;
  const uint8_t* k = (const uint8_t*)p.k;
  const uint8_t* v = (const uint8_t*)p.v;
  uint8_t* kp = (uint8_t*)p.k_pool;
  uint8_t* vp = (uint8_t*)p.v_pool;
  auto quant_launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kWriteThreads), 0, st, ss, p.num_tokens, k, v, kp, vp,
                       p.k_scale, p.v_scale, p.scale_mode, p.num_blocks, p.block_size,
                       p.num_kv_heads, p.head_dim, p.bstride);
  };
  if (p.kv_dtype == DT_F32)
    hipLaunchKernelGGL(kv_write_copy_kernel<4>, grid, dim3(kWriteThreads), 0, st, ss,
                       p.num_tokens, k, v, kp, vp, p.num_blocks, p.block_size, p.num_kv_heads,
                       p.head_dim, p.bstride);
  else if (p.kv_dtype == DT_F16 || p.kv_dtype == DT_BF16)
    hipLaunchKernelGGL(kv_write_copy_kernel<2>, grid, dim3(kWriteThreads), 0, st, ss,
                       p.num_tokens, k, v, kp, vp, p.num_blocks, p.block_size, p.num_kv_heads,
                       p.head_dim, p.bstride);
  else if (p.kv_dtype == DT_FP8 && p.src_dtype == DT_BF16)
    quant_launch(kv_write_quant_kernel<DT_BF16, DT_FP8>);
  else if (p.kv_dtype == DT_FP8 && p.src_dtype == DT_F16)
    quant_launch(kv_write_quant_kernel<DT_F16, DT_FP8>);
  else if (p.kv_dtype == DT_FP8 && p.src_dtype == DT_F32)
    quant_launch(kv_write_quant_kernel<DT_F32, DT_FP8>);
  else if (p.kv_dtype == DT_I8 && p.src_dtype == DT_BF16)
    quant_launch(kv_write_quant_kernel<DT_BF16, DT_I8>);
  else if (p.kv_dtype == DT_I8 && p.src_dtype == DT_F16)
    quant_launch(kv_write_quant_kernel<DT_F16, DT_I8>);
  else if (p.kv_dtype == DT_I8 && p.src_dtype == DT_F32)
    quant_launch(kv_write_quant_kernel<DT_F32, DT_I8>);
  else
    return -3;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace pkv
