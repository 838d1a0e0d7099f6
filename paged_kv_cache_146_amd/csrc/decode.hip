// decode.hip — paged decode attention for gfx950 on the matrix cores, plus the
// split-KV log-sum-exp merges.
//
// Method: "03 | PagedAttention and the KV-cache memory system", §4 — per
// sequence and query head, walk the logical blocks of the visible context,
// look each one up in the block table, load its K/V page, and fold the partial
// attention into an online-softmax state (max, exp_sum, weighted_value); long
// contexts are scanned in parallel pieces whose states are merged.
//
// A wavefront works on 64 consecutive tokens of one (sequence, kv head) at a
// time ("chunk"), for all G = H_q/H_kv query heads of that kv head, so every
// K/V byte is read from HBM once per step (GQA grouping).  Both products run
// on 16x16 MFMA tiles with the query heads as the N = 16 columns (heads past G
// are zero columns):
//   S^T = K . Q^T   A = 16 K rows (tokens) x 32 dims, from the K pool
//                   [block][head][D/X][B][X]: one 16-byte piece per lane;
//                   B = q, loaded once per (sequence, kv head).
//   O^T = V^T . P^T A = 16 dims x 32 tokens, from the V pool
//                   [block][head][B/TG][D][TG] (runs of TG = min(X, B) tokens
//                   per dim): four consecutive tokens of a dim per lane piece;
//                   B = P, which S^T's output layout already leaves in place.
// Lane L = 16 g + n.  Tile T's row n is token 16 T + n, so each K load of a
// wavefront reads 16 consecutive tokens of four consecutive K pieces: 1 KB of
// one page, contiguous.  In S^T's output the lane holds head n at the tokens
// 16 T + 4 g + r (rows 4 g + r of tile T).  P.V takes its k-slots in the same
// order, so the online softmax (max over the four lane groups by permlane
// swaps, p = 2^(z - m) with log2(e) folded into the scale) feeds the second
// product without any data exchange, and a lane's V operand is two runs of four
// consecutive tokens of one dim (each V load of a wavefront: 16 dims x 16
// tokens, 16-byte-or-longer runs of the V pool).  O^T leaves head n, dims 16 dt + 4 g + r in
// the lane.  With block_size >= 16 the 16 tokens of a tile share one block, so
// the table entries of a chunk are wave-uniform (scalar loads).
//
// fp8 (OCP E4M3) and int8 pages are widened exactly to the query's 16-bit type for
// S^T and to f16 for P.V; K's scale (per page, per pool or per token) multiplies the
// scores and V's is folded into P, which enters P.V as one f16 term (p <= 1 against
// the running max).  With a 16-bit pool P enters as a hi + lo pair of that type.
// The 8-bit V pages are loaded by rows: lane group g takes the whole 16-token row of
// tile g for its dims (one 16-byte load per dim tile), and a 4 x 4 transpose across
// the lane groups (permlane swaps) hands each lane its four tokens of every tile.
// f32 pools use the 16x16x4 f32 product with one k-slot per lane.
//
// Three ways to cut the work:
//   unsplit / fixed partitions — one workgroup (4 waves) per (kv head,
//         sequence, partition), kv heads first in launch order (workgroups go to
//         the 8 XCDs round-robin, so with H_kv a multiple of 8 each XCD takes one
//         kv head of every item) and, up to 256 sequences, longest context first;
//         the waves take chunks round-robin and merge in LDS; partitions are
//         merged by split_reduce_kernel.
//   balanced — the chunks of all (sequence, kv head) pairs form one stream that
//         is cut into equal contiguous shares, one per wavefront ("worker").  A
//         worker finishes every pair it covers entirely and leaves a partial
//         state for at most two pairs it shares with neighbours; those are
//         merged by the last worker to finish one (a per-pair counter tells it).
//   shared prefix — shared_prefix_kernel reads the blocks every sequence of the
//         batch shares once per kv head, with 16/G sequences x G heads in the 16
//         product columns; the balanced kernel takes the private tails and
//         merge_slots_kernel merges the two.
// Both main kernels also take a sliding window (a sequence's chunk grid starts
// at its window's first 16-token tile), and both can store each sequence's
// newest token themselves before decoding it (the fused decode step).
// The workgroup kernel's chunk loop is software-pipelined on one buffer for 16-
// and 32-bit pools: the next chunk's K pieces are requested as soon as the
// current scores are done and its V pieces as soon as the current P.V is done,
// the table entries one chunk further ahead.  Over 8-bit pools, whose chunks are
// half the bytes, it runs two buffers deep (chunk i+1 in flight while chunk i is
// computed, chunk i+2 requested into chunk i's buffer in the same two halves), so
// that a wavefront keeps as many bytes in flight as over a 16-bit pool.  The
// balanced kernel's loop runs on two buffers (the next chunk in flight while the
// current one is computed).  Both are compiled with the whole register file open
// to a wavefront, whose registers hold the buffers; where an instantiation needs at
// most 256 of them (the workgroup kernel over 16-bit pools, and over 8-bit pools
// with page or pool scales), the hardware keeps two wavefronts per SIMD.
#include "device.hpp"
#include "internal.hpp"
#include "tile.hpp"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace pkv {

struct DecodeScalars {
  int W;            // max_blocks_per_seq
  int ctx_cap;      // clamp for context_lens
  int S, Hq, Hkv, G;
  int blog2;        // log2(block_size)
  int num_blocks;
  int part_size;    // tokens per partition, multiple of 64 (WG kernel)
  int max_parts;
  int split;
  int out_dtype;
  int num_workers;  // balanced kernel: wavefront workers in the grid
  uint32_t epoch;   // balanced kernel: call tag of the shared-pair counters
  int scale_mode;   // quantised pools: SCALE_BLOCK / SCALE_TENSOR / SCALE_TOKEN
  float scale_log2; // softmax scale * log2(e)
  // balanced kernel over the private tails of a batch with a shared prefix:
  // every sequence starts ctx_off tokens (tbl_off table entries) in, and its
  // result goes to partial slot tail_part of the part arrays (stride max_parts)
  // instead of `out`; tail_part < 0: plain decode
  int ctx_off, tbl_off, tail_part;
  float* tail_out;
  float* tail_max;
  float* tail_sum;
  int window;       // > 0: a sequence of context c sees only the keys [c - window, c)
  long long bstride;  // 16-byte units from one block to the next in each pool
  // decode fused with the append of each sequence's newest token (position ctx - 1):
  // its K / V rows [S][H_kv][D], in the pool's 16-bit type, and where its slots go
  const uint8_t* k_new;
  const uint8_t* v_new;
  int64_t* slot_out;
  int lpt;  // workgroup kernel, S <= kThreads: sequences go out longest first
};

// 16-byte unit where block b's K pages start, and element where its V pages start
__device__ __forceinline__ size_t block_k16(const DecodeScalars& sc, int b) {
  return (size_t)b * (size_t)sc.bstride;
}

// The oldest key a sequence of (clamped) context ctx sees, and where its chunk grid
// starts: that key rounded down to a 16-token tile.  With block_size >= 16 the tile
// lies in the key's own block, so no table entry of an older block is ever read
// (those blocks may have been released); the keys of the tile older than the
// window are masked.
__device__ __forceinline__ int window_lo(int ctx, int window) {
  return window > 0 && ctx > window ? ctx - window : 0;
}

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// ---- per-instantiation geometry ----------------------------------------------------
// KVT = pool element type, CT = product type (the query's type), D = head dim.
template <int KVT, int CT, int D>
struct Cfg {
  static constexpr int Dim = D;
  static constexpr int EB = Elem<KVT>::bytes;
  static constexpr int E = 16 / EB;           // elements per 16-byte piece (the pool's X)
  static constexpr int ELOG = EB == 4 ? 2 : (EB == 2 ? 3 : 4);  // log2(E)
  static constexpr int NC = D / E;            // pieces per K row
  static constexpr int NPL = NC / 4;          // K pieces per lane per token (lane group g
                                              // takes pieces 4 q + g)
  static constexpr bool F32 = (CT == DT_F32);
  static constexpr int SPP = F32 ? E : E / 8; // MFMA k-steps per K piece
  static constexpr int NQ = NPL * SPP;        // q operands
  static constexpr int NDT = D / 16;          // dim tiles of O^T
  static constexpr int NK = 4 * NPL;          // K pieces per lane per chunk: [T][q]
  static constexpr int NV = NDT * 4;          // V pieces per lane per chunk: [dt][T]
  static constexpr int QEB = F32 ? 4 : 2;     // bytes per q element
  // chunk buffers in the balanced kernel's software pipeline (for 16-bit pools the
  // second lives in AGPRs, which measured faster than one buffer whose next chunk is
  // requested in two halves as in the workgroup kernel; a third costs more in copies
  // than it gains)
  static constexpr int NBUF = 2;
  using QOp = std::conditional_t<F32, float, u32x4>;
  // a V piece: four consecutive tokens of one dim
  using VPiece = std::conditional_t<EB == 4, u32x4, std::conditional_t<EB == 2, u32x2, uint32_t>>;
  static_assert(NPL >= 1, "head_dim too small for four lane groups");
  static_assert((KVT == DT_F32) == F32, "f32 pools pair with f32 queries only");
};

template <class C>
struct Chunk {
  u32x4 k[C::NK];                // [T][q]: pieces 4 q + g of token 16 T + n
  typename C::VPiece v[C::NV];  // [dt][T]: dim 16 dt + n, tokens 16 T + 4 g + (0..3)
};

// per-lane softmax state: head n; m is shared by the four lane groups, l is the
// lane's own share of the exp-sum
template <class C>
struct State {
  f32x4 acc[C::NDT];
  float m, l;
};

template <class C>
__device__ __forceinline__ void state_init(State<C>& st) {
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) st.acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  st.m = -INFINITY;
  st.l = 0.0f;
}

// q operands (B of S^T = K . Q^T) for the kv head's G query heads.  Lanes of
// heads >= G load head 0's row; q_live() zeroes those columns afterwards (kept
// apart so that a prefetch of the next pair's q does not wait on its own load).
// Operand (pq, h) of lane group g covers the dims of K piece c = 4 pq + g, step h.
template <class C>
__device__ __forceinline__ void load_q_row(typename C::QOp (&qop)[C::NQ],
                                           const uint8_t* __restrict__ row, int g) {
#pragma unroll
  for (int pq = 0; pq < C::NPL; ++pq) {
    const int c = 4 * pq + g;
    if constexpr (C::F32) {  // four dims per piece, one per step
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + (size_t)c * 16);
#pragma unroll
      for (int h = 0; h < C::SPP; ++h) qop[pq * C::SPP + h] = as_f32(w[h]);
    } else {  // eight dims per step: [c E + 8 h, c E + 8 h + 8)
#pragma unroll
      for (int h = 0; h < C::SPP; ++h)
        qop[pq * C::SPP + h] = *reinterpret_cast<const u32x4*>(row + ((size_t)c * C::E + 8 * h) * 2);
    }
  }
}

template <class C>
__device__ __forceinline__ void load_q(typename C::QOp (&qop)[C::NQ],
                                       const uint8_t* __restrict__ q, int s, int kvh,
                                       const DecodeScalars& sc, int n, int g) {
  const bool live = n < sc.G;
  load_q_row<C>(qop, q + ((size_t)s * sc.Hq + (size_t)kvh * sc.G + (live ? n : 0)) * C::Dim * C::QEB,
                g);
}

template <class C>
__device__ __forceinline__ void q_live(typename C::QOp (&dst)[C::NQ],
                                       const typename C::QOp (&src)[C::NQ], bool live) {
#pragma unroll
  for (int k = 0; k < C::NQ; ++k) {
    if constexpr (C::F32)
      dst[k] = live ? src[k] : 0.0f;
    else
      dst[k] = live ? src[k] : u32x4{0u, 0u, 0u, 0u};
  }
}

// ---- loads of one chunk (block_size >= 16) ------------------------------------------
// Tile T's tokens 16 T .. 16 T + 15 lie in one block, so the chunk needs four
// wave-uniform table entries.  Tiles at or past `end` are clamped onto the last
// visible block (their values are masked).
struct Pages {
  int b[4];
  int off;  // base mod block_size: tile T starts at offset (off + 16 T) mod block_size
};

__device__ __forceinline__ Pages pages_of(const int32_t* __restrict__ trow, int base, int end,
                                          const DecodeScalars& sc) {
  Pages pg;
  pg.off = uniform(base & ((1 << sc.blog2) - 1));
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int t = uniform(min(base + 16 * T, end - 1));
    pg.b[T] = uniform(clamp_block(trow[t >> sc.blog2], sc.num_blocks));
  }
  return pg;
}

// The decode reads each K/V byte once per step, so its page loads carry the
// non-temporal hint (STREAM = true): the lines stream through the caches instead
// of being kept there.  The shared-prefix kernel, whose column tiles re-read the
// prefix from their XCD's L2, loads with the default policy.
template <class C, bool STREAM = true>
__device__ __forceinline__ void issue_k(u32x4 (&kr)[C::NK], const uint8_t* __restrict__ k_pool,
                                        const Pages& pg, int kvh, const DecodeScalars& sc, int n,
                                        int g) {
  const int B = 1 << sc.blog2;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const size_t page = block_k16(sc, pg.b[T]) + (size_t)kvh * C::NC * B;  // 16-byte units
    const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + page +
                      ((pg.off + 16 * T) & (B - 1)) + n + (size_t)g * B;
#pragma unroll
    for (int pq = 0; pq < C::NPL; ++pq) {
      if constexpr (STREAM)
        kr[T * C::NPL + pq] = __builtin_nontemporal_load(&kp[(size_t)pq * 4 * B]);
      else
        kr[T * C::NPL + pq] = kp[(size_t)pq * 4 * B];
    }
  }
}

template <class C, bool STREAM = true>
__device__ __forceinline__ void issue_v(typename C::VPiece (&vr)[C::NV],
                                        const uint8_t* __restrict__ v_pool, const Pages& pg,
                                        int kvh, const DecodeScalars& sc, int n, int g) {
  using VP = typename C::VPiece;
  const int B = 1 << sc.blog2;
  if constexpr (C::EB == 1) {
    // 8-bit pools: lane group g loads tile g's whole 16-token row of each dim (one
    // 16-byte load per dim tile instead of four 4-byte ones); v_rows_to_tiles then
    // hands each lane its four tokens of every tile
    const int bg = g == 0 ? pg.b[0] : (g == 1 ? pg.b[1] : (g == 2 ? pg.b[2] : pg.b[3]));
    const int t = (pg.off + 16 * g) & (B - 1);  // the group's tile: 16 tokens, one row
    const uint8_t* vp = v_pool + block_k16(sc, bg) * 16 +
                        ((size_t)kvh * C::Dim * B + ((size_t)(t / 16) * C::Dim + n) * 16);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const u32x4* a = reinterpret_cast<const u32x4*>(vp + (size_t)16 * dt * 16);
      const u32x4 w = STREAM ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[dt * 4 + r] = w[r];
    }
    return;
  }
  // V page [B/E][D][E] (block_size >= 16 >= E): token t of dim d at (t/E * D + d) E + t%E
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int t = ((pg.off + 16 * T) & (B - 1)) + 4 * g;  // the lane's first token
    const uint8_t* vp = v_pool + block_k16(sc, pg.b[T]) * 16 +
                        ((size_t)kvh * C::Dim * B + ((size_t)(t / C::E) * C::Dim + n) * C::E +
                         (t % C::E)) * C::EB;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {  // 16 dims on
      const VP* a = reinterpret_cast<const VP*>(vp + (size_t)16 * dt * C::E * C::EB);
      if constexpr (STREAM)
        vr[dt * 4 + T] = __builtin_nontemporal_load(a);
      else
        vr[dt * 4 + T] = *a;
    }
  }
}

// 8-bit pools loaded by rows (issue_v): lane group g holds, for each dim tile, the
// four 4-token words of tile g; a 4 x 4 transpose across the lane groups (two
// permlane32 and two permlane16 swaps per dim tile) leaves word T = tokens
// 16 T + 4 g + (0..3), the layout the P.V products take
template <class C>
__device__ __forceinline__ void v_rows_to_tiles(typename C::VPiece (&vr)[C::NV]) {
  if constexpr (C::EB == 1) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      uint32_t* w = &vr[dt * 4];
      // across lane-group halves (g and g ^ 2): words 0/2 and 1/3
      auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
      w[0] = a[0];
      w[2] = a[1];
      auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
      w[1] = b[0];
      w[3] = b[1];
      // within each half (g and g ^ 1): words 0/1 and 2/3
      auto c = __builtin_amdgcn_permlane16_swap(w[0], w[1], false, false);
      w[0] = c[0];
      w[1] = c[1];
      auto d = __builtin_amdgcn_permlane16_swap(w[2], w[3], false, false);
      w[2] = d[0];
      w[3] = d[1];
    }
  }
}

// index of the scale of (page, token offset) in the pool's scale mode
__device__ __forceinline__ size_t scale_at(const DecodeScalars& sc, size_t page, int off) {
  return sc.scale_mode == SCALE_TENSOR ? 0
                                       : (sc.scale_mode == SCALE_TOKEN ? (page << sc.blog2) + off
                                                                       : page);
}

// scales of the lane's 16 keys of a quantised chunk (key 16 T + 4 g + r at slot
// 4 T + r): one per page, one for the pool, or one per token (four consecutive
// tokens of a page for each tile)
__device__ __forceinline__ void chunk_scales(float (&ks)[16], float (&vs)[16],
                                             const float* __restrict__ k_scale,
                                             const float* __restrict__ v_scale, const Pages& pg,
                                             int kvh, const DecodeScalars& sc, int g) {
  const int B = 1 << sc.blog2;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const size_t page = (size_t)pg.b[T] * sc.Hkv + kvh;
    if (sc.scale_mode == SCALE_TOKEN) {
      const size_t i0 = page * B + ((pg.off + 16 * T) & (B - 1)) + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ks[4 * T + r] = k_scale[i0 + r];
        vs[4 * T + r] = v_scale[i0 + r];
      }
    } else {
      const size_t i = sc.scale_mode == SCALE_TENSOR ? 0 : page;
      const float a = k_scale[i], b = v_scale[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ks[4 * T + r] = a;
        vs[4 * T + r] = b;
      }
    }
  }
}

// The same scales with the mode fixed at compile time: per token (TOK) the lane's 16
// keys, else one per tile (page or pool scale), so a software pipeline that holds the
// scales of two chunks keeps 8 registers per chunk instead of 32 outside token mode
template <bool TOK>
struct ChunkScales {
  float k[TOK ? 16 : 4], v[TOK ? 16 : 4];
};

template <bool TOK>
__device__ __forceinline__ void load_scales(ChunkScales<TOK>& cs, const float* __restrict__ k_scale,
                                            const float* __restrict__ v_scale, const Pages& pg,
                                            int kvh, const DecodeScalars& sc, int g) {
  const int B = 1 << sc.blog2;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const size_t page = (size_t)pg.b[T] * sc.Hkv + kvh;
    if constexpr (TOK) {
      const size_t i0 = page * B + ((pg.off + 16 * T) & (B - 1)) + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cs.k[4 * T + r] = k_scale[i0 + r];
        cs.v[4 * T + r] = v_scale[i0 + r];
      }
    } else {
      const size_t i = sc.scale_mode == SCALE_TENSOR ? 0 : page;
      cs.k[T] = k_scale[i];
      cs.v[T] = v_scale[i];
    }
  }
}

// the 16 per-key scales (key 16 T + 4 g + r at slot 4 T + r) the softmax takes
template <bool TOK>
__device__ __forceinline__ void expand_scales(const ChunkScales<TOK>& cs, float (&ks)[16],
                                              float (&vs)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (TOK) {
      ks[i] = cs.k[i];
      vs[i] = cs.v[i];
    } else {
      ks[i] = cs.k[i >> 2];
      vs[i] = cs.v[i >> 2];
    }
  }
}

// ---- loads of one chunk (block_size < 16): every token looks up its own block -----
template <class C>
__device__ __forceinline__ void load_small(Chunk<C>& ch, float (&ks)[16], float (&vs)[16],
                                           const uint8_t* __restrict__ k_pool,
                                           const uint8_t* __restrict__ v_pool,
                                           const float* __restrict__ k_scale,
                                           const float* __restrict__ v_scale,
                                           const int32_t* __restrict__ trow, int base, int end,
                                           int kvh, const DecodeScalars& sc, int n, int g,
                                           int lo = 0) {
  // tokens outside [lo, end) load the nearest visible one instead (masked later):
  // the blocks outside may have been released
  const int B = 1 << sc.blog2;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int t = max(min(base + 16 * T + n, end - 1), lo);
    const int blk = clamp_block(trow[t >> sc.blog2], sc.num_blocks);
    const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + block_k16(sc, blk) +
                      (size_t)kvh * C::NC * B + (t & (B - 1)) + (size_t)g * B;
#pragma unroll
    for (int pq = 0; pq < C::NPL; ++pq) ch.k[T * C::NPL + pq] = kp[(size_t)pq * 4 * B];
  }
  uint32_t w[C::NV][4];
#pragma unroll
  for (int a = 0; a < C::NV; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) w[a][b] = 0u;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * T + e;  // the lane's score index of this token
      const int t = max(min(base + 16 * T + 4 * g + e, end - 1), lo);
      const int blk = clamp_block(trow[t >> sc.blog2], sc.num_blocks);
      const size_t page = (size_t)blk * sc.Hkv + kvh;  // scale index base
      if constexpr (C::EB == 1) {  // quantised
        const size_t si = scale_at(sc, page, t & (B - 1));
        ks[i] = k_scale[si];
        vs[i] = v_scale[si];
      } else {
        ks[i] = vs[i] = 1.0f;
      }
      // element of dim n: V page [B/TG][D][TG], TG = min(E, B) tokens per dim run
      const int tgl = min(C::ELOG, sc.blog2), tb = t & (B - 1);
      const size_t e0 = block_k16(sc, blk) * C::E + (size_t)kvh * C::Dim * B +
                        (((size_t)(tb >> tgl) * C::Dim + n) << tgl) + (tb & ((1 << tgl) - 1));
      const int word = e * C::EB / 4, sh = (e * C::EB % 4) * 8;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const size_t el = e0 + ((size_t)16 * dt << tgl);
        uint32_t x;
        if constexpr (C::EB == 4)
          x = reinterpret_cast<const uint32_t*>(v_pool)[el];
        else if constexpr (C::EB == 2)
          x = reinterpret_cast<const uint16_t*>(v_pool)[el];
        else
          x = v_pool[el];
        w[dt * 4 + T][word] |= x << sh;
      }
    }
#pragma unroll
  for (int a = 0; a < C::NV; ++a) {
    if constexpr (C::EB == 4)
      ch.v[a] = u32x4{w[a][0], w[a][1], w[a][2], w[a][3]};
    else if constexpr (C::EB == 2)
      ch.v[a] = u32x2{w[a][0], w[a][1]};
    else
      ch.v[a] = w[a][0];
  }
}

// ---- the two products and the online softmax of one chunk ------------------------
template <class C, int KVT, int CT>
__device__ __forceinline__ void chunk_qk(f32x4 (&S)[4], const u32x4 (&kr)[C::NK],
                                         const typename C::QOp (&qop)[C::NQ]) {
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int pq = 0; pq < C::NPL; ++pq) {
      const u32x4 piece = kr[T * C::NPL + pq];
#pragma unroll
      for (int h = 0; h < C::SPP; ++h) {
        if constexpr (C::F32)
          acc = mma_f32(as_f32(piece[h]), qop[pq * C::SPP + h], acc);
        else if constexpr (C::EB == 1)
          acc = mma16<CT>(widen8<KVT, CT>(piece[2 * h], piece[2 * h + 1]), qop[pq * C::SPP + h],
                          acc);
        else
          acc = mma16<CT>(piece, qop[pq], acc);
      }
    }
    S[T] = acc;
  }
}

// zero the V elements of masked tokens (0xFF-filled or stale slots may hold NaN,
// and 0 * NaN would poison the product).  Piece [dt][T] holds tokens
// 16 T + 4 g + e, e < 4; a token is visible when below nvalid.
template <class C>
__device__ __forceinline__ void mask_v(typename C::VPiece (&vr)[C::NV], int nvalid, int g) {
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int t0 = 16 * T + 4 * g;
      auto& x = vr[dt * 4 + T];
      if constexpr (C::EB == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = t0 + e < nvalid ? x[e] : 0u;
      } else if constexpr (C::EB == 2) {
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
          const uint32_t m = (t0 + 2 * wd < nvalid ? 0x0000ffffu : 0u) |
                             (t0 + 2 * wd + 1 < nvalid ? 0xffff0000u : 0u);
          x[wd] &= m;
        }
      } else {
        uint32_t m = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) m |= t0 + e < nvalid ? (0xffu << (8 * e)) : 0u;
        x &= m;
      }
    }
}

// Scores x[4 T + r] belong to token 16 T + 4 g + r, and so do the scales ks[4 T + r]
// and vs[4 T + r] of a quantised pool.  Keys from nvalid on (wave-uniform) are
// past the context of every column.  COLMASK: the lane's column also hides the
// keys from xvalid on, and may see no key of the chunk at all.  Keys below nlow
// (wave-uniform; the first chunk of a sliding window) are older than the window:
// their values are finite (the window's own first tile, or a clamped load) and
// only their scores are masked.
template <class C, int KVT, int CT, bool COLMASK = false>
__device__ __forceinline__ void chunk_softmax_pv(State<C>& st, const f32x4 (&S)[4],
                                                 typename C::VPiece (&vr)[C::NV], float zscale,
                                                 const float (&ks)[16], float (&vs)[16],
                                                 int nvalid, int g, int xvalid = 64,
                                                 int nlow = 0) {
  constexpr bool kFp8 = (KVT == DT_FP8 || KVT == DT_I8);  // quantised: scaled 8-bit codes
  float x[16];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * T + r;
      x[i] = S[T][r] * (kFp8 ? zscale * ks[i] : zscale);
    }
  if (nvalid < 64) {
    // a key past the context gets weight 0; its V codes and its scale (read from a
    // slot nothing wrote, or from a page past the table's live entries) may hold
    // anything, NaN included, so both are cleared rather than multiplied by 0
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool live = 16 * T + 4 * g + r < nvalid;
        x[4 * T + r] = live ? x[4 * T + r] : -INFINITY;
        if constexpr (kFp8) vs[4 * T + r] = live ? vs[4 * T + r] : 0.0f;
      }
    mask_v<C>(vr, nvalid, g);
  }
  if (nlow > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      x[i] = 16 * (i >> 2) + 4 * g + (i & 3) >= nlow ? x[i] : -INFINITY;
  }
  if constexpr (COLMASK) {
    if (xvalid < 64) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        x[i] = 16 * (i >> 2) + 4 * g + (i & 3) < xvalid ? x[i] : -INFINITY;
    }
  }
  float cm = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) cm = fmaxf(cm, x[i]);
  cm = max_groups(cm);  // finite unless COLMASK: token 0 of every chunk is visible
  const float mn = fmaxf(st.m, cm);
  // a column that has seen no key yet keeps m = -inf and adds nothing
  const float mref = COLMASK && mn == -INFINITY ? 0.0f : mn;
  const float alpha = __builtin_amdgcn_exp2f(st.m - mref);
  st.m = mn;
  float p[16], ps = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
    ps += p[i];
  }
  st.l = st.l * alpha + ps;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) st.acc[dt] *= alpha;
  }
  if constexpr (C::F32) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const u32x4 piece = vr[dt * 4 + T];
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[dt] = mma_f32(as_f32(piece[r]), p[4 * T + r], st.acc[dt]);
      }  // the f32 pool: VPiece is u32x4
  } else if constexpr (kFp8) {
    // 8-bit pools: the codes widen exactly to f16, and P (times V's scale, p <= 1)
    // enters P.V as one f16 term: 11 significant bits, one product per operand
    u32x4 pv[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t w[4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int i0 = 8 * s2 + 2 * wd;
        w[wd] = pack2<DT_F16>(p[i0] * vs[i0], p[i0 + 1] * vs[i0 + 1]);
      }
      pv[s2] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        // slots 0-3: tokens 32 s2 + 4 g + (0..3) (tile 2 s2); 4-7: tile 2 s2 + 1
        const u32x4 a = widen8<KVT, DT_F16>(vr[dt * 4 + 2 * s2], vr[dt * 4 + 2 * s2 + 1]);
        st.acc[dt] = mma16<DT_F16>(a, pv[s2], st.acc[dt]);
      }
  } else {
    // P = hi + lo, both in CT: the pair carries about twice CT's significand, so
    // the weights reach the product essentially unrounded (a single 16-bit P
    // would cost up to 2^-9 relative per term, visible where outputs cancel)
    u32x4 phi[2], plo[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int i0 = 8 * s2 + 2 * wd;
        float a = p[i0], b = p[i0 + 1];
        if constexpr (kFp8) {
          a *= vs[i0];
          b *= vs[i0 + 1];
        }
        wh[wd] = pack2<CT>(a, b);
        const f32x2 h = unpack2<CT>(wh[wd]);
        wl[wd] = pack2<CT>(a - h[0], b - h[1]);
      }
      phi[s2] = u32x4{wh[0], wh[1], wh[2], wh[3]};
      plo[s2] = u32x4{wl[0], wl[1], wl[2], wl[3]};
    }
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        // slots 0-3: tokens 32 s2 + 4 g + (0..3) (tile 2 s2); 4-7: tile 2 s2 + 1
        u32x4 a;
        if constexpr (kFp8) {
          a = widen8<KVT, CT>(vr[dt * 4 + 2 * s2], vr[dt * 4 + 2 * s2 + 1]);
        } else {
          const u32x2 lo = vr[dt * 4 + 2 * s2], hi = vr[dt * 4 + 2 * s2 + 1];
          a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        st.acc[dt] = mma16<CT>(a, phi[s2], st.acc[dt]);
        st.acc[dt] = mma16<CT>(a, plo[s2], st.acc[dt]);
      }
  }
}

// ---- the newest token of a pair (decode fused with the append) -------------------
// Its K and V rows come from the caller (k_new / v_new [S][H_kv][D], the pool's
// 16-bit type).  The wave that reads the pair's last visible chunk does not read
// that token back from the pool: once the chunk's loads have arrived it replaces
// the token's K pieces and V elements in its registers by the caller's row
// (patch_k, patch_v).  So no read of the launch depends on the store of the new
// row into the pool, and the store may complete at any time before the launch
// ends.  Between its load and its use the row sits in LDS, 2 NC pieces of 16
// bytes: K pieces 0 .. NC-1 (8 dims each), then V pieces 0 .. NC-1 (8 dims each).

// lane L < NC loads K piece L of the row, NC <= L < 2 NC the V piece L - NC
template <class C>
__device__ __forceinline__ u32x4 new_row_load(const DecodeScalars& sc, int s, int kvh, int lane) {
  const size_t row = ((size_t)s * sc.Hkv + kvh) * C::NC;  // in 16-byte pieces
  u32x4 w = {0u, 0u, 0u, 0u};
  if (lane < C::NC)
    w = reinterpret_cast<const u32x4*>(sc.k_new)[row + lane];
  else if (lane < 2 * C::NC)
    w = reinterpret_cast<const u32x4*>(sc.v_new)[row + lane - C::NC];
  return w;
}

// Store the row held in LDS into the slot of position pos of the sequence, as the
// append does: no store (slot -1) when pos / B is past the table or the table
// entry lies outside the pool; slot_out receives the slot.  The pool pointers are
// the kernel's own (const only for the decode's reads).
template <class C>
__device__ __forceinline__ void new_row_store(const DecodeScalars& sc, const uint8_t* k_pool,
                                              const uint8_t* v_pool, const int32_t* trow,
                                              const u32x4* row, int pos, int s, int kvh,
                                              int lane) {
  const int B = 1 << sc.blog2;
  const int j = pos >> sc.blog2, off = pos & (B - 1);
  const int blk = j < sc.W ? trow[j] : -1;
  const bool inside = blk >= 0 && blk < sc.num_blocks;
  if (sc.slot_out && kvh == 0 && lane == 0) sc.slot_out[s] = inside ? (int64_t)blk * B + off : -1;
  if (!inside) return;
  const size_t blk16 = block_k16(sc, blk);
  u32x4* kp = reinterpret_cast<u32x4*>(const_cast<uint8_t*>(k_pool));
  if (lane < C::NC) __builtin_nontemporal_store(row[lane], &kp[blk16 + ((size_t)kvh * C::NC + lane) * B + off]);
  // V page [B/TG][D][TG], TG = min(E, B): dims lane and lane + 64
  const uint16_t* vrow = reinterpret_cast<const uint16_t*>(row + C::NC);
  const int tgl = min(C::ELOG, sc.blog2);
  uint16_t* vp = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(v_pool)) + blk16 * C::E +
                 (size_t)kvh * C::Dim * B + ((size_t)(off >> tgl) * C::Dim << tgl) +
                 (off & ((1 << tgl) - 1));
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (lane + 64 * i < C::Dim)
      __builtin_nontemporal_store(vrow[lane + 64 * i], &vp[(size_t)(lane + 64 * i) << tgl]);
}

// The newest token is key r (0 <= r < 64, wave-uniform) of the chunk in registers.
// K: tile r / 16, row r % 16, so lanes n = r % 16 hold its pieces 4 pq + g.
template <class C>
__device__ __forceinline__ void patch_k(u32x4 (&kr)[C::NK], const u32x4* row, int r, int n, int g) {
  const int T = r >> 4;
  const bool mine = n == (r & 15);
#pragma unroll
  for (int pq = 0; pq < C::NPL; ++pq) {
    const u32x4 x = row[4 * pq + g];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t == T) kr[t * C::NPL + pq] = mine ? x : kr[t * C::NPL + pq];
  }
}

// V: piece [dt][T] of lane (n, g) holds dim 16 dt + n at keys 16 T + 4 g + (0..3),
// two 16-bit elements per word; the lanes g = (r % 16) / 4 hold key r as element r % 4.
template <class C>
__device__ __forceinline__ void patch_v(typename C::VPiece (&vr)[C::NV], const u32x4* row, int r,
                                        int n, int g) {
  static_assert(C::EB == 2, "the fused step stores 16-bit pools");
  const uint16_t* vrow = reinterpret_cast<const uint16_t*>(row + C::NC);
  const int T = r >> 4, wd = (r >> 1) & 1, sh = 16 * (r & 1);
  const bool mine = g == ((r >> 2) & 3);
  const uint32_t keep = ~(0xffffu << sh);
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) {
    const uint32_t x = (uint32_t)vrow[16 * dt + n] << sh;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t == T) {
        auto& pc = vr[dt * 4 + t];
        const uint32_t w = wd ? pc[1] : pc[0];
        const uint32_t nw = mine ? (w & keep) | x : w;
        if (wd)
          pc[1] = nw;
        else
          pc[0] = nw;
      }
  }
}

// The sequence with the r-th longest context (ties to the lower index), for S <=
// kThreads: thread t counts the sequences that go before sequence t.  The workgroup
// kernel runs one workgroup per CU and the hardware hands workgroups out in launch
// order as CUs free up, so taking the longest contexts first (longest processing
// time first) leaves the short ones to fill the end of the launch; with fixed
// partitions each partition index is a slice of the launch, taken the same way.  Called by the
// whole workgroup; the ranks form a permutation, so exactly one thread matches r.
__device__ int seq_by_rank(const int32_t* __restrict__ context_lens, int S, int r) {
  __shared__ int c_lds[kThreads];
  __shared__ int pick;
  const int t = threadIdx.x;
  if (t < S) c_lds[t] = context_lens[t];
  __syncthreads();
  if (t < S) {
    const int c = c_lds[t];
    int before = 0;
    for (int u = 0; u < S; ++u) {
      const int cu = c_lds[u];
      before += (cu > c) | ((cu == c) & (u < t));
    }
    if (before == r) pick = t;
  }
  __syncthreads();
  return uniform(pick);
}

// A wave's chunks of one (sequence, kv head) over an 8-bit pool (block_size >= 16):
// chunks c, c + 4, ... for c = wave, each base(i) = t_begin + 64 (wave + 4 i).  An
// 8-bit chunk is half the bytes of a 16-bit one, so the pipeline runs two chunks
// deep on two buffers: while chunk i is computed, chunk i+1 is in flight in the
// other buffer, and chunk i+2's K pieces are requested into the current buffer as
// soon as chunk i's scores are done, its V pieces as soon as chunk i's P.V is done.
// A chunk's scales are requested one stage ahead of their use.
template <class C, int KVT, int CT, bool TOK>
__device__ __forceinline__ void wave_chunks_8bit(
    State<C>& st, const typename C::QOp (&qop)[C::NQ], const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ trow, int t_begin, int t_end,
    int lo, int wave, int cnt, int kvh, const DecodeScalars& sc, int n, int g) {
  static_assert(C::EB == 1, "two-deep pipeline for 8-bit pools");
  auto base_of = [&](int i) { return t_begin + 64 * (wave + kWaves * min(i, cnt - 1)); };
  Chunk<C> RA, RB;
  ChunkScales<TOK> sa, sb;
  Pages pg1 = pages_of(trow, base_of(0), t_end, sc);
  issue_k<C>(RA.k, k_pool, pg1, kvh, sc, n, g);
  load_scales<TOK>(sa, k_scale, v_scale, pg1, kvh, sc, g);
  issue_v<C>(RA.v, v_pool, pg1, kvh, sc, n, g);
  pg1 = pages_of(trow, base_of(1), t_end, sc);
  if (cnt > 1) {
    issue_k<C>(RB.k, k_pool, pg1, kvh, sc, n, g);
    issue_v<C>(RB.v, v_pool, pg1, kvh, sc, n, g);
  }
  Pages pg2 = pages_of(trow, base_of(2), t_end, sc);
  // chunk i sits in R with its scales in cur; chunk i+1 (pages pg1) is in flight in
  // the other buffer and its scales go to nxt; chunk i+2 (pages pg2) goes to R
  auto stage = [&](Chunk<C>& R, ChunkScales<TOK>& cur, ChunkScales<TOK>& nxt, int i)
      __attribute__((always_inline)) {
    const int b0 = base_of(i);
    f32x4 S[4];
    chunk_qk<C, KVT, CT>(S, R.k, qop);
    issue_point();
    if (i + 1 < cnt) load_scales<TOK>(nxt, k_scale, v_scale, pg1, kvh, sc, g);
    if (i + 2 < cnt) issue_k<C>(R.k, k_pool, pg2, kvh, sc, n, g);
    const Pages pg3 = pages_of(trow, base_of(i + 3), t_end, sc);
    issue_point();
    float ks[16], vs[16];
    expand_scales<TOK>(cur, ks, vs);
    v_rows_to_tiles<C>(R.v);
    chunk_softmax_pv<C, KVT, CT>(st, S, R.v, sc.scale_log2, ks, vs, min(64, t_end - b0), g, 64,
                                 lo - b0);
    issue_point();
    if (i + 2 < cnt) issue_v<C>(R.v, v_pool, pg2, kvh, sc, n, g);
    issue_point();
    pg1 = pg2;
    pg2 = pg3;
  };
  for (int i = 0; i < cnt; i += 2) {
    stage(RA, sa, sb, i);
    if (i + 1 >= cnt) break;
    stage(RB, sb, sa, i + 1);
  }
}

// =================================================================================
// Kernel A: one workgroup per (partition, kv head, sequence)
// =================================================================================
// FUSE: the wave that reads a pair's last visible chunk (in the workgroup whose
// partition reaches the end of the clamped context) also appends the newest token
// (position ctx - 1, from sc.k_new / sc.v_new): it stores the row into its slot at
// the start and patches it into its registers at that chunk.
template <int KVT, int CT, int D, bool SMALLB, bool FUSE = false, bool TOKSC = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out,
    float* __restrict__ part_out, float* __restrict__ part_max, float* __restrict__ part_sum,
    const DecodeScalars sc) {
  using C = Cfg<KVT, CT, D>;
  constexpr bool kFp8 = (KVT == DT_FP8 || KVT == DT_I8);  // quantised: scaled 8-bit codes

  __shared__ float c_acc[kWaves][16][D];
  __shared__ float c_m[kWaves][16];
  __shared__ float c_l[kWaves][16];
  __shared__ u32x4 new_lds[FUSE ? 2 * C::NC : 1];  // the appended row (FUSE)

  // grid (kv head, sequence, partition): launch order runs over the kv heads first,
  // so with H_kv a multiple of 8 every XCD (workgroups go to the 8 XCDs round-robin)
  // takes the same kv head of every (sequence, partition), the same work.  8-bit
  // pools instead keep the kv heads of a sequence on one XCD, so that they share, in
  // its L2, the lines that hold their blocks' scales ([block][kv head] floats): the
  // launch runs in groups of 8 sequences x H_kv heads, the i-th workgroup of a group
  // takes sequence i mod 8 (reversed in every other group, which evens out the XCDs'
  // shares of the longest-first order) and kv head i / 8.
  const int part = blockIdx.z;
  int kvh = blockIdx.x, srank = blockIdx.y;
  if constexpr (C::EB == 1) {
    const int L = blockIdx.x + sc.Hkv * blockIdx.y;  // launch order in the partition
    const int full = (sc.S / 8) * 8 * sc.Hkv;        // workgroups in whole groups
    if (L < full) {
      const int grp = L / (8 * sc.Hkv), r = L - grp * 8 * sc.Hkv, x = r & 7;
      kvh = r >> 3;
      srank = 8 * grp + ((grp & 1) ? 7 - x : x);
    } else {
      kvh = (L - full) % sc.Hkv;
      srank = (sc.S / 8) * 8 + (L - full) / sc.Hkv;
    }
    kvh = uniform(kvh);
    srank = uniform(srank);
  }
  const int s = sc.lpt ? seq_by_rank(context_lens, sc.S, srank) : srank;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;

  const int ctx_raw = max(context_lens[s], 0);
  const int ctx = min(ctx_raw, sc.ctx_cap);
  const int lo = window_lo(ctx, sc.window);
  const int t_begin = max(part * sc.part_size, lo & ~15);
  const int t_end = min(part * sc.part_size + sc.part_size, ctx);
  if (t_begin >= t_end) {
    if constexpr (FUSE) {
      // a new token past a clamped context of 0 is still appended (by partition 0)
      if (part == 0 && ctx == 0 && ctx_raw > 0 && wave == 0) {
        const u32x4 w = new_row_load<C>(sc, s, kvh, lane);
        if (lane < 2 * C::NC) new_lds[lane] = w;
        wave_lds_sync();
        new_row_store<C>(sc, k_pool, v_pool, block_table + (size_t)s * sc.W, new_lds, ctx_raw - 1,
                         s, kvh, lane);
      }
    }
    if (!sc.split && part == 0) {  // empty context: zeros
      for (int i = threadIdx.x; i < sc.G * D; i += kThreads) {
        size_t o = ((size_t)s * sc.Hq + (size_t)kvh * sc.G) * D + i;
        store_any(out, sc.out_dtype, o, 0.0f);
      }
    } else if (sc.split && part * sc.part_size < ctx) {
      // a partition older than the window: an empty state for the merge
      for (int i = threadIdx.x; i < sc.G * D; i += kThreads) {
        const int h = i / D, d = i - h * D;
        const size_t pi = ((size_t)s * sc.Hq + (size_t)kvh * sc.G + h) * sc.max_parts + part;
        part_out[pi * D + d] = 0.0f;
        if (d == 0) {
          part_max[pi] = -INFINITY;
          part_sum[pi] = 0.0f;
        }
      }
    }
    return;
  }

  typename C::QOp qop[C::NQ];
  load_q<C>(qop, q, s, kvh, sc, n, g);
  q_live<C>(qop, qop, n < sc.G);
  State<C> st;
  state_init(st);
  const int32_t* trow = block_table + (size_t)s * sc.W;
  const int nch = (t_end - t_begin + 63) >> 6;
  const int cnt = nch > wave ? (nch - wave + kWaves - 1) / kWaves : 0;  // chunks wave, wave+4, ...
  auto base_of = [&](int i) { return t_begin + 64 * (wave + kWaves * min(i, cnt - 1)); };
  // FUSE: the wave that reads the last chunk requests the new row first (its first
  // chunk's loads go out behind it), parks it in LDS, patches it into its last chunk
  // when the newest token is visible (the context was not clamped; r_new is that
  // token's key index in the chunk), and stores it into the pool after its chunk
  // loop (stores issued while the launch streams cost more than stores at its end).
  const bool fuse_wave = FUSE && t_end == ctx && wave == (nch - 1) % kWaves;
  const bool patch = fuse_wave && ctx == ctx_raw;
  const int r_new = ctx - 1 - base_of(cnt - 1);
  u32x4 new_w;
  if constexpr (FUSE)
    if (fuse_wave) new_w = new_row_load<C>(sc, s, kvh, lane);
  auto park_new_row = [&]() {
    if constexpr (FUSE) {
      if (fuse_wave) {
        issue_point();  // behind the first chunk's requests
        if (lane < 2 * C::NC) new_lds[lane] = new_w;
        wave_lds_sync();
      }
    }
  };

  if constexpr (SMALLB) {
    park_new_row();
    for (int i = 0; i < cnt; ++i) {
      const int base = base_of(i);
      Chunk<C> ch;
      float ks[16], vs[16];
      load_small<C>(ch, ks, vs, k_pool, v_pool, k_scale, v_scale, trow, base, t_end, kvh, sc, n, g,
                    lo);
      if constexpr (FUSE)
        if (patch && i == cnt - 1) {
          patch_k<C>(ch.k, new_lds, r_new, n, g);
          patch_v<C>(ch.v, new_lds, r_new, n, g);
        }
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, ch.k, qop);
      chunk_softmax_pv<C, KVT, CT>(st, S, ch.v, sc.scale_log2, ks, vs, min(64, t_end - base), g,
                                   64, lo - base);
    }
  } else if (C::EB == 1 && cnt > 0) {
    if constexpr (C::EB == 1)
      wave_chunks_8bit<C, KVT, CT, TOKSC>(st, qop, k_pool, v_pool, k_scale, v_scale, trow,
                                          t_begin, t_end, lo, wave, cnt, kvh, sc, n, g);
  } else if (cnt > 0) {
    // Single-buffered pipeline: chunk i+1's K pieces are requested as soon as
    // chunk i's scores are computed and its V pieces as soon as chunk i's P.V is
    // done; the table entries run one chunk further ahead.  The load order keeps
    // every wait on the in-order memory counter narrow (K(i) never waits for
    // V(i), and so on).
    Chunk<C> R;
    float ks0[16], vs0[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ks0[i] = vs0[i] = 1.0f;
    {
      const Pages p0 = pages_of(trow, base_of(0), t_end, sc);
      issue_k<C>(R.k, k_pool, p0, kvh, sc, n, g);
      if constexpr (kFp8) chunk_scales(ks0, vs0, k_scale, v_scale, p0, kvh, sc, g);
      issue_v<C>(R.v, v_pool, p0, kvh, sc, n, g);
    }
    park_new_row();
    Pages p1 = pages_of(trow, base_of(1), t_end, sc);
    for (int i = 0; i < cnt; ++i) {
      const int b0 = base_of(i);
      const bool more = i + 1 < cnt;
      const bool patch_now = FUSE && patch && !more;
      if constexpr (FUSE)
        if (patch_now) patch_k<C>(R.k, new_lds, r_new, n, g);
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, R.k, qop);
      issue_point();
      float ks1[16], vs1[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) ks1[k] = vs1[k] = 1.0f;
      Pages p2 = p1;
      if (more) {
        issue_k<C>(R.k, k_pool, p1, kvh, sc, n, g);
        if constexpr (kFp8) chunk_scales(ks1, vs1, k_scale, v_scale, p1, kvh, sc, g);
        p2 = pages_of(trow, base_of(i + 2), t_end, sc);
      }
      issue_point();
      if constexpr (FUSE)
        if (patch_now) patch_v<C>(R.v, new_lds, r_new, n, g);
      v_rows_to_tiles<C>(R.v);
      chunk_softmax_pv<C, KVT, CT>(st, S, R.v, sc.scale_log2, ks0, vs0, min(64, t_end - b0),
                                   g, 64, lo - b0);
      issue_point();
      if (more) issue_v<C>(R.v, v_pool, p1, kvh, sc, n, g);
      issue_point();
      p1 = p2;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        ks0[k] = ks1[k];
        vs0[k] = vs1[k];
      }
    }
  }

  if constexpr (FUSE)
    if (fuse_wave) new_row_store<C>(sc, k_pool, v_pool, trow, new_lds, ctx_raw - 1, s, kvh, lane);

  // ---- merge the four waves' states in LDS ------------------------------------------
  const float lw = sum_groups(st.l);
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
    *reinterpret_cast<f32x4*>(&c_acc[wave][n][16 * dt + 4 * g]) = st.acc[dt];
  if (g == 0) {
    c_m[wave][n] = st.m;
    c_l[wave][n] = lw;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < sc.G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, c_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = __builtin_amdgcn_exp2f(c_m[w][h] - M);
      L += a * c_l[w][h];
      O += a * c_acc[w][h][d];
    }
    const int hq = kvh * sc.G + h;
    const float val = O / L;
    if (!sc.split) {
      store_any(out, sc.out_dtype, ((size_t)s * sc.Hq + hq) * D + d, val);
    } else {
      const size_t pi = ((size_t)s * sc.Hq + hq) * sc.max_parts + part;
      part_out[pi * D + d] = val;
      if (d == 0) {
        part_max[pi] = M * kLn2;  // back to natural-log units of z
        part_sum[pi] = L;
      }
    }
  }
}

// =================================================================================
// Kernel B: balanced wavefront workers
// =================================================================================
// Unit = one 64-token chunk of one (sequence, kv head) pair.  Units are ordered
// sequence-major, then kv head, then chunk; unit_prefix[s] = units before s.
// Worker w of NWe owns units [floor(w*U/NWe), floor((w+1)*U/NWe)).

// exclusive prefix of per-sequence unit counts into lds[0..S], by one workgroup:
// tiles of 256 sequences, each scanned by wave shuffles plus the wave totals
__device__ void unit_prefix(const int32_t* __restrict__ context_lens, int S, int ctx_off,
                            int ctx_cap, int window, int Hkv, int* lds, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + threadIdx.x;
    int v = 0;
    if (s < S) {
      int c = context_lens[s];
      c = c < ctx_off ? 0 : c - ctx_off;
      c = c > ctx_cap ? ctx_cap : c;
      c -= window_lo(c, window) & ~15;  // keys from the window's first tile on
      v = ((c + 63) >> 6) * Hkv;
    }
    int x = v;  // inclusive scan inside the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += tmp[w];
    if (s < S) lds[s] = before + x - v;
    int tile = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tile += tmp[w];
    carry += tile;
    __syncthreads();  // tmp is rewritten by the next tile
  }
  if (threadIdx.x == 0) lds[S] = carry;
  __syncthreads();
}

// sequence owning unit u: the last s with prefix[s] <= u (prefix non-decreasing)
__device__ __forceinline__ int find_seq(const int* prefix, int S, int u) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= u)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int worker_start(int w, int U, int NWe) {
  return (int)(((long long)w * U) / NWe);
}
// the worker whose share contains unit u
__device__ __forceinline__ int worker_of(int u, int U, int NWe) {
  return (int)((((long long)u + 1) * NWe - 1) / U);
}

// Count one finished piece of a shared (sequence, kv head) pair; returns 1 for the
// worker that brings the count to npieces.  The counter word holds (epoch << 32 |
// count): a word from another call (other epoch) counts as zero, and the last
// finisher leaves (epoch, 0) behind, so no zero-fill is ever needed and replays
// of the same call stay correct.  Lock-free: a failed exchange means another
// worker made progress; nothing waits on anyone.
// Memory order: the pieces and the counter are touched only by agent-scope atomic
// operations, ordered by a wait on the wave's outstanding stores before the
// exchange and by the exchange's returned value before the merge's loads (the
// caller, the claim in paged_decode_balanced_kernel, explains why no release /
// acquire pair is used).
__device__ __forceinline__ int claim_last(unsigned long long* c, uint32_t epoch, uint32_t npieces) {
  unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (true) {
    const uint32_t ep = (uint32_t)(old >> 32), n = (uint32_t)old;
    const uint32_t n2 = (ep == epoch ? n : 0u) + 1u;
    const bool last = n2 >= npieces;
    const unsigned long long nw = ((unsigned long long)epoch << 32) | (last ? 0u : n2);
    unsigned long long expected = old;
    if (__hip_atomic_compare_exchange_strong(c, &expected, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return last ? 1 : 0;
    old = expected;
  }
}

// The result of query head hq of sequence s as partial slot sc.tail_part: the
// normalised output, its log-sum-exp (natural-log units of z) and weight 1.
// acc * inv is the output; m is the log2-domain max and l the exp-sum.
template <int NDT>
__device__ __forceinline__ void tail_emit(const DecodeScalars& sc, int s, int hq,
                                          const f32x4 (&acc)[NDT], float inv, float m, float l,
                                          int g) {
  const size_t pi = ((size_t)s * sc.Hq + hq) * sc.max_parts + sc.tail_part;
  float* o = sc.tail_out + pi * (16 * NDT) + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = acc[dt] * inv;
  if (g == 0) {
    sc.tail_max[pi] = m * kLn2 + logf(l);
    sc.tail_sum[pi] = 1.0f;
  }
}

// One wavefront merges the partial states of a shared pair (pieces of workers wa..wb,
// log2-domain maxima) in a single online pass over the pieces.  Lane (n, g) takes
// head n and dims 16 dt + 4 g + r, the layout the pieces were written in.  Reads
// are device-scope loads, matching the device-scope stores of the writers.
template <int QDT, int D>
__device__ void merge_pair(float* slot_out, float* slot_ml, uint8_t* __restrict__ out,
                           const DecodeScalars& sc, int s, int kvh, int u0, int wa, int wb,
                           int U, int NWe, int n, int g) {
  constexpr int NDT = D / 16;
  const int first_slot = worker_start(wa, U, NWe) != u0 ? 2 * wa + 1 : 2 * wa;
  const int hh = n < sc.G ? n : sc.G - 1;
  float M = -INFINITY, L = 0.0f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int w = wa; w <= wb; ++w) {
    const int slot = w == wa ? first_slot : 2 * w;
    float* ml = slot_ml + ((size_t)slot * sc.G + hh) * 2;
    const float m = __hip_atomic_load(ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float l = __hip_atomic_load(ml + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float* so = slot_out + ((size_t)slot * sc.G + hh) * D + 4 * g;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[dt][r] = __hip_atomic_load(so + 16 * dt + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float mn = fmaxf(M, m);
    const float a_old = __builtin_amdgcn_exp2f(M - mn);
    const float a_new = __builtin_amdgcn_exp2f(m - mn) * l;
    L = L * a_old + a_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[dt] = O[dt] * a_old + o[dt] * a_new;
    M = mn;
  }
  if (n < sc.G) {
    const float inv = 1.0f / L;
    if (sc.tail_part >= 0) {
      tail_emit<NDT>(sc, s, kvh * sc.G + n, O, inv, M, L, g);
    } else {
      const size_t orow = ((size_t)s * sc.Hq + (size_t)kvh * sc.G + n) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) store4(out, QDT, orow + 16 * dt, O[dt] * inv);
    }
  }
}

// where a worker is in the unit stream: unit u = chunk j of pair (s, kvh), the
// k-th unit of the worker's share; the chunk covers keys [st + 64 j, st + 64 j + 64)
// of which those below lo (a sliding window's) and from ctx on are masked
struct Pos {
  int u, s, kvh, j, nch, ctx, k, lo, st;
};

// FUSE: the worker that reads a pair's last chunk also appends the pair's newest
// token (position ctx - 1, from sc.k_new / sc.v_new): the row is requested with
// that chunk's loads, stored into its slot when the chunk is computed, and patched
// into the chunk's registers (never read back from the pool).
template <int KVT, int CT, int D, bool SMALLB, bool FUSE = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
paged_decode_balanced_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out, float* slot_out,
    float* slot_ml, unsigned long long* counters, const DecodeScalars sc) {
  using C = Cfg<KVT, CT, D>;
  constexpr bool kFp8 = (KVT == DT_FP8 || KVT == DT_I8);  // quantised: scaled 8-bit codes

  extern __shared__ int prefix[];  // [S + 1]
  __shared__ int tmp[kThreads];
  __shared__ u32x4 new_lds[kWaves][FUSE ? 2 * C::NC : 1];  // each wave's appended row (FUSE)

  unit_prefix(context_lens, sc.S, sc.ctx_off, sc.ctx_cap, sc.window, sc.Hkv, prefix, tmp);
  const int U = prefix[sc.S];
  if (blockIdx.x == 0) {  // sequences with an empty context own no unit: their output is zero
    for (int s0 = 0; s0 < sc.S; ++s0) {
      if (prefix[s0 + 1] != prefix[s0]) continue;
      if (sc.tail_part >= 0) {  // an empty partial: weight 0
        for (int i = threadIdx.x; i < sc.Hq * D; i += kThreads) {
          const int hq = i / D, d = i - hq * D;
          const size_t pi = ((size_t)s0 * sc.Hq + hq) * sc.max_parts + sc.tail_part;
          sc.tail_out[pi * D + d] = 0.0f;
          if (d == 0) {
            sc.tail_max[pi] = -INFINITY;
            sc.tail_sum[pi] = 0.0f;
          }
        }
      } else {
        for (int i = threadIdx.x; i < sc.Hq * D; i += kThreads)
          store_any(out, CT, (size_t)s0 * sc.Hq * D + i, 0.0f);
      }
      if constexpr (FUSE) {
        // a new token past a clamped context of 0 is still appended
        const int raw = max(context_lens[s0], 0);
        const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
        if (raw > 0)
          for (int h = wv; h < sc.Hkv; h += kWaves) {
            const u32x4 w = new_row_load<C>(sc, s0, h, ln);
            if (ln < 2 * C::NC) new_lds[wv][ln] = w;
            wave_lds_sync();
            new_row_store<C>(sc, k_pool, v_pool, block_table + (size_t)s0 * sc.W, new_lds[wv],
                             raw - 1, s0, h, ln);
            wave_lds_sync();
          }
      }
    }
  }
  const int NWe = min(sc.num_workers, U);
  // wave-uniform values go through readfirstlane so that the compiler keeps them,
  // and the addresses derived from them, scalar
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int w = blockIdx.x * kWaves + wave;
  if (w >= NWe) return;  // no barrier below this point
  const int u_begin = worker_start(w, U, NWe);
  const int u_end = worker_start(w + 1, U, NWe);

  auto clamp_ctx = [&](int s) {
    int c = context_lens[s];
    c = c < sc.ctx_off ? 0 : c - sc.ctx_off;
    return uniform(c > sc.ctx_cap ? sc.ctx_cap : c);
  };
  auto locate = [&](int u) {
    Pos p;
    p.u = u;
    p.s = uniform(find_seq(prefix, sc.S, u));
    const int pfx = uniform(prefix[p.s]);
    p.nch = uniform((prefix[p.s + 1] - pfx) / sc.Hkv);
    const int rel = u - pfx;
    p.kvh = rel / p.nch;
    p.j = rel - p.kvh * p.nch;
    p.ctx = clamp_ctx(p.s);
    p.lo = uniform(window_lo(p.ctx, sc.window));
    p.st = p.lo & ~15;
    return p;
  };
  // the unit after p, or p itself at the end of the share (its loads are then
  // repeated and never used)
  const int n_units = u_end - u_begin;
  auto first_pos = [&]() {
    Pos p = locate(u_begin);
    p.k = 0;
    return p;
  };
  // the unit after p, or p itself after the last one (its loads are then never
  // issued)
  auto advance = [&](Pos p) {
    if (p.k + 1 >= n_units) return p;
    ++p.u;
    ++p.k;
    if (++p.j < p.nch) return p;
    p.j = 0;
    if (++p.kvh < sc.Hkv) return p;
    p.kvh = 0;
    do {
      ++p.s;
    } while (prefix[p.s + 1] == prefix[p.s]);  // stops: unit p.u exists
    p.s = uniform(p.s);
    p.nch = uniform((prefix[p.s + 1] - prefix[p.s]) / sc.Hkv);
    p.ctx = clamp_ctx(p.s);
    p.lo = uniform(window_lo(p.ctx, sc.window));
    p.st = p.lo & ~15;
    return p;
  };
  // a piece ends at the last chunk of its pair or of the worker's share
  auto piece_ends = [&](const Pos& p) { return p.j == p.nch - 1 || p.k + 1 >= n_units; };
  auto trow_of = [&](const Pos& p) { return block_table + (size_t)p.s * sc.W + sc.tbl_off; };

  // FUSE: append the newest token of the pair whose last chunk is at p (the row
  // w was requested with that chunk) and, when that token is visible, patch it
  // into the chunk's registers
  auto append_at = [&](const Pos& p, const u32x4& w, Chunk<C>& ch, int base) {
    if constexpr (FUSE) {
      u32x4* row = new_lds[wave];
      if (lane < 2 * C::NC) row[lane] = w;
      wave_lds_sync();
      const int raw = max(context_lens[p.s], 0);
      new_row_store<C>(sc, k_pool, v_pool, trow_of(p), row, raw - 1, p.s, p.kvh, lane);
      if (raw == p.ctx) {
        patch_k<C>(ch.k, row, p.ctx - 1 - base, n, g);
        patch_v<C>(ch.v, row, p.ctx - 1 - base, n, g);
      }
    }
  };

  State<C> st;
  state_init(st);
  typename C::QOp qop[C::NQ];
  Pos pc = first_pos();
  load_q<C>(qop, q, pc.s, pc.kvh, sc, n, g);
  q_live<C>(qop, qop, n < sc.G);
  int piece_j0 = pc.j, piece_u0 = pc.u;

  // Shared pairs whose piece this worker has published but not yet counted: at
  // most the first and the last piece of the share.  The count (a release of the
  // piece's stores) comes at the end of the share, where no prefetched chunk is in
  // flight: a release waits for all of the wave's outstanding memory operations,
  // loads included, so an earlier count would drain the pipeline.
  int pend_s0 = 0, pend_k0 = 0, pend_n0 = 0, pend_s1 = 0, pend_k1 = 0, pend_n1 = 0;
  int n_pend = 0;
  auto claim = [&](int ps, int pk, int pn) {
    ps = uniform(ps);
    pk = uniform(pk);
    pn = uniform(pn);
    const int seg_first = uniform(prefix[ps]) + pk * pn;
    const int wa = worker_of(seg_first, U, NWe);
    const int wb = worker_of(seg_first + pn - 1, U, NWe);
    // Publish, then claim.  The partial states were stored with agent-scope atomic
    // stores (coherent across the XCDs' L2 caches); the wait below holds the claim
    // until every store of the wave has completed at that scope, and the compiler
    // barriers keep the compiler from moving memory operations across the claim.
    // The winner's merge loads are agent-scope atomic loads issued only after the
    // exchange has returned.  (A release exchange plus an acquire fence would say
    // the same in the language's memory model, but on this chip they add a
    // write-back of the whole L2 before every claim and an invalidation of it in
    // every merge; measured, that slows the balanced decode by 40-50%.)
    int last = 0;
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (lane == 0)
      last = claim_last(counters + (size_t)ps * sc.Hkv + pk, sc.epoch, (uint32_t)(wb - wa + 1));
    last = uniform(last);  // lane 0's answer
    asm volatile("" ::: "memory");
    if (last) merge_pair<CT, D>(slot_out, slot_ml, out, sc, ps, pk, seg_first, wa, wb, U, NWe, n, g);
  };
  auto claim_pending = [&]() {
    if (n_pend > 0) claim(pend_s0, pend_k0, pend_n0);
    if (n_pend > 1) claim(pend_s1, pend_k1, pend_n1);
    n_pend = 0;
  };

  // close the piece that ends with chunk pc: whole pairs go straight to `out`,
  // shared ones to this worker's slot, merged by the last of their workers
  auto finish_piece = [&](const Pos& p) {
    const float lw = sum_groups(st.l);
    const bool whole = (piece_j0 == 0 && p.j == p.nch - 1);
    if (whole) {
      if (n < sc.G) {
        const float inv = 1.0f / lw;
        if (sc.tail_part >= 0) {
          tail_emit<C::NDT>(sc, p.s, p.kvh * sc.G + n, st.acc, inv, st.m, lw, g);
        } else {
          const size_t orow = ((size_t)p.s * sc.Hq + (size_t)p.kvh * sc.G + n) * D + 4 * g;
#pragma unroll
          for (int dt = 0; dt < C::NDT; ++dt) store4(out, CT, orow + 16 * dt, st.acc[dt] * inv);
        }
      }
    } else {
      // Publish the partial state with device-scope stores (coherent across the
      // XCDs' L2 caches without a cache-wide write-back); no cache-wide fence is
      // needed on either side.
      // slot 2w: the piece that starts the worker's share; 2w+1: the one that ends it
      const int slot = 2 * w + (piece_u0 == u_begin ? 0 : 1);
      if (n < sc.G) {
        const float inv = 1.0f / lw;
        float* so = slot_out + ((size_t)slot * sc.G + n) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __hip_atomic_store(so + 16 * dt + r, st.acc[dt][r] * inv, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (g == 0) {
          float* ml = slot_ml + ((size_t)slot * sc.G + n) * 2;
          __hip_atomic_store(ml, st.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // log2
          __hip_atomic_store(ml + 1, lw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // counted at the end of the share (claim_pending)
      if (n_pend == 0) {
        pend_s0 = p.s;
        pend_k0 = p.kvh;
        pend_n0 = p.nch;
      } else {
        pend_s1 = p.s;
        pend_k1 = p.kvh;
        pend_n1 = p.nch;
      }
      ++n_pend;
    }
    state_init(st);
  };

  if constexpr (SMALLB) {
    while (true) {
      const Pos pn = advance(pc);
      Chunk<C> ch;
      float ks[16], vs[16];
      const int base = pc.st + 64 * pc.j;
      load_small<C>(ch, ks, vs, k_pool, v_pool, k_scale, v_scale, trow_of(pc), base, pc.ctx,
                    pc.kvh, sc, n, g, pc.lo);
      if constexpr (FUSE)
        if (pc.j == pc.nch - 1) append_at(pc, new_row_load<C>(sc, pc.s, pc.kvh, lane), ch, base);
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, ch.k, qop);
      chunk_softmax_pv<C, KVT, CT>(st, S, ch.v, sc.scale_log2, ks, vs, min(64, pc.ctx - base),
                                   g, 64, pc.lo - base);
      const bool done = pc.k + 1 >= n_units;
      if (done || piece_ends(pc)) {
        finish_piece(pc);
        if (done) break;
        if (pn.s != pc.s || pn.kvh != pc.kvh) {
          load_q<C>(qop, q, pn.s, pn.kvh, sc, n, g);
          q_live<C>(qop, qop, n < sc.G);
        }
        piece_j0 = pn.j;
        piece_u0 = pn.u;
      }
      pc = pn;
    }
  } else {
    // Software pipeline over a ring of NBUF chunk buffers: on entry to a stage
    // the loads of the next NBUF-2 chunks are in flight; the stage requests
    // chunk +NBUF-1 into the buffer freed by the previous stage, then computes
    // the current one.  The table entries run one chunk ahead of the requests.
    // The next pair's q is requested a whole stage before its first chunk is
    // computed.
    constexpr int NB = C::NBUF;
    Chunk<C> R[NB];
    Pos pp[NB];          // pp[k]: position of the chunk k stages ahead of pc
    float ksr[NB][16], vsr[NB][16];
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int i = 0; i < 16; ++i) ksr[k][i] = vsr[k][i] = 1.0f;
    pp[0] = pc;
    u32x4 nwr[NB];  // FUSE: the new row of the pair whose last chunk is in buffer k
    auto issue = [&](Chunk<C>& dst, const Pos& p, const Pages& pg, float (&ks)[16],
                     float (&vs)[16], u32x4& nw) {
      if constexpr (FUSE)
        if (p.j == p.nch - 1) nw = new_row_load<C>(sc, p.s, p.kvh, lane);
      issue_k<C>(dst.k, k_pool, pg, p.kvh, sc, n, g);
      issue_v<C>(dst.v, v_pool, pg, p.kvh, sc, n, g);
      if constexpr (kFp8) chunk_scales(ks, vs, k_scale, v_scale, pg, p.kvh, sc, g);
    };
    auto pages_at = [&](const Pos& p) {
      return pages_of(trow_of(p), p.st + 64 * p.j, p.ctx, sc);
    };
#pragma unroll
    for (int k = 0; k + 1 < NB; ++k) {
      if (k > 0) pp[k] = advance(pp[k - 1]);
      issue(R[k], pp[k], pages_at(pp[k]), ksr[k], vsr[k], nwr[k]);
    }
    pp[NB - 1] = advance(pp[NB - 2]);
    Pages en = pages_at(pp[NB - 1]);
    bool done = false;
    // The q of the pair that starts at pp[1] is requested a whole stage before its
    // first chunk is computed (into qn, moved to qop when the pair starts)
    typename C::QOp qn[C::NQ];
    auto switch_next = [&]() {
      return pp[0].k + 1 < n_units && (pp[1].s != pp[0].s || pp[1].kvh != pp[0].kvh);
    };
    if (switch_next()) load_q<C>(qn, q, pp[1].s, pp[1].kvh, sc, n, g);
    // stage: chunk pp[0] sits in R[c]; chunk pp[NB-1] goes to R[f]
    auto stage = [&](Chunk<C>& cur, Chunk<C>& fill, int c, int f) {
      const Pos& p0 = pp[0];
      const bool last = p0.k + 1 >= n_units;
      const bool fetch = pp[NB - 1].k != pp[NB - 2].k;  // a chunk that is not a repeat
      Pages en2 = en;
      Pos pnext = pp[NB - 1];
      if (fetch) {
        issue(fill, pp[NB - 1], en, ksr[f], vsr[f], nwr[f]);
        pnext = advance(pp[NB - 1]);
        en2 = pages_at(pnext);
      }
      issue_point();
      const int base0 = p0.st + 64 * p0.j;
      if constexpr (FUSE)
        if (p0.j == p0.nch - 1) append_at(p0, nwr[c], cur, base0);
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, cur.k, qop);
      issue_point();
      const bool new_pair = !last && (pp[1].s != p0.s || pp[1].kvh != p0.kvh);
      issue_point();
      v_rows_to_tiles<C>(cur.v);
      chunk_softmax_pv<C, KVT, CT>(st, S, cur.v, sc.scale_log2, ksr[c], vsr[c],
                                   min(64, p0.ctx - base0), g, 64, p0.lo - base0);
      issue_point();
      if (last || piece_ends(p0)) {
        finish_piece(p0);
        piece_j0 = pp[1].j;
        piece_u0 = pp[1].u;
        if (new_pair) q_live<C>(qop, qn, n < sc.G);
      }
      done = last;
#pragma unroll
      for (int k = 0; k + 1 < NB; ++k) pp[k] = pp[k + 1];
      pp[NB - 1] = pnext;
      en = en2;
      if (!done && switch_next()) load_q<C>(qn, q, pp[1].s, pp[1].kvh, sc, n, g);
    };
    while (true) {
      if constexpr (NB == 3) {
        stage(R[0], R[2], 0, 2);
        if (done) break;
        stage(R[1], R[0], 1, 0);
        if (done) break;
        stage(R[2], R[1], 2, 1);
        if (done) break;
      } else {
        stage(R[0], R[1], 0, 1);
        if (done) break;
        stage(R[1], R[0], 1, 0);
        if (done) break;
      }
    }
  }
  if (n_pend) claim_pending();
}

// =================================================================================
// Split-KV reduce for fixed partitions: one workgroup per (query head, sequence).
// A sequence's partitions are those of its context clamped to ctx_cap (the clamp
// the decode applied; the decode writes no partition past it).  Without
// context_lens every one of the max_parts slots is merged (empty ones, with
// exp-sum 0, weigh nothing).
// =================================================================================
template <int D>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, const int32_t* __restrict__ context_lens,
    uint8_t* __restrict__ out, int out_dtype, int Hq, int part_size, int max_parts, int ctx_cap) {
  extern __shared__ float w_lds[];  // [max_parts] merge weights
  __shared__ float red[kWaves];
  __shared__ float o_lds[kWaves][D];
  const int h = blockIdx.x, s = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int np = max_parts;
  if (context_lens) {
    const long long cap = min((long long)max_parts * part_size, (long long)ctx_cap);
    long long ctx = context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    np = (int)((ctx + part_size - 1) / part_size);
  }
  const size_t orow = ((size_t)s * Hq + h) * D;
  if (np == 0) {
    for (int d = threadIdx.x; d < D; d += kThreads) store_any(out, out_dtype, orow + d, 0.0f);
    return;
  }
  const size_t base = ((size_t)s * Hq + h) * max_parts;

  float m = -INFINITY;
  for (int i = threadIdx.x; i < np; i += kThreads) m = fmaxf(m, part_max[base + i]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  float lsum = 0.0f;
  for (int i = threadIdx.x; i < np; i += kThreads) {
    const float l = part_sum[base + i];
    const float w = l > 0.0f ? __builtin_amdgcn_exp2f((part_max[base + i] - M) * kLog2e) * l : 0.0f;
    w_lds[i] = w;
    lsum += w;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  const float L = (red[0] + red[1]) + (red[2] + red[3]);

  constexpr int PER = D / 64;  // output elements per lane
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
  for (int i = wave; i < np; i += kWaves) {
    const float w = w_lds[i];
    const float* po = part_out + (base + i) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, po[lane + 64 * k], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) o_lds[wave][lane + 64 * k] = acc[k];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kThreads) {
    const float o = (o_lds[0][d] + o_lds[1][d]) + (o_lds[2][d] + o_lds[3][d]);
    store_any(out, out_dtype, orow + d, L > 0.0f ? o / L : 0.0f);
  }
}

// A merge of every one of a few slots per (sequence, query head) (the shared-prefix
// decode's): one wavefront per row, lane L taking dims L, L + 64; the same weights
// as split_reduce_kernel, exp(m_i - M) l_i.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_slots_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, uint8_t* __restrict__ out, int out_dtype, int n_rows,
    int max_parts) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + uniform(threadIdx.x >> 6);  // s * H_q + h
  if (row >= n_rows) return;
  const size_t base = (size_t)row * max_parts;
  float M = -INFINITY;
  for (int i = 0; i < max_parts; ++i) M = fmaxf(M, part_max[base + i]);
  float L = 0.0f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
  for (int i = 0; i < max_parts; ++i) {
    const float l = part_sum[base + i];
    const float w = l > 0.0f ? __builtin_amdgcn_exp2f((part_max[base + i] - M) * kLog2e) * l : 0.0f;
    L += w;
    const float* po = part_out + (base + i) * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, po[lane + 64 * k], acc[k]);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k)
    store_any(out, out_dtype, (size_t)row * D + lane + 64 * k, L > 0.0f ? acc[k] / L : 0.0f);
}

// =================================================================================
// Kernel C: the shared prefix of a batch, read once per kv head
// =================================================================================
// Every sequence of the batch holds its first shared_len tokens in the same
// physical blocks (the caller's table rows agree there; row 0 is read).  A
// wavefront takes one kv head, one slice of the prefix and a tile of 16 query
// columns, here 16/G sequences x the G heads of that kv head, so one K/V chunk
// feeds the scores of 16/G sequences instead of one: the product S^T = K . Q^T
// has distinct queries in every column even for G = 1.  Column (sequence s,
// head h) sees the keys below min(ctx_s, shared_len).  The slice's state goes to
// partial slot `slice` of (s, query head); the tails and the merge follow.
struct PrefixGrid {
  int shared_len;
  int n_slices;    // slices of the prefix (partial slots 0 .. n_slices-1)
  int slice_chunks;  // 64-token chunks per slice
  int spt;         // sequences per column tile: 16 / G
  int n_tiles;     // column tiles: ceil(S / spt)
  int wg_per_group;  // workgroups per (kv head, slice): ceil(n_tiles / 4)
  int n_groups;    // Hkv * n_slices
};

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return uniform(x);
}

template <int KVT, int CT, int D, bool SMALLB>
__global__ __launch_bounds__(kThreads) void shared_prefix_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, float* __restrict__ part_out,
    float* __restrict__ part_max, float* __restrict__ part_sum, const DecodeScalars sc,
    const PrefixGrid pg) {
  using C = Cfg<KVT, CT, D>;
  constexpr bool kFp8 = (KVT == DT_FP8 || KVT == DT_I8);
  // The workgroups of one (kv head, slice) share a residue of blockIdx mod 8, so
  // they run on one XCD and read the slice's pages through one L2.
  const int x = blockIdx.x;
  const int grp = (x >> 3) / pg.wg_per_group * 8 + (x & 7);
  if (grp >= pg.n_groups) return;  // no barrier in this kernel
  const int kvh = grp / pg.n_slices, slice = grp - kvh * pg.n_slices;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int tile = ((x >> 3) % pg.wg_per_group) * kWaves + wave;
  if (tile >= pg.n_tiles) return;

  const int sl = n / sc.G, h = n - sl * sc.G;
  const int s = tile * pg.spt + sl;
  const bool live = sl < pg.spt && s < sc.S;
  int lim = 0;  // keys of the prefix this column sees
  if (live) {
    int c = context_lens[s];
    c = c < 0 ? 0 : (c > sc.ctx_cap ? sc.ctx_cap : c);
    lim = min(c, pg.shared_len);
  }
  const int lim_tile = wave_max_int(lim);
  const int t_begin = slice * pg.slice_chunks * 64;
  const int t_end = min(t_begin + pg.slice_chunks * 64, lim_tile);

  typename C::QOp qop[C::NQ];
  load_q_row<C>(qop, q + ((size_t)(live ? s : 0) * sc.Hq + (size_t)kvh * sc.G + h) * D * C::QEB,
                g);
  q_live<C>(qop, qop, live);
  State<C> st;
  state_init(st);
  const int32_t* trow = block_table;  // row 0: the shared blocks
  const int cnt = t_end > t_begin ? (t_end - t_begin + 63) >> 6 : 0;
  auto base_of = [&](int i) { return t_begin + 64 * min(i, cnt - 1); };

  if constexpr (SMALLB) {
    for (int i = 0; i < cnt; ++i) {
      const int base = base_of(i);
      Chunk<C> ch;
      float ks[16], vs[16];
      load_small<C>(ch, ks, vs, k_pool, v_pool, k_scale, v_scale, trow, base, t_end, kvh, sc, n, g);
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, ch.k, qop);
      chunk_softmax_pv<C, KVT, CT, true>(st, S, ch.v, sc.scale_log2, ks, vs,
                                         min(64, t_end - base), g, lim - base);
    }
  } else if (cnt > 0) {
    // the single-buffered pipeline of paged_decode_kernel
    Chunk<C> R;
    float ks0[16], vs0[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ks0[i] = vs0[i] = 1.0f;
    {
      const Pages p0 = pages_of(trow, base_of(0), t_end, sc);
      issue_k<C, false>(R.k, k_pool, p0, kvh, sc, n, g);
      if constexpr (kFp8) chunk_scales(ks0, vs0, k_scale, v_scale, p0, kvh, sc, g);
      issue_v<C, false>(R.v, v_pool, p0, kvh, sc, n, g);
    }
    Pages p1 = pages_of(trow, base_of(1), t_end, sc);
    for (int i = 0; i < cnt; ++i) {
      const int b0 = base_of(i);
      const bool more = i + 1 < cnt;
      f32x4 S[4];
      chunk_qk<C, KVT, CT>(S, R.k, qop);
      issue_point();
      float ks1[16], vs1[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) ks1[k] = vs1[k] = 1.0f;
      Pages p2 = p1;
      if (more) {
        issue_k<C, false>(R.k, k_pool, p1, kvh, sc, n, g);
        if constexpr (kFp8) chunk_scales(ks1, vs1, k_scale, v_scale, p1, kvh, sc, g);
        p2 = pages_of(trow, base_of(i + 2), t_end, sc);
      }
      issue_point();
      v_rows_to_tiles<C>(R.v);
      chunk_softmax_pv<C, KVT, CT, true>(st, S, R.v, sc.scale_log2, ks0, vs0,
                                         min(64, t_end - b0), g, lim - b0);
      issue_point();
      if (more) issue_v<C, false>(R.v, v_pool, p1, kvh, sc, n, g);
      issue_point();
      p1 = p2;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        ks0[k] = ks1[k];
        vs0[k] = vs1[k];
      }
    }
  }

  // the slice's state of column (s, h): normalised output, max (natural-log units
  // of z) and exp-sum; a column that saw no key leaves an empty state (weight 0)
  const float lw = sum_groups(st.l);
  if (live) {
    const size_t pi = ((size_t)s * sc.Hq + (size_t)kvh * sc.G + h) * sc.max_parts + slice;
    const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;
    float* o = part_out + pi * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = st.acc[dt] * inv;
    if (g == 0) {
      part_max[pi] = lw > 0.0f ? st.m * kLn2 : -INFINITY;
      part_sum[pi] = lw;
    }
  }
}

// ---------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------
namespace {

template <int KVT, int CT, int D, bool SMALLB>
int launch_t(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  if (p.prefix) {
    PrefixGrid pg;
    pg.shared_len = p.shared_len;
    pg.n_slices = p.n_slices;
    pg.slice_chunks = p.slice_chunks;
    pg.spt = 16 / sc.G;
    pg.n_tiles = (p.num_seqs + pg.spt - 1) / pg.spt;
    pg.wg_per_group = (pg.n_tiles + kWaves - 1) / kWaves;
    pg.n_groups = p.num_kv_heads * p.n_slices;
    const long long wgs = (long long)(pg.n_groups + 7) / 8 * 8 * pg.wg_per_group;
    if (pg.n_groups < 1 || wgs >= (1LL << 31)) return -3;
    hipLaunchKernelGGL((shared_prefix_kernel<KVT, CT, D, SMALLB>), dim3((unsigned)wgs),
                       dim3(kThreads), 0, st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                       (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                       p.context_lens, p.part_out, p.part_max, p.part_sum, sc, pg);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (p.balanced && p.fuse) {  // decode fused with the append: 16-bit pools only
    if constexpr (KVT == CT && (KVT == DT_F16 || KVT == DT_BF16)) {
      const size_t lds = ((size_t)p.num_seqs + 1) * sizeof(int);
      dim3 grid((sc.num_workers + kWaves - 1) / kWaves);
      hipLaunchKernelGGL((paged_decode_balanced_kernel<KVT, CT, D, SMALLB, true>), grid,
                         dim3(kThreads), lds, st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                         (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                         p.context_lens, (uint8_t*)p.out, p.part_out, p.part_max, p.counters,
                         sc);
      return hipGetLastError() == hipSuccess ? 0 : -5;
    } else {
      return -3;
    }
  }
  if (p.balanced) {
    const size_t lds = ((size_t)p.num_seqs + 1) * sizeof(int);
    dim3 grid((sc.num_workers + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((paged_decode_balanced_kernel<KVT, CT, D, SMALLB>), grid, dim3(kThreads),
                       lds, st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                       (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                       p.context_lens, (uint8_t*)p.out, p.part_out, p.part_max, p.counters, sc);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (p.max_parts > 65535) return -3;  // grid z (the reduce takes at most 8192)
  const dim3 grid(p.num_kv_heads, p.num_seqs, p.max_parts);
  if (p.fuse) {  // decode fused with the append: 16-bit pools only
    if constexpr (KVT == CT && (KVT == DT_F16 || KVT == DT_BF16)) {
      hipLaunchKernelGGL((paged_decode_kernel<KVT, CT, D, SMALLB, true>), grid, dim3(kThreads), 0,
                         st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                         (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                         p.context_lens, (uint8_t*)p.out, p.part_out, p.part_max, p.part_sum, sc);
      return hipGetLastError() == hipSuccess ? 0 : -5;
    } else {
      return -3;
    }
  }
  // 8-bit pools with per-token scales: an instantiation of their own, so that the
  // others keep 8 scale registers per chunk in flight (and two waves per SIMD)
  if constexpr (Elem<KVT>::bytes == 1 && !SMALLB) {
    if (sc.scale_mode == SCALE_TOKEN) {
      hipLaunchKernelGGL((paged_decode_kernel<KVT, CT, D, SMALLB, false, true>), grid,
                         dim3(kThreads), 0, st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                         (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                         p.context_lens, (uint8_t*)p.out, p.part_out, p.part_max, p.part_sum,
                         sc);
      return hipGetLastError() == hipSuccess ? 0 : -5;
    }
  }
  hipLaunchKernelGGL((paged_decode_kernel<KVT, CT, D, SMALLB>), grid, dim3(kThreads), 0, st,
                     (const uint8_t*)p.q, (const uint8_t*)p.k_pool, (const uint8_t*)p.v_pool,
                     p.k_scale, p.v_scale, p.block_table, p.context_lens, (uint8_t*)p.out,
                     p.part_out, p.part_max, p.part_sum, sc);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int KVT, int CT, int D>
int pick_b(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  return p.block_size >= 16 ? launch_t<KVT, CT, D, false>(p, sc, st)
                            : launch_t<KVT, CT, D, true>(p, sc, st);
}

template <int KVT, int CT>
int pick_d(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  if (p.head_dim == 64) return pick_b<KVT, CT, 64>(p, sc, st);
  if (p.head_dim == 128) return pick_b<KVT, CT, 128>(p, sc, st);
  return -3;
}

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

}  // namespace

namespace {

DecodeScalars scalars_of(const DecodeLaunch& p) {
  DecodeScalars sc;
  sc.W = p.max_blocks_per_seq;
  sc.ctx_cap = p.ctx_cap;
  sc.S = p.num_seqs;
  sc.Hq = p.num_q_heads;
  sc.Hkv = p.num_kv_heads;
  sc.G = p.num_q_heads / p.num_kv_heads;
  sc.blog2 = log2_exact(p.block_size);
  sc.num_blocks = p.num_blocks;
  sc.part_size = p.part_size;
  sc.max_parts = p.max_parts;
  sc.split = p.split;
  sc.out_dtype = p.q_dtype;
  sc.num_workers = p.num_workers;
  sc.epoch = p.epoch;
  sc.scale_mode = p.scale_mode;
  sc.scale_log2 = p.scale * kLog2e;
  sc.ctx_off = p.ctx_off;
  sc.tbl_off = p.tbl_off;
  sc.tail_part = p.tail_part;
  sc.tail_out = p.tail_out;
  sc.tail_max = p.tail_max;
  sc.tail_sum = p.tail_sum;
  sc.window = p.window;
  sc.bstride = p.bstride;
  sc.k_new = static_cast<const uint8_t*>(p.k_new);
  sc.v_new = static_cast<const uint8_t*>(p.v_new);
  sc.slot_out = p.slot_out;
  sc.lpt = !p.balanced && !p.prefix && p.num_seqs <= kThreads;
  return sc;
}

}  // namespace

int launch_decode(const DecodeLaunch& p, hipStream_t st) {
  const DecodeScalars sc = scalars_of(p);
  if (sc.blog2 < 0 || p.block_size > 64 || sc.G > 16) return -3;
  const int kv = p.kv_dtype, qd = p.q_dtype;
  if (kv == DT_F32 && qd == DT_F32) return pick_d<DT_F32, DT_F32>(p, sc, st);
  if (kv == DT_F16 && qd == DT_F16) return pick_d<DT_F16, DT_F16>(p, sc, st);
  if (kv == DT_BF16 && qd == DT_BF16) return pick_d<DT_BF16, DT_BF16>(p, sc, st);
  if (kv == DT_FP8 && qd == DT_BF16) return pick_d<DT_FP8, DT_BF16>(p, sc, st);
  if (kv == DT_FP8 && qd == DT_F16) return pick_d<DT_FP8, DT_F16>(p, sc, st);
  if (kv == DT_I8 && qd == DT_BF16) return pick_d<DT_I8, DT_BF16>(p, sc, st);
  if (kv == DT_I8 && qd == DT_F16) return pick_d<DT_I8, DT_F16>(p, sc, st);
  return -3;
}

// ---- resident-worker capacity (device property x kernel occupancy), cached -------
namespace {

template <int KVT, int CT, int D, bool SMALLB>
int blocks_per_cu() {
  static const int v = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&paged_decode_balanced_kernel<KVT, CT, D, SMALLB>),
            kThreads, 4096) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  return v;
}

template <int KVT, int CT>
int bpc(int D, int B) {
  if (D == 64) return B >= 16 ? blocks_per_cu<KVT, CT, 64, false>() : blocks_per_cu<KVT, CT, 64, true>();
  return B >= 16 ? blocks_per_cu<KVT, CT, 128, false>() : blocks_per_cu<KVT, CT, 128, true>();
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace

int balanced_worker_capacity(int kv, int qd, int D, int block_size) {
  int n = 1;
  if (kv == DT_F32) n = bpc<DT_F32, DT_F32>(D, block_size);
  else if (kv == DT_F16) n = bpc<DT_F16, DT_F16>(D, block_size);
  else if (kv == DT_BF16) n = bpc<DT_BF16, DT_BF16>(D, block_size);
  else if (kv == DT_I8) n = qd == DT_F16 ? bpc<DT_I8, DT_F16>(D, block_size)
                                         : bpc<DT_I8, DT_BF16>(D, block_size);
  else if (qd == DT_F16) n = bpc<DT_FP8, DT_F16>(D, block_size);
  else n = bpc<DT_FP8, DT_BF16>(D, block_size);
  return device_cus() * n * kWaves;
}

int launch_split_reduce(const ReduceLaunch& p, hipStream_t st) {
  if (p.max_parts > kMaxPartitions) return -3;
  if (!p.context_lens && p.max_parts <= 64) {  // every slot, few of them: a wavefront per row
    const long long rows = (long long)p.num_seqs * p.num_q_heads;
    dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    if (p.head_dim == 64)
      hipLaunchKernelGGL(merge_slots_kernel<64>, grid, dim3(kThreads), 0, st, p.part_out,
                         p.part_max, p.part_sum, (uint8_t*)p.out, p.out_dtype, (int)rows,
                         p.max_parts);
    else if (p.head_dim == 128)
      hipLaunchKernelGGL(merge_slots_kernel<128>, grid, dim3(kThreads), 0, st, p.part_out,
                         p.part_max, p.part_sum, (uint8_t*)p.out, p.out_dtype, (int)rows,
                         p.max_parts);
    else
      return -3;
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  dim3 grid(p.num_q_heads, p.num_seqs);
  size_t lds = (size_t)p.max_parts * sizeof(float);
  if (p.head_dim == 64)
    hipLaunchKernelGGL(split_reduce_kernel<64>, grid, dim3(kThreads), lds, st, p.part_out,
                       p.part_max, p.part_sum, p.context_lens, (uint8_t*)p.out, p.out_dtype,
                       p.num_q_heads, p.part_size, p.max_parts, p.ctx_cap);
  else if (p.head_dim == 128)
    hipLaunchKernelGGL(split_reduce_kernel<128>, grid, dim3(kThreads), lds, st, p.part_out,
                       p.part_max, p.part_sum, p.context_lens, (uint8_t*)p.out, p.out_dtype,
                       p.num_q_heads, p.part_size, p.max_parts, p.ctx_cap);
  else
    return -3;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace pkv
