// prefill.hip — chunked prefill over the paged cache on the matrix cores.
//
// Method: "03 | PagedAttention and the KV-cache memory system", §4 — prefill
// reuses flash-style tiling over the paged cache, handed the block table; a
// query row i of an n-token chunk sits at position a = ctx - n + i and sees the
// keys 0..a (the whole cache, causal inside the chunk).
//
// Work cut: one workgroup (4 waves; 8 for fp8 pools of 128 dims) per (query block,
// kv head, sequence).  A "row" is a (query token, query head) pair; a 16-row tile
// holds 16/G tokens x the G heads of the kv head, so every K/V tile is reused by all
// G heads.  Each wave owns two row tiles, the workgroup 128/G tokens (256/G with 8
// waves, which share each staged chunk: half the staging per wave and half the
// pool reads per query, at the same two waves per SIMD).  The query blocks of one
// (sequence, kv head) pair run on one XCD, so their shared K/V hits in its L2.
//
// Per 64-key chunk the workgroup stages K and V once into LDS, widened to 16
// bits (fp8 E4M3 -> bf16 for K, -> f16 for V; both exact), double-buffered,
// with the pool loads issued two chunks ahead.  Then every wave computes, per
// row tile, the same products as decode:
//   S^T = K . Q^T   16x16x32 bf16 MFMA, K rows from LDS, q columns in registers;
//   O^T = V^T . P^T 16x16x32 MFMA in the V staging type, P from the lane's own
//                   scores (tile T row n is key 16 T + n, so S^T leaves lane
//                   (n, g) the keys 16 T + 4 g + r, the k-slots P.V needs).
// The softmax first takes a chunk's p against each row's current reference and
// computes the chunk's maxima only where that would leave the P operand's range.
// fp8 pools: K's page scale multiplies the scores; V's multiplies V as it is
// widened to f16 in LDS; P.V runs in f16 (P keeps 11 significant bits) and the
// softmax sum adds the same f16 values of P.  bf16 pools: P.V in bf16 with P split
// into hi + lo bf16 terms.
//
// LDS rows are XOR-swizzled in 16-byte units (K rows by token mod 16, V rows by
// dim / 2 mod 8) so that the lanes of one LDS cycle hit distinct banks, for the
// staging writes and for the operand reads.  The chunk's block ids and fp8
// scales come from a small LDS window, refilled every 32 chunks, so that no
// scalar load is outstanding when the loop waits on LDS (both share a counter).
#include "device.hpp"
#include "internal.hpp"
#include "prefill.hpp"
#include "tile.hpp"

#include <math.h>

namespace pkv {

struct PrefillScalars {
  int W;           // max_blocks_per_seq
  int S, Hq, Hkv, G;
  int blog2, num_blocks, ctx_cap;
  int causal;
  int nqb;         // query blocks per pair (grid)
  int pairs;       // (sequence, kv head) pairs; prefix mode: (kv head, slice) pairs
  float scale_log2;
  long long bstride;  // 16-byte units from one block to the next in each pool
  // prefix mode: slices of the shared prefix and the partial states they leave
  int shared_len, n_slices, slice_chunks, max_parts;
  float* part_out;
  float* part_max;
  float* part_sum;
};

// Workgroups are dealt to the XCDs round robin by id (id mod 8), and each XCD has
// its own L2.  The query blocks of one (sequence, kv head) pair read the same K/V
// chunks, so they are given ids of one residue mod 8: pair p lives on XCD p mod 8
// as that XCD's (p / 8)-th pair, and its query blocks take consecutive slots there.
constexpr int kXcds = 8;

constexpr int kPfThreads = 256;

template <int KVT, int D, int NT_ = kPfThreads>
struct PCfg {
  static constexpr int KV = KVT;                    // pool element type
  static constexpr int Dim = D;
  static constexpr int NT = NT_;                    // threads per workgroup
  static constexpr int EB = Elem<KVT>::bytes;       // pool bytes per element
  static constexpr int X = 16 / EB;                 // K dims per pool piece
  static constexpr int NC = D / X;                  // K pieces per token
  static constexpr int TP = 16 / EB;                // V tokens per pool piece
  static constexpr int NKS = D / 32;                // k-steps of S^T
  static constexpr int NDT = D / 16;                // dim tiles of O^T
  static constexpr int NR = 2;                      // row tiles per wave
  static constexpr int KUNITS = D * 2 / 16;         // 16-byte units per staged K row
  static constexpr int KROW = D * 2;                // staged K row (one token, bf16)
  static constexpr int VROW = 64 * 2;               // staged V row (one dim, 64 tokens)
  static constexpr int KBUF = 64 * KROW;
  static constexpr int VBUF = D * VROW;
  static constexpr int QT = KVT == DT_F16 ? DT_F16 : DT_BF16;  // q, staged K and the output
  static constexpr int PT = KVT == DT_BF16 ? DT_BF16 : DT_F16;  // type of the P.V product
  static constexpr bool SPLIT = (PT == DT_BF16);                // P as hi + lo
  // two resident workgroups per CU where the registers allow it (LDS holds two)
  static constexpr int WPE = (KVT == DT_BF16 && D == 128) ? 1 : 2;
  // chunks of pool bytes held in registers: two (loads issued two chunks ahead) where
  // they are small; one (a chunk ahead) for 16-bit pools of 128 dims, whose 32
  // registers per chunk would not leave two workgroups per CU
  static constexpr int NRAW = (EB == 2 && D == 128) ? 1 : 2;
  static constexpr int KP = 64 * NC / NT;           // K pool pieces per thread per chunk
  static constexpr int VP = D * (64 / TP) / NT;     // V pool pieces per thread
  static_assert(KP >= 1 && VP >= 1, "chunk too small for the workgroup");
};

// pool bytes of one chunk held by a thread between its load and its staging
template <class C>
struct Raw {
  u32x4 k[C::KP];
  u32x4 v[C::VP];
};

__device__ __forceinline__ int pick4(const int (&v)[4], int i) {
  return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
}

// Pieces of a chunk and who loads them.  Every wavefront loads from one 16-token
// tile per piece index, so the page is wave-uniform: its base address is scalar
// and each lane adds an offset that is the same for every chunk (recomputed only
// in a chunk that runs past the context, whose tokens are clamped).
//   K piece i of thread (w, l): token 16 (w % 4) + l % 16, dims [c X, c X + X) with
//     c = l / 16 + 4 (w / 4) + 4 (NT / 256) i (tile w % 4; NT threads per workgroup).
//   V piece i: vp = NT i + 64 w + l covers tokens [TP p, TP p + TP) of dim
//     vp % D, p = vp / D (tile TP p / 16, the same for the whole wavefront as
//     64 divides D).  A V page is [B/TP][D][TP] (block_size >= 16 >= TP), so the
//     piece of tokens [t, t + TP) of dim d is the 16 bytes at (t/TP * D + d) * 16.
template <class C>
struct PieceMap {
  int k_tok;               // chunk-relative token of this lane's K pieces
  int k_c[C::KP];          // K piece index c
  int v_p[C::VP], v_d[C::VP];
  uint32_t k_off[C::KP];   // byte offset within the page, full chunks
  uint32_t v_off[C::VP];

  __device__ __forceinline__ PieceMap(int wave, int lane, int blog2) {
    const int B = 1 << blog2;
    const int tile = C::NT == 256 ? wave : (wave & 3), half = C::NT == 256 ? 0 : (wave >> 2);
    k_tok = 16 * tile + (lane & 15);
#pragma unroll
    for (int i = 0; i < C::KP; ++i) {
      k_c[i] = (lane >> 4) + 4 * half + 4 * (C::NT / 256) * i;
      k_off[i] = (uint32_t)((k_c[i] * B + (k_tok & (B - 1))) * 16);
    }
#pragma unroll
    for (int i = 0; i < C::VP; ++i) {
      const int vp = C::NT * i + 64 * wave + lane;
      v_p[i] = vp / C::Dim;
      v_d[i] = vp % C::Dim;
      v_off[i] = (uint32_t)(((((v_p[i] * C::TP) & (B - 1)) / C::TP) * C::Dim + v_d[i]) * 16);
    }
  }
};

// Issue the pool loads of the chunk at `base` (tokens clamped below `end`).
template <class C>
__device__ __forceinline__ void chunk_load(Raw<C>& r, const uint8_t* __restrict__ k_pool,
                                           const uint8_t* __restrict__ v_pool, const int (&pg)[4],
                                           int base, int end, int kvh, int wave,
                                           const PieceMap<C>& pm, const PrefillScalars& ps) {
  constexpr int D = C::Dim;
  const int B = 1 << ps.blog2;
  const bool full = base + 64 <= end;  // uniform
  {
    const uint8_t* pb = k_pool + ((size_t)pick4(pg, C::NT == 256 ? wave : (wave & 3)) *
                                      (size_t)ps.bstride +
                                  (size_t)kvh * C::NC * B) * 16;
#pragma unroll
    for (int i = 0; i < C::KP; ++i) {
      uint32_t off = pm.k_off[i];
      if (!full) {
        const int t = min(base + pm.k_tok, end - 1);
        off = (uint32_t)((pm.k_c[i] * B + (t & (B - 1))) * 16);
      }
      r.k[i] = *reinterpret_cast<const u32x4*>(pb + off);
    }
  }
#pragma unroll
  for (int i = 0; i < C::VP; ++i) {
    const int t0 = uniform(pm.v_p[i]) * C::TP;  // first token of the piece within the chunk
    const uint8_t* pb = v_pool + (size_t)pick4(pg, t0 >> 4) * (size_t)ps.bstride * 16 +
                        (size_t)kvh * (D * B * C::EB);
    uint32_t off = pm.v_off[i];
    if (!full) {
      const int t = (min(base + t0, end - 1) & (B - 1)) & ~(C::TP - 1);
      off = (uint32_t)(((t / C::TP) * D + pm.v_d[i]) * 16);
    }
    r.v[i] = *reinterpret_cast<const u32x4*>(pb + off);
  }
}

// Widen K piece i of the thread to 16 bits and write it into a K buffer.
template <class C>
__device__ __forceinline__ void stage_k_piece(const Raw<C>& r, uint8_t* kbuf,
                                              const PieceMap<C>& pm, int i) {
  constexpr int KVT = C::KV;
  const int c = pm.k_c[i], tok = pm.k_tok;
  uint8_t* row = kbuf + tok * C::KROW;
  if constexpr (KVT == DT_FP8) {
    const u32x4 w = r.k[i];
    const u32x4 lo = fp8x8<DT_BF16>(w[0], w[1]), hi = fp8x8<DT_BF16>(w[2], w[3]);
    const int u0 = 2 * c, u1 = 2 * c + 1;
    *reinterpret_cast<u32x4*>(row + ((u0 ^ (tok & (C::KUNITS - 1))) << 4)) = lo;
    *reinterpret_cast<u32x4*>(row + ((u1 ^ (tok & (C::KUNITS - 1))) << 4)) = hi;
  } else {
    *reinterpret_cast<u32x4*>(row + ((c ^ (tok & (C::KUNITS - 1))) << 4)) = r.k[i];
  }
}

// Widen the thread's K pieces to 16 bits and write them into a K buffer.
template <class C>
__device__ __forceinline__ void stage_k(const Raw<C>& r, uint8_t* kbuf, const PieceMap<C>& pm) {
#pragma unroll
  for (int i = 0; i < C::KP; ++i) stage_k_piece<C>(r, kbuf, pm, i);
}

// Widen V piece i of the thread to 16 bits and write it into a V buffer.  MASK: the
// tokens at or past `end` (chunk at `base`) become zero, as their slots may hold
// anything; only the chunk that reaches `end` needs it.
template <class C, bool MASK>
__device__ __forceinline__ void stage_v_piece(const Raw<C>& r, uint8_t* vbuf, int base, int end,
                                              const PieceMap<C>& pm, int i, float vsc) {
  constexpr int KVT = C::KV;
  const int p = pm.v_p[i], d = pm.v_d[i];
  const int t0 = p * C::TP;
  uint8_t* row = vbuf + d * C::VROW;
  u32x4 w = r.v[i];
  if constexpr (MASK) {
    const int lim = end - (base + t0);  // tokens of the piece below end
    if (lim < C::TP) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok_e = e / C::EB;
        if (tok_e >= lim) w[e >> 2] &= ~(0xffu << (8 * (e & 3)));
      }
    }
  }
  // 16-bit values of the piece's tokens t0 + i; a row keeps, per 16-byte unit
  // u = 4 s2 + g, the keys 32 s2 + 4 g + (0..3) and 32 s2 + 16 + 4 g + (0..3)
  // (the k-slots of one P.V operand), so key t sits at unit 4 (t / 32) + (t / 4) % 4,
  // half (t / 16) % 2
  uint32_t h16[C::TP / 2];
  if constexpr (KVT == DT_FP8) {
    // f16(code) times the page's V scale (rounded to f16), one packed multiply per pair
    const u32x4 lo = fp8x8<DT_F16>(w[0], w[1]), hi = fp8x8<DT_F16>(w[2], w[3]);
    const f16x2 sc = {(_Float16)vsc, (_Float16)vsc};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h16[k] = __builtin_bit_cast(uint32_t, as_f16x2(lo[k]) * sc);
      h16[4 + k] = __builtin_bit_cast(uint32_t, as_f16x2(hi[k]) * sc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) h16[k] = w[k];
  }
#pragma unroll
  for (int q4 = 0; q4 < C::TP / 4; ++q4) {  // runs of four keys
    const int t = t0 + 4 * q4;
    const int u = 4 * (t >> 5) + ((t >> 2) & 3);
    *reinterpret_cast<u32x2*>(row + ((u ^ ((d >> 1) & 7)) << 4) + 8 * ((t >> 4) & 1)) =
        u32x2{h16[2 * q4], h16[2 * q4 + 1]};
  }
}

// Widen the thread's V pieces to 16 bits and write them into a V buffer (MASK as above);
// fp8: piece i is scaled by vsc[i], the V scale of its page.
template <class C, bool MASK>
__device__ __forceinline__ void stage_v(const Raw<C>& r, uint8_t* vbuf, int base, int end,
                                        const PieceMap<C>& pm, const float (&vsc)[C::VP]) {
#pragma unroll
  for (int i = 0; i < C::VP; ++i) stage_v_piece<C, MASK>(r, vbuf, base, end, pm, i, vsc[i]);
}

// Both halves; V tokens at or past `end` become zero.  Only the chunk that reaches
// `end` has such tokens: the check sits behind a wave-uniform branch.
template <class C>
__device__ __forceinline__ void chunk_stage(const Raw<C>& r, uint8_t* kbuf, uint8_t* vbuf,
                                            int base, int end, const PieceMap<C>& pm,
                                            const float (&vsc)[C::VP]) {
  stage_k<C>(r, kbuf, pm);
  if (uniform(base + 64 > end ? 1 : 0) != 0)
    stage_v<C, true>(r, vbuf, base, end, pm, vsc);
  else
    stage_v<C, false>(r, vbuf, base, end, pm, vsc);
}

// Headroom of the lazily moved softmax reference, in log2 units: p <= 2^kLazyMax.
// With the fp8 V scale folded into P (f16), scales up to 65504 / 2^kLazyMax keep P finite.
constexpr float kLazyMax = 4.0f;

// LDS operand reads in flight ahead of the MFMA that uses them
constexpr int kPrefetch = 4;

// maximum of four floats (NaN-propagating: v_maximum3, no operand quieting)
__device__ __forceinline__ float fmax4(float a, float b, float c, float d) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                       __builtin_elementwise_maximum(c, d));
}

// per-row online-softmax state of one row tile: lane (n, g) holds column n
template <int D>
struct RowState {
  f32x4 acc[D / 16];
  float m, l;
};

// S^T = K . Q^T of every row tile for the chunk staged at kbuf.  K operands
// (i = T * NKS + ks) are read kPrefetch ahead of their MFMAs, so the LDS latency hides
// behind the products of the operands before them.
template <class C>
__device__ __forceinline__ void chunk_scores(f32x4 (&S)[C::NR][4], const uint8_t* kbuf,
                                             const int (&k_off)[4], const int (&k_unit)[C::NKS],
                                             const u32x4 (&qop)[C::NR][C::NKS]) {
  constexpr int NR = C::NR, NI = 4 * C::NKS;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  auto rd = [&](int i) {
    return *reinterpret_cast<const u32x4*>(kbuf + k_off[i / C::NKS] + k_unit[i % C::NKS]);
  };
  u32x4 kop[kPrefetch + 1];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) kop[i] = rd(i);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i + kPrefetch < NI) kop[(i + kPrefetch) % (kPrefetch + 1)] = rd(i + kPrefetch);
    const int T = i / C::NKS, ks = i % C::NKS;
#pragma unroll
    for (int rt = 0; rt < NR; ++rt)
      S[rt][T] = mma16<C::QT>(kop[i % (kPrefetch + 1)], qop[rt][ks], ks == 0 ? zero : S[rt][T]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 1);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i + kPrefetch < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, NR, 1);
  }
}

// S^T = K . q^T of one row tile (the rare second pass of a chunk's softmax)
template <class C>
__device__ __forceinline__ void tile_scores(f32x4 (&S)[4], const uint8_t* kbuf,
                                            const int (&k_off)[4], const int (&k_unit)[C::NKS],
                                            const u32x4 (&q)[C::NKS]) {
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
      S[T] = mma16<C::QT>(*reinterpret_cast<const u32x4*>(kbuf + k_off[T] + k_unit[ks]), q[ks],
                          ks == 0 ? zero : S[T]);
}

// scores of keys at or past a row's bound become -inf (the softmax then gives them 0)
__device__ __forceinline__ void mask_scores(f32x4 (&S)[4], int rlim, int base, int g) {
  const int lim = rlim - base - 4 * g;  // keys 16 T + r below lim are visible
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[T][r] = 16 * T + r < lim ? S[T][r] : -INFINITY;
}

// p = 2^(S zs - mref) of one row tile's 16 keys, packed into the P operands of P.V,
// and the row sum of the same values (masked keys: S = -inf, p = 0)
template <class C>
__device__ __forceinline__ float chunk_p(const f32x4 (&S)[4], const float (&zs)[4], float mref,
                                         u32x4 (&phi)[2], u32x4 (&plo)[2]) {
  float p[16];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) p[4 * T + r] = __builtin_amdgcn_exp2f(fmaf(S[T][r], zs[T], -mref));
  float psum = 0.0f;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const int i0 = 8 * s2 + 2 * wd;  // keys 32 s2 + 16 (wd / 2) + 4 g + 2 (wd % 2) + {0, 1}
      const float a = p[i0], b = p[i0 + 1];
      wh[wd] = pack2<C::PT>(a, b);
      if constexpr (C::SPLIT) {
        const f32x2 h = unpack2<C::PT>(wh[wd]);
        wl[wd] = pack2<C::PT>(a - h[0], b - h[1]);
        psum += a + b;
      } else {
        // fp8 and f16 pools: P is f16(p) (fp8: V carries its page scale); the row sum
        // adds the same rounded values (exact f16 products, fp32 sum)
        wl[wd] = 0u;
        psum = __builtin_amdgcn_fdot2(as_f16x2(wh[wd]), f16x2{(_Float16)1.0f, (_Float16)1.0f},
                                      psum, false);
      }
    }
    phi[s2] = u32x4{wh[0], wh[1], wh[2], wh[3]};
    plo[s2] = u32x4{wl[0], wl[1], wl[2], wl[3]};
  }
  return psum;
}

// Online softmax of one chunk (keys base ..) for every row tile: the P operands, the
// reference and the sum updated, the accumulators rescaled when a reference moves.
// Keys at or past a row's bound (rlim) exist only where need_mask says so.
//
// The softmax does not depend on the reference a row's p are taken against, as long
// as they stay finite in the P operand's type.  So a chunk first takes p against the
// row's current reference without computing the chunk's maxima; that is kept when
// every row of the tile has a reference and its chunk sum is at most 2^15 (each p is
// then at most 2^15, inside f16 and bf16).  Otherwise (a row's first keys, or scores
// that passed the reference by about 9 or more in log2 units) the chunk takes the
// maxima: the reference moves only when a chunk's max passes it by more than
// kLazyMax, so the accumulators are rescaled rarely, and p is taken again (after a
// failed first pass from scores computed again, so that the first pass need not keep
// them).
template <class C, bool TWO_PASS>
__device__ __forceinline__ void chunk_softmax(f32x4 (&S)[C::NR][4], RowState<C::Dim> (&st)[C::NR],
                                              const float (&zs)[4], const int (&rlim)[C::NR],
                                              int base, int g, bool need_mask,
                                              u32x4 (&phi)[C::NR][2], u32x4 (&plo)[C::NR][2],
                                              const uint8_t* kbuf, const int (&k_off)[4],
                                              const int (&k_unit)[C::NKS],
                                              const u32x4 (&qop)[C::NR][C::NKS]) {
  constexpr int NR = C::NR;
  constexpr float kFastSum = 32768.0f;
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    // scores in log2 units are S zs (zs > 0: the softmax scale times K's page
    // scale); masked keys become -inf in place, which the same path turns into 0
    if (need_mask) mask_scores(S[rt], rlim[rt], base, g);
    if (TWO_PASS && __builtin_amdgcn_ballot_w64(st[rt].m == -INFINITY) == 0) {
      const float psum = chunk_p<C>(S[rt], zs, st[rt].m, phi[rt], plo[rt]);
      if (__builtin_amdgcn_ballot_w64(!(psum <= kFastSum)) == 0) {
        st[rt].l += psum;
        continue;
      }
      tile_scores<C>(S[rt], kbuf, k_off, k_unit, qop[rt]);
      if (need_mask) mask_scores(S[rt], rlim[rt], base, g);
    }
    float tm[4];
#pragma unroll
    for (int T = 0; T < 4; ++T)
      tm[T] = fmax4(S[rt][T][0], S[rt][T][1], S[rt][T][2], S[rt][T][3]) * zs[T];
    float cm = max_groups(fmax4(tm[0], tm[1], tm[2], tm[3]));
    const bool moves = cm > st[rt].m + kLazyMax;
    if (__builtin_amdgcn_ballot_w64(moves) != 0) {
      // 0 for a row's first keys; 1 for a row that does not move (which may not have
      // seen a key yet: m = -inf, where m - m would be NaN)
      const float mn = moves ? cm : st[rt].m;
      const float alpha = moves ? __builtin_amdgcn_exp2f(st[rt].m - mn) : 1.0f;
      st[rt].m = mn;
      st[rt].l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) st[rt].acc[dt] *= alpha;
    }
    const float mref = st[rt].m == -INFINITY ? 0.0f : st[rt].m;  // rows that have seen no key yet
    st[rt].l += chunk_p<C>(S[rt], zs, mref, phi[rt], plo[rt]);
  }
}

// O^T += V^T . P^T of every row tile for the chunk staged at vbuf.  V operands
// (i = 2 dt + s2) are read kPrefetch ahead as the K operands above.
template <class C>
__device__ __forceinline__ void chunk_pv(RowState<C::Dim> (&st)[C::NR], const uint8_t* vbuf,
                                         int v_off, const int (&v_unit)[2],
                                         const u32x4 (&phi)[C::NR][2],
                                         const u32x4 (&plo)[C::NR][2]) {
  constexpr int NR = C::NR, NI = 2 * C::NDT;
  constexpr int MPI = NR * (C::SPLIT ? 2 : 1);  // MFMAs per operand
  auto rd = [&](int i) {
    return *reinterpret_cast<const u32x4*>(vbuf + v_off + (i / 2) * 16 * C::VROW + v_unit[i % 2]);
  };
  u32x4 vop[kPrefetch + 1];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) vop[i] = rd(i);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i + kPrefetch < NI) vop[(i + kPrefetch) % (kPrefetch + 1)] = rd(i + kPrefetch);
    const int dt = i / 2, s2 = i % 2;
    const u32x4 a = vop[i % (kPrefetch + 1)];
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      st[rt].acc[dt] = mma16<C::PT>(a, phi[rt][s2], st[rt].acc[dt]);
      if constexpr (C::SPLIT) st[rt].acc[dt] = mma16<C::PT>(a, plo[rt][s2], st[rt].acc[dt]);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kPrefetch, 2);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i + kPrefetch < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
    __builtin_amdgcn_sched_group_barrier(0x008, MPI, 2);
  }
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return uniform(x);
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return uniform(x);
}

// PREFIX: the shared prefix of a decode batch instead of a prefill chunk.  The rows
// are then (sequence, query head) pairs of one kv head (16/G sequences per row tile,
// every sequence's one query token), the keys one slice of the prefix that every
// sequence reads from the same blocks (table row 0); row (s, h) sees the prefix keys
// below min(ctx_s, shared_len), without a causal bound.  The slice's state of each
// row (normalised output, reference max in natural-log units, sum) goes to partial
// slot `slice`, which a log-sum-exp merge combines with the other slices and the
// sequence's private tail.
template <int KVT, int D, bool PREFIX = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(
    PCfg<KVT, D>::WPE, PCfg<KVT, D>::WPE))) void paged_prefill_kernel(const uint8_t* __restrict__ q, const int32_t* __restrict__ cu_seqlens_q,
                     const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
                     const float* __restrict__ k_scale, const float* __restrict__ v_scale,
                     const int32_t* __restrict__ block_table,
                     const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out,
                     const PrefillScalars ps) {
  using C = PCfg<KVT, D, 64 * NW>;
  constexpr bool kFp8 = (KVT == DT_FP8);
  constexpr int NR = C::NR;
  // two chunk buffers as separate arrays, so that the staging writes into one are
  // provably independent of the operand reads from the other
  __shared__ __attribute__((aligned(16))) uint8_t lds0[C::KBUF + C::VBUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[C::KBUF + C::VBUF];
  constexpr int kWinChunks = 32;
  constexpr int kWinBlocks = (kWinChunks + 2) * 4;  // chunks of 64 tokens, blocks of >= 16
  __shared__ int w_blk[kWinBlocks];
  __shared__ float w_ks[kWinBlocks], w_vs[kWinBlocks];

  const int xcd = blockIdx.x % kXcds, xslot = blockIdx.x / kXcds;
  const int pair = (xslot / ps.nqb) * kXcds + xcd, qb = xslot % ps.nqb;
  if (pair >= ps.pairs) return;  // the grid is rounded up to whole XCD rows
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int G = ps.G, tpr = 16 / G;           // tokens (prefix: sequences) per row tile
  const int tpw = NR * tpr, tpg = NW * tpw;   // per wave / per workgroup
  const int tok0 = qb * tpg;

  // the workgroup's rows and keys [kbeg, kend); row t of the pair is token q0 + t
  // of the query array
  int s, kvh, slice = 0, q0, nq, ctx = 0, pos0 = 0, kbeg = 0, kend;
  if constexpr (PREFIX) {
    kvh = pair / ps.n_slices;
    slice = pair - kvh * ps.n_slices;
    s = 0;  // the shared blocks: table row 0
    q0 = 0;
    nq = ps.S;
    if (tok0 >= nq) return;
    kbeg = slice * ps.slice_chunks * 64;
    kend = min(kbeg + ps.slice_chunks * 64, ps.shared_len);
  } else {
    s = pair / ps.Hkv;
    kvh = pair - s * ps.Hkv;
    q0 = cu_seqlens_q[s];
    nq = cu_seqlens_q[s + 1] - q0;
    if (tok0 >= nq) return;
    ctx = context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > ps.ctx_cap ? ps.ctx_cap : ctx);
    pos0 = ctx - nq;  // absolute position of query token 0
    const int tok_end = min(nq, tok0 + tpg);
    kend = ps.causal ? max(0, min(ctx, pos0 + tok_end)) : ctx;
  }

  // ---- this lane's rows: token and head of column n in each row tile
  const int hq = kvh * G + n % G;
  int rtok[NR];  // query token (chunk-relative) of column n, or -1 when past the chunk
  int rlim[NR];  // keys [0, rlim) visible to that row
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    const int t = tok0 + wave * tpw + rt * tpr + n / G;
    rtok[rt] = t < nq ? t : -1;
    if constexpr (PREFIX) {
      int c = rtok[rt] < 0 ? 0 : context_lens[rtok[rt] < 0 ? 0 : t];  // never past S
      c = c < 0 ? 0 : (c > ps.ctx_cap ? ps.ctx_cap : c);
      rlim[rt] = min(c, ps.shared_len);
    } else {
      rlim[rt] = rtok[rt] < 0 ? 0 : (ps.causal ? max(0, min(ctx, pos0 + t + 1)) : ctx);
    }
  }

  // ---- q operands (B of S^T), one per row tile and k-step; dead rows are zero
  u32x4 qop[NR][C::NKS];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    const int t = rtok[rt] < 0 ? 0 : rtok[rt];
    const uint8_t* row = q + ((size_t)(q0 + t) * ps.Hq + hq) * D * 2;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(row + (32 * ks + 8 * g) * 2);
      qop[rt][ks] = rtok[rt] < 0 ? u32x4{0u, 0u, 0u, 0u} : w;
    }
  }

  RowState<D> st[NR];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) st[rt].acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st[rt].m = -INFINITY;
    st[rt].l = 0.0f;
  }

  // keys [0, wave_min_lim) are visible to every row of the wave (a dead row counts as
  // seeing none); [0, wave_max_lim) to at least one (wave-uniform)
  const int wave_min_lim = wave_min_i(min(rlim[0], rlim[NR - 1]));
  const int wave_max_lim = wave_max_i(max(rlim[0], rlim[NR - 1]));
  static_assert(NR == 2, "the wave bounds above take the two row tiles");
  if constexpr (PREFIX) {
    // keys past every row's bound are never read: they need not have been written
    // (a prefix token lies in the context of some sequence that sees it)
    __shared__ int wg_lim[NW];
    if (lane == 0) wg_lim[wave] = wave_max_lim;
    __syncthreads();
    int wl = wg_lim[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) wl = max(wl, wg_lim[w]);
    kend = min(kend, wl);
  }
  // this lane's LDS offsets (swizzled 16-byte units), the same for every chunk
  int k_off[4], k_unit[C::NKS], v_off, v_unit[2];
#pragma unroll
  for (int T = 0; T < 4; ++T) k_off[T] = (16 * T + n) * C::KROW;
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) k_unit[ks] = ((4 * ks + g) ^ (n & (C::KUNITS - 1))) << 4;
  v_off = n * C::VROW;
  // rows d = 16 dt + n share (d >> 1) & 7 = (n >> 1) & 7 for every dt
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) v_unit[s2] = ((4 * s2 + g) ^ ((n >> 1) & 7)) << 4;
  const int nch = kend > kbeg ? (kend - kbeg + 63) >> 6 : 0;  // chunk j: keys kbeg + 64 j ..
  if (nch > 0) {
    const int32_t* trow = block_table + (size_t)s * ps.W;
    // window k holds the blocks of chunks [32 k, 32 k + 34) (two chunks of lookahead);
    // kbeg is a multiple of 64, so of the block size
    auto fill_window = [&](int wk) {
      const int blk0 = (kbeg + wk * kWinChunks * 64) >> ps.blog2;
      const int last = (kend - 1) >> ps.blog2;
      for (int t = threadIdx.x; t < kWinBlocks; t += 64 * NW) {
        const int e = clamp_block(trow[min(blk0 + t, last)], ps.num_blocks);
        w_blk[t] = e;
        if constexpr (kFp8) {
          const size_t page = (size_t)e * ps.Hkv + kvh;
          w_ks[t] = ps.scale_log2 * k_scale[page];
          w_vs[t] = v_scale[page];
        }
      }
    };
    // block ids of chunk c's four tiles from window wk (which must cover c)
    auto win_pages = [&](int c, int wk, int (&pg)[4]) {
      const int blk0 = (kbeg + wk * kWinChunks * 64) >> ps.blog2;
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const int t = min(kbeg + 64 * c + 16 * T, kend - 1);
        pg[T] = uniform(w_blk[(t >> ps.blog2) - blk0]);
      }
    };
    fill_window(0);
    __syncthreads();
    const PieceMap<C> pm(wave, lane, ps.blog2);
    // V scales of the thread's pieces of the chunk at `base` from window wk (fp8; a
    // piece's 16 tokens sit in one tile, the same for the whole wavefront)
    auto piece_scales = [&](int base, int wk, float (&vsc)[C::VP]) {
      const int blk0 = (kbeg + wk * kWinChunks * 64) >> ps.blog2;
#pragma unroll
      for (int i = 0; i < C::VP; ++i) {
        if constexpr (kFp8) {
          const int t = min(base + uniform(pm.v_p[i]) * C::TP, kend - 1);
          vsc[i] = w_vs[(t >> ps.blog2) - blk0];
        } else {
          vsc[i] = 1.0f;
        }
      }
    };
    constexpr bool kOneRaw = (C::NRAW == 1);
    Raw<C> ra, rb;
    {
      int pg[4];
      win_pages(0, 0, pg);
      chunk_load<C>(ra, k_pool, v_pool, pg, kbeg, kend, kvh, wave, pm, ps);
      if (!kOneRaw && nch > 1) {
        win_pages(1, 0, pg);
        chunk_load<C>(rb, k_pool, v_pool, pg, kbeg + 64, kend, kvh, wave, pm, ps);
      }
    }
    {
      float vsc[C::VP];
      piece_scales(kbeg, 0, vsc);
      chunk_stage<C>(ra, lds0, lds0 + C::KBUF, kbeg, kend, pm, vsc);
    }
    __syncthreads();

    // one chunk: loads of chunk j+2 go to `nxt2` (one raw buffer: chunk j+1's to
    // `nxt1`), chunk j+1's pieces (in `nxt1`) are staged after chunk j is computed
    auto step = [&](int j, Raw<C>& nxt2, Raw<C>& nxt1, uint8_t* cur_buf, uint8_t* nxt_buf) {
      const int base = kbeg + 64 * j;
      const int wk = j / kWinChunks;
      const int ahead = kOneRaw ? 1 : 2;
      if (j + ahead < nch) {
        int pg[4];
        win_pages(j + ahead, wk, pg);
        chunk_load<C>(kOneRaw ? nxt1 : nxt2, k_pool, v_pool, pg, base + 64 * ahead, kend,
                           kvh, wave, pm, ps);
      }
      float zs[4];  // per tile: softmax scale x K's page scale, log2 units
      {
        const int blk0 = (kbeg + wk * kWinChunks * 64) >> ps.blog2;
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          if constexpr (kFp8) {
            const int i = (min(base + 16 * T, kend - 1) >> ps.blog2) - blk0;
            zs[T] = w_ks[i];
          } else {
            zs[T] = ps.scale_log2;
          }
        }
      }
      const uint8_t* kbuf = cur_buf;
      const uint8_t* vbuf = cur_buf + C::KBUF;
      issue_point();
      if (base < wave_max_lim) {  // some row of the wave sees a key of this chunk
      // ---- S^T for every row tile (a tile past its rows' keys is masked below).
      // The matrix phases run at raised wave priority: of the two waves on a SIMD,
      // the one with MFMAs ready issues first while the other works on its softmax.
      __builtin_amdgcn_s_setprio(2);
      f32x4 S[NR][4];
      chunk_scores<C>(S, kbuf, k_off, k_unit, qop);
      __builtin_amdgcn_s_setprio(0);
      // ---- online softmax per row tile; P operands
      u32x4 phi[NR][2], plo[NR][2];
      // the first pass without the chunk's maxima where the registers allow it (not in
      // prefix mode, nor over f16 pools of 128 dims: there it would not leave two
      // workgroups per CU)
      constexpr bool kTwoPass = !PREFIX && !(KVT == DT_F16 && D == 128);
      chunk_softmax<C, kTwoPass>(S, st, zs, rlim, base, g, base + 64 > wave_min_lim, phi, plo,
                                 kbuf, k_off, k_unit, qop);
      // ---- stage chunk j+1 into the other buffer (free since the last barrier)
      // while the matrix cores run O^T += V^T . P^T: the conversions and LDS writes
      // fill the issue slots between the MFMAs
      if (j + 1 < nch) {
        float vsc[C::VP];
        piece_scales(base + 64, wk, vsc);
        chunk_stage<C>(nxt1, nxt_buf, nxt_buf + C::KBUF, base + 64, kend, pm, vsc);
      }
      __builtin_amdgcn_s_setprio(2);
      chunk_pv<C>(st, vbuf, v_off, v_unit, phi, plo);
      __builtin_amdgcn_s_setprio(0);
      } else if (j + 1 < nch) {  // no key of this chunk for the wave: only the staging
        float vsc[C::VP];
        piece_scales(base + 64, wk, vsc);
        chunk_stage<C>(nxt1, nxt_buf, nxt_buf + C::KBUF, base + 64, kend, pm, vsc);
      }
      issue_point();
      // ---- advance the page window
      if ((j + 1) % kWinChunks == 0 && j + 1 < nch) {  // the next step starts a new window
        __syncthreads();  // every wave has read the old window
        fill_window((j + 1) / kWinChunks);
      }
      __syncthreads();
    };
    // chunk j's raw pieces live in ra (j even) / rb (j odd) until staged (one raw
    // buffer: in ra)
    for (int j = 0; j < nch; j += 2) {
      if constexpr (kOneRaw) {
        step(j, ra, ra, lds0, lds1);
        if (j + 1 < nch) step(j + 1, ra, ra, lds1, lds0);
      } else {
        step(j, ra, rb, lds0, lds1);
        if (j + 1 < nch) step(j + 1, rb, ra, lds1, lds0);
      }
    }
  }

  // ---- normalise and store the live rows (prefix: the slice's partial state; a row
  // that saw no key leaves an empty state, weight 0)
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    const float lw = sum_groups(st[rt].l);
    if (rtok[rt] < 0) continue;
    const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;
    if constexpr (PREFIX) {
      const size_t pi = ((size_t)rtok[rt] * ps.Hq + hq) * ps.max_parts + slice;
      float* o = ps.part_out + pi * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
        *reinterpret_cast<f32x4*>(o + 16 * dt) = st[rt].acc[dt] * inv;
      if (g == 0) {
        ps.part_max[pi] = lw > 0.0f ? st[rt].m * kLn2 : -INFINITY;
        ps.part_sum[pi] = lw;
      }
    } else {
      const size_t orow = ((size_t)(q0 + rtok[rt]) * ps.Hq + hq) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) store4(out, C::QT, orow + 16 * dt, st[rt].acc[dt] * inv);
    }
  }
}

namespace {

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

template <int KVT, int D, bool PREFIX>
int launch_pf(const PrefillLaunch& p, const PrefillScalars& ps, hipStream_t st) {
  // fp8 pools of 128 dims: one 8-wave workgroup per CU staging each chunk for 256/G
  // tokens (two waves per SIMD, as two 4-wave workgroups would be)
  constexpr int NW = (!PREFIX && KVT == DT_FP8 && D == 128) ? 8 : 4;
  const int tpg = NW * PCfg<KVT, D>::NR * (16 / ps.G);
  PrefillScalars q = ps;
  const long long rows = PREFIX ? p.num_seqs : p.max_q_len;  // per pair
  q.nqb = (int)((rows + tpg - 1) / tpg);
  const long long pairs = PREFIX ? (long long)p.num_kv_heads * p.n_slices
                                 : (long long)p.num_seqs * p.num_kv_heads;
  const long long per_xcd = (pairs + kXcds - 1) / kXcds;
  const long long blocks = per_xcd * kXcds * q.nqb;
  if (blocks > 0x7fffffffLL) return -3;
  q.pairs = (int)pairs;
  dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL((paged_prefill_kernel<KVT, D, PREFIX, NW>), grid, dim3(64 * NW), 0, st,
                     (const uint8_t*)p.q, p.cu_seqlens_q, (const uint8_t*)p.k_pool,
                     (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                     p.context_lens, (uint8_t*)p.out, q);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int KVT, int D>
int pick_mode(const PrefillLaunch& p, const PrefillScalars& ps, hipStream_t st) {
  return p.prefix ? launch_pf<KVT, D, true>(p, ps, st) : launch_pf<KVT, D, false>(p, ps, st);
}

}  // namespace

int launch_prefill(const PrefillLaunch& p, hipStream_t st) {
  PrefillScalars ps;
  ps.W = p.max_blocks_per_seq;
  ps.S = p.num_seqs;
  ps.Hq = p.num_q_heads;
  ps.Hkv = p.num_kv_heads;
  ps.G = p.num_q_heads / p.num_kv_heads;
  ps.blog2 = log2_exact(p.block_size);
  ps.num_blocks = p.num_blocks;
  ps.ctx_cap = p.ctx_cap;
  ps.causal = p.causal;
  ps.scale_log2 = p.scale * kLog2e;
  ps.bstride = p.bstride;
  ps.shared_len = p.shared_len;
  ps.n_slices = p.n_slices;
  ps.slice_chunks = p.slice_chunks;
  ps.max_parts = p.max_parts;
  ps.part_out = p.part_out;
  ps.part_max = p.part_max;
  ps.part_sum = p.part_sum;
  if (ps.blog2 < 4 || p.block_size > 64) return -3;  // a 16-token tile must sit in one block
  if (ps.G < 1 || ps.G > 16 || (16 % ps.G) != 0) return -3;
  // q (and the output) in bf16 over bf16 and fp8 pools, in f16 over f16 pools
  if (p.q_dtype != (p.kv_dtype == DT_F16 ? DT_F16 : DT_BF16)) return -3;
  if (p.prefix) {
    if (p.n_slices < 1 || p.slice_chunks < 1 || p.max_parts < p.n_slices) return -3;
    if (p.num_seqs <= 0 || p.shared_len <= 0) return 0;
  } else if (p.max_q_len <= 0) {
    return 0;
  }
  if (p.kv_dtype == DT_FP8) {
    if (p.head_dim == 128) return pick_mode<DT_FP8, 128>(p, ps, st);
    if (p.head_dim == 64) return pick_mode<DT_FP8, 64>(p, ps, st);
  } else if (p.kv_dtype == DT_BF16) {
    if (p.head_dim == 128) return pick_mode<DT_BF16, 128>(p, ps, st);
    if (p.head_dim == 64) return pick_mode<DT_BF16, 64>(p, ps, st);
  } else if (p.kv_dtype == DT_F16) {
    if (p.head_dim == 128) return pick_mode<DT_F16, 128>(p, ps, st);
    if (p.head_dim == 64) return pick_mode<DT_F16, 64>(p, ps, st);
  }
  return -3;
}

}  // namespace pkv
