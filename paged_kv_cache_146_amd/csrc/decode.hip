// decode.hip — paged decode attention for gfx950, plus the split-KV
// log-sum-exp merges.
//
// Method: "03 | PagedAttention and the KV-cache memory system", §4 — per
// sequence and query head, walk the logical blocks of the visible context,
// look each one up in the block table, load its K/V page, and fold the partial
// attention into an online-softmax state (max, exp_sum, weighted_value); long
// contexts are scanned in parallel pieces whose states are merged.
//
// Shared by all kernels: a wavefront works on 64 consecutive tokens of one
// (sequence, kv head) at a time ("chunk"), for all G = H_q/H_kv query heads of
// that kv head, so every K/V byte is read from HBM once per step (GQA grouping).
//   QK^T  lane = token.  The K pool is [block][head][D/X][B][X]: a lane's 16-byte
//         loads walk its token's row and the 64 lanes of one load cover
//         contiguous 16-byte pieces of the pages; the dot product over D stays in
//         the lane.  q is wave-uniform and read through the scalar cache.
//   soft  chunk max per head by DPP row ops + lane reads; p = 2^(z - m) with
//         log2(e) folded into the scale.
//   P.V   lane = 16-byte slice of one V row (V pool [block][head][B][D]); each
//         pass covers 64/(D/X) tokens; p comes from LDS.
//
// Three ways to cut the work:
//   unsplit / fixed partitions — one workgroup (4 waves) per (partition, kv
//         head, sequence); the waves take chunks round-robin and merge in LDS;
//         partitions are merged by split_reduce_kernel.
//   balanced — the chunks of all (sequence, kv head) pairs form one stream that
//         is cut into equal contiguous shares, one per wavefront ("worker").  A
//         worker finishes every pair it covers entirely and leaves a partial
//         state for at most two pairs it shares with neighbours; those are
//         merged by the last worker to finish one (a per-pair counter tells it).  Inside a worker the chunk loop is
//         software-pipelined: the next chunk's table entry and K rows are in
//         flight while the current chunk's P.V runs.
#include "device.hpp"
#include "internal.hpp"

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
  float scale_log2; // softmax scale * log2(e)
};

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ void store_any(uint8_t* out, int dt, size_t idx, float x) {
  if (dt == DT_F32)
    reinterpret_cast<float*>(out)[idx] = x;
  else if (dt == DT_BF16)
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(x);
  else
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(x);
}

// q elements [c*X, c*X + X) of one (wave-uniform) query row, as floats
template <int QDT, int X>
__device__ __forceinline__ void q_chunk_f32(const uint8_t* __restrict__ qrow, int c, float* qf) {
  if constexpr (QDT == DT_F32) {
    const float* p = reinterpret_cast<const float*>(qrow) + c * X;
#pragma unroll
    for (int i = 0; i < X; ++i) qf[i] = p[i];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(qrow) + c * (X / 2);
#pragma unroll
    for (int i = 0; i < X / 2; ++i) {
      uint32_t w = p[i];
      if constexpr (QDT == DT_BF16) {
        qf[2 * i] = bf16_lo(w);
        qf[2 * i + 1] = bf16_hi(w);
      } else {
        qf[2 * i] = f16_lo(w);
        qf[2 * i + 1] = f16_hi(w);
      }
    }
  }
}

template <int KVT, int QDT, int D>
struct Shape {
  static constexpr int X = Elem<KVT>::per16;  // elements per 16 bytes
  static constexpr int ES = Elem<KVT>::bytes;
  static constexpr int NC = D / X;            // 16-byte pieces per row (= lanes per V row)
  static constexpr int R = 64 / NC;           // V rows per pass
  static constexpr int NPASS = 64 / R;        // passes per 64-token chunk
  static constexpr int QES = (QDT == DT_F32) ? 4 : 2;
  static_assert(NC <= 64 && 64 % NC == 0, "row must split into 16-byte lane slices");
};

// acc[h] = <q_h, K row held in kr> for every head of the group
template <int KVT, int QDT, int D, int GM>
__device__ __forceinline__ void chunk_scores(const u32x4 (&kr)[Shape<KVT, QDT, D>::NC],
                                             const uint8_t* const (&qrow)[GM], float (&acc)[GM]) {
  using S = Shape<KVT, QDT, D>;
#pragma unroll
  for (int h = 0; h < GM; ++h) acc[h] = 0.0f;
  if constexpr (KVT == DT_BF16 || KVT == DT_F16) {
    // q slices are scalar loads; only the next 16-byte slice of each head is
    // prefetched (sched_barrier per slice) so q never floods the scalar registers
    u32x4 qn[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) qn[h] = *reinterpret_cast<const u32x4*>(qrow[h]);
#pragma unroll
    for (int c = 0; c < S::NC; ++c) {
      u32x4 qc[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) qc[h] = qn[h];
      if (c + 1 < S::NC) {
#pragma unroll
        for (int h = 0; h < GM; ++h) qn[h] = *(reinterpret_cast<const u32x4*>(qrow[h]) + c + 1);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t kw = kr[c][w], qw = qc[h][w];
          if constexpr (KVT == DT_BF16)
            acc[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw), as_bf16x2(qw), acc[h], false);
          else
            acc[h] = __builtin_amdgcn_fdot2(as_f16x2(kw), as_f16x2(qw), acc[h], false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < S::NC; ++c) {
    {
      float kf[S::X];
      unpack16<KVT>(kr[c], kf);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        float qf[S::X];
        q_chunk_f32<QDT, S::X>(qrow[h], c, qf);
#pragma unroll
        for (int e = 0; e < S::X; ++e) acc[h] = fmaf(kf[e], qf[e], acc[h]);
      }
    }
  }
}

// online-softmax update for one chunk: new running max, rescale, p to LDS
template <int X, int GM, bool FP8>
__device__ __forceinline__ void chunk_softmax(const float (&acc)[GM], bool valid, float zscale,
                                              float vs, float (&m_run)[GM], float (&l_lane)[GM],
                                              float (&pacc)[GM][X], float* pl) {
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const float z = valid ? acc[h] * zscale : -INFINITY;
    const float mn = fmaxf(m_run[h], wave_max(z));
    const float alpha = __builtin_amdgcn_exp2f(m_run[h] - mn);
    const float p = __builtin_amdgcn_exp2f(z - mn);
    l_lane[h] = l_lane[h] * alpha + p;
#pragma unroll
    for (int e = 0; e < X; ++e) pacc[h][e] *= alpha;
    m_run[h] = mn;
    pl[h] = FP8 ? p * vs : p;
  }
}

// pacc[h][:] += sum over this lane's rows of p[tok][h] * V row slice.  Each pass
// is fenced off from the next (sched_barrier) with only the next pass's p
// prefetched, so that no more than one V row is ever held unpacked.  Rows past
// the context hold garbage: their packed words are zeroed (every storage type
// decodes all-zero bits to +0) before the unpack, so 0 * NaN never happens.
template <int KVT, int GM, int X, int R, int NPASS>
__device__ __forceinline__ void chunk_pv(const u32x4 (&vr)[NPASS], const float* p_wave, int r,
                                         int n_valid, float (&pacc)[GM][X]) {
  float pn[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) pn[h] = p_wave[r * GM + h];
#pragma unroll
  for (int i = 0; i < NPASS; ++i) {
    const int tok = i * R + r;
    float pc[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) pc[h] = pn[h];
    if (i + 1 < NPASS) {
#pragma unroll
      for (int h = 0; h < GM; ++h) pn[h] = p_wave[(tok + R) * GM + h];
    }
    const uint32_t keep = tok < n_valid ? 0xffffffffu : 0u;
    const u32x4 vw = {vr[i][0] & keep, vr[i][1] & keep, vr[i][2] & keep, vr[i][3] & keep};
    float vf[X];
    unpack16<KVT>(vw, vf);
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int e = 0; e < X; ++e) pacc[h][e] = fmaf(pc[h], vf[e], pacc[h][e]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// X consecutive outputs of one row, converted to DT and stored with 16-byte stores
template <int DT, int X>
__device__ __forceinline__ void store_row(uint8_t* __restrict__ out, size_t elem_idx,
                                          const float* v) {
  if constexpr (DT == DT_F32) {
    u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<float*>(out) + elem_idx);
#pragma unroll
    for (int k = 0; k < X / 4; ++k) {
      const u32x4 w = {__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                       __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
      p[k] = w;
    }
  } else {
    u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + elem_idx);
#pragma unroll
    for (int k = 0; k < X / 8; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = v[8 * k + 2 * i], b = v[8 * k + 2 * i + 1];
        const uint32_t lo = DT == DT_BF16 ? f32_to_bf16_bits(a) : f32_to_f16_bits(a);
        const uint32_t hi = DT == DT_BF16 ? f32_to_bf16_bits(b) : f32_to_f16_bits(b);
        w[i] = lo | (hi << 16);
      }
      p[k] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

__device__ __forceinline__ int clamp_block(int phys, int num_blocks) {
  return phys < 0 ? 0 : (phys >= num_blocks ? num_blocks - 1 : phys);
}

// =================================================================================
// Kernel A: one workgroup per (partition, kv head, sequence)
// =================================================================================
template <int KVT, int QDT, int D, int GM>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out,
    float* __restrict__ part_out, float* __restrict__ part_max, float* __restrict__ part_sum,
    const DecodeScalars sc) {
  using SH = Shape<KVT, QDT, D>;
  constexpr int X = SH::X, ES = SH::ES, NC = SH::NC, R = SH::R, NPASS = SH::NPASS;
  constexpr bool kFp8 = (KVT == DT_FP8);

  __shared__ float p_lds[kWaves][64 * GM];
  __shared__ float c_acc[kWaves][GM][D];
  __shared__ float c_m[kWaves][GM];
  __shared__ float c_l[kWaves][GM];

  const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int B = 1 << sc.blog2;

  int ctx = context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > sc.ctx_cap ? sc.ctx_cap : ctx);
  const int t_begin = part * sc.part_size;
  const int t_end = min(t_begin + sc.part_size, ctx);
  if (t_begin >= t_end) {
    if (!sc.split && part == 0) {  // empty context: zeros
      for (int i = threadIdx.x; i < sc.G * D; i += kThreads) {
        size_t o = ((size_t)s * sc.Hq + (size_t)kvh * sc.G) * D + i;
        store_any(out, sc.out_dtype, o, 0.0f);
      }
    }
    return;
  }

  const uint8_t* qrow[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    int hq = kvh * sc.G + (h < sc.G ? h : sc.G - 1);
    qrow[h] = q + ((size_t)s * sc.Hq + hq) * D * SH::QES;
  }

  float m_run[GM], l_lane[GM];
  float pacc[GM][X];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < X; ++e) pacc[h][e] = 0.0f;
  }

  const int r = lane / NC, col = lane % NC;
  const int32_t* trow = block_table + (size_t)s * sc.W;
  float* pw = p_lds[wave];

  for (int cbase = t_begin + wave * 64; cbase < t_end; cbase += kThreads) {
    const int t = cbase + lane;
    const bool valid = t < t_end;
    const int tt = valid ? t : cbase;  // masked lanes address a valid token
    const int phys = clamp_block(trow[tt >> sc.blog2], sc.num_blocks);
    const size_t page = (size_t)phys * sc.Hkv + kvh;
    const int off = tt & (B - 1);
    const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + (page * NC * B + off);
    const uint32_t vrow = (uint32_t)(page * B + off);

    u32x4 kr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = kp[(size_t)c * B];
    u32x4 vr[NPASS];
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      uint32_t rowi = (uint32_t)__builtin_amdgcn_ds_bpermute((i * R + r) << 2, (int)vrow);
      vr[i] = *(reinterpret_cast<const u32x4*>(v_pool + (size_t)rowi * (D * ES)) + col);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) materialize(kr[c]);

    float acc[GM];
    chunk_scores<KVT, QDT, D, GM>(kr, qrow, acc);
    float zscale = sc.scale_log2, vs = 1.0f;
    if constexpr (kFp8) {
      zscale *= k_scale[page];
      vs = v_scale[page];
    }
    chunk_softmax<X, GM, kFp8>(acc, valid, zscale, vs, m_run, l_lane, pacc, pw + lane * GM);
    wave_lds_sync();
    chunk_pv<KVT, GM, X, R, NPASS>(vr, pw, r, t_end - cbase, pacc);
    wave_lds_sync();  // p_lds is rewritten by the next chunk
  }

  // ---- combine the rows of each wave, then the waves --------------------------
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < X; ++e)
#pragma unroll
      for (int o = NC; o < 64; o <<= 1) pacc[h][e] += __shfl_xor(pacc[h][e], o);
  float lw[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) lw[h] = wave_sum(l_lane[h]);
  if (lane < NC) {
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int e = 0; e < X; ++e) c_acc[wave][h][col * X + e] = pacc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      c_m[wave][h] = m_run[h];
      c_l[wave][h] = lw[h];
    }
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
__device__ void unit_prefix(const int32_t* __restrict__ context_lens, int S, int ctx_cap, int Hkv,
                            int* lds, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + threadIdx.x;
    int v = 0;
    if (s < S) {
      int c = context_lens[s];
      c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
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

// One wavefront merges the partial states of a shared pair (pieces of workers wa..wb,
// log2-domain maxima) in a single online pass: every piece's (m, l, o) for all heads
// is loaded together (device-scope loads) and pieces are unrolled, so the merge
// costs a few memory round trips, not two per head.
template <int QDT, int D, int GM>
__device__ void merge_pair(float* slot_out, float* slot_ml, uint8_t* __restrict__ out,
                           const DecodeScalars& sc, int s, int kvh, int u0, int wa, int wb,
                           int U, int NWe, int lane) {
  constexpr int PER = D / 64;
  const int first_slot = worker_start(wa, U, NWe) != u0 ? 2 * wa + 1 : 2 * wa;
  const int stride = sc.G * D;
  float M[GM], L[GM], O[GM][PER];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    M[h] = -INFINITY;
    L[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < PER; ++k) O[h][k] = 0.0f;
  }
#pragma unroll 4
  for (int w = wa; w <= wb; ++w) {
    const int slot = w == wa ? first_slot : 2 * w;
    float m[GM], l[GM], o[GM][PER];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const int hh = h < sc.G ? h : sc.G - 1;
      float* ml = slot_ml + ((size_t)slot * sc.G + hh) * 2;
      m[h] = __hip_atomic_load(ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      l[h] = __hip_atomic_load(ml + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float* so = slot_out + (size_t)slot * stride + hh * D + lane;
#pragma unroll
      for (int k = 0; k < PER; ++k)
        o[h][k] = __hip_atomic_load(so + 64 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float mn = fmaxf(M[h], m[h]);
      const float a_old = __builtin_amdgcn_exp2f(M[h] - mn);
      const float a_new = __builtin_amdgcn_exp2f(m[h] - mn) * l[h];
      L[h] = L[h] * a_old + a_new;
#pragma unroll
      for (int k = 0; k < PER; ++k) O[h][k] = O[h][k] * a_old + a_new * o[h][k];
      M[h] = mn;
    }
  }
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < sc.G) {
      const float inv = 1.0f / L[h];
      const size_t orow = ((size_t)s * sc.Hq + (size_t)kvh * sc.G + h) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) store_any(out, QDT, orow + lane + 64 * k, O[h][k] * inv);
    }
  }
}

template <int KVT, int QDT, int D, int GM>
// two resident waves per SIMD: the pipeline needs the second wave to cover its gaps
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
paged_decode_balanced_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out, float* slot_out,
    float* slot_ml, unsigned long long* counters, const DecodeScalars sc) {
  using SH = Shape<KVT, QDT, D>;
  constexpr int X = SH::X, ES = SH::ES, NC = SH::NC, R = SH::R, NPASS = SH::NPASS;
  constexpr bool kFp8 = (KVT == DT_FP8);

  extern __shared__ int prefix[];  // [S + 1]
  __shared__ int tmp[kThreads];
  __shared__ float p_lds[kWaves][64 * GM];

  unit_prefix(context_lens, sc.S, sc.ctx_cap, sc.Hkv, prefix, tmp);
  const int U = prefix[sc.S];
  if (blockIdx.x == 0) {  // sequences with an empty context own no unit: their output is zero
    for (int s0 = 0; s0 < sc.S; ++s0) {
      if (prefix[s0 + 1] != prefix[s0]) continue;
      for (int i = threadIdx.x; i < sc.Hq * D; i += kThreads)
        store_any(out, QDT, (size_t)s0 * sc.Hq * D + i, 0.0f);
    }
  }
  const int NWe = min(sc.num_workers, U);
  // wave-uniform values are passed through readfirstlane so that the compiler
  // keeps them (and every address derived from them, q's in particular) scalar
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWaves + wave;
  if (w >= NWe) return;  // no barrier below this point
  const int u_begin = worker_start(w, U, NWe);
  const int u_end = worker_start(w + 1, U, NWe);

  const int B = 1 << sc.blog2;
  const int r = lane / NC, col = lane % NC;
  float* pw = p_lds[wave];
  const int slot_stride = sc.G * D;

  int u = u_begin;
  bool first_piece = true;
  while (u < u_end) {
    // ---- locate the (sequence, kv head) pair of unit u and this worker's piece of it
    const int s = uniform(find_seq(prefix, sc.S, u));
    const int pfx = uniform(prefix[s]);
    const int seg_units = uniform((prefix[s + 1] - pfx) / sc.Hkv);  // chunks per kv head
    const int rel = u - pfx;
    const int kvh = rel / seg_units;
    const int j0 = rel - kvh * seg_units;
    const int seg_first = pfx + kvh * seg_units;
    const int j1 = min(seg_units, u_end - seg_first);
    int ctx = context_lens[s];
    ctx = ctx < 0 ? 0 : (ctx > sc.ctx_cap ? sc.ctx_cap : ctx);

    const uint8_t* qrow[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      int hq = kvh * sc.G + (h < sc.G ? h : sc.G - 1);
      qrow[h] = q + ((size_t)s * sc.Hq + hq) * D * SH::QES;
    }
    const int32_t* trow = block_table + (size_t)s * sc.W;

    float m_run[GM], l_lane[GM];
    float pacc[GM][X];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      m_run[h] = -INFINITY;
      l_lane[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < X; ++e) pacc[h][e] = 0.0f;
    }

    // token-lane addressing of chunk j: masked lanes address the chunk's first token
    auto lane_token = [&](int j) {
      const int t = j * 64 + lane;
      return t < ctx ? t : j * 64;
    };
    // ---- prologue: table entry and K rows of the first chunk
    int tt = lane_token(j0);
    int phys = clamp_block(trow[tt >> sc.blog2], sc.num_blocks);
    u32x4 kr[NC];
    {
      const size_t page = (size_t)phys * sc.Hkv + kvh;
      const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + (page * NC * B + (tt & (B - 1)));
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[c] = kp[(size_t)c * B];
    }

    // Chunk j; chunk j+1's table entry is fetched during the scores and its K
    // rows during P.V, overwriting kr only after K(j) is dead.  On the piece's
    // last chunk the "next" chunk is the same one (a re-read, never used).
    for (int j = j0; j < j1; ++j) {
      const size_t page = (size_t)phys * sc.Hkv + kvh;
      const int off = tt & (B - 1);
      const bool valid = j * 64 + lane < ctx;
      u32x4 vr[NPASS];
      if (B >= R) {
        // The R rows of pass i are consecutive tokens of one page (R divides B), so the
        // page is wave-uniform: its table entry comes through the scalar cache and the
        // lane's byte offset inside the pass is just lane*16.  Passes wholly past the
        // context re-read the last valid group of rows (selected out later).
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
          const int tok0 = j * 64 + i * R;
          const int tokc = uniform(tok0 < ctx ? tok0 : ((ctx - 1) & ~(R - 1)));
          const int pv = clamp_block(trow[tokc >> sc.blog2], sc.num_blocks);
          const size_t row0 = ((size_t)pv * sc.Hkv + kvh) * B + (tokc & (B - 1));
          vr[i] = *reinterpret_cast<const u32x4*>(v_pool + row0 * (D * ES) + lane * 16);
        }
      } else {
        const uint32_t vrow = (uint32_t)(page * B + off);
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
          uint32_t rowi = (uint32_t)__builtin_amdgcn_ds_bpermute((i * R + r) << 2, (int)vrow);
          vr[i] = *(reinterpret_cast<const u32x4*>(v_pool + (size_t)rowi * (D * ES)) + col);
        }
      }
      const int jn = uniform(j + 1 < j1 ? j + 1 : j);
      const int tt_next = lane_token(jn);
      const int phys_next_raw = trow[tt_next >> sc.blog2];
      float zscale = sc.scale_log2, vs = 1.0f;
      if constexpr (kFp8) {
        zscale *= k_scale[page];
        vs = v_scale[page];
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) materialize(kr[c]);
      issue_point();

      float acc[GM];
      chunk_scores<KVT, QDT, D, GM>(kr, qrow, acc);
      chunk_softmax<X, GM, kFp8>(acc, valid, zscale, vs, m_run, l_lane, pacc, pw + lane * GM);
      issue_point();  // K(j) is dead from here on

      phys = clamp_block(phys_next_raw, sc.num_blocks);
      tt = tt_next;
      {
        const size_t pg = (size_t)phys * sc.Hkv + kvh;
        const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + (pg * NC * B + (tt & (B - 1)));
#pragma unroll
        for (int c = 0; c < NC; ++c) kr[c] = kp[(size_t)c * B];
      }
      wave_lds_sync();
      chunk_pv<KVT, GM, X, R, NPASS>(vr, pw, r, ctx - j * 64, pacc);
      wave_lds_sync();
    }

    // ---- finish the piece ------------------------------------------------------
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int e = 0; e < X; ++e)
#pragma unroll
        for (int o = NC; o < 64; o <<= 1) pacc[h][e] += __shfl_xor(pacc[h][e], o);
    float lw[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) lw[h] = wave_sum(l_lane[h]);

    const bool whole = (j0 == 0 && j1 == seg_units);
    if (whole) {
      if (lane < NC) {
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h < sc.G) {
            const size_t o = ((size_t)s * sc.Hq + kvh * sc.G + h) * D + col * X;
            const float inv = 1.0f / lw[h];
            float v[X];
#pragma unroll
            for (int e = 0; e < X; ++e) v[e] = pacc[h][e] * inv;
            store_row<QDT, X>(out, o, v);
          }
        }
      }
    } else {
      // Publish the partial state with device-scope stores (coherent across the
      // XCDs' L2 caches without whole-cache write-back), wait until they have
      // completed, and only then count the piece.  The merging worker reads with
      // device-scope loads.  No cache-wide fence is needed on either side.
      const int slot = 2 * w + (first_piece ? 0 : 1);
      if (lane < NC) {
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h < sc.G) {
            const float inv = 1.0f / lw[h];
            float* so = slot_out + (size_t)slot * slot_stride + h * D + col * X;
#pragma unroll
            for (int e = 0; e < X; ++e)
              __hip_atomic_store(so + e, pacc[h][e] * inv, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      if (lane == 0) {
        for (int h = 0; h < sc.G && h < GM; ++h) {
          float* ml = slot_ml + ((size_t)slot * sc.G + h) * 2;
          __hip_atomic_store(ml, m_run[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // log2
          __hip_atomic_store(ml + 1, lw[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // every store above has completed
      // ---- the last worker to finish a piece of this pair merges all of them
      const int wa = worker_of(seg_first, U, NWe);
      const int wb = worker_of(seg_first + seg_units - 1, U, NWe);
      int last = 0;
      if (lane == 0)
        last = claim_last(counters + (size_t)s * sc.Hkv + kvh, sc.epoch, (uint32_t)(wb - wa + 1));
      last = uniform(last);  // lane 0's answer
      if (last)
        merge_pair<QDT, D, GM>(slot_out, slot_ml, out, sc, s, kvh, seg_first, wa, wb, U, NWe, lane);
    }
    first_piece = false;
    u = seg_first + j1;
  }
}

// =================================================================================
// Split-KV reduce for fixed partitions: one workgroup per (query head, sequence).
// =================================================================================
template <int D>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, const int32_t* __restrict__ context_lens,
    uint8_t* __restrict__ out, int out_dtype, int Hq, int part_size, int max_parts) {
  extern __shared__ float w_lds[];  // [max_parts] merge weights
  __shared__ float red[kWaves];
  __shared__ float o_lds[kWaves][D];
  const int h = blockIdx.x, s = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  long long cap = (long long)max_parts * part_size;
  long long ctx = context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int np = (int)((ctx + part_size - 1) / part_size);
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
    store_any(out, out_dtype, orow + d, o / L);
  }
}

// ---------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------
namespace {

template <int KVT, int QDT, int D, int GM>
int launch_t(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  if (p.balanced) {
    const size_t lds = ((size_t)p.num_seqs + 1) * sizeof(int);
    dim3 grid((sc.num_workers + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((paged_decode_balanced_kernel<KVT, QDT, D, GM>), grid, dim3(kThreads), lds,
                       st, (const uint8_t*)p.q, (const uint8_t*)p.k_pool,
                       (const uint8_t*)p.v_pool, p.k_scale, p.v_scale, p.block_table,
                       p.context_lens, (uint8_t*)p.out, p.part_out, p.part_max, p.counters, sc);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  dim3 grid(p.max_parts, p.num_kv_heads, p.num_seqs);
  hipLaunchKernelGGL((paged_decode_kernel<KVT, QDT, D, GM>), grid, dim3(kThreads), 0, st,
                     (const uint8_t*)p.q, (const uint8_t*)p.k_pool, (const uint8_t*)p.v_pool,
                     p.k_scale, p.v_scale, p.block_table, p.context_lens, (uint8_t*)p.out,
                     p.part_out, p.part_max, p.part_sum, sc);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int KVT, int QDT, int D>
int pick_g(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  const int G = sc.G;
  if (G <= 1) return launch_t<KVT, QDT, D, 1>(p, sc, st);
  if (G <= 2) return launch_t<KVT, QDT, D, 2>(p, sc, st);
  if (G <= 4) return launch_t<KVT, QDT, D, 4>(p, sc, st);
  if (G <= 8) return launch_t<KVT, QDT, D, 8>(p, sc, st);
  if (G <= 16) return launch_t<KVT, QDT, D, 16>(p, sc, st);
  return -3;
}

template <int KVT, int QDT>
int pick_d(const DecodeLaunch& p, const DecodeScalars& sc, hipStream_t st) {
  if (p.head_dim == 64) return pick_g<KVT, QDT, 64>(p, sc, st);
  if (p.head_dim == 128) return pick_g<KVT, QDT, 128>(p, sc, st);
  return -3;
}

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

}  // namespace

int launch_decode(const DecodeLaunch& p, hipStream_t st) {
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
  sc.scale_log2 = p.scale * kLog2e;
  if (sc.blog2 < 0 || p.block_size > 64) return -3;
  const int kv = p.kv_dtype, qd = p.q_dtype;
  if (kv == DT_F32 && qd == DT_F32) return pick_d<DT_F32, DT_F32>(p, sc, st);
  if (kv == DT_F16 && qd == DT_F16) return pick_d<DT_F16, DT_F16>(p, sc, st);
  if (kv == DT_BF16 && qd == DT_BF16) return pick_d<DT_BF16, DT_BF16>(p, sc, st);
  if (kv == DT_FP8 && qd == DT_BF16) return pick_d<DT_FP8, DT_BF16>(p, sc, st);
  if (kv == DT_FP8 && qd == DT_F16) return pick_d<DT_FP8, DT_F16>(p, sc, st);
  return -3;
}

// ---- resident-worker capacity (device property x kernel occupancy), cached -------
namespace {

template <int KVT, int QDT, int D, int GM>
int blocks_per_cu() {
  static const int v = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&paged_decode_balanced_kernel<KVT, QDT, D, GM>),
            kThreads, 4096) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  return v;
}

template <int KVT, int QDT, int D>
int bpc_g(int G) {
  if (G <= 1) return blocks_per_cu<KVT, QDT, D, 1>();
  if (G <= 2) return blocks_per_cu<KVT, QDT, D, 2>();
  if (G <= 4) return blocks_per_cu<KVT, QDT, D, 4>();
  if (G <= 8) return blocks_per_cu<KVT, QDT, D, 8>();
  return blocks_per_cu<KVT, QDT, D, 16>();
}

template <int KVT, int QDT>
int bpc_d(int D, int G) {
  return D == 64 ? bpc_g<KVT, QDT, 64>(G) : bpc_g<KVT, QDT, 128>(G);
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

int balanced_worker_capacity(int kv, int qd, int D, int G) {
  int bpc = 1;
  if (kv == DT_F32) bpc = bpc_d<DT_F32, DT_F32>(D, G);
  else if (kv == DT_F16) bpc = bpc_d<DT_F16, DT_F16>(D, G);
  else if (kv == DT_BF16) bpc = bpc_d<DT_BF16, DT_BF16>(D, G);
  else if (qd == DT_F16) bpc = bpc_d<DT_FP8, DT_F16>(D, G);
  else bpc = bpc_d<DT_FP8, DT_BF16>(D, G);
  return device_cus() * bpc * kWaves;
}

int launch_split_reduce(const ReduceLaunch& p, hipStream_t st) {
  if (p.max_parts > 8192) return -3;
  dim3 grid(p.num_q_heads, p.num_seqs);
  size_t lds = (size_t)p.max_parts * sizeof(float);
  if (p.head_dim == 64)
    hipLaunchKernelGGL(split_reduce_kernel<64>, grid, dim3(kThreads), lds, st, p.part_out,
                       p.part_max, p.part_sum, p.context_lens, (uint8_t*)p.out, p.out_dtype,
                       p.num_q_heads, p.part_size, p.max_parts);
  else if (p.head_dim == 128)
    hipLaunchKernelGGL(split_reduce_kernel<128>, grid, dim3(kThreads), lds, st, p.part_out,
                       p.part_max, p.part_sum, p.context_lens, (uint8_t*)p.out, p.out_dtype,
                       p.num_q_heads, p.part_size, p.max_parts);
  else
    return -3;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace pkv
