// decode.hip — paged decode attention for gfx950, plus the split-KV
// log-sum-exp reduce.
//
// Method: "03 | PagedAttention and the KV-cache memory system", §4 — per
// sequence and query head, walk the logical blocks of the visible context,
// look each one up in the block table, load its K/V page, and fold the partial
// attention into an online-softmax state (max, exp_sum, weighted_value); long
// contexts are scanned in parallel partitions whose states are merged.
//
// Work mapping (one workgroup = 4 wavefronts):
//   workgroup  <- (partition, kv head, sequence); all G = H_q/H_kv query heads
//                 of the kv head are handled together, so every K/V byte is
//                 read from HBM once per step (GQA grouping).
//   wavefront  <- 64 consecutive tokens per iteration ("chunk"); the waves of
//                 a workgroup take chunks round-robin inside the partition.
//   QK^T       <- lane = token.  With the K pool laid out
//                 [block][head][D/X][B][X], a lane's 16-byte loads walk its
//                 token's row while the 64 lanes of one load instruction cover
//                 contiguous 16-byte pieces of the pages; the dot product over D
//                 stays inside the lane (no cross-lane reduction).  q is
//                 wave-uniform and read through the scalar cache.
//   softmax    <- chunk max per head by DPP row ops + lane reads; p = 2^(z - m)
//                 with log2(e) folded into the scale.
//   P.V        <- lane = 16-byte slice of one V row (V pool [block][head][B][D]);
//                 each pass covers 64/(D/X) tokens, p comes from LDS.
//   merge      <- per-wave states combined in LDS; the partition's state is
//                 written (split) or normalised into the output (unsplit).
#include "device.hpp"
#include "internal.hpp"

#include <math.h>

#include <type_traits>

namespace pkv {

struct DecodeScalars {
  int W;            // max_blocks_per_seq
  int ctx_cap;      // clamp for context_lens
  int Hq, Hkv, G;
  int blog2;        // log2(block_size)
  int num_blocks;
  int part_size;    // tokens per partition, multiple of 64
  int max_parts;
  int split;
  int out_dtype;
  float scale_log2; // softmax scale * log2(e)
};

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <int DT>
__device__ __forceinline__ void store_out(uint8_t* out, size_t idx, float x);

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

template <int KVT, int QDT, int D, int GM>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, uint8_t* __restrict__ out,
    float* __restrict__ part_out, float* __restrict__ part_max, float* __restrict__ part_sum,
    const DecodeScalars sc) {
  constexpr int X = Elem<KVT>::per16;     // elements per 16 bytes
  constexpr int ES = Elem<KVT>::bytes;
  constexpr int NC = D / X;               // 16-byte chunks per K row (= lanes per V row)
  constexpr int R = 64 / NC;              // V rows per pass
  constexpr int NPASS = 64 / R;           // passes per 64-token chunk
  constexpr int QES = (QDT == DT_F32) ? 4 : 2;
  constexpr bool kFp8 = (KVT == DT_FP8);
  static_assert(NC <= 64 && 64 % NC == 0, "row must split into 16-byte lane slices");

  __shared__ float p_lds[kWaves][64][GM];
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

  // query rows of this kv head's group (wave-uniform addresses)
  const uint8_t* qrow[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    int hq = kvh * sc.G + (h < sc.G ? h : sc.G - 1);
    qrow[h] = q + ((size_t)s * sc.Hq + hq) * D * QES;
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

  auto chunk = [&](int cbase, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // ---- token-lane addressing: one token per lane --------------------------------
    const int t = cbase + lane;
    const bool valid = !MASK || t < t_end;
    const int tt = valid ? t : cbase;  // masked lanes read a valid token's page
    int phys = trow[tt >> sc.blog2];
    phys = phys < 0 ? 0 : (phys >= sc.num_blocks ? sc.num_blocks - 1 : phys);
    const size_t page = (size_t)phys * sc.Hkv + kvh;
    const int off = tt & (B - 1);
    const u32x4* kp = reinterpret_cast<const u32x4*>(k_pool) + (page * NC * B + off);
    const uint32_t vrow = (uint32_t)(page * B + off);

    u32x4 kr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = kp[(size_t)c * B];

    // V rows of this lane's passes: token i*R + r of the chunk
    u32x4 vr[NPASS];
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      uint32_t rowi = (uint32_t)__builtin_amdgcn_ds_bpermute((i * R + r) << 2, (int)vrow);
      vr[i] = *(reinterpret_cast<const u32x4*>(v_pool + (size_t)rowi * (D * ES)) + col);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) materialize(kr[c]);

    // ---- scores ---------------------------------------------------------------
    float acc[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (KVT == DT_BF16 || KVT == DT_F16) {
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const u32x4 qv = *(reinterpret_cast<const u32x4*>(qrow[h]) + c);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t kw = kr[c][w], qw = qv[w];
            if constexpr (KVT == DT_BF16)
              acc[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw), as_bf16x2(qw), acc[h],
                                                       false);
            else
              acc[h] = __builtin_amdgcn_fdot2(as_f16x2(kw), as_f16x2(qw), acc[h], false);
          }
        }
      } else {
        float kf[X];
        unpack16<KVT>(kr[c], kf);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          float qf[X];
          q_chunk_f32<QDT, X>(qrow[h], c, qf);
#pragma unroll
          for (int e = 0; e < X; ++e) acc[h] = fmaf(kf[e], qf[e], acc[h]);
        }
      }
    }
    float zscale = sc.scale_log2;
    float vs = 1.0f;
    if constexpr (kFp8) {
      zscale *= k_scale[page];
      vs = v_scale[page];
    }

    // ---- online softmax per head; p to LDS ------------------------------------
    float* pl = &p_lds[wave][lane][0];
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
      pl[h] = kFp8 ? p * vs : p;
    }
    wave_lds_sync();

    // ---- P.V ------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int tok = i * R + r;
      float vf[X];
      unpack16<KVT>(vr[i], vf);
      if constexpr (MASK) {
        const bool vvalid = cbase + tok < t_end;
#pragma unroll
        for (int e = 0; e < X; ++e) vf[e] = vvalid ? vf[e] : 0.0f;
      }
      const float* pt = &p_lds[wave][tok][0];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        const float ph = pt[h];
#pragma unroll
        for (int e = 0; e < X; ++e) pacc[h][e] = fmaf(ph, vf[e], pacc[h][e]);
      }
    }
    wave_lds_sync();  // p_lds is rewritten by the next chunk
  };

  for (int cbase = t_begin + wave * 64; cbase < t_end; cbase += kThreads) {
    if (cbase + 64 <= t_end)
      chunk(cbase, std::integral_constant<bool, false>{});
    else
      chunk(cbase, std::integral_constant<bool, true>{});
  }

  // ---- combine the rows of each wave, then the waves --------------------------
#pragma unroll
  for (int h = 0; h < GM; ++h) {
#pragma unroll
    for (int e = 0; e < X; ++e) {
#pragma unroll
      for (int o = NC; o < 64; o <<= 1) pacc[h][e] += __shfl_xor(pacc[h][e], o);
    }
  }
  float lw[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) lw[h] = wave_sum(l_lane[h]);
  if (lane < NC) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
#pragma unroll
      for (int e = 0; e < X; ++e) c_acc[wave][h][col * X + e] = pacc[h][e];
    }
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

// ---------------------------------------------------------------------------------
// Split-KV reduce: one workgroup per (query head, sequence).
// ---------------------------------------------------------------------------------
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
  sc.Hq = p.num_q_heads;
  sc.Hkv = p.num_kv_heads;
  sc.G = p.num_q_heads / p.num_kv_heads;
  sc.blog2 = log2_exact(p.block_size);
  sc.num_blocks = p.num_blocks;
  sc.part_size = p.part_size;
  sc.max_parts = p.max_parts;
  sc.split = p.split;
  sc.out_dtype = p.q_dtype;
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

int launch_split_reduce(const ReduceLaunch& p, hipStream_t st) {
  if (p.max_parts > 16384) return -3;
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
