// device.hpp — gfx950 device helpers for the paged KV-cache kernels.
//
// Element codecs, 16-byte vector types and wavefront (64-lane) reductions built
// on DPP row operations plus lane reads.  Used by the kernels of this library
// only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_I8 = 4 };
// where a quantised element's scale lives (the C ABI's pkv_scale_mode)
enum : int { SCALE_BLOCK = 0, SCALE_TENSOR = 1, SCALE_TOKEN = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bytes per element and elements per 16-byte vector for each storage type
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4, per16 = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2, per16 = 8; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2, per16 = 8; };
template <> struct Elem<DT_FP8> { static constexpr int bytes = 1, per16 = 16; };
template <> struct Elem<DT_I8> { static constexpr int bytes = 1, per16 = 16; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reinterpret one 32-bit word as a packed pair.  The word is taken BY VALUE on
// purpose: with this compiler, __builtin_bit_cast applied directly to a vector
// element subscript v[i] inside an unrolled loop reads element 0 for every i.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  bf16x2 r;
  __builtin_memcpy(&r, &w, 4);
  return r;
}
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) {
  f16x2 r;
  __builtin_memcpy(&r, &w, 4);
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Unpack the 16-byte vector `v` of storage type DT into per16 floats (exact).
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4& v, float* out) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(v[i]);
      out[2 * i + 1] = bf16_hi(v[i]);
    }
  } else if constexpr (DT == DT_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = f16_lo(v[i]);
      out[2 * i + 1] = f16_hi(v[i]);
    }
  } else {  // OCP E4M3 -> f32 with the gfx950 packed converter (bytes 0,1 then 2,3)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], false);
      f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i], true);
      out[4 * i + 0] = a[0];
      out[4 * i + 1] = a[1];
      out[4 * i + 2] = b[0];
      out[4 * i + 3] = b[1];
    }
  }
}

// fp32 -> storage bits, round to nearest even (f16 and bf16; NaN kept NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// fp32 -> OCP E4M3 code: round to nearest, ties to even; |y| >= 448 and
// infinities saturate to +-448; NaN -> 0x7F with the sign bit of y.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // 448.0f
  if (a < 0x3c800000u) {                      // below 2^-6: subnormal codes m * 2^-9
    float t = __uint_as_float(a) * 512.0f;    // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(t);  // rint: nearest, ties to even
  }
  uint32_t mant = a & 0x7fffffu;
  uint32_t code = (((a >> 23) - 120u) << 3) | (mant >> 20);
  uint32_t rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;  // carry may bump exponent
  return sign | code;
}

// ---- wavefront reductions -------------------------------------------------
// DPP controls (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// all 16 lanes of each row end with the row's max / sum
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowRor4>(x));
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  return x;
}

// a value the caller knows to be equal in all lanes, made provably wave-uniform
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float lane_read(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// wave-uniform max / sum over all 64 lanes
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  float a = fmaxf(lane_read(x, 0), lane_read(x, 16));
  float b = fmaxf(lane_read(x, 32), lane_read(x, 48));
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}

// Keep a 16-byte value whole in registers at this point.  Without it the
// optimiser may split a 16-byte load whose lanes are only read one word at a
// time into four 4-byte loads issued next to their uses, which serialises the
// memory latency; with it every load issued before the call stays one
// dwordx4 request in flight.
__device__ __forceinline__ void materialize(u32x4& v) { asm volatile("" : "+v"(v)); }

// Compiler-only fence: no instruction is moved across it (neither memory
// operations nor arithmetic; a plain memory clobber would still let matrix-core
// products float above the loads).  Pins where a software-pipelined loop issues
// its next loads relative to the products that consume the current ones.
__device__ __forceinline__ void issue_point() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Synchronise the lanes of this wave: every lane's memory operations before the
// call happen before every lane's operations after it (a wave-local exchange
// through LDS, or one lane's release / acquire on behalf of the wave).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ void wave_lds_sync() { wave_sync(); }

}  // namespace pkv
