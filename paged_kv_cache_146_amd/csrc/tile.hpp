// tile.hpp — matrix-core and cross-lane helpers shared by the decode and prefill
// kernels of this library (gfx950, wave64).
#pragma once

#include "device.hpp"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float as_f32(uint32_t w) {
  float f;
  __builtin_memcpy(&f, &w, 4);
  return f;
}

// ---- matrix-core products ---------------------------------------------------------
template <int CT>
__device__ __forceinline__ f32x4 mma16(const u32x4 a, const u32x4 b, const f32x4 c) {
  if constexpr (CT == DT_BF16) {
    bf16x8 x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  } else {
    f16x8 x, y;
    __builtin_memcpy(&x, &a, 16);
    __builtin_memcpy(&y, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// two floats -> one packed pair of CT, round to nearest even
template <int CT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  uint32_t w;
  if constexpr (CT == DT_BF16) {
    const bf16x2 b = __builtin_convertvector(v, bf16x2);
    __builtin_memcpy(&w, &b, 4);
  } else {
    const f16x2 h = __builtin_convertvector(v, f16x2);
    __builtin_memcpy(&w, &h, 4);
  }
  return w;
}

// one packed pair of CT -> two floats (exact)
template <int CT>
__device__ __forceinline__ f32x2 unpack2(uint32_t w) {
  if constexpr (CT == DT_BF16) {
    return f32x2{bf16_lo(w), bf16_hi(w)};
  } else {
    return f32x2{f16_lo(w), f16_hi(w)};
  }
}

// eight E4M3 codes (two words) -> eight CT values; exact, as every E4M3 value is
// representable in bf16 and in f16.  The scaled conversion widens two codes per
// instruction; it applies only the power-of-two part of its scale, so with 1.0
// it is the plain widening (checked against every code, NaN included).
template <int CT>
__device__ __forceinline__ u32x4 fp8x8(uint32_t w0, uint32_t w1) {
  if constexpr (CT == DT_F16) {
    const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
    return r;
  } else {
    static_assert(CT == DT_BF16, "fp8 widens to f16 or bf16");
    const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
    return r;
  }
}

// byte B of a word, sign-extended, as f32: one conversion that selects the byte in
// its operand (written out so that the compiler cannot split it into a shift, kept
// alive, and a conversion of byte 0)
template <int B>
__device__ __forceinline__ float sbyte_f32(uint32_t w) {
  float f;
  if constexpr (B == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
        : "=v"(f) : "v"(w));
  else if constexpr (B == 1)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
        : "=v"(f) : "v"(w));
  else if constexpr (B == 2)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
        : "=v"(f) : "v"(w));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
        : "=v"(f) : "v"(w));
  return f;
}

// eight int8 codes (two words) -> eight CT values; exact, as every int8 value is
// an integer of at most 8 bits.  f16: each byte, sign bit flipped (u = x + 128),
// becomes the f16 1024 + u by its bits (one byte permute places two of them under
// the exponent byte 0x64), and a packed subtraction of 1152 leaves x.
// bf16: each byte sign-extended and converted to f32 (one instruction per code:
// the conversion reads the byte in place), then a conversion that is exact.
template <int CT>
__device__ __forceinline__ u32x4 i8x8(uint32_t w0, uint32_t w1) {
  const uint32_t w[2] = {w0, w1};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {  // bytes 2 hp, 2 hp + 1
      if constexpr (CT == DT_F16) {
        const uint32_t x = w[i] ^ 0x80808080u;
        // bytes [u(2 hp), 0x64, u(2 hp + 1), 0x64]: selector values 0-3 take x's
        // bytes, 4 takes a byte of the 0x64 word
        const uint32_t bits =
            __builtin_amdgcn_perm(0x64646464u, x, hp == 0 ? 0x04010400u : 0x04030402u);
        const f16x2 h = __builtin_bit_cast(f16x2, bits);
        r[2 * i + hp] = __builtin_bit_cast(uint32_t, h - f16x2{(_Float16)1152.0f, (_Float16)1152.0f});
      } else {
        static_assert(CT == DT_BF16, "int8 widens to f16 or bf16");
        r[2 * i + hp] = hp == 0 ? pack2<DT_BF16>(sbyte_f32<0>(w[i]), sbyte_f32<1>(w[i]))
                                : pack2<DT_BF16>(sbyte_f32<2>(w[i]), sbyte_f32<3>(w[i]));
      }
    }
  }
  return r;
}

// the 16-bit CT values of eight 8-bit codes of a quantised pool type
template <int KVT, int CT>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  if constexpr (KVT == DT_I8)
    return i8x8<CT>(w0, w1);
  else
    return fp8x8<CT>(w0, w1);
}

// max / sum over the four lane groups {L, L^16, L^32, L^48}; every lane of the
// set gets the same bits (each swap hands both partners the same operand order)
__device__ __forceinline__ float max_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(as_f32(a[0]), as_f32(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(as_f32(b[0]), as_f32(b[1]));
}
__device__ __forceinline__ float sum_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = as_f32(a[0]) + as_f32(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return as_f32(b[0]) + as_f32(b[1]);
}

__device__ __forceinline__ void store_any(uint8_t* out, int dt, size_t idx, float x) {
  if (dt == DT_F32)
    reinterpret_cast<float*>(out)[idx] = x;
  else if (dt == DT_BF16)
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(x);
  else
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(x);
}

// four consecutive output elements starting at idx (a multiple of 4)
__device__ __forceinline__ void store4(uint8_t* out, int dt, size_t idx, const f32x4 v) {
  if (dt == DT_F32) {
    *reinterpret_cast<f32x4*>(out + idx * 4) = v;
  } else {
    const u32x2 w = dt == DT_BF16 ? u32x2{pack2<DT_BF16>(v[0], v[1]), pack2<DT_BF16>(v[2], v[3])}
                                  : u32x2{pack2<DT_F16>(v[0], v[1]), pack2<DT_F16>(v[2], v[3])};
    *reinterpret_cast<u32x2*>(out + idx * 2) = w;
  }
}

__device__ __forceinline__ int clamp_block(int phys, int num_blocks) {
  return phys < 0 ? 0 : (phys >= num_blocks ? num_blocks - 1 : phys);
}

}  // namespace pkv
