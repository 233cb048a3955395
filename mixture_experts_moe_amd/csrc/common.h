// Device-side helpers shared by the gfx950 kernels of the fused MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // bf16 bit pattern as stored in memory
typedef uint8_t fp8_t;    // OCP e4m3fn byte

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two e4m3fn bytes (the low or high 16 bits of q) -> two bf16 values packed
// in one 32-bit word, exactly (every e4m3fn value is a bf16 value).  gfx950
// converts OCP e4m3fn in hardware; scale 1.0 leaves the value unchanged.
// Results are kept as whole packed words (never split into elements).
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t q, bool high) {
  return high ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false));
}

// Eight e4m3fn bytes (two words) -> one MFMA operand fragment of eight bf16.
__device__ __forceinline__ uint4 e4m3x8_to_frag_bits(uint32_t lo, uint32_t hi) {
  return uint4{e4m3x2_to_bf16x2(lo, false), e4m3x2_to_bf16x2(lo, true),
               e4m3x2_to_bf16x2(hi, false), e4m3x2_to_bf16x2(hi, true)};
}

__device__ __forceinline__ bf16x8 as_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- MFMA

// D(16x16,f32) += A(16x32,bf16) * B(32x16,bf16).  Lane l supplies A row l%16
// and B column l%16, both for k = 8*(l/16) .. +8; it receives D column l%16,
// rows 4*(l/16) .. +4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16,f32) += A(16x4,f32) * B(4x16,f32).  Lane l supplies A row l%16 and
// B column l%16 for k = l/16; D layout as above.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace moe
