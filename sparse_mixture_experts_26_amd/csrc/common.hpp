// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, vector
// types, wave reductions and the launch descriptors passed between the C ABI
// layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's uint4 is a wrapper struct the optimiser cannot
// always keep in registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float softplus_f32(float z) {
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ float gelu_f32(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.70710678118654752440f));
}

// Activation codes match moe_act_t.
__device__ __forceinline__ float apply_act(int act, float a, float u) {
  if (act == 2) return silu_f32(a) * u;
  if (act == 1) return fmaxf(a, 0.0f);
  return gelu_f32(a);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// One entry of the grouped-GEMM tile schedule: `rows` (<= tile height) rows
// of weight group `group`, reading operand rows from a_row0 and writing
// output rows from c_row0.
struct TileEntry {
  int32_t group;
  int32_t a_row0;
  int32_t rows;
  int32_t c_row0;
};

}  // namespace moe
