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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
// gfx950 converts in one instruction (v_cvt_pk_bf16_f32, two values at once
// when the compiler can pair them).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float softplus_f32(float z) {
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}

// 1 / (1 + e^-a) from the hardware base-2 exponential and reciprocal (each
// within about an ulp); e^-a = 2^(-a log2 e).  Large positive a gives 1, large
// negative a gives 0, as the exact function does in float32.
__device__ __forceinline__ float sigmoid_f32(float a) {
  const float e = __builtin_amdgcn_exp2f(-a * 1.44269504088896340736f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float silu_f32(float a) { return a * sigmoid_f32(a); }

__device__ __forceinline__ float gelu_f32(float a) {
  return 0.5f * a * (1.0f + erff(a * 0.70710678118654752440f));
}

// Activation codes match moe_act_t.
__device__ __forceinline__ float apply_act(int act, float a, float u) {
  if (act == 2) return silu_f32(a) * u;
  if (act == 1) return fmaxf(a, 0.0f);
  return gelu_f32(a);
}

// Backward of the activation: from dh (gradient of the hidden value) and the
// pre-activations u (v: the SwiGLU up projection), the gradients du and dv.
//   GELU   d/du u Phi(u) = Phi(u) + u phi(u)
//   ReLU   [u > 0]
//   SwiGLU d/du silu(u) v = v s (1 + u (1 - s)), d/dv = silu(u), s = 1/(1+e^-u)
__device__ __forceinline__ void act_backward(int act, float dh, float u, float v, float& du,
                                             float& dv) {
  dv = 0.0f;
  if (act == 2) {
    const float s = sigmoid_f32(u);
    du = dh * v * s * (1.0f + u * (1.0f - s));
    dv = dh * u * s;
  } else if (act == 1) {
    du = u > 0.0f ? dh : 0.0f;
  } else {
    const float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752440f));
    const float pdf = 0.39894228040143267794f * expf(-0.5f * u * u);
    du = dh * (cdf + u * pdf);
  }
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

// DPP lane permutations within each 16-lane row: swap neighbours (quad
// permutation [1,0,3,2]), swap pairs ([2,3,0,1]), reverse each half row,
// reverse the row.  Applied in that order they leave every lane of a row
// combined with all 16 lanes of its row.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);  // every source lane exists
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Maximum and sum over the wave, the same value in every lane.  The sum's
// order is fixed: pairs, quads, half rows, rows, then (row 0 + row 1) +
// (row 2 + row 3).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
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

// Reduction layout of one group for the weight gradients: its rows are
// rows [row0, row0 + rows) of the row-major operands, and in the transposed
// operands (feature-major, one block per group) its block starts at column
// poff of a feature row and holds kp = rows rounded up to 64 (zero padded).
struct GroupDesc {
  int32_t poff;
  int32_t kp;
  int32_t row0;
  int32_t rows;
};

}  // namespace moe
