// Gate-weighted combine back to token order, and the load-balance statistics.
//
// "Mixture-of-Experts & Sparse Model Scaling", Mathematical Formulation: the
// output is the gate-weighted sum of the selected experts' outputs, and
// L_aux = N * sum_i f_i P_i; "Large Language Models part 09", s.4: f_i and P_i
// over a batch of T tokens; "Mixture-of-experts Models", overflow contract: a
// dropped assignment contributes nothing.  Shared experts add with weight 1.
//
// One block per token gathers its <= k expert rows (each contiguous, 16-byte
// loads; float32 rows, or the bf16 rows a bf16 layer call keeps) and
// accumulates in float32 in a fixed order: shared experts first, then slot 0,
// 1, ...; the result is stored in the layer dtype.
#include "launch.hpp"

namespace moe {

namespace {

// Every expert row is read exactly once, so the loads are non-temporal; each
// slot's row gets a buffer resource of its own (an empty one for a dropped
// slot, whose loads then read zeros and move nothing), and a chunk's loads
// for all slots are issued before the fixed-order accumulation.
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, bytes, 0x00020000);
}

// the VW values of one 16-byte load: float32, or bf16 pairs.  (The element
// is copied to a scalar first: a bit cast applied to a vector element
// expression itself reads element 0 whatever the index.)
template <bool RB>
__device__ __forceinline__ float lane_val(const u32x4& v, int j) {
  if constexpr (RB) {
    const uint32_t w = v[j >> 1];
    return __builtin_bit_cast(float, (j & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    const uint32_t w = v[j];
    return __builtin_bit_cast(float, w);
  }
}

// KM: slots per token the instance handles (k <= KM); RB: expert rows (and
// shared rows) in bf16, 8 columns per 16-byte load instead of 4
template <int KM, bool RB>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int VW = RB ? 8 : 4;   // columns per 16-byte load
  constexpr int ES = RB ? 2 : 4;   // bytes per row element
  const int64_t t = blockIdx.x;
  const int d = p.d;
  const char* rows = static_cast<const char*>(p.y_rows);
  const char* shared = static_cast<const char*>(p.y_shared);
  int dst[KM];
  float g[KM];
  __amdgpu_buffer_rsrc_t rs[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    dst[s] = s < p.k ? p.dest[t * p.k + s] : -1;
    g[s] = s < p.k ? p.gate[t * p.k + s] : 0.f;
    rs[s] = row_rsrc(rows + (int64_t)(dst[s] >= 0 ? dst[s] : 0) * d * ES, dst[s] >= 0 ? d * ES : 0);
  }
  for (int c = threadIdx.x * VW; c < d; c += blockDim.x * VW) {
    float acc[VW];
#pragma unroll
    for (int j = 0; j < VW; ++j) acc[j] = 0.f;
    for (int s = 0; s < p.S; ++s) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
          row_rsrc(shared + ((int64_t)s * p.T + t) * d * ES, d * ES), (uint32_t)c * ES, 0, kNT);
#pragma unroll
      for (int j = 0; j < VW; ++j) acc[j] += lane_val<RB>(v, j);
    }
    u32x4 v[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s) v[s] = __builtin_amdgcn_raw_buffer_load_b128(rs[s], (uint32_t)c * ES, 0, kNT);
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      if (dst[s] < 0) continue;
#pragma unroll
      for (int j = 0; j < VW; ++j) acc[j] = fmaf(g[s], lane_val<RB>(v[s], j), acc[j]);
    }
    if (p.out_bf16) {
      uint32_t w[VW / 2];
#pragma unroll
      for (int j = 0; j < VW / 2; ++j)
        w[j] = (uint32_t)f32_to_bf16(acc[2 * j]) | ((uint32_t)f32_to_bf16(acc[2 * j + 1]) << 16);
      uint16_t* o = static_cast<uint16_t*>(p.y) + t * d + c;
      if constexpr (RB) {
        *reinterpret_cast<u32x4*>(o) = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        uint2 pk;
        pk.x = w[0];
        pk.y = w[1];
        *reinterpret_cast<uint2*>(o) = pk;
      }
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.y) + t * d + c) =
          f32x4{acc[0], acc[1], acc[2], acc[3]};
    }
  }
}

// stats = [f (E), P (E), L_aux, drop_rate]; one block, fixed summation order
// (a pairwise tree over the 256 threads for the sums over experts and over
// the slots left unplaced).
__global__ __launch_bounds__(256) void stats_kernel(StatsParams p) {
  __shared__ double prod[256];
  __shared__ long long kept[256];
  __shared__ int lost[256];
  const int e = threadIdx.x;
  const double tk = (double)p.T * (double)p.k;
  prod[e] = 0.0;
  kept[e] = 0;
  if (e < p.E) {
    const int c = p.counts[e];
    const double f = (double)c / tk;
    const double P = (double)p.prob_sum[e] / (double)p.T;
    p.stats[e] = (float)f;
    p.stats[p.E + e] = (float)P;
    prod[e] = f * P;
    kept[e] = c < p.C ? c : p.C;
  }
  // slots left unplaced (re-routing): counted over dest, each thread a fixed
  // strided subset
  int my_lost = 0;
  if (p.dest) {
    const int64_t n = (int64_t)p.T * p.k, n4 = n >> 2;
    const int4* d4 = reinterpret_cast<const int4*>(p.dest);  // 16-byte aligned
    int64_t i = e;
    for (; i + 3 * 256 < n4; i += 4 * 256) {  // four loads in flight
      const int4 a = d4[i], b = d4[i + 256], c = d4[i + 512], d = d4[i + 768];
      my_lost += (a.x < 0) + (a.y < 0) + (a.z < 0) + (a.w < 0) + (b.x < 0) + (b.y < 0) +
                 (b.z < 0) + (b.w < 0) + (c.x < 0) + (c.y < 0) + (c.z < 0) + (c.w < 0) +
                 (d.x < 0) + (d.y < 0) + (d.z < 0) + (d.w < 0);
    }
    for (; i < n4; i += 256) {
      const int4 v = d4[i];
      my_lost += (v.x < 0) + (v.y < 0) + (v.z < 0) + (v.w < 0);
    }
    for (int64_t i = 4 * n4 + e; i < n; i += 256) my_lost += p.dest[i] < 0;
  }
  lost[e] = my_lost;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) {
      prod[e] += prod[e + o];
      kept[e] += kept[e + o];
      lost[e] += lost[e + o];
    }
    __syncthreads();
  }
  if (e == 0) {
    p.stats[2 * p.E] = (float)((double)p.E * prod[0]);
    p.stats[2 * p.E + 1] = p.dest ? (float)((double)lost[0] / tk) : (float)(1.0 - (double)kept[0] / tk);
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int threads = p.d >= 1024 ? 256 : (p.d >= 512 ? 128 : 64);
  if (p.T > 0) {
    const dim3 g((unsigned)p.T), b((unsigned)threads);
#define MOE_COMBINE(RBV)                                                                   \
  if (p.k <= 1) hipLaunchKernelGGL((combine_kernel<1, RBV>), g, b, 0, stream, p);         \
  else if (p.k <= 2) hipLaunchKernelGGL((combine_kernel<2, RBV>), g, b, 0, stream, p);    \
  else if (p.k <= 4) hipLaunchKernelGGL((combine_kernel<4, RBV>), g, b, 0, stream, p);    \
  else hipLaunchKernelGGL((combine_kernel<8, RBV>), g, b, 0, stream, p);
    // bf16 rows only feed a bf16 output
    if (p.rows_bf16 && !p.out_bf16) return hipErrorInvalidValue;
    if (p.rows_bf16) { MOE_COMBINE(true) } else { MOE_COMBINE(false) }
#undef MOE_COMBINE
  }
  return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
