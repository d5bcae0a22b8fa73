// Gate-weighted combine back to token order, and the load-balance statistics.
//
// "Mixture-of-Experts & Sparse Model Scaling", Mathematical Formulation: the
// output is the gate-weighted sum of the selected experts' outputs, and
// L_aux = N * sum_i f_i P_i; "Large Language Models part 09", s.4: f_i and P_i
// over a batch of T tokens; "Mixture-of-experts Models", overflow contract: a
// dropped assignment contributes nothing.  Shared experts add with weight 1.
//
// One block per token gathers its <= k expert rows (each contiguous, 16-byte
// loads) and accumulates in float32 in a fixed order: shared experts first,
// then slot 0, 1, ...; the result is stored in the layer dtype.
#include "launch.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int64_t t = blockIdx.x;
  int dst[8];
  float g[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    dst[s] = s < p.k ? p.dest[t * p.k + s] : -1;
    g[s] = s < p.k ? p.gate[t * p.k + s] : 0.f;
  }
  for (int c = threadIdx.x * 4; c < p.d; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.S; ++s)
      acc += *reinterpret_cast<const f32x4*>(p.y_shared + ((int64_t)s * p.T + t) * p.d + c);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (dst[s] < 0) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.y_rows + (int64_t)dst[s] * p.d + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(g[s], v[j], acc[j]);
    }
    if (p.out_bf16) {
      uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      uint2 pk;
      pk.x = lo;
      pk.y = hi;
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + t * p.d + c) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.y) + t * p.d + c) = acc;
    }
  }
}

// stats = [f (E), P (E), L_aux, drop_rate]; one block, fixed summation order.
__global__ __launch_bounds__(256) void stats_kernel(StatsParams p) {
  __shared__ double prod[256];
  __shared__ long long kept[256];
  const int e = threadIdx.x;
  const double tk = (double)p.T * (double)p.k;
  if (e < p.E) {
    const int c = p.counts[e];
    const double f = (double)c / tk;
    const double P = (double)p.prob_sum[e] / (double)p.T;
    p.stats[e] = (float)f;
    p.stats[p.E + e] = (float)P;
    prod[e] = f * P;
    kept[e] = c < p.C ? c : p.C;
  }
  __syncthreads();
  // slots left unplaced (re-routing): counted over dest in a fixed order
  __shared__ int lost[256];
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
  if (e == 0) {
    double s = 0.0;
    long long ks = 0, ls = 0;
    for (int i = 0; i < p.E; ++i) {
      s += prod[i];
      ks += kept[i];
    }
    for (int i = 0; i < 256; ++i) ls += lost[i];
    p.stats[2 * p.E] = (float)((double)p.E * s);
    p.stats[2 * p.E + 1] = p.dest ? (float)((double)ls / tk) : (float)(1.0 - (double)ks / tk);
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int threads = p.d >= 1024 ? 256 : (p.d >= 512 ? 128 : 64);
  if (p.T > 0)
    hipLaunchKernelGGL(combine_kernel, dim3(p.T), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
