// Router logits, top-k selection, gates and full-softmax partial sums.
//
// "Mixture-of-Experts & Sparse Model Scaling", Mathematical Formulation: a
// linear router scores every expert, the k best are kept and weighted by their
// softmax scores; "Large Language Models part 09", s.2: optional noise
// eps * softplus(x W_noise) on the logits and a softmax over the selected
// logits; "Mixture-of-experts Models", Level 2: a fixed tie rule.
//
// One block handles 64 tokens.  Phase 1 (skipped when replaying logits) computes
// the [64, E(+E)] logit tile with bf16 MFMA 16x16x32 (float32 accumulate): each
// wave owns 16 tokens and walks all expert columns 64 at a time.  The tile lands
// in LDS, bias and noise are applied and the logits are written out.  Phase 2
// gives every token to one wave: lanes hold experts e = lane + 64j, k rounds of a
// wave-wide argmax on (value desc, index asc) pick the experts, and the same
// registers yield the full softmax whose per-expert sums are reduced per block
// in a fixed order (no atomics, so the result is deterministic).
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// Phase 1, bf16: raw products into sH[m*ldh + n], n < ncols (gate columns,
// then noise columns).
__device__ void router_tile_bf16(const RouteParams& p, float* sH, int ldh, int t_base,
                                 int ncols) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* wg = static_cast<const uint16_t*>(p.w_g);
  const uint16_t* wn = static_cast<const uint16_t*>(p.w_noise);
  const int row = t_base + w * 16 + (lane & 15);
  const bool row_ok = row < p.T;
  const uint16_t* xrow = x + (int64_t)(row_ok ? row : 0) * p.d;
  const int kofs = (lane >> 4) * 8;
  const bf16x8 zero = {};
  for (int nb = 0; nb < ncols; nb += 64) {
    const uint16_t* wrow[4];
    bool n_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      n_ok[j] = n < ncols;
      const int nn = n_ok[j] ? n : 0;
      wrow[j] = nn < p.E ? wg + (int64_t)nn * p.d : wn + (int64_t)(nn - p.E) * p.d;
    }
    f32x4 acc[4] = {};
#pragma unroll 4
    for (int k0 = 0; k0 < p.d; k0 += 32) {
      const int kk = k0 + kofs;
      const bool k_ok = kk < p.d;
      const bf16x8 a = (row_ok && k_ok) ? load_bf16x8(xrow + kk) : zero;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = (n_ok[j] && k_ok) ? load_bf16x8(wrow[j] + kk) : zero;
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    // 16x16 result layout: lane holds column lane%16, rows 4*(lane/16) + i.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      if (n < ncols) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sH[(w * 16 + (lane >> 4) * 4 + i) * ldh + n] = acc[j][i];
      }
    }
  }
}

// Phase 1, float32: plain sequential-k dot products (small fp32 layers).
__device__ void router_tile_f32(const RouteParams& p, float* sH, int ldh, int t_base,
                                int ncols) {
  const float* x = static_cast<const float*>(p.x);
  const float* wg = static_cast<const float*>(p.w_g);
  const float* wn = static_cast<const float*>(p.w_noise);
  for (int i = threadIdx.x; i < kRouteTokens * ncols; i += kThreads) {
    const int m = i / ncols, n = i - m * ncols, t = t_base + m;
    if (t >= p.T) continue;
    const float* xr = x + (int64_t)t * p.d;
    const float* wr = n < p.E ? wg + (int64_t)n * p.d : wn + (int64_t)(n - p.E) * p.d;
    float s = 0.0f;
    for (int c = 0; c < p.d; ++c) s = fmaf(xr[c], wr[c], s);
    sH[m * ldh + n] = s;
  }
}

__global__ __launch_bounds__(kThreads) void route_kernel(RouteParams p) {
  extern __shared__ float sH[];
  __shared__ double sP[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_base = blockIdx.x * kRouteTokens;
  const bool noise = p.w_noise != nullptr;
  const int ncols = p.E * (noise ? 2 : 1);
  const int ldh = ncols + 1;

  if (p.x != nullptr) {
    if (p.bf16) router_tile_bf16(p, sH, ldh, t_base, ncols);
    else router_tile_f32(p, sH, ldh, t_base, ncols);
    __syncthreads();
    for (int i = threadIdx.x; i < kRouteTokens * p.E; i += kThreads) {
      const int m = i / p.E, e = i - m * p.E, t = t_base + m;
      if (t >= p.T) continue;
      float v = sH[m * ldh + e];
      if (p.b_g) v += p.b_g[e];
      if (noise) v += p.eps[(int64_t)t * p.E + e] * softplus_f32(sH[m * ldh + p.E + e]);
      sH[m * ldh + e] = v;
      p.logits[(int64_t)t * p.E + e] = v;
    }
  } else {
    for (int i = threadIdx.x; i < kRouteTokens * p.E; i += kThreads) {
      const int m = i / p.E, e = i - m * p.E, t = t_base + m;
      if (t < p.T) sH[m * ldh + e] = p.logits[(int64_t)t * p.E + e];
    }
  }
  __syncthreads();

  // Phase 2: one token per wave iteration; lane owns experts lane + 64*j.
  const int nj = (p.E + 63) >> 6;
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int mi = 0; mi < 16; ++mi) {
    const int m = w * 16 + mi, t = t_base + m;
    if (t >= p.T) break;
    float v[4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = (j < nj && e < p.E) ? sH[m * ldh + e] : -INFINITY;
      mx = fmaxf(mx, v[j]);
    }
    mx = wave_max(mx);
    float ex[4], s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      ex[j] = (j < nj && e < p.E) ? expf(v[j] - mx) : 0.f;
      s += ex[j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) pacc[j] += ex[j] / s;

    unsigned taken = 0;
    float v0 = 0.f, z = 0.f;
    float my_v = 0.f;
    int my_i = 0;
    for (int sl = 0; sl < p.k; ++sl) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (j < nj && e < p.E && !((taken >> j) & 1u) && (v[j] > bv || bi == 0x7fffffff)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (sl == 0) v0 = bv;
      z += expf(bv - v0);
      if (lane == sl) {
        my_v = bv;
        my_i = bi;
      }
    }
    if (lane < p.k) {
      p.idx[(int64_t)t * p.k + lane] = my_i;
      p.gate[(int64_t)t * p.k + lane] = expf(my_v - v0) / z;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < 256) sP[w][e] = (double)pacc[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += kThreads)
    p.prob_partial[(int64_t)blockIdx.x * p.E + e] =
        (float)(((sP[0][e] + sP[1][e]) + sP[2][e]) + sP[3][e]);
}

// prob_sum[e] = sum over routing blocks, in block order, accumulated in double.
__global__ __launch_bounds__(256) void prob_reduce_kernel(const float* partial, float* out,
                                                          int nblocks, int E) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double s = 0.0;
    for (int b = 0; b < nblocks; ++b) s += (double)partial[(int64_t)b * E + e];
    out[e] = (float)s;
  }
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t stream) {
  const int blocks = route_blocks(p.T);
  const int ncols = p.E * (p.w_noise ? 2 : 1);
  const size_t lds = (size_t)kRouteTokens * (ncols + 1) * sizeof(float);
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kThreads), lds, stream, p);
  hipLaunchKernelGGL(prob_reduce_kernel, dim3(1), dim3(256), 0, stream,
                     (const float*)p.prob_partial, p.prob_sum, blocks, p.E);
  return hipGetLastError();
}

}  // namespace moe
