// Router logits, top-k selection, gates and full-softmax partial sums.
//
// "Mixture-of-Experts & Sparse Model Scaling", Mathematical Formulation: a
// linear router scores every expert, the k best are kept and weighted by their
// softmax scores; "Large Language Models part 09", s.2: optional noise
// eps * softplus(x W_noise) on the logits and a softmax over the selected
// logits; "Mixture-of-experts Models", Level 2: a fixed tie rule.
//
// One block handles 16 tokens with up to 16 waves.  Phase 1 (skipped when
// replaying logits) computes the [16, E(+E)] logit tile with bf16 MFMA 16x16x32
// (float32 accumulate): the waves split the model width into contiguous
// ranges, so even a decode batch of a few tokens keeps many waves streaming x
// and W_g, and wide tiles (more than 64 columns) also give their 64-column
// groups to different waves; the partial tiles are summed in LDS in a fixed
// order.  Bias and
// noise are applied and the logits written out.  Phase 2 gives every token to
// one wave: lanes hold experts e = lane + 64j, k rounds of a wave-wide argmax
// on (value desc, index asc) pick the experts, and the same registers yield
// the full softmax, whose per-expert sums over the block's tokens are written
// per block and reduced in a fixed order by a second kernel (no atomics, so
// results are deterministic).
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kMaxThreads = 64 * kMaxWaves;
constexpr uint32_t kOOB = 0x80000000u;

// Phase 1, bf16: this wave's partial products over its model-width range into
// part[m*ldh + n] (gate columns, then noise columns).  The block's waves form
// nk x nc: nk contiguous model-width ranges, and nc interleaved sets of
// 64-column groups (wide tiles: the column groups run in parallel instead of
// one after another); wave w takes range w % nk and set w / nk.
__device__ void router_tile_bf16(const RouteParams& p, float* part, int ldh, int t_base,
                                 int ncols, int nk, int nc) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wid % nk, wc = wid / nk;
  const int d = p.d;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.x), (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.w_g), (short)0, (int)((int64_t)p.E * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t nr = p.w_noise ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.w_noise), (short)0, (int)((int64_t)p.E * d * 2), 0x00020000) : gr;
  const int row = t_base + (lane & 15);
  const int kofs = (lane >> 4) * 8;
  const uint32_t a_base = row < p.T ? (uint32_t)row * (uint32_t)d * 2u : kOOB;
  // contiguous model-width range of this wave, in steps of 32
  const int steps = (d + 31) / 32, per = (steps + nk - 1) / nk;
  const int kb = w * per * 32, ke = min(d, (w + 1) * per * 32);
  for (int nb = wc * 64; nb < ncols; nb += nc * 64) {
    uint32_t b_base[4];
    bool noise_col[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      noise_col[j] = n >= p.E;
      const int nn = noise_col[j] ? n - p.E : n;
      b_base[j] = n < ncols ? (uint32_t)nn * (uint32_t)d * 2u : kOOB;
    }
    f32x4 acc[4] = {};
    // batches of 3 steps: all of a batch's loads are issued before its MFMAs
    // (steps past the range read zeros), so a wave waits for memory once per
    // batch rather than once per step
    constexpr int kBatch = 3;
    for (int k0 = kb; k0 < ke; k0 += 32 * kBatch) {
      bf16x8 a[kBatch];
      u32x4 bv[kBatch][4];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int kk = k0 + u * 32 + kofs;
        const uint32_t kadd = kk < ke ? (uint32_t)kk * 2u : kOOB;
        a[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, a_base + kadd, 0, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[u][j] = noise_col[j] ? __builtin_amdgcn_raw_buffer_load_b128(nr, b_base[j] + kadd, 0, 0)
                                  : __builtin_amdgcn_raw_buffer_load_b128(gr, b_base[j] + kadd, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], __builtin_bit_cast(bf16x8, bv[u][j]),
                                                          acc[j], 0, 0, 0);
    }
    // 16x16 result layout: lane holds column lane%16, rows 4*(lane/16) + i.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      if (n < ncols) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[((lane >> 4) * 4 + i) * ldh + n] = acc[j][i];
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
  for (int i = threadIdx.x; i < kRouteTokens * ncols; i += blockDim.x) {
    const int m = i / ncols, n = i - m * ncols, t = t_base + m;
    if (t >= p.T) continue;
    const float* xr = x + (int64_t)t * p.d;
    const float* wr = n < p.E ? wg + (int64_t)n * p.d : wn + (int64_t)(n - p.E) * p.d;
    float s = 0.0f;
    for (int c = 0; c < p.d; ++c) s = fmaf(xr[c], wr[c], s);
    sH[m * ldh + n] = s;
  }
}

__global__ __launch_bounds__(kMaxThreads) void route_kernel(RouteParams p) {
  extern __shared__ float lds[];  // nw partial tiles [16][ldh]; tile 0 becomes the logits
  __shared__ float sP[kMaxWaves][256];  // per-wave probability sums (float)
  const int nt = blockDim.x, nw = nt >> 6;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_base = blockIdx.x * kRouteTokens;
  const bool noise = p.w_noise != nullptr;
  const int ncols = p.E * (noise ? 2 : 1);
  const int ldh = ncols + 1;
  const int tile = kRouteTokens * ldh;
  float* sH = lds;

  if (p.x != nullptr) {
    if (p.bf16) {
      // wide tiles: up to 4 column-group sets, the rest of the waves split
      // the model width; every (range, column) partial lands in tile w % nk
      const int nc = ncols > 64 ? min(4, min(nw, (ncols + 63) / 64)) : 1;
      const int nk = nw / nc;
      router_tile_bf16(p, lds + (w % nk) * tile, ldh, t_base, ncols, nk, nc);
      __syncthreads();
      for (int i = threadIdx.x; i < tile; i += nt) {
        float v = lds[i];
        for (int q = 1; q < nk; ++q) v += lds[q * tile + i];  // fixed order
        sH[i] = v;
      }
    } else {
      router_tile_f32(p, sH, ldh, t_base, ncols);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kRouteTokens * p.E; i += nt) {
      const int m = i / p.E, e = i - m * p.E, t = t_base + m;
      if (t >= p.T) continue;
      float v = sH[m * ldh + e];
      if (p.b_g) v += p.b_g[e];
      if (noise) {
        const float n = sH[m * ldh + p.E + e];
        v += p.eps[(int64_t)t * p.E + e] * softplus_f32(n);
        if (p.noise_pre) p.noise_pre[(int64_t)t * p.E + e] = n;
      }
      sH[m * ldh + e] = v;
      p.logits[(int64_t)t * p.E + e] = v;
    }
  } else {
    for (int i = threadIdx.x; i < kRouteTokens * p.E; i += nt) {
      const int m = i / p.E, e = i - m * p.E, t = t_base + m;
      if (t < p.T) sH[m * ldh + e] = p.logits[(int64_t)t * p.E + e];
    }
  }
  __syncthreads();

  // Phase 2: one token per wave iteration; lane owns experts lane + 64*j.
  const int nj = (p.E + 63) >> 6;
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
  const int tpw = kRouteTokens / nw;  // tokens per wave
  for (int mi = 0; mi < tpw; ++mi) {
    const int m = w * tpw + mi, t = t_base + m;
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
    if (e < 256) sP[w][e] = pacc[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.E; e += nt) {
    double v = (double)sP[0][e];
    for (int q = 1; q < nw; ++q) v += (double)sP[q][e];  // fixed order, double
    p.prob_partial[(int64_t)blockIdx.x * p.E + e] = (float)v;
  }
}

// prob_sum[e] = sum over routing blocks: one wave per expert, each lane sums a
// fixed strided subset in double, then a fixed butterfly; deterministic.
__global__ __launch_bounds__(256) void prob_reduce_kernel(const float* partial, float* out,
                                                          int nblocks, int E) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;
  double s = 0.0;
  for (int b = lane; b < nblocks; b += 64) s += (double)partial[(int64_t)b * E + e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) out[e] = (float)s;
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t stream) {
  const int blocks = route_blocks(p.T);
  const int ncols = p.E * (p.w_noise ? 2 : 1);
  const size_t tile = (size_t)kRouteTokens * (ncols + 1) * sizeof(float);
  // bf16 tiles: up to 4 column-group sets run in parallel (wide tiles) and
  // the other waves split the model width, 16 waves in all unless the
  // partial tiles (one per width range) and the 16 KiB of probability
  // partials outgrow the 160 KiB of LDS; narrow tiles give up width ranges
  // (down to 8) so that two blocks share a CU.  float32 and replay use 4
  // waves and one tile.
  const bool mma = p.bf16 && p.x;
  const int nc = (mma && ncols > 64) ? std::min(4, (ncols + 63) / 64) : 1;
  int nk = mma ? kMaxWaves / nc : 4;
  const size_t fixed = sizeof(float) * kMaxWaves * 256, cap = 160 * 1024;
  while (mma && nk > 1 && nk * tile + fixed > cap) nk >>= 1;
  while (mma && nc == 1 && nk > 8 && 2 * (nk * tile + fixed) > cap) nk >>= 1;
  const int nw = mma ? nk * nc : 4;
  const size_t lds = (mma ? nk : 1) * tile;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(64 * nw), lds, stream, p);
  hipLaunchKernelGGL(prob_reduce_kernel, dim3((p.E + 3) / 4), dim3(256), 0, stream,
                     (const float*)p.prob_partial, p.prob_sum, blocks, p.E);
  return hipGetLastError();
}

}  // namespace moe
