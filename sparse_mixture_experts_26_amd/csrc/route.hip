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
// results are deterministic).  Phase 2's wave reductions run within 16-lane
// rows on DPP lane permutations (register-speed, where a general shuffle
// goes through the LDS crossbar and costs a round trip per step), and the
// four row results are read as scalars and combined in a fixed order.
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kMaxThreads = 64 * kMaxWaves;
constexpr uint32_t kOOB = 0x80000000u;

// (value desc, index asc): the candidate (ov, oi) beats (bv, bi).  A strict
// total order on distinct indices, so any reduction order picks the same one.
__device__ __forceinline__ void take_better(float& bv, int& bi, float ov, int oi) {
  const bool win = (ov > bv) | ((ov == bv) & (oi < bi));  // both sides evaluated: no branch
  bv = win ? ov : bv;
  bi = win ? oi : bi;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  take_better(bv, bi, dpp<CTRL>(bv), dpp<CTRL>(bi));
}
// the wave's best (value, index), the same in every lane
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_step<kDppXor1>(bv, bi);
  argmax_step<kDppXor2>(bv, bi);
  argmax_step<kDppHalfMirror>(bv, bi);
  argmax_step<kDppMirror>(bv, bi);
  float v = lane_value(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    take_better(v, i, lane_value(bv, r), __builtin_amdgcn_readlane(bi, r));
  bv = v;
  bi = i;
}

// Phase 1, bf16: this wave's partial products over its model-width range into
// part[m*ldh + n] (gate columns, then noise columns).  The block's waves form
// nk x nc: nk contiguous model-width ranges, and nc interleaved sets of
// 64-column groups (wide tiles: the column groups run in parallel instead of
// one after another); wave w takes range w % nk and set w / nk.  NJ: 16-column
// groups per 64-column set that can hold columns (narrow tiles skip the rest);
// NOISE: the tile has noise columns, so each group loads from both sets (a
// lane's offset into the set its column is not in reads zeros) and ORs them.
template <int NJ, bool NOISE>
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
  const __amdgpu_buffer_rsrc_t nr = NOISE ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.w_noise), (short)0, (int)((int64_t)p.E * d * 2), 0x00020000) : gr;
  const int row = t_base + (lane & 15);
  const int kofs = (lane >> 4) * 8;
  const uint32_t a_base = row < p.T ? (uint32_t)row * (uint32_t)d * 2u : kOOB;
  // contiguous model-width range of this wave, in steps of 32
  const int steps = (d + 31) / 32, per = (steps + nk - 1) / nk;
  const int kb = w * per * 32, ke = min(d, (w + 1) * per * 32);
  for (int nb = wc * 64; nb < ncols; nb += nc * 64) {
    // Column n < E is gate row n, E <= n < 2E noise row n - E: each lane has
    // an offset into both sets, out of range in the set its column is not in.
    uint32_t g_off[NJ], n_off[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      g_off[j] = n < p.E ? (uint32_t)n * (uint32_t)d * 2u : kOOB;
      n_off[j] = (NOISE && n >= p.E && n < ncols) ? (uint32_t)(n - p.E) * (uint32_t)d * 2u : kOOB;
    }
    f32x4 acc[NJ] = {};
    // batches of 3 steps (2 for 4 groups with noise, within the 16-wave
    // block's 128 registers): all of a batch's loads are issued before its
    // MFMAs (steps past the range read zeros), so a wave waits for memory once
    // per batch rather than once per step
    constexpr int kBatch = (NOISE && NJ == 4) ? 2 : 3;
    for (int k0 = kb; k0 < ke; k0 += 32 * kBatch) {
      bf16x8 a[kBatch];
      u32x4 bg[kBatch][NJ], bn[kBatch][NJ];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        // past the range every offset is out of range (no sum of two
        // out-of-range offsets, which could wrap into range)
        const int kk = k0 + u * 32 + kofs;
        const bool kin = kk < ke;
        const uint32_t kk2 = (uint32_t)kk * 2u;
        a[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            xr, kin ? a_base + kk2 : kOOB, 0, 0));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          bg[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
              gr, kin && g_off[j] != kOOB ? g_off[j] + kk2 : kOOB, 0, 0);
          if constexpr (NOISE)
            bn[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
                nr, kin && n_off[j] != kOOB ? n_off[j] + kk2 : kOOB, 0, 0);
        }
      }
      // keep the batch's loads ahead of its MFMAs (the scheduler would
      // otherwise pair each load with its use and wait on it)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          u32x4 b = bg[u][j];
          if constexpr (NOISE) b |= bn[u][j];
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], __builtin_bit_cast(bf16x8, b),
                                                          acc[j], 0, 0, 0);
        }
    }
    // 16x16 result layout: lane holds column lane%16, rows 4*(lane/16) + i.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = nb + j * 16 + (lane & 15);
      if (n < ncols) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[((lane >> 4) * 4 + i) * ldh + n] = acc[j][i];
      }
    }
  }
}

// Router logits of a large bf16 batch, ahead of route_kernel's replay form.
// The fused kernel's 16-token blocks each read the whole router matrix, so a
// batch of T tokens reads it T/16 times from L2 (a 128-expert noisy router
// over 4096 tokens: 100 MB; 64 experts over 16384 tokens: 268 MB).  Here a
// block takes 64 tokens and one block of columns: EB experts' gate rows (and,
// with noise, the same experts' noise rows), 16 NG weight rows in all.  Its KW
// waves split the model width into contiguous ranges and each computes the
// whole 64 x 16NG tile over its range (4 x NG tiles of
// v_mfma_f32_16x16x32_bf16, float32 accumulate), so no operand is loaded
// twice within a block; the KW partial tiles are summed in LDS in wave order
// (fixed, deterministic), then bias and noise are applied as in the fused
// kernel and the logits (and the pre-softplus noise sums) written out.
// Columns: gate expert e0 + c for c < EB; with noise, noise expert e0 + c - EB
// for EB <= c < 2 EB (EB = 8 NG with noise, 16 NG without).
constexpr int kLogitRows = 64;
#ifndef MOE_LOGIT_WAVES
#define MOE_LOGIT_WAVES 8
#endif
constexpr int kLogitWaves = MOE_LOGIT_WAVES;
template <int NG, bool NOISE, int KW>
__global__ __launch_bounds__(64 * KW) void router_logits_kernel(RouteParams p) {
  constexpr int NC = 16 * NG, EB = NOISE ? NC / 2 : NC, LD = NC + 1;
  __shared__ float part[KW][kLogitRows * LD];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kLogitRows, e0 = blockIdx.y * EB;
  const int d = p.d;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.x), (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.w_g), (short)0, (int)((int64_t)p.E * d * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t nr = NOISE ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.w_noise), (short)0, (int)((int64_t)p.E * d * 2), 0x00020000) : gr;
  const int kofs = (lane >> 4) * 8;
  uint32_t a_off[4], b_off[NG];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = t0 + 16 * m + (lane & 15);
    a_off[m] = t < p.T ? (uint32_t)t * (uint32_t)d * 2u : kOOB;
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int e = e0 + (16 * j) % EB + (lane & 15);
    b_off[j] = e < min(p.E, e0 + EB) ? (uint32_t)e * (uint32_t)d * 2u : kOOB;
  }
  // this wave's contiguous model-width range, in steps of 32
  const int steps = (d + 31) / 32, per = (steps + KW - 1) / KW;
  const int kb = w * per * 32, ke = min(d, (w + 1) * per * 32);
  f32x4 acc[4][NG] = {};
  // batches of kBatch steps: all of a batch's loads are issued before its
  // MFMAs, so a wave waits for memory once per batch
  constexpr int kBatch = NG >= 4 ? 4 : 6;
  for (int k0 = kb; k0 < ke; k0 += 32 * kBatch) {
    bf16x8 a[kBatch][4], b[kBatch][NG];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int kk = k0 + u * 32 + kofs;
      const bool kin = kk < ke;
      const uint32_t kk2 = (uint32_t)kk * 2u;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        a[u][m] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            xr, kin && a_off[m] != kOOB ? a_off[m] + kk2 : kOOB, 0, 0));
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        // gate rows, then (with noise) the noise rows of the same experts
        const bool from_noise = NOISE && j >= NG / 2;
        b[u][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            from_noise ? nr : gr, kin && b_off[j] != kOOB ? b_off[j] + kk2 : kOOB, 0, 0));
      }
    }
    // keep the batch's loads ahead of its MFMAs (the scheduler would otherwise
    // pair each load with its use and wait on it, one load in flight at a time)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < NG; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][m], b[u][j], acc[m][j], 0, 0, 0);
  }
  // 16x16 result layout: lane holds column lane%16, rows 4*(lane/16) + i
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part[w][(16 * m + 4 * (lane >> 4) + i) * LD + 16 * j + (lane & 15)] = acc[m][j][i];
  __syncthreads();
  // thread -> column c = tid % EB, rows tid / EB + (64 KW / EB) i: the bias
  // is loaded once and every eps load of the thread is issued before any is
  // used
  constexpr int RS = 64 * KW / EB, NR = kLogitRows / RS;
  const int c = threadIdx.x % EB, r0 = threadIdx.x / EB, e = e0 + c;
  const bool col_ok = e < p.E;
  const float bias = (p.b_g && col_ok) ? p.b_g[e] : 0.f;
  float eps[NR];
  if constexpr (NOISE) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int t = t0 + r0 + RS * i;
      eps[i] = (col_ok && t < p.T) ? p.eps[(int64_t)t * p.E + e] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + RS * i, t = t0 + r;
    if (!col_ok || t >= p.T) continue;
    const int o = r * LD + c;
    float v = part[0][o];
#pragma unroll
    for (int q = 1; q < KW; ++q) v += part[q][o];  // wave order
    v += bias;
    if constexpr (NOISE) {
      const int on = o + EB;
      float n = part[0][on];
#pragma unroll
      for (int q = 1; q < KW; ++q) n += part[q][on];
      v += eps[i] * softplus_f32(n);
      if (p.noise_pre) p.noise_pre[(int64_t)t * p.E + e] = n;
    }
    p.logits[(int64_t)t * p.E + e] = v;
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

// Phase 2 for the block's tokens, NJ logits per lane (expert lane + 64 j; E
// <= 64 NJ).  A lane's slot that holds no expert, or whose expert has been
// selected, reads (-inf, kNone), which loses to every expert still
// selectable (a tie on -inf goes to the lower index), so each of the k
// rounds is a plain wave-wide argmax.  The gates' normaliser sums
// exp(logit - best) in slot order.
constexpr int kNone = 0x7fffffff;

template <int NJ>
__device__ __forceinline__ void route_tokens(const RouteParams& p, const float* sH, int ldh,
                                             int t_base, int w, int nw, int lane,
                                             float (&pacc)[4]) {
  for (int m = w; m < kRouteTokens; m += nw) {
    const int t = t_base + m;
    if (t >= p.T) break;
    float v[NJ];
    int id[NJ];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      const bool ok = e < p.E;
      v[j] = ok ? sH[m * ldh + e] : -INFINITY;
      id[j] = ok ? e : kNone;
      mx = fmaxf(mx, v[j]);
    }
    mx = wave_max_dpp(mx);
    float ex[NJ], s = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      ex[j] = id[j] != kNone ? expf(v[j] - mx) : 0.f;
      s += ex[j];
    }
    s = wave_sum_dpp(s);
#pragma unroll
    for (int j = 0; j < NJ; ++j) pacc[j] += ex[j] / s;

    float v0 = 0.f, z = 0.f, my_v = 0.f;
    int my_i = 0;
    for (int sl = 0; sl < p.k; ++sl) {
      float bv = v[0];
      int bi = id[0];
#pragma unroll
      for (int j = 1; j < NJ; ++j) take_better(bv, bi, v[j], id[j]);
      wave_argmax(bv, bi);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool mine = id[j] == bi;
        v[j] = mine ? -INFINITY : v[j];
        id[j] = mine ? kNone : id[j];
      }
      v0 = sl == 0 ? bv : v0;
      z += expf(bv - v0);
      my_v = lane == sl ? bv : my_v;
      my_i = lane == sl ? bi : my_i;
    }
    if (lane < p.k) {
      p.idx[(int64_t)t * p.k + lane] = my_i;
      p.gate[(int64_t)t * p.k + lane] = expf(my_v - v0) / z;
    }
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
      float* part = lds + (w % nk) * tile;
      // 16-column groups a 64-column set can hold: 1, 2 or 4
      const int nj = ncols > 32 ? 4 : (ncols > 16 ? 2 : 1);
      if (noise) {
        if (nj == 4) router_tile_bf16<4, true>(p, part, ldh, t_base, ncols, nk, nc);
        else if (nj == 2) router_tile_bf16<2, true>(p, part, ldh, t_base, ncols, nk, nc);
        else router_tile_bf16<1, true>(p, part, ldh, t_base, ncols, nk, nc);
      } else {
        if (nj == 4) router_tile_bf16<4, false>(p, part, ldh, t_base, ncols, nk, nc);
        else if (nj == 2) router_tile_bf16<2, false>(p, part, ldh, t_base, ncols, nk, nc);
        else router_tile_bf16<1, false>(p, part, ldh, t_base, ncols, nk, nc);
      }
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
    // the block's 16 x E logits, 4 per thread per pass: a pass issues its
    // bias and eps loads before it uses any of them
    for (int i0 = 0; i0 < kRouteTokens * p.E; i0 += 4 * nt) {
      float bias[4], ep[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nt + threadIdx.x;
        const int m = i / p.E, e = i - m * p.E, t = t_base + m;
        const bool ok = i < kRouteTokens * p.E && t < p.T;
        bias[u] = (ok && p.b_g) ? p.b_g[e] : 0.f;
        ep[u] = (ok && noise) ? p.eps[(int64_t)t * p.E + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nt + threadIdx.x;
        const int m = i / p.E, e = i - m * p.E, t = t_base + m;
        if (i >= kRouteTokens * p.E || t >= p.T) continue;
        float v = sH[m * ldh + e] + bias[u];
        if (noise) {
          const float n = sH[m * ldh + p.E + e];
          v += ep[u] * softplus_f32(n);
          if (p.noise_pre) p.noise_pre[(int64_t)t * p.E + e] = n;
        }
        sH[m * ldh + e] = v;
        p.logits[(int64_t)t * p.E + e] = v;
      }
    }
  } else {
    // replay: 4 loads per thread in flight per pass
    for (int i0 = 0; i0 < kRouteTokens * p.E; i0 += 4 * nt) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nt + threadIdx.x;
        const int m = i / p.E, e = i - m * p.E, t = t_base + m;
        v[u] = (i < kRouteTokens * p.E && t < p.T) ? p.logits[(int64_t)t * p.E + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nt + threadIdx.x;
        const int m = i / p.E, e = i - m * p.E;
        if (i < kRouteTokens * p.E) sH[m * ldh + e] = v[u];
      }
    }
  }
  __syncthreads();

  // Phase 2: one token per wave iteration; lane owns experts lane + 64*j.
  // Wave w takes tokens w, w + nw, w + 2nw, ... of the block, so every one of
  // the 16 tokens is handled whatever the wave count (which need not divide 16).
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
  const int nj = (p.E + 63) >> 6;
  if (nj == 1) route_tokens<1>(p, sH, ldh, t_base, w, nw, lane, pacc);
  else if (nj == 2) route_tokens<2>(p, sH, ldh, t_base, w, nw, lane, pacc);
  else route_tokens<4>(p, sH, ldh, t_base, w, nw, lane, pacc);
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
  // the block's tokens' output rows, zeroed last (nothing is loaded after)
  if (p.zero_rows) {
    const int chunks = p.row_bytes >> 4;
    const int rows = min(kRouteTokens, p.T - t_base);
    for (int c = threadIdx.x; c < rows * chunks; c += nt) {
      const int m = c / chunks, q = c - m * chunks;
      reinterpret_cast<uint4*>(static_cast<char*>(p.zero_rows) +
                               (int64_t)(t_base + m) * p.row_bytes)[q] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// prob_sum[e] = sum over routing blocks: one wave per expert, each lane sums a
// fixed strided subset in double, then a fixed butterfly; deterministic.  A
// lane's loads are issued 8 at a time before their adds (in the same order),
// so a large batch waits for memory once per 8 partials, not once per partial.
__global__ __launch_bounds__(256) void prob_reduce_kernel(const float* partial, float* out,
                                                          int nblocks, int E) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;
  double s = 0.0;
  int b = lane;
  for (; b + 7 * 64 < nblocks; b += 8 * 64) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = partial[(int64_t)(b + j * 64) * E + e];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (double)v[j];
  }
  for (; b < nblocks; b += 64) s += (double)partial[(int64_t)b * E + e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) out[e] = (float)s;
}

}  // namespace

// bf16 tiles: up to 4 column-group sets run in parallel (wide tiles) and the
// other waves split the model width, 16 waves in all unless the partial tiles
// (one per width range) and the 16 KiB of probability partials outgrow the
// 160 KiB of LDS; narrow tiles give up width ranges (down to 8) so that two
// blocks share a CU.  float32 and replay use 4 waves and one tile.  The wave
// count need not divide the block's 16 tokens (phase 2 strides by it).
RoutePlan route_plan(int E, bool noise, bool mma) {
  const int ncols = E * (noise ? 2 : 1);
  const size_t tile = (size_t)kRouteTokens * (ncols + 1) * sizeof(float);
  const int nc = (mma && ncols > 64) ? std::min(4, (ncols + 63) / 64) : 1;
  int nk = mma ? kMaxWaves / nc : 4;
  const size_t fixed = sizeof(float) * kMaxWaves * 256, cap = 160 * 1024;
  while (mma && nk > 1 && nk * tile + fixed > cap) nk >>= 1;
  while (mma && nc == 1 && nk > 8 && 2 * (nk * tile + fixed) > cap) nk >>= 1;
  RoutePlan r;
  r.waves = mma ? nk * nc : 4;
  r.lds_bytes = (mma ? nk : 1) * tile;
  r.static_lds_bytes = fixed;
  return r;
}

hipError_t launch_route(const RouteParams& p, hipStream_t stream) {
  const int blocks = route_blocks(p.T);
  if (p.bf16 && p.x && route_split_logits(p.T, p.E, p.w_noise != nullptr)) {
    // logits first (bias and noise applied), then the router kernel replays them
    const bool noise = p.w_noise != nullptr;
    // (at least 32 columns: two groups of 16, or four past 32 columns)
    const int ng = (noise ? 2 * p.E : p.E) > 32 ? 4 : 2;
    const int eb = noise ? 8 * ng : 16 * ng;
    const dim3 g((unsigned)((p.T + kLogitRows - 1) / kLogitRows), (unsigned)((p.E + eb - 1) / eb));
#define MOE_LOGITS(NGV, NZ) \
  hipLaunchKernelGGL((router_logits_kernel<NGV, NZ, kLogitWaves>), g, dim3(64 * kLogitWaves), 0, stream, p)
    if (noise) {
      if (ng == 4) MOE_LOGITS(4, true); else MOE_LOGITS(2, true);
    } else {
      if (ng == 4) MOE_LOGITS(4, false); else MOE_LOGITS(2, false);
    }
#undef MOE_LOGITS
    RouteParams q = p;
    q.x = nullptr; q.w_g = nullptr; q.b_g = nullptr; q.w_noise = nullptr; q.eps = nullptr;
    q.noise_pre = nullptr;
    const RoutePlan rp = route_plan(p.E, false, false);
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(64 * rp.waves), rp.lds_bytes, stream, q);
  } else {
    const RoutePlan rp = route_plan(p.E, p.w_noise != nullptr, p.bf16 && p.x);
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(64 * rp.waves), rp.lds_bytes, stream, p);
  }
  hipLaunchKernelGGL(prob_reduce_kernel, dim3((p.E + 3) / 4), dim3(256), 0, stream,
                     (const float*)p.prob_partial, p.prob_sum, blocks, p.E);
  return hipGetLastError();
}

}  // namespace moe
