// Expert-choice routing: every expert takes the tokens it scores highest, up
// to its capacity ("Mixture-of-Experts & Sparse Model Scaling", Advanced
// Theory & Extensions), so every expert is full and a token may be taken by
// no expert or by several.
//
// Readings where the page is silent: the score of token t for expert e is the
// float32 softmax over experts of t's logits; each expert takes
// C' = min(C, T) tokens; equal scores go to the lower token index; the gate of
// a (token, expert) pair is that raw score; an expert's rows are laid out in
// ascending token order.
//
// Selection is one block per expert: a most-significant-digit-first radix
// select (4 passes of 8 bits over order-preserving keys of the float32
// scores) finds the C'-th largest score s* and how many of the tokens scoring
// exactly s* are still needed; a compaction pass in token order then takes
// every token above s* and the lowest-index tokens at s*, and writes each
// chosen token to the next row.  Histograms are integer LDS counts, so the
// result is exact and deterministic.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Order-preserving unsigned key of a float (-0.0 counts as +0.0).
__device__ __forceinline__ uint32_t score_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// scores[t, :] = softmax(logits[t, :]) in float32; one wave per token, lane
// owns experts lane + 64 j.
__global__ __launch_bounds__(256) void ec_scores_kernel(const float* logits, float* scores,
                                                        int T, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* h = logits + t * E;
  float v[4], mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? h[e] : -INFINITY;
    mx = fmaxf(mx, v[j]);
  }
  mx = wave_max(mx);
  float ex[4], s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    ex[j] = e < E ? expf(v[j] - mx) : 0.f;
    s += ex[j];
  }
  s = wave_sum(s);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) scores[t * E + e] = ex[j] / s;
  }
}

// Exclusive prefix count of `flag` over the block's threads in thread order,
// and the block total.  Uses wtot (kSelWaves ints of LDS); ends synchronised.
__device__ __forceinline__ int block_excl_count(bool flag, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wtot[w] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    const int c = wtot[i];
    before += i < w ? c : 0;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(EcParams p) {
  __shared__ int hist[256];
  __shared__ int pick[2];
  __shared__ int wtot[kSelWaves];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int T = p.T, E = p.E, Cp = p.Cp;
  const float* sc = p.scores;
  if (tid == 0) {
    p.counts[e] = Cp;
    p.offsets[e] = e * Cp;
    if (e == E - 1) p.offsets[E] = E * Cp;
  }
  // radix select of the Cp-th largest key: `prefix` holds its digits found so
  // far, `need` how many keys matching the prefix are still to be taken
  uint32_t prefix = 0, mask = 0;
  int need = Cp;
  if (Cp > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int t = tid; t < T; t += kSelThreads) {
        const uint32_t k = score_key(sc[(int64_t)t * E + e]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0, b = 255;
        for (; b > 0; --b) {
          if (above + hist[b] >= need) break;
          above += hist[b];
        }
        pick[0] = b;
        pick[1] = need - above;
      }
      __syncthreads();
      prefix |= (uint32_t)pick[0] << shift;
      mask |= 255u << shift;
      need = pick[1];
      __syncthreads();
    }
  }
  // compaction in token order: keys above the threshold, then the first
  // `need` tokens whose key equals it
  int base_eq = 0, base_sel = 0;
  for (int t0 = 0; t0 < T; t0 += kSelThreads) {
    const int t = t0 + tid;
    const bool valid = t < T && Cp > 0;
    const uint32_t k = valid ? score_key(sc[(int64_t)t * E + e]) : 0u;
    const bool eq = valid && k == prefix;
    int n_eq, n_sel;
    const int eq_rank = base_eq + block_excl_count(eq, wtot, n_eq);
    const bool sel = valid && (k > prefix || (eq && eq_rank < need));
    const int pos = base_sel + block_excl_count(sel, wtot, n_sel);
    if (t < T) {
      p.slot[(int64_t)t * E + e] = sel ? e * Cp + pos : -1;
      if (sel && pos < Cp) p.row_token[e * Cp + pos] = t;
    }
    base_eq += n_eq;
    base_sel += n_sel;
  }
}

// y[t] = shared experts + sum over e ascending of scores[t,e] * y_rows[slot[t,e]]
// in float32; one block per token.
__global__ __launch_bounds__(256) void ec_combine_kernel(EcCombineParams p) {
  __shared__ int s_row[256];
  __shared__ float s_gate[256];
  __shared__ int s_n;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // ordered list of the experts that took t (E <= 256: thread e looks at e)
  __shared__ int wcnt[4];
  const int r = tid < p.E ? p.slot[t * p.E + tid] : -1;
  const uint64_t b = __ballot(r >= 0);
  if (lane == 0) wcnt[w] = __popcll(b);
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wcnt[i];
  if (r >= 0) {
    const int pos = base + __popcll(b & ((1ull << lane) - 1ull));
    s_row[pos] = r;
    s_gate[pos] = p.scores[t * p.E + tid];
  }
  if (tid == 0) s_n = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  __syncthreads();
  const int n = s_n;
  for (int c = tid * 4; c < p.d; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.S; ++s)
      acc += *reinterpret_cast<const f32x4*>(p.y_shared + ((int64_t)s * p.T + t) * p.d + c);
    for (int i = 0; i < n; ++i) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p.y_rows + (int64_t)s_row[i] * p.d + c);
      const float g = s_gate[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(g, v[j], acc[j]);
    }
    if (p.out_bf16) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + t * p.d + c) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.y) + t * p.d + c) = acc;
    }
  }
}

// stats = [f (E), P (E), L_aux, drop rate]: f = rows of e / all rows,
// P = prob_sum / T, L_aux = E sum f P, drop rate = tokens no expert took / T.
// One block; integer counts and a fixed summation order.
__global__ __launch_bounds__(1024) void ec_stats_kernel(EcStatsParams p) {
  __shared__ int wtot[16];
  __shared__ double prod[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int uncovered = 0;
  for (int t = tid; t < p.T; t += 1024) {
    bool any = false;
    for (int e = 0; e < p.E; ++e) any |= p.slot[(int64_t)t * p.E + e] >= 0;
    uncovered += any ? 0 : 1;
  }
  for (int o = 32; o > 0; o >>= 1) uncovered += __shfl_xor(uncovered, o, kWave);
  if (lane == 0) wtot[w] = uncovered;
  long long rows = 0;
  for (int e = 0; e < p.E; ++e) rows += p.counts[e];
  __syncthreads();
  if (tid < p.E) {
    const double f = rows > 0 ? (double)p.counts[tid] / (double)rows : 0.0;
    const double P = (double)p.prob_sum[tid] / (double)p.T;
    p.stats[tid] = (float)f;
    p.stats[p.E + tid] = (float)P;
    prod[tid] = f * P;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int i = 0; i < p.E; ++i) s += prod[i];
    int un = 0;
    for (int i = 0; i < 16; ++i) un += wtot[i];
    p.stats[2 * p.E] = (float)((double)p.E * s);
    p.stats[2 * p.E + 1] = (float)((double)un / (double)p.T);
  }
}

}  // namespace

hipError_t launch_expert_choice(const EcParams& p, const float* logits, hipStream_t stream) {
  if (logits && p.T > 0)
    hipLaunchKernelGGL(ec_scores_kernel, dim3((p.T + 3) / 4), dim3(256), 0, stream, logits,
                       p.scores, p.T, p.E);
  hipLaunchKernelGGL(ec_select_kernel, dim3(p.E), dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine_ec(const EcCombineParams& p, hipStream_t stream) {
  if (p.T > 0) hipLaunchKernelGGL(ec_combine_kernel, dim3(p.T), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_stats_ec(const EcStatsParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(ec_stats_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
