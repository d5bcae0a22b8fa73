// Router z-loss and routing diagnostics of a token-choice batch.
//
// "Mixture-of-Experts & Sparse Model Scaling": Advanced Theory & Extensions
// (a z-loss keeps router logits from growing large) and Benchmark Datasets &
// Evaluation (utilisation, routing entropy, fraction of tokens dropped);
// "Mixture-of-experts Models", Level 3 (overflow and an imbalance measure).
// The z-loss is read as the mean over tokens of the squared log-partition of
// the float32 logits; entropy is in nats.
//
// Per-token terms: one wave per token (lane owns experts lane + 64 j), 16
// tokens per block, partial sums per block in double in a fixed order; a
// one-block kernel reduces the partials in a fixed order (strided per thread,
// then over the threads) and adds the count-based metrics.  No atomics:
// results are deterministic.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kDiagTokens = 16;

__global__ __launch_bounds__(256) void diag_token_kernel(DiagParams p) {
  __shared__ double s_z[4], s_h[4];
  __shared__ int s_full[4], s_part[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double zsum = 0.0, hsum = 0.0;
  int full = 0, part = 0;
  for (int i = 0; i < kDiagTokens / 4; ++i) {
    const int64_t t = (int64_t)blockIdx.x * kDiagTokens + w * (kDiagTokens / 4) + i;
    if (t >= p.T) break;
    const float* h = p.logits + t * p.E;
    float v[4], mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < p.E ? h[e] : -INFINITY;
      mx = fmaxf(mx, v[j]);
    }
    mx = wave_max(mx);
    float ex[4], s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      ex[j] = e < p.E ? expf(v[j] - mx) : 0.f;
      s += ex[j];
    }
    s = wave_sum(s);
    const float lse = mx + logf(s);
    float ph = 0.f;  // sum_e p_e h_e
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < p.E) ph += (ex[j] / s) * v[j];
    }
    ph = wave_sum(ph);
    int lost = lane < p.k && p.dest[t * p.k + lane] < 0 ? 1 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lost += __shfl_xor(lost, o, kWave);
    zsum += (double)lse * (double)lse;
    hsum += (double)lse - (double)ph;
    full += lost == p.k;
    part += lost > 0 && lost < p.k;
  }
  if (lane == 0) {
    s_z[w] = zsum;
    s_h[w] = hsum;
    s_full[w] = full;
    s_part[w] = part;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* pd = p.partial_d + (int64_t)blockIdx.x * 2;
    int* pi = p.partial_i + (int64_t)blockIdx.x * 2;
    pd[0] = ((s_z[0] + s_z[1]) + s_z[2]) + s_z[3];
    pd[1] = ((s_h[0] + s_h[1]) + s_h[2]) + s_h[3];
    pi[0] = s_full[0] + s_full[1] + s_full[2] + s_full[3];
    pi[1] = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  }
}

__global__ __launch_bounds__(256) void diag_final_kernel(DiagParams p, int nblocks) {
  __shared__ double s_ov[256];
  const int e = threadIdx.x;
  const double tk = (double)p.T * (double)p.k;
  double mean = 0.0;
  int mx = 0;
  for (int i = 0; i < p.E; ++i) {
    mean += (double)p.counts[i];
    mx = max(mx, p.counts[i]);
  }
  mean /= (double)p.E;
  if (e < p.E) {
    const int c = p.counts[e];
    const int kept = c < p.C ? c : p.C;
    p.diag[8 + e] = (float)(c - kept);
    p.diag[8 + p.E + e] = p.C > 0 ? (float)((double)kept / (double)p.C) : 0.f;
    s_ov[e] = (double)(c - kept);
  }
  // partials: thread e sums blocks e, e+256, ... (fixed order), then thread 0
  // sums the 256 thread sums in order
  __shared__ double s_zs[256], s_hs[256];
  __shared__ long long s_full[256], s_part[256];
  {
    double zs = 0.0, hs = 0.0;
    long long full = 0, part = 0;
    for (int b = e; b < nblocks; b += 256) {
      zs += p.partial_d[2 * b];
      hs += p.partial_d[2 * b + 1];
      full += p.partial_i[2 * b];
      part += p.partial_i[2 * b + 1];
    }
    s_zs[e] = zs;
    s_hs[e] = hs;
    s_full[e] = full;
    s_part[e] = part;
  }
  __syncthreads();
  if (e == 0) {
    double zs = 0.0, hs = 0.0, var = 0.0, dev = 0.0, ov = 0.0;
    long long full = 0, part = 0;
    for (int b = 0; b < 256; ++b) {
      zs += s_zs[b];
      hs += s_hs[b];
      full += s_full[b];
      part += s_part[b];
    }
    for (int i = 0; i < p.E; ++i) {
      const double c = (double)p.counts[i];
      var += (c - mean) * (c - mean);
      dev += fabs(c - tk / (double)p.E);
      ov += s_ov[i];
    }
    var /= (double)p.E;
    p.diag[0] = (float)(zs / (double)p.T);
    p.diag[1] = (float)(hs / (double)p.T);
    p.diag[2] = mean > 0.0 ? (float)(sqrt(var) / mean) : 0.f;
    p.diag[3] = (float)dev;
    p.diag[4] = mean > 0.0 ? (float)((double)mx / mean) : 0.f;
    p.diag[5] = (float)ov;
    p.diag[6] = (float)((double)full / (double)p.T);
    p.diag[7] = (float)((double)part / (double)p.T);
  }
}

}  // namespace

int diag_blocks(int64_t T) { return (int)((T + kDiagTokens - 1) / kDiagTokens); }

hipError_t launch_diagnostics(const DiagParams& p, hipStream_t stream) {
  const int blocks = diag_blocks(p.T);
  if (blocks > 0) hipLaunchKernelGGL(diag_token_kernel, dim3(blocks), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(diag_final_kernel, dim3(1), dim3(256), 0, stream, p, blocks);
  return hipGetLastError();
}

}  // namespace moe
