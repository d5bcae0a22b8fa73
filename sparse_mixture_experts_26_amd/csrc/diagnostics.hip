// Router z-loss and routing diagnostics of a token-choice batch.
//
// "Mixture-of-Experts & Sparse Model Scaling": Advanced Theory & Extensions
// (a z-loss keeps router logits from growing large) and Benchmark Datasets &
// Evaluation (utilisation, routing entropy, fraction of tokens dropped);
// "Mixture-of-experts Models", Level 3 (overflow and an imbalance measure).
// The z-loss is read as the mean over tokens of the squared log-partition of
// the float32 logits; entropy is in nats.
//
// Per-token terms: one wave per token (lane owns experts lane + 64 j; wave
// reductions on DPP row permutations, the token's lost slots by one ballot),
// 16 tokens per block, partial sums per block in double in a fixed order; a
// one-block kernel reduces the partials (strided per thread, then a fixed
// pairwise tree over the threads) and adds the count-based metrics, whose
// sums over experts use the same tree.  No atomics: results are
// deterministic.
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
  // the wave's 4 tokens: every logit load is issued before any is used
  constexpr int kPer = kDiagTokens / 4;
  const int64_t t0 = (int64_t)blockIdx.x * kDiagTokens + w * kPer;
  float v[kPer][4];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[i][j] = (t0 + i < p.T && e < p.E) ? p.logits[(t0 + i) * p.E + e] : -INFINITY;
    }
  int lost[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    lost[i] = __popcll(__ballot(t0 + i < p.T && lane < p.k && p.dest[(t0 + i) * p.k + lane] < 0));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (t0 + i >= p.T) break;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, v[i][j]);
    mx = wave_max_dpp(mx);
    float ex[4], s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      ex[j] = e < p.E ? expf(v[i][j] - mx) : 0.f;
      s += ex[j];
    }
    s = wave_sum_dpp(s);
    const float lse = mx + logf(s);
    float ph = 0.f;  // sum_e p_e h_e
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < p.E) ph += (ex[j] / s) * v[i][j];
    }
    ph = wave_sum_dpp(ph);
    zsum += (double)lse * (double)lse;
    hsum += (double)lse - (double)ph;
    full += lost[i] == p.k;
    part += lost[i] > 0 && lost[i] < p.k;
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
  __shared__ double s_a[256], s_b[256], s_c[256], s_d[256];
  __shared__ long long s_full[256], s_part[256];
  __shared__ int s_mx[256];
  const int e = threadIdx.x;
  const double tk = (double)p.T * (double)p.k;
  const bool ex = e < p.E;
  const int c = ex ? p.counts[e] : 0;
  const int kept = c < p.C ? c : p.C;
  if (ex) {
    p.diag[8 + e] = (float)(c - kept);
    p.diag[8 + p.E + e] = p.C > 0 ? (float)((double)kept / (double)p.C) : 0.f;
  }
  // per-token partials: thread e sums blocks e, e + 256, ... in order
  double zs = 0.0, hs = 0.0;
  long long full = 0, part = 0;
  for (int b = e; b < nblocks; b += 256) {
    zs += p.partial_d[2 * b];
    hs += p.partial_d[2 * b + 1];
    full += p.partial_i[2 * b];
    part += p.partial_i[2 * b + 1];
  }
  s_a[e] = (double)c;
  s_b[e] = zs;
  s_c[e] = hs;
  s_d[e] = (double)(c - kept);
  s_full[e] = full;
  s_part[e] = part;
  s_mx[e] = c;
  __syncthreads();
  // pairwise trees over the 256 slots, all seven in step (slot 0 ends with
  // each total; the same pairing every call)
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) {
      s_a[e] += s_a[e + o];
      s_b[e] += s_b[e + o];
      s_c[e] += s_c[e + o];
      s_d[e] += s_d[e + o];
      s_full[e] += s_full[e + o];
      s_part[e] += s_part[e + o];
      s_mx[e] = max(s_mx[e], s_mx[e + o]);
    }
    __syncthreads();
  }
  const double mean = s_a[0] / (double)p.E;
  const double z_sum = s_b[0], h_sum = s_c[0], ov = s_d[0];
  const long long n_full = s_full[0], n_part = s_part[0];
  const int mx = s_mx[0];
  __syncthreads();  // every thread has read the totals before the slots are reused
  s_a[e] = ex ? ((double)c - mean) * ((double)c - mean) : 0.0;
  s_b[e] = ex ? fabs((double)c - tk / (double)p.E) : 0.0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) {
      s_a[e] += s_a[e + o];
      s_b[e] += s_b[e + o];
    }
    __syncthreads();
  }
  if (e == 0) {
    const double var = s_a[0] / (double)p.E;
    p.diag[0] = (float)(z_sum / (double)p.T);
    p.diag[1] = (float)(h_sum / (double)p.T);
    p.diag[2] = mean > 0.0 ? (float)(sqrt(var) / mean) : 0.f;
    p.diag[3] = (float)s_b[0];
    p.diag[4] = mean > 0.0 ? (float)((double)mx / mean) : 0.f;
    p.diag[5] = (float)ov;
    p.diag[6] = (float)((double)n_full / (double)p.T);
    p.diag[7] = (float)((double)n_part / (double)p.T);
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
