// Overflow re-routing: assignments that find their expert full go to the
// token's lower-ranked experts ("Mixture-of-experts Models", Level 2,
// "Overflow handling defines an output contract"; "3D mixture-of-experts
// routing lab", Capacity panel).
//
// The pages fix no policy; the one implemented: a token's fallbacks are its
// experts ranked below its top k (float32 logits, ties to the lower index),
// each tried at most once.  In rounds, every unplaced assignment proposes its
// token's next untried fallback (a token's unplaced slots, in slot order, take
// consecutive ones); every expert accepts the proposals in arrival order up to
// its spare capacity; the rest retry next round; an assignment whose token has
// no untried fallback left is dropped.  A re-routed slot keeps its gate.
// Rows of an expert: its primary kept assignments, then each round's
// accepted ones, in arrival order.
//
// Three steps after the primary dispatch (which leaves counts, offsets and
// dest of the arrival-order pass):
//   1. fallback lists, one wave per token that lost a slot;
//   2. the rounds, in one block: per chunk of 1024 proposals in arrival order,
//      ranks per expert from 9 ballots per 64-lane slice and slice
//      histograms, a running count per expert across chunks, acceptance
//      against the expert's load at the start of the round, and an ordered
//      compaction of the assignments still unplaced;
//   3. offsets over the final loads, dest, row_token and final_expert.
// Every step is ordered, so the integer results are exact and deterministic.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRrThreads = 1024;
constexpr int kRrWaves = kRrThreads / 64;
constexpr int kNoExpert = 511;  // matches no expert in the ballot ranking

// F[t, r] = expert ranked k + r of token t, for tokens that lost a slot.
__global__ __launch_bounds__(256) void fallback_kernel(RerouteParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  int lost = 0;
  for (int s = 0; s < p.k; ++s) lost |= p.dest[t * p.k + s] < 0;
  if (!lost) return;
  const float* h = p.logits + t * p.E;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < p.E ? h[e] + 0.0f : 0.f;
  }
  int rank[4] = {0, 0, 0, 0};
  for (int e2 = 0; e2 < p.E; ++e2) {
    const float o = __shfl(v[e2 >> 6], e2 & 63, kWave);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      rank[j] += (o > v[j] || (o == v[j] && e2 < e)) ? 1 : 0;
    }
  }
  const int nf = p.E - p.k;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < p.E && rank[j] >= p.k) p.fallback[t * nf + (rank[j] - p.k)] = (uint8_t)e;
  }
}

// Exclusive count of `flag` over the block in thread order, block total.
__device__ __forceinline__ int rr_excl_count(bool flag, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  if (lane == 0) wtot[w] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < kRrWaves; ++i) {
    const int c = wtot[i];
    before += i < w ? c : 0;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + __popcll(b & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kRrThreads) void reroute_kernel(RerouteParams p) {
  __shared__ int hist[kRrWaves][256];   // per-slice counts, then slice bases
  __shared__ int load[256], run[256], ctot[256], off_prim[257];
  __shared__ int wtot[kRrWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = p.E, k = p.k, C = p.C, nf = p.E - p.k;
  const int n_all = p.T * k;
  for (int e = tid; e < E; e += kRrThreads) {
    const int c = p.counts[e];
    load[e] = c < C ? c : C;
  }
  for (int e = tid; e <= E; e += kRrThreads) off_prim[e] = p.offsets[e];
  for (int t = tid; t < p.T; t += kRrThreads) p.ptr[t] = 0;
  // the unplaced list, in arrival order
  int n = 0;
  for (int i0 = 0; i0 < n_all; i0 += kRrThreads) {
    const int i = i0 + tid;
    const bool un = i < n_all && p.dest[i] < 0;
    int tot;
    const int pos = n + rr_excl_count(un, wtot, tot);
    if (un) {
      p.list_a[pos] = i;
      p.fe[i] = -1;
    }
    n += tot;
  }
  int* cur = p.list_a;
  int* nxt = p.list_b;
  __syncthreads();
  for (int round = 0; round <= nf && n > 0; ++round) {
    for (int e = tid; e < 256; e += kRrThreads) run[e] = 0;
    __syncthreads();
    int m = 0;
    for (int c0 = 0; c0 < n; c0 += kRrThreads) {
      const int pos = c0 + tid;
      const bool valid = pos < n;
      const int i = valid ? cur[pos] : 0;
      const int t = i / k;
      // j = earlier unplaced slots of the same token (contiguous in the list)
      int j = 0;
      bool last = true;
      if (valid) {
        for (int b = 1; b < k && pos - b >= 0 && cur[pos - b] / k == t; ++b) ++j;
        last = !(pos + 1 < n && cur[pos + 1] / k == t);
      }
      const int q = valid ? p.ptr[t] + j : 0;
      const int e = (valid && q < nf) ? (int)p.fallback[(int64_t)t * nf + q] : kNoExpert;
      // rank among this chunk's proposals to the same expert (slice = wave)
      for (int x = tid; x < kRrWaves * 256; x += kRrThreads) (&hist[0][0])[x] = 0;
      __syncthreads();
      uint64_t peers = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const bool on = (e >> bit) & 1;
        const uint64_t bal = __ballot(on);
        peers &= on ? bal : ~bal;
      }
      const int r_slice = __popcll(peers & ((1ull << lane) - 1ull));
      if (e != kNoExpert && r_slice == 0) hist[w][e] = __popcll(peers);
      __syncthreads();
      // slice bases within the chunk, and this chunk's total per expert
      for (int x = tid; x < E; x += kRrThreads) {
        int acc = 0;
        for (int sl = 0; sl < kRrWaves; ++sl) {
          const int c = hist[sl][x];
          hist[sl][x] = acc;
          acc += c;
        }
        ctot[x] = acc;
      }
      __syncthreads();
      bool accepted = false, still = false;
      if (e != kNoExpert) {
        const int rank = run[e] + hist[w][e] + r_slice;
        accepted = load[e] + rank < C;
        still = !accepted;
        if (accepted) {
          p.fe[i] = e;
          p.rin[i] = load[e] + rank;
        }
      }
      // token pointers advance past every proposal of this round (after the
      // reads above); the last slot of a token in the list writes it
      __syncthreads();
      if (valid && last) p.ptr[t] = p.ptr[t] + j + 1;
      int tot;
      const int spos = m + rr_excl_count(still, wtot, tot);
      if (still) nxt[spos] = i;
      m += tot;
      for (int x = tid; x < E; x += kRrThreads) run[x] += ctot[x];
      __syncthreads();
    }
    // accepted this round per expert: the proposals ranked below the spare capacity
    for (int x = tid; x < E; x += kRrThreads) {
      const int spare = C - load[x];
      load[x] += run[x] < spare ? run[x] : spare;
    }
    int* sw = cur;
    cur = nxt;
    nxt = sw;
    n = m;
    __syncthreads();
  }
  // offsets over the final loads
  if (tid == 0) {
    int acc = 0;
    for (int x = 0; x < E; ++x) {
      p.offsets[x] = acc;
      acc += load[x];
    }
    p.offsets[E] = acc;
  }
  __syncthreads();
  // final placement of every assignment
  for (int i = tid; i < n_all; i += kRrThreads) {
    const int dp = p.dest[i];
    int e, r;
    if (dp >= 0) {
      e = p.idx[i];
      r = dp - off_prim[e];
    } else {
      e = p.fe[i];
      r = e >= 0 ? p.rin[i] : 0;
    }
    const int d = e >= 0 ? p.offsets[e] + r : -1;
    p.final_expert[i] = e;
    p.dest_out[i] = d;
    if (d >= 0) p.row_token[d] = i / k;
  }
}

}  // namespace

hipError_t launch_reroute(const RerouteParams& p, hipStream_t stream) {
  if (p.T > 0 && p.E > p.k)
    hipLaunchKernelGGL(fallback_kernel, dim3((p.T + 3) / 4), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(reroute_kernel, dim3(1), dim3(kRrThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moe
