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
//   2. the rounds.  Large batches build the unplaced list and run the first
//      rounds (the large ones) as multi-block passes over chunks of 1024 list
//      positions: proposals with their stable rank per expert inside the
//      chunk; one block for the per-expert chunk bases, the acceptance
//      totals and the ordered bases of the rejected pairs; acceptance and the
//      ordered compaction.  The remaining rounds run in one block: per chunk
//      of 1024 proposals in arrival order,
//      ranks per expert from 9 ballots per 64-lane slice and slice
//      histograms, a running count per expert across chunks, acceptance
//      against the expert's load at the start of the round, and an ordered
//      compaction of the assignments still unplaced;
//   3. offsets over the final loads (same block), then dest, row_token and
//      final_expert in a kernel of one thread per assignment.
// Every step is ordered, so the integer results are exact and deterministic.
#include <algorithm>

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

// Exclusive sum of v over the block in thread order, block total.
__device__ __forceinline__ int rr_excl_sum(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < kRrWaves; ++i) {
    const int c = wtot[i];
    before += i < w ? c : 0;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// ---- multi-block list build and rounds ------------------------------------------
// Chunk c covers slots (list positions) [1024 c, 1024 c + 1024); thread order
// is arrival order inside a chunk, chunk order across chunks.

__global__ __launch_bounds__(kRrThreads) void rr_list_count_kernel(RerouteParams p) {
  __shared__ int wtot[kRrWaves];
  const int64_t i = (int64_t)blockIdx.x * kRrChunk + threadIdx.x;
  const bool f = i < (int64_t)p.T * p.k && p.dest[i] < 0;
  int total;
  rr_excl_count(f, wtot, total);
  if (threadIdx.x == 0) p.chunk_cnt[blockIdx.x] = total;
}

// chunk bases of the unplaced list, its length, the loads after the primary
// pass (both load buffers), the primary offsets
__global__ __launch_bounds__(kRrThreads) void rr_list_scan_kernel(RerouteParams p, int chunks) {
  __shared__ int wtot[kRrWaves];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < chunks; c0 += kRrThreads) {
    const int c = c0 + tid;
    const int v = c < chunks ? p.chunk_cnt[c] : 0;
    int total;
    const int ex = rr_excl_sum(v, wtot, total);
    if (c < chunks) p.chunk_base[c] = carry + ex;
    carry += total;
  }
  if (tid == 0) p.n_g[0] = carry;
  for (int e = tid; e < 256; e += kRrThreads) {
    const int c = e < p.E ? p.counts[e] : 0;
    const int l = c < p.C ? c : p.C;
    p.load_g[e] = l;
    p.load_g[256 + e] = l;
  }
  for (int e = tid; e <= p.E; e += kRrThreads) p.off_prim[e] = p.offsets[e];
}

__global__ __launch_bounds__(kRrThreads) void rr_list_write_kernel(RerouteParams p) {
  __shared__ int wtot[kRrWaves];
  const int64_t i = (int64_t)blockIdx.x * kRrChunk + threadIdx.x;
  const bool f = i < (int64_t)p.T * p.k && p.dest[i] < 0;
  int total;
  const int ex = rr_excl_count(f, wtot, total);
  if (f) {
    const int pos = p.chunk_base[blockIdx.x] + ex;
    p.list_a[2 * pos] = (int)i;
    p.list_a[2 * pos + 1] = 0;
    p.fe[i] = -1;
  }
}

// Round r, pass 1: every pair of the chunk proposes its token's next untried
// fallback (its position j among the token's unplaced slots picks the j-th
// one after the pointer); its rank among the chunk's proposals to the same
// expert, in arrival order; the chunk's count per expert.
__global__ __launch_bounds__(kRrThreads) void rr_propose_kernel(RerouteParams p, int r) {
  __shared__ int hist[kRrWaves][257];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = p.k, nf = p.E - p.k;
  const int* cur = (r & 1) ? p.list_b : p.list_a;
  const int n = p.n_g[r & 1];
  const int c = blockIdx.x;
  if (c * kRrChunk >= n) return;  // the whole block: no list positions here
  for (int x = tid; x < kRrWaves * 257; x += kRrThreads) (&hist[0][0])[x] = 0;
  const int pos = c * kRrChunk + tid;
  int e = kNoExpert;
  if (pos < n) {
    const int i = cur[2 * pos], ptr = cur[2 * pos + 1], t = i / k;
    int jn = 0, after = 0;
    for (int b = 1; b < k && pos - b >= 0 && cur[2 * (pos - b)] / k == t; ++b) ++jn;
    for (int b = 1; b < k && pos + b < n && cur[2 * (pos + b)] / k == t; ++b) ++after;
    const int q = ptr + jn;
    if (q < nf) e = p.fallback[(int64_t)t * nf + q];
    p.prop[pos] = e == kNoExpert ? -1 : e;
    p.pcnt[pos] = jn + 1 + after;
  }
  // lanes of the wave with the same proposal: 9 ballots on the expert bits
  uint64_t peers = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const bool on = (e >> bit) & 1;
    const uint64_t bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  const int r_w = __popcll(peers & ((1ull << lane) - 1ull));
  __syncthreads();  // hist is zero
  if (e != kNoExpert && r_w == 0) hist[w][e] = __popcll(peers);
  __syncthreads();
  for (int x = tid; x < p.E; x += kRrThreads) {  // per expert, exclusive over the waves
    int run = 0;
    for (int q = 0; q < kRrWaves; ++q) {
      const int v = hist[q][x];
      hist[q][x] = run;
      run += v;
    }
    p.chunk_hist[(int64_t)c * p.E + x] = run;
  }
  __syncthreads();
  if (pos < n && e != kNoExpert) p.local_rank[pos] = hist[w][e] + r_w;
}

// Round r, pass 2 (one block): per expert, the chunk bases (exclusive over the
// chunks), the proposals in all and the load after the round; per chunk, how
// many of its proposals are rejected (those of expert e ranked at or past the
// expert's spare capacity), their bases in chunk order, and the next list's
// length.
__global__ __launch_bounds__(kRrThreads) void rr_round_scan_kernel(RerouteParams p, int r) {
  __shared__ int s_spare[256];
  __shared__ int wtot[kRrWaves];
  const int tid = threadIdx.x;
  const int E = p.E;
  const int n = p.n_g[r & 1];
  const int chunks = (n + kRrChunk - 1) / kRrChunk;
  const int* load_in = p.load_g + (r & 1) * 256;
  int* load_out = p.load_g + ((r + 1) & 1) * 256;
  constexpr int kBatch = 16;
  for (int e = tid; e < E; e += kRrThreads) {
    int run = 0;
    for (int c0 = 0; c0 < chunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        v[j] = c0 + j < chunks ? p.chunk_hist[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < chunks) p.chunk_ebase[(int64_t)(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
    const int spare = p.C - load_in[e];
    s_spare[e] = spare;
    load_out[e] = load_in[e] + (run < spare ? run : spare);
  }
  __syncthreads();  // the bases written above are visible to the whole block
  int carry = 0;
  for (int c0 = 0; c0 < chunks; c0 += kRrThreads) {
    const int c = c0 + tid;
    int rej = 0;
    if (c < chunks) {
      for (int e = 0; e < E; ++e) {
        const int cnt = p.chunk_hist[(int64_t)c * E + e];
        int ok = s_spare[e] - p.chunk_ebase[(int64_t)c * E + e];
        ok = ok < 0 ? 0 : (ok > cnt ? cnt : ok);
        rej += cnt - ok;
      }
    }
    int total;
    const int ex = rr_excl_sum(rej, wtot, total);
    if (c < chunks) p.chunk_base[c] = carry + ex;
    carry += total;
  }
  if (tid == 0) p.n_g[(r + 1) & 1] = carry;
}

// Round r, pass 3: acceptance against the load at the start of the round, and
// the ordered compaction of the rejected pairs into the next list (their
// token pointer moves past all of the token's proposals of the round).
__global__ __launch_bounds__(kRrThreads) void rr_accept_kernel(RerouteParams p, int r) {
  __shared__ int wtot[kRrWaves];
  const int tid = threadIdx.x;
  const int* cur = (r & 1) ? p.list_b : p.list_a;
  int* nxt = (r & 1) ? p.list_a : p.list_b;
  const int n = p.n_g[r & 1];
  const int c = blockIdx.x;
  if (c * kRrChunk >= n) return;
  const int pos = c * kRrChunk + tid;
  const int* load_in = p.load_g + (r & 1) * 256;
  bool rej = false;
  int i = 0, ptr = 0;
  if (pos < n) {
    const int e = p.prop[pos];
    i = cur[2 * pos];
    ptr = cur[2 * pos + 1];
    if (e >= 0) {
      const int rank = p.chunk_ebase[(int64_t)c * p.E + e] + p.local_rank[pos];
      const int l = load_in[e];
      if (l + rank < p.C) {
        p.fe[i] = e;
        p.rin[i] = l + rank;
      } else {
        rej = true;
      }
    }
  }
  int total;
  const int ex = rr_excl_count(rej, wtot, total);
  if (rej) {
    const int o = p.chunk_base[c] + ex;
    nxt[2 * o] = i;
    nxt[2 * o + 1] = ptr + p.pcnt[pos];
  }
}

// The rounds, in one block of 1024 threads.  The unplaced list holds pairs
// (assignment i, its token's fallback pointer at the start of the round) in
// arrival order.  Chunks of proposals go through a three-stage software
// pipeline, so no step waits on a dependent global load; a step takes 4096
// proposals (four per thread, 64 slices of 64 lanes in arrival order):
//   step s loads the pairs of chunk s+3 into registers,
//          writes the tokens of chunk s+2 (loaded a step ago) into an LDS ring
//          of three chunks,
//          lets each slot of chunk s+1 find, in the ring, its position j among
//          its token's unplaced slots and how many follow it, and loads its
//          proposal F[t, ptr + j],
//          and settles chunk s: ranks per expert (9 ballots per slice, slice
//          histograms tagged with the chunk number so they need no zeroing),
//          acceptance against the expert's load at the start of the round,
//          and the ordered compaction of the rejected pairs, whose token
//          pointer moves past all of the token's proposals of the round.
struct Pair { int i, ptr; };
constexpr int kSub = 4;                        // 1024-proposal sub-chunks per step
constexpr int kStep = kSub * kRrThreads;       // proposals per step
constexpr int kSlices = kSub * kRrWaves;       // 64-lane slices per step
constexpr int kRing = 3 * kStep;
static_assert(kSlices == 64, "one lane per slice in the scans");

// start_round > 0: the multi-block passes built the list and ran rounds
// 0 .. start_round-1; the list, its length and the loads continue from there.
__global__ __launch_bounds__(kRrThreads) void reroute_kernel(RerouteParams p, int start_round) {
  // (tag << 16) | count, then | base; rows padded to 257 words so the scan's
  // column reads (lane = slice) fall in 64 distinct banks
  __shared__ uint32_t hist[kSlices][257];
  __shared__ int load[256], run[256], ctot[256];
  __shared__ int wtot[kSlices];
  __shared__ int ring[kRing];              // token of list position pos % kRing
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = p.E, k = p.k, C = p.C, nf = p.E - p.k;
  const int n_all = p.T * k;
  for (int x = tid; x < kSlices * 257; x += kRrThreads) (&hist[0][0])[x] = 0u;
  int n = 0;
  int* cur = p.list_a;
  int* nxt = p.list_b;
  if (start_round > 0) {
    for (int e = tid; e < 256; e += kRrThreads) load[e] = p.load_g[(start_round & 1) * 256 + e];
    n = p.n_g[start_round & 1];
    if (start_round & 1) {
      cur = p.list_b;
      nxt = p.list_a;
    }
  } else {
    for (int e = tid; e < 256; e += kRrThreads) {
      const int c = e < E ? p.counts[e] : 0;
      load[e] = c < C ? c : C;
    }
    for (int e = tid; e <= E; e += kRrThreads) p.off_prim[e] = p.offsets[e];
  }
  // the unplaced list, in arrival order, with pointer 0; four slots a thread
  for (int i0 = 0; start_round == 0 && i0 < n_all; i0 += 4 * kRrThreads) {
    int cnt = 0, fl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 4 * tid + u;
      fl[u] = i < n_all && p.dest[i] < 0;
      cnt += fl[u];
    }
    int incl = cnt;  // inclusive prefix over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int x = 0; x < kRrWaves; ++x) {
      before += x < w ? wtot[x] : 0;
      all += wtot[x];
    }
    __syncthreads();
    int pos = n + before + incl - cnt;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (fl[u]) {
        const int i = i0 + 4 * tid + u;
        p.list_a[2 * pos] = i;
        p.list_a[2 * pos + 1] = 0;
        p.fe[i] = -1;
        ++pos;
      }
    }
    n += all;
  }
  uint32_t tag = 0;
  __syncthreads();

  for (int round = start_round; round <= nf && n > 0; ++round) {
    for (int e = tid; e < 256; e += kRrThreads) run[e] = 0;
    int m = 0;
    // position of this thread's proposal u in step-chunk c
    auto at = [&](int c, int u) { return c * kStep + u * kRrThreads + tid; };
    auto load_pair = [&](int pos) -> Pair {
      Pair r{-1, 0};
      if (pos < n) {
        r.i = cur[2 * pos];
        r.ptr = cur[2 * pos + 1];
      }
      return r;
    };
    Pair pa[kSub], p1[kSub], pc[kSub];
    int ec[kSub], cntc[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      pa[u] = load_pair(at(0, u));
      p1[u] = Pair{-1, 0};
      pc[u] = Pair{-1, 0};
      ec[u] = kNoExpert;
      cntc[u] = 0;
    }
    // sub-chunks of step-chunk c that hold proposals (uniform)
    auto live = [&](int c) {
      const int left = n - c * kStep;
      return left <= 0 ? 0 : (left >= kStep ? kSub : (left + kRrThreads - 1) / kRrThreads);
    };
    for (int s_ = -2; s_ * kStep < n; ++s_) {
      Pair pb[kSub];
      const int live_cur = live(s_), live_2 = live(s_ + 2), live_3 = live(s_ + 3);
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        pb[u] = u < live_3 ? load_pair(at(s_ + 3, u)) : Pair{-1, 0};  // chunk s+3
        if (u < live_2) {                  // chunk s+2's tokens into the ring
          const int pos = at(s_ + 2, u);
          ring[pos % kRing] = pa[u].i >= 0 ? pa[u].i / k : -1 - pos;
        }
      }
      const bool cur_ok = s_ >= 0;
      // ---- current chunk s: ballots and slice counts
      int r_slice[kSub];
      if (cur_ok) {
        ++tag;
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          r_slice[u] = 0;
          if (u >= live_cur) continue;   // no proposals there: slices stay empty
          const int e = ec[u];
          uint64_t peers = ~0ull;
#pragma unroll
          for (int bit = 0; bit < 9; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bal = __ballot(on);
            peers &= on ? bal : ~bal;
          }
          r_slice[u] = __popcll(peers & ((1ull << lane) - 1ull));
          if (e != kNoExpert && r_slice[u] == 0)
            hist[u * kRrWaves + w][e] = (tag << 16) | (uint32_t)__popcll(peers);
        }
      }
      __syncthreads();  // A: ring and slice counts are in
      // ---- chunk s+1: position among its token's slots, proposal
      int en[kSub], cntn[kSub];
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        en[u] = kNoExpert;
        cntn[u] = 0;
        if (p1[u].i >= 0) {
          const int pos = at(s_ + 1, u);
          const int t = p1[u].i / k;
          int jn = 0, after = 0;
          for (int b = 1; b < k && pos - b >= 0 && ring[(pos - b) % kRing] == t; ++b) ++jn;
          for (int b = 1; b < k && pos + b < n && ring[(pos + b) % kRing] == t; ++b) ++after;
          cntn[u] = jn + 1 + after;
          const int q = p1[u].ptr + jn;
          if (q < nf) en[u] = p.fallback[(int64_t)t * nf + q];
        }
      }
      if (cur_ok) {
        // per expert, an exclusive scan over the 64 slices: one wave per
        // expert, lane = slice
        for (int x = w; x < E; x += kRrWaves) {
          const uint32_t h = hist[lane][x];
          const int c = (h >> 16) == tag ? (int)(h & 0xffffu) : 0;
          int incl = c;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
          }
          hist[lane][x] = (tag << 16) | (uint32_t)(incl - c);
          if (lane == 63) ctot[x] = incl;
        }
      }
      __syncthreads();  // B: slice bases and chunk totals are in
      if (cur_ok) {
        uint64_t sb[kSub];
        bool still[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          const int e = ec[u];
          still[u] = false;
          if (e != kNoExpert) {
            const int rank = run[e] + (int)(hist[u * kRrWaves + w][e] & 0xffffu) + r_slice[u];
            if (load[e] + rank < C) {
              p.fe[pc[u].i] = e;
              p.rin[pc[u].i] = load[e] + rank;
            } else {
              still[u] = true;
            }
          }
          sb[u] = __ballot(still[u]);
          if (lane == 0) wtot[u * kRrWaves + w] = __popcll(sb[u]);
        }
        __syncthreads();  // C: every slice's count of rejected pairs is in
        // exclusive scan of the slice counts, lane = slice, in every wave
        const int wc = wtot[lane];
        int wincl = wc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_up(wincl, o, kWave);
          if (lane >= o) wincl += v;
        }
        const int all = __shfl(wincl, 63, kWave);
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
          const int before = __shfl(wincl - wc, u * kRrWaves + w, kWave);
          if (still[u]) {
            const int o = m + before + __popcll(sb[u] & ((1ull << lane) - 1ull));
            nxt[2 * o] = pc[u].i;
            nxt[2 * o + 1] = pc[u].ptr + cntc[u];  // past all of the token's proposals
          }
        }
        m += all;
        for (int x = tid; x < E; x += kRrThreads) run[x] += ctot[x];
      }
      // next step: chunk s+1 is current, s+2 becomes s+1, s+3 becomes s+2
#pragma unroll
      for (int u = 0; u < kSub; ++u) {
        pc[u] = p1[u];
        ec[u] = en[u];
        cntc[u] = cntn[u];
        p1[u] = pa[u];
        pa[u] = pb[u];
      }
    }
    __syncthreads();
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
  if (tid == 0) {
    int acc = 0;
    for (int x = 0; x < E; ++x) {
      p.offsets[x] = acc;
      acc += load[x];
    }
    p.offsets[E] = acc;
  }
}

// Final placement of every assignment: primary kept rows keep their rank,
// re-routed ones take theirs from the rounds.
__global__ __launch_bounds__(256) void reroute_place_kernel(RerouteParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)p.T * p.k) return;
  const int dp = p.dest[i];
  int e, r;
  if (dp >= 0) {
    e = p.idx[i];
    r = dp - p.off_prim[e];
  } else {
    e = p.fe[i];
    r = e >= 0 ? p.rin[i] : 0;
  }
  const int d = e >= 0 ? p.offsets[e] + r : -1;
  p.final_expert[i] = e;
  p.dest_out[i] = d;
  if (d >= 0) p.row_token[d] = (int)(i / p.k);
}

}  // namespace

hipError_t launch_reroute(const RerouteParams& p, hipStream_t stream) {
  if (p.T > 0 && p.E > p.k)
    hipLaunchKernelGGL(fallback_kernel, dim3((p.T + 3) / 4), dim3(256), 0, stream, p);
  // batches of 4096 assignments or more run the list build and the first
  // (up to 3) rounds as multi-block passes; the rest stay in one block
  const int64_t n_all = (int64_t)p.T * p.k;
  const int chunks = reroute_chunks(n_all);
  const int mb = n_all >= 4096 ? std::min(3, p.E - p.k + 1) : 0;
  if (mb > 0) {
    hipLaunchKernelGGL(rr_list_count_kernel, dim3(chunks), dim3(kRrThreads), 0, stream, p);
    hipLaunchKernelGGL(rr_list_scan_kernel, dim3(1), dim3(kRrThreads), 0, stream, p, chunks);
    hipLaunchKernelGGL(rr_list_write_kernel, dim3(chunks), dim3(kRrThreads), 0, stream, p);
    for (int r = 0; r < mb; ++r) {
      hipLaunchKernelGGL(rr_propose_kernel, dim3(chunks), dim3(kRrThreads), 0, stream, p, r);
      hipLaunchKernelGGL(rr_round_scan_kernel, dim3(1), dim3(kRrThreads), 0, stream, p, r);
      hipLaunchKernelGGL(rr_accept_kernel, dim3(chunks), dim3(kRrThreads), 0, stream, p, r);
    }
  }
  hipLaunchKernelGGL(reroute_kernel, dim3(1), dim3(kRrThreads), 0, stream, p, mb);
  const int64_t n = (int64_t)p.T * p.k;
  if (n > 0)
    hipLaunchKernelGGL(reroute_place_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace moe
