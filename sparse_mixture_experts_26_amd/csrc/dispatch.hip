// Per-expert counts, capacity and expert-contiguous dispatch tables.
//
// "Mixture-of-Experts & Sparse Model Scaling", lab 3 and Advanced Theory: each
// expert accepts assignments in arrival order until it holds C of them, the
// rest are dropped; "Mixture-of-experts Models", Level 2: loads and overflow
// per expert; "Scaling Capacity via Sparse MoE Architectures": tokens are
// grouped by their expert.  Arrival order is the flat index i = t*k + s.
//
// The sequential walk becomes a stable counting sort in three launches:
//   1. rank:   per 1024-assignment chunk, each 64-lane slice finds the lanes
//              holding the same expert with 9 ballots, so its stable rank within
//              the slice is a popcount; slice histograms in LDS are prefix-summed
//              in slice order to give the rank within the chunk and the chunk's
//              per-expert histogram.
//   2. scan:   one block turns the chunk histograms into per-chunk bases (chunk
//              order), counts, kept = min(counts, C) and the offsets.
//   3. assign: rank = base + local rank; kept iff rank < C; dest and row_token.
// A batch of at most four chunks (decode- and Switch-sized) runs all three
// steps in a single block of 16 waves, one to four slices per wave, with the
// tables kept in LDS.
// Every step is ordered, so the integer outputs are exact and deterministic.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kSlices = kDispatchChunk / 64;  // 16 slices of 64 per chunk
constexpr int kInvalid = 511;                 // expert id that matches no expert

// Stable rank of lane's expert among the 64 lanes of its slice; `count` gets
// the number of lanes holding the same expert.
__device__ __forceinline__ int slice_rank(int e, int lane, int& count) {
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  count = __popcll(peers);
  return __popcll(peers & ((1ull << lane) - 1ull));
}

// n <= NS * kDispatchChunk: rank, scan and assign in one block of 16 waves;
// wave w takes slices w, w + 16, ..., w + 16 (NS - 1), and the slices are
// prefix-summed per expert in slice (= arrival) order.
template <int NS>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(DispatchParams p) {
  __shared__ int hist[NS * kSlices][256];
  __shared__ int sscan[256];
  __shared__ int soff[256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, x = threadIdx.x;
  for (int i = x; i < NS * kSlices * 256; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();
  int my_e[NS], my_r[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int s = w + kSlices * j;
    const int i = s * 64 + lane;
    int e = kInvalid;
    if (i < p.n) {
      e = p.idx[i];
      if (e < 0 || e >= p.E) e = kInvalid;
    }
    int cnt;
    const int r = slice_rank(e, lane, cnt);
    if (e != kInvalid && r == 0) hist[s][e] = cnt;
    my_e[j] = e;
    my_r[j] = r;
  }
  __syncthreads();
  int kept = 0;
  if (x < 256) {
    if (x < p.E) {
      // the expert's slice counts, read together, then their exclusive
      // prefix in slice order
      int c[NS * kSlices];
#pragma unroll
      for (int q = 0; q < NS * kSlices; ++q) c[q] = hist[q][x];
      int run = 0;
#pragma unroll
      for (int q = 0; q < NS * kSlices; ++q) {
        hist[q][x] = run;
        run += c[q];
      }
      p.counts[x] = run;
      kept = run < p.C ? run : p.C;
    }
    sscan[x] = kept;
  }
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // Hillis-Steele inclusive scan
    const int v = (x < 256 && x >= o) ? sscan[x - o] : 0;
    __syncthreads();
    if (x < 256) sscan[x] += v;
    __syncthreads();
  }
  if (x < p.E) {
    soff[x] = sscan[x] - kept;
    p.offsets[x] = sscan[x] - kept;
    if (x == p.E - 1) p.offsets[p.E] = sscan[x];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int s = w + kSlices * j;
    const int i = s * 64 + lane;
    if (i < p.n) {
      const int e = my_e[j];
      int d = -1;
      if (e != kInvalid) {
        const int rank = hist[s][e] + my_r[j];
        if (rank < p.C) {
          d = soff[e] + rank;
          p.row_token[d] = i / p.k;
        }
      }
      p.dest[i] = d;
    }
  }
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(DispatchParams p) {
  __shared__ int hist[kSlices][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kSlices * 256; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t chunk0 = (int64_t)blockIdx.x * kDispatchChunk;
  int my_e[4], my_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = w + 4 * r;
    const int64_t i = chunk0 + s * 64 + lane;
    int e = kInvalid;
    if (i < p.n) {
      e = p.idx[i];
      if (e < 0 || e >= p.E) e = kInvalid;
    }
    int cnt;
    const int rank = slice_rank(e, lane, cnt);
    if (e != kInvalid && rank == 0) hist[s][e] = cnt;
    my_e[r] = e;
    my_r[r] = rank;
  }
  __syncthreads();
  if ((int)threadIdx.x < p.E) {
    const int e = threadIdx.x;
    int run = 0;
    for (int s = 0; s < kSlices; ++s) {
      const int c = hist[s][e];
      hist[s][e] = run;
      run += c;
    }
    p.chunk_hist[(int64_t)blockIdx.x * p.E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = w + 4 * r;
    const int64_t i = chunk0 + s * 64 + lane;
    if (i < p.n) p.local_rank[i] = my_e[r] == kInvalid ? -1 : hist[s][my_e[r]] + my_r[r];
  }
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(DispatchParams p, int nchunks) {
  __shared__ int skept[256];
  const int tid = threadIdx.x;
  // per expert (one thread each): the chunk histograms become per-chunk base
  // ranks in chunk order, and the total is the expert's count; the column is
  // read 16 chunks at a time so that its loads are in flight together
  constexpr int kBatch = 16;
  int run = 0;
  if (tid < p.E) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int* col = p.chunk_hist + (int64_t)c0 * p.E + tid;
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < nchunks ? col[(int64_t)j * p.E] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < nchunks) col[(int64_t)j * p.E] = run;
        run += v[j];
      }
    }
    p.counts[tid] = run;
  }
  skept[tid] = tid < p.E ? (run < p.C ? run : p.C) : 0;
  __syncthreads();
  const int e = tid;
  const int kept = skept[e];
  // Hillis-Steele inclusive scan over 256 experts.
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? skept[e - o] : 0;
    __syncthreads();
    skept[e] += v;
    __syncthreads();
  }
  if (e < p.E) p.offsets[e] = skept[e] - kept;
  if (e == p.E - 1) p.offsets[p.E] = skept[e];
}

__global__ __launch_bounds__(256) void dispatch_assign_kernel(DispatchParams p) {
  const int64_t chunk0 = (int64_t)blockIdx.x * kDispatchChunk;
  for (int j = threadIdx.x; j < kDispatchChunk; j += 256) {
    const int64_t i = chunk0 + j;
    if (i >= p.n) break;
    const int lr = p.local_rank[i];
    int d = -1;
    if (lr >= 0) {
      const int e = p.idx[i];
      const int rank = p.chunk_hist[(int64_t)blockIdx.x * p.E + e] + lr;
      if (rank < p.C) {
        d = p.offsets[e] + rank;
        p.row_token[d] = (int)(i / p.k);
      }
    }
    p.dest[i] = d;
  }
}

// One wave per destination row; 16-byte copies.
__global__ __launch_bounds__(256) void permute_kernel(const uint4* x, const int32_t* row_token,
                                                      const int32_t* total, uint4* xp,
                                                      int64_t row_vecs) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= *total) return;
  const int64_t t = row_token[r];
  const uint4* src = x + t * row_vecs;
  uint4* dst = xp + r * row_vecs;
  for (int64_t c = lane; c < row_vecs; c += 64) dst[c] = src[c];
}

}  // namespace

hipError_t launch_dispatch(const DispatchParams& p, hipStream_t stream) {
  const int chunks = dispatch_chunks(p.n);
  if (chunks == 1) {
    hipLaunchKernelGGL(dispatch_small_kernel<1>, dim3(1), dim3(1024), 0, stream, p);
    return hipGetLastError();
  }
  if (chunks <= 4) {  // (a 64 KiB slice table in LDS)
    hipLaunchKernelGGL(dispatch_small_kernel<4>, dim3(1), dim3(1024), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_rank_kernel, dim3(chunks), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, stream, p, chunks);
  hipLaunchKernelGGL(dispatch_assign_kernel, dim3(chunks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_permute(const void* x, const int32_t* row_token, const int32_t* total,
                          void* x_perm, int64_t row_bytes, int64_t rows_bound,
                          hipStream_t stream) {
  const int64_t blocks = (rows_bound + 3) / 4;
  if (blocks > 0)
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint4*)x, row_token, total, (uint4*)x_perm, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
