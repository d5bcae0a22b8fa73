// Grouped expert GEMM for many rows per expert (prefill-shaped), bf16 MFMA.
//
// Each expert is an FFN with its own weights that runs once over the tokens
// routed to it ("Mixture-of-Experts & Sparse Model Scaling", Core Concepts;
// "Scaling Capacity via Sparse MoE Architectures", the layer groups tokens by
// expert).  Both operands are contiguous along the reduction axis (C = A B^T).
//
// Tile schedule: a one-block kernel turns the device-side group offsets into a
// list of (group, first row, rows, first output row) entries of at most 256
// rows, so no host synchronisation is needed; the GEMM grid is sized for the
// worst case and surplus blocks exit at once.  Blocks are mapped to tiles so
// that each of the 8 XCDs (which receive workgroups round-robin) walks a
// contiguous range of tiles, and within it groups of 4 row-tiles sweep the
// output columns together, so the A and B slabs of concurrent tiles are shared
// through that XCD's L2.
//
// Block tile: 256 rows x 256 weight rows x 64 deep, 4 waves in a 2x2 grid, each
// wave 128x128 as 4x4 tiles of v_mfma_f32_32x32x16_bf16 with float32 accumulators.
// For the gated (SwiGLU) form the 256 weight rows are 128 rows of w1 and the
// same 128 rows of w3, and every wave holds matching gate and up accumulators,
// so silu(gate) * up is formed in registers.  Operands are staged through a
// double-buffered LDS tile whose 16-byte chunks are XOR-swizzled per row, so
// both the row-wise stores and the MFMA operand reads are bank-conflict-free.
// Routed rows may be gathered from the token matrix through row_token, which
// removes the separate permuted copy from the layer.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int BM = 256;      // output rows per tile
constexpr int BR = 256;      // weight rows per tile
constexpr int BK = 64;       // reduction depth per stage
constexpr int kThreads = 256;
constexpr int kGroupM = 4;   // row-tiles that sweep the columns together
constexpr int kTileBytes = BM * BK * 2;  // one operand tile, 32 KiB

// Kept out of line so the fully unrolled epilogue stays small enough to keep
// every accumulator in registers.
__device__ __noinline__ float gelu_outlined(float a) { return gelu_f32(a); }

__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * 128 + ((kc ^ ((row + (row >> 3)) & 7)) << 4);
}

// Workgroup P runs on XCD P % 8; give every XCD a contiguous range of tiles.
__device__ __forceinline__ int xcd_remap(int P, int nb) {
  const int x = P & 7, q = P >> 3, per = nb >> 3, rem = nb & 7;
  return x < rem ? x * (per + 1) + q : rem * (per + 1) + (x - rem) * per + q;
}

// Entries beyond max_entries (possible only if a caller's rows_bound is below
// offsets[G]) are not written, so the schedule never overruns its workspace.
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* offsets, int G,
                                                          int S, int T, int64_t rows_bound,
                                                          int max_entries, TileEntry* entries,
                                                          int32_t* n_entries) {
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  int base = 0;
  for (int g0 = 0; g0 < G + S; g0 += 256) {
    const int g = g0 + tid;
    int nt = 0, r0 = 0, rows = 0;
    if (g < G) {
      r0 = offsets[g];
      rows = offsets[g + 1] - r0;
    } else if (g < G + S) {
      rows = T;
    }
    nt = (rows + BM - 1) / BM;
    scan[tid] = nt;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = base + scan[tid] - nt;
    for (int i = 0; i < nt && first + i < max_entries; ++i) {
      TileEntry e;
      e.group = g;
      e.rows = min(BM, rows - i * BM);
      if (g < G) {
        e.a_row0 = r0 + i * BM;
        e.c_row0 = r0 + i * BM;
      } else {
        e.a_row0 = i * BM;
        e.c_row0 = (int)(rows_bound + (int64_t)(g - G) * T) + i * BM;
      }
      entries[first + i] = e;
    }
    base += scan[255];
    __syncthreads();
  }
  if (tid == 0) *n_entries = min(base, max_entries);
}

// ACT: moe_act_t for the up projection (2 = gated SwiGLU), -1 for none.
template <int ACT>
__global__ __launch_bounds__(kThreads, 1) void ffn_tiled_kernel(FfnParams p, int n_tiles_n,
                                                                int max_entries) {
  constexpr bool GATED = ACT == 2;
  __shared__ __attribute__((aligned(16))) char lds[4 * kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- which tile ----
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * n_tiles_n;
  const int grp = L / per_group, rem = L - grp * per_group;
  const int gsize = min(kGroupM, max_entries - grp * kGroupM);
  const int e_idx = grp * kGroupM + rem % gsize;
  const int n_idx = rem / gsize;
  if (e_idx >= *p.n_entries) return;
  const TileEntry te = p.entries[e_idx];
  const bool routed = te.group < p.G;
  const int gw = routed ? te.group : te.group - p.G;
  const int K = p.K, N = p.N;
  const int64_t wstride = (int64_t)N * K;
  const uint16_t* W = static_cast<const uint16_t*>(routed ? p.w_main : p.w_shared) + gw * wstride;
  const uint16_t* U = nullptr;
  if (GATED) U = static_cast<const uint16_t*>(routed ? p.u_main : p.u_shared) + gw * wstride;
  const uint16_t* A = static_cast<const uint16_t*>(routed ? p.a_main : p.a_shared);
  const int n_out0 = n_idx * (GATED ? BR / 2 : BR);

  // ---- global -> register staging assignment: rows r_ld + 32 i, chunk kc_ld ----
  // Element offsets stay 32-bit (the host rejects operands of 2^31 elements or
  // more); the weight rows of stage i are b_row0 + 32 (i mod 4) for the gated
  // form (w1 for i < 4, w3 after) and b_row0 + 32 i otherwise.
  const int kc_ld = tid & 7, r_ld = tid >> 3;
  uint32_t a_off[8];
  unsigned a_ok = 0, b_ok = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r_ld + 32 * i;
    const bool ok = row < te.rows;
    int arow = p.a_from_c ? te.c_row0 + row : te.a_row0 + row;
    if (ok && routed && p.gather && !p.a_from_c) arow = p.gather[arow];
    a_off[i] = (uint32_t)(ok ? arow : 0) * (uint32_t)K + kc_ld * 8;
    a_ok |= (unsigned)ok << i;
    const int n = n_out0 + r_ld + 32 * (GATED ? (i & 3) : i);
    b_ok |= (unsigned)(n < N) << i;
  }
  const uint32_t b_off0 = (uint32_t)min(n_out0 + r_ld, N - 1) * (uint32_t)K + kc_ld * 8;
  const uint32_t b_step = 32u * (uint32_t)K;

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16{};

  const int lr = lane & 31, lh = lane >> 5;
  int brow[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
    brow[ni] = GATED ? (ni < 2 ? wn * 64 + ni * 32 : 128 + wn * 64 + (ni - 2) * 32)
                     : wn * 128 + ni * 32;
  int st_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) st_off[i] = lds_off(r_ld + 32 * i, kc_ld);

  const int nk = (K + BK - 1) / BK;
  u32x4 ra[8], rb[8];
  const u32x4 z4 = {0u, 0u, 0u, 0u};
#define MOE_LOAD_STAGE(k0)                                                                 \
  {                                                                                        \
    const bool k_ok = (k0) + kc_ld * 8 < K;                                                \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
      ra[i] = (((a_ok >> i) & 1u) && k_ok)                                                 \
                  ? *reinterpret_cast<const u32x4*>(A + a_off[i] + (k0))                   \
                  : z4;                                                                    \
      const uint16_t* Bb = (GATED && i >= 4) ? U : W;                                      \
      const uint32_t bo = b_off0 + (uint32_t)(GATED ? (i & 3) : i) * b_step + (k0);        \
      rb[i] = (((b_ok >> i) & 1u) && k_ok) ? *reinterpret_cast<const u32x4*>(Bb + bo) : z4; \
    }                                                                                      \
  }
#define MOE_STORE_STAGE(buf)                                                               \
  {                                                                                        \
    char* As_ = lds + (buf) * 2 * kTileBytes;                                              \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
      *reinterpret_cast<u32x4*>(As_ + st_off[i]) = ra[i];                                  \
      *reinterpret_cast<u32x4*>(As_ + kTileBytes + st_off[i]) = rb[i];                     \
    }                                                                                      \
  }

  MOE_LOAD_STAGE(0)
  MOE_STORE_STAGE(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) MOE_LOAD_STAGE((kt + 1) * BK)
    const char* As = lds + (kt & 1) * 2 * kTileBytes;
    const char* Bs = As + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kc = kk * 2 + lh;
      bf16x8 af[4], bv[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 128 + mi * 32 + lr, kc));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bv[ni] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(brow[ni] + lr, kc));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) MOE_STORE_STAGE((kt + 1) & 1)
    __syncthreads();
  }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE

  // ---- epilogue: 32x32 result layout, lane holds column lane%32,
  //      rows 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15 ----
  const float* bias = routed ? p.bias_main : p.bias_shared;
  constexpr int NJ = GATED ? 2 : 4;  // output column blocks per wave
  int col[NJ];
  float bcol[NJ];
#pragma unroll
  for (int nj = 0; nj < NJ; ++nj) {
    col[nj] = n_out0 + (GATED ? wn * 64 : wn * 128) + nj * 32 + lr;
    bcol[nj] = (bias && col[nj] < N) ? bias[(int64_t)gw * N + col[nj]] : 0.f;
  }
  uint16_t* __restrict__ out16 = static_cast<uint16_t*>(p.out);
  float* __restrict__ out32 = static_cast<float*>(p.out);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * 128 + mi * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
      const bool row_ok = row < te.rows;
      const int64_t orow = (int64_t)(te.c_row0 + row) * N;
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        if (!row_ok || col[nj] >= N) continue;
        float o;
        if (GATED) {
          o = silu_f32(acc[mi][nj][v] + bcol[nj]) * acc[mi][nj + 2][v];
        } else {
          o = acc[mi][nj][v] + bcol[nj];
          if (ACT == 0) o = gelu_outlined(o);
          if (ACT == 1) o = fmaxf(o, 0.f);
        }
        if (p.out_bf16) {
          out16[orow + col[nj]] = f32_to_bf16(o);
        } else {
          float* dst = out32 + orow + col[nj];
          *dst = p.accumulate ? *dst + o : o;
        }
      }
    }
  }
}

}  // namespace

int64_t ffn_max_entries(int64_t rows_bound, int G, int S, int T) {
  return (rows_bound + BM - 1) / BM + G + (int64_t)S * ((T + BM - 1) / BM);
}

hipError_t launch_ffn_tiled(const FfnParams& p, hipStream_t stream) {
  const int64_t max_entries = ffn_max_entries(p.rows_bound, p.G, p.S, p.T);
  const bool gated = p.act == 2;
  const int cols = gated ? BR / 2 : BR;
  const int n_tiles_n = (p.N + cols - 1) / cols;
  const int64_t blocks = max_entries * n_tiles_n;
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, p.offsets, p.G, p.S,
                     p.T, p.rows_bound, (int)max_entries, p.entries, p.n_entries);
  if (blocks > 0) {
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (p.act) {
      case 2: hipLaunchKernelGGL(ffn_tiled_kernel<2>, grid, block, 0, stream, p, n_tiles_n, (int)max_entries); break;
      case 1: hipLaunchKernelGGL(ffn_tiled_kernel<1>, grid, block, 0, stream, p, n_tiles_n, (int)max_entries); break;
      case 0: hipLaunchKernelGGL(ffn_tiled_kernel<0>, grid, block, 0, stream, p, n_tiles_n, (int)max_entries); break;
      default: hipLaunchKernelGGL(ffn_tiled_kernel<-1>, grid, block, 0, stream, p, n_tiles_n, (int)max_entries); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
