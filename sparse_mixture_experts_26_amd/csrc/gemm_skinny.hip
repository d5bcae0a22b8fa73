// Grouped expert GEMM for at most 32 rows per expert (decode- and
// Switch-shaped layers), bf16 MFMA.
//
// With a handful of rows per expert the expert FFN is a stream over the
// expert's weights ("Mixture-of-Experts & Sparse Model Scaling", Computational
// Considerations: MoE layers are more memory-bound than dense ones of equal
// active size), so the kernel is built to keep HBM busy rather than to reuse
// operands.  Work is cut into units of (expert, 32-column slab of its weight
// rows); the grid is two resident blocks per CU and each block walks an equal,
// contiguous run of units, so neighbouring slabs of one expert stream through
// the same CU and no partial last wave of blocks is left.  Each unit's weight
// rows are read exactly once with 16-byte buffer loads; the 4 waves of a block
// split the reduction axis, and each wave keeps the next 64-deep step's loads
// in flight (register double buffer) while it multiplies the current one.  The
// expert's <= 32 operand rows ride along as the A operand of
// v_mfma_f32_16x16x32_bf16 (two 16-row fragments; the second reads zeros when
// the expert holds 16 rows or fewer).  The 4 partial products are summed in
// LDS in wave order (deterministic) and the activation is applied there.
// Experts that received no rows read no weights at all.
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNF = 4;  // 16-column fragments per unit: 32 or 64 output columns
constexpr int UNR = 2;     // 32-deep k-steps per pipeline stage
constexpr int kStep = 32 * UNR;  // depth of one pipeline stage
constexpr uint32_t kOOB = 0x80000000u;
#ifndef MOE_SKINNY_BLOCKS_PER_CU
#define MOE_SKINNY_BLOCKS_PER_CU 2
#endif
constexpr int kBlocksPerCU = MOE_SKINNY_BLOCKS_PER_CU;

// Where a unit's operands live: the load side runs one pipeline step ahead of
// the multiply side, so each keeps its own copy across unit boundaries.
struct UnitDesc {
  int g, rows, c_row0;
  uint32_t a_off[2];
  uint32_t b_off[kMaxNF];
  const uint16_t* W;
  const uint16_t* U;
  const void* A;
};

// The unit's base pointers are the same for the whole wave; say so, or the
// buffer resources built from them are taken as per-lane and every load
// becomes a waterfall loop (which also makes the wait counts conservative).
__device__ __forceinline__ void* uniform_ptr(const void* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// NF: 16-column fragments per unit (2 or 4); wider units put more bytes in
// flight per step and halve the number of unit reductions.
// WU: every wave owns whole units (the full reduction axis, no LDS reduction,
// no barriers), for short reductions with units enough for every wave;
// otherwise the block's 4 waves split each unit's reduction axis.
template <int ACT, int NF, bool WU>
__global__ __launch_bounds__(kThreads) void ffn_skinny_kernel(FfnParams p, int n_slabs,
                                                              int n_units) {
  constexpr int kCols = NF * 16;
  constexpr bool GATED = ACT == 2;
  constexpr int NB = GATED ? 2 : 1;           // weight sets (w1 and w3 when gated)
  constexpr int NFRAG = 2 * NF * NB;          // (row fragment, column fragment, set)
  __shared__ float red[WU ? 1 : 4][NFRAG][4][64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = p.K, N = p.N;
  const int64_t wstride = (int64_t)N * K;
  // a contiguous run of units per block (per wave with WU)
  const int64_t workers = WU ? (int64_t)gridDim.x * 4 : gridDim.x;
  const int64_t me = WU ? (int64_t)blockIdx.x * 4 + w : blockIdx.x;
  const int u_begin = (int)(me * n_units / workers);
  const int u_end = (int)((me + 1) * n_units / workers);
  // this wave's contiguous reduction range; every wave runs `per` steps
  // per unit (steps past its range read zeros), so the waves stay in step
  const int kch = (K + kStep - 1) / kStep, per = WU ? kch : (kch + 3) / 4;
  const int kb = WU ? 0 : min(K, w * per * kStep), ke = WU ? K : min(K, (w + 1) * per * kStep);
  const int kl = (lane >> 4) * 8;
  const int total = (u_end - u_begin) * per;

  // Unit descriptor.  The expert's row range and gathered rows are re-read
  // only when the expert changes (consecutive units are slabs of one expert):
  // those loads are needed at once, and waiting for them would also wait for
  // the stage in flight.  The stage loads themselves are unconditional, so the
  // compiler's wait counts stay exact.
  int cached_g = -1, cached_rows = 0, cached_r0 = 0;
  uint32_t cached_a[2] = {kOOB, kOOB};
  auto describe = [&](int u, UnitDesc& d) __attribute__((always_inline)) {
    const int g = u / n_slabs, slab = u - g * n_slabs;
    const bool routed = g < p.G;
    if (g != cached_g) {
      int rows, a_row0;
      if (routed) {
        a_row0 = p.offsets[g];
        rows = p.offsets[g + 1] - a_row0;
        cached_r0 = a_row0;
      } else {
        a_row0 = 0;
        rows = p.T;
        cached_r0 = (int)(p.rows_bound + (int64_t)(g - p.G) * p.T);
      }
      rows = min(rows, 32);
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        const int r = mf * 16 + (lane & 15);
        const bool ok = r < rows;
        int arow = p.a_from_c ? cached_r0 + r : a_row0 + r;
        if (ok && routed && p.gather && !p.a_from_c) arow = p.gather[arow];
        cached_a[mf] = ok ? ((uint32_t)arow * (uint32_t)K + kl) * 2u : kOOB;
      }
      cached_g = g;
      cached_rows = rows;
    }
    const int gw = routed ? g : g - p.G;
    d.g = g;
    d.rows = cached_rows;
    d.c_row0 = cached_r0;
    d.a_off[0] = cached_a[0];
    d.a_off[1] = cached_a[1];
    d.W = static_cast<const uint16_t*>(routed ? p.w_main : p.w_shared) + gw * wstride;
    d.U = GATED ? static_cast<const uint16_t*>(routed ? p.u_main : p.u_shared) + gw * wstride : d.W;
    d.A = routed ? p.a_main : p.a_shared;
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      const int n = slab * kCols + nf * 16 + (lane & 15);
      // an expert with no rows reads no weights: every offset is out of range
      d.b_off[nf] = (n < N && cached_rows > 0) ? ((uint32_t)n * (uint32_t)K + kl) * 2u : kOOB;
    }
  };

  f32x4 acc[2][NF][NB];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s) acc[mf][nf][s] = f32x4{};
  };

  // `red` is the only memory the waves share: a barrier needs this wave's LDS
  // operations done, not its loads in flight (which __syncthreads would drain)
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };

  struct Stage { u32x4 a[UNR][2], b[UNR][NF][NB]; };
  // loads of step `st` (0..per-1) of the unit described by d; `past` (past the
  // block's last step) turns every offset out of range: the loads read zeros
  // and move no data, and the code stays branch-free
  auto load = [&](Stage& sg, const UnitDesc& d, int st, uint32_t past) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.A), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.W), (short)0, (int)(wstride * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t u_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.U), (short)0, (int)(wstride * 2), 0x00020000);
    const int k0 = kb + st * kStep;
#pragma unroll
    for (int v = 0; v < UNR; ++v) {
      const int kk = k0 + v * 32 + kl;
      const uint32_t kadd = (kk < ke ? (uint32_t)(k0 + v * 32) * 2u : kOOB) | past;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
        sg.a[v][mf] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, (d.a_off[mf] + kadd) | past, 0, 0);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        sg.b[v][nf][0] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, (d.b_off[nf] + kadd) | past, 0, 0);
        if (GATED)
          sg.b[v][nf][NB - 1] =
              __builtin_amdgcn_raw_buffer_load_b128(u_rs, (d.b_off[nf] + kadd) | past, 0, 0);
      }
    }
  };
  // Both row fragments are always multiplied: the second reads zeros when the
  // expert holds 16 rows or fewer, and branch-free code keeps the compiler's
  // wait counts exact (MFMA time is negligible here).
  auto compute = [&](const Stage& sg) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < UNR; ++v)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, sg.b[v][nf][s]);
#pragma unroll
          for (int mf = 0; mf < 2; ++mf)
            acc[mf][nf][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, sg.a[v][mf]), b, acc[mf][nf][s], 0, 0, 0);
        }
  };
  // one output element of the unit: bias, pre-activations, activation, store
  auto emit = [&](const UnitDesc& d, int row, int col, float a, float up)
      __attribute__((always_inline)) {
    const bool routed = d.g < p.G;
    const int gw = routed ? d.g : d.g - p.G;
    const float* bias = routed ? p.bias_main : p.bias_shared;
    if (bias) a += bias[(int64_t)gw * N + col];
    if (ACT >= 0 && p.pre) {  // pre-activations for the backward
      uint16_t* pre = static_cast<uint16_t*>(p.pre) +
                      (int64_t)(d.c_row0 + row) * (GATED ? 2 * N : N) + col;
      pre[0] = f32_to_bf16(a);
      if (GATED) pre[N] = f32_to_bf16(up);
    }
    float out;
    if (GATED) {
      out = silu_f32(a) * up;
    } else if (ACT == 0) {
      out = gelu_f32(a);
    } else if (ACT == 1) {
      out = fmaxf(a, 0.f);
    } else {
      out = a;
    }
    const int64_t idx = (int64_t)(d.c_row0 + row) * N + col;
    if (p.out_bf16) {
      static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(out);
    } else {
      float* dst = static_cast<float*>(p.out) + idx;
      *dst = p.accumulate ? *dst + out : out;
    }
  };
  // sum the 4 waves' partial products in wave order, activation, store (with
  // WU the wave's own products, straight from the 16x16 result layout: lane
  // holds column lane%16 of rows 4*(lane/16) + i)
  auto finish = [&](const UnitDesc& d, int u) __attribute__((always_inline)) {
    if constexpr (WU) {
      const int slab = u - d.g * n_slabs;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = mf * 16 + (lane >> 4) * 4 + i;
            const int col = slab * kCols + nf * 16 + (lane & 15);
            if (row < d.rows && col < N)
              emit(d, row, col, acc[mf][nf][0][i], GATED ? acc[mf][nf][NB - 1][i] : 0.f);
          }
      return;
    }
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[w][(mf * NF + nf) * NB + s][i][lane] = acc[mf][nf][s][i];
    lds_barrier();
    const int slab = u - d.g * n_slabs;
    for (int o = threadIdx.x; o < 2 * NF * 256; o += kThreads) {
      const int mf = o / (NF * 256), rem = o - mf * NF * 256;
      const int nf = rem >> 8, i = (rem >> 6) & 3, l = rem & 63;
      const int row = mf * 16 + (l >> 4) * 4 + i;
      const int col = slab * kCols + nf * 16 + (l & 15);
      if (row >= d.rows || col >= N) continue;
      const int f0 = (mf * NF + nf) * NB;
      const float a = ((red[0][f0][i][l] + red[1][f0][i][l]) + red[2][f0][i][l]) + red[3][f0][i][l];
      float up = 0.f;
      if (GATED)
        up = ((red[0][f0 + 1][i][l] + red[1][f0 + 1][i][l]) + red[2][f0 + 1][i][l]) +
             red[3][f0 + 1][i][l];
      emit(d, row, col, a, up);
    }
    lds_barrier();  // red is reused by the next unit
  };

  // One continuous pipeline over the block's units: the loads of step i+1 (of
  // this unit or the next) are in flight while step i is multiplied, so a
  // unit's reduction and stores overlap the next unit's first loads.
  if (total <= 0) return;
  UnitDesc ld, cd;  // load side, multiply side
  describe(u_begin, ld);
  cd = ld;
  zero_acc();
  Stage s0, s1;
  load(s0, ld, 0, 0u);
#define MOE_SKINNY_STEP(Scur, Snext, i)                                    \
  {                                                                        \
    const int nl = (i) + 1;                                                \
    const int nq = nl < total ? nl : total - 1;                            \
    describe(u_begin + nq / per, ld);                                      \
    load(Snext, ld, nq % per, nl < total ? 0u : kOOB);                     \
    compute(Scur);                                                         \
    if ((i) % per == per - 1) {                                            \
      finish(cd, u_begin + (i) / per);                                     \
      zero_acc();                                                          \
      cd = ld;                                                             \
    }                                                                      \
  }
  // the loop body has no exit of its own: an exit between the two steps
  // would join the loop's back edge with loads still in flight, and the
  // compiler would then wait for all of them at the top of every iteration
  int i = 0;
  for (; i + 1 < total; i += 2) {
    MOE_SKINNY_STEP(s0, s1, i)
    MOE_SKINNY_STEP(s1, s0, i + 1)
  }
  if (i < total) MOE_SKINNY_STEP(s0, s1, i)
#undef MOE_SKINNY_STEP
}

}  // namespace

int device_cus();

hipError_t launch_ffn_skinny(const FfnParams& p, hipStream_t stream) {
  // Unit width and work split from a cost model in wave-steps of one
  // 16-column fragment: the busiest worker's units times their steps (the
  // K-split pays about 3 more steps per unit for its LDS reduction), times
  // the width.  Whole-unit waves must beat the K-split by 15% to be chosen;
  // between widths, ties go to the wider unit.
  const int64_t groups = p.G + p.S;
  const int64_t cap = (int64_t)device_cus() * kBlocksPerCU;
  const int64_t kch = (p.K + kStep - 1) / kStep;
  int nf = 2;
  bool wu = false;
  double best = 1e300;
  for (int cand = 4; cand >= 2; cand -= 2) {
    const int64_t units = groups * ((p.N + cand * 16 - 1) / (cand * 16));
    if (units == 0) continue;
    const int64_t blocks = std::min<int64_t>(units, cap);
    const double ksplit = (double)((units + blocks - 1) / blocks) * ((kch + 3) / 4 + 3) * cand;
    const int64_t wblocks = std::min<int64_t>((units + 3) / 4, cap);
    const double whole = (double)((units + 4 * wblocks - 1) / (4 * wblocks)) * kch * cand * 1.15;
    if (ksplit < best) { best = ksplit; nf = cand; wu = false; }
    if (whole < best) { best = whole; nf = cand; wu = true; }
  }
  const int n_slabs = (p.N + nf * 16 - 1) / (nf * 16);
  const int64_t n_units = groups * n_slabs;
  // two resident blocks per CU walk equal runs of units (of whole-unit
  // waves: a block's 4 waves take 4 consecutive runs)
  const int64_t grid = std::min<int64_t>(wu ? (n_units + 3) / 4 : n_units, cap);
  if (grid > 0) {
    const dim3 g((unsigned)grid), block(kThreads);
    const int nu = (int)n_units;
#define MOE_SKINNY_LAUNCH(NFV, WUV)                                                              \
  switch (p.act) {                                                                               \
    case 2: hipLaunchKernelGGL((ffn_skinny_kernel<2, NFV, WUV>), g, block, 0, stream, p, n_slabs, nu); break;  \
    case 1: hipLaunchKernelGGL((ffn_skinny_kernel<1, NFV, WUV>), g, block, 0, stream, p, n_slabs, nu); break;  \
    case 0: hipLaunchKernelGGL((ffn_skinny_kernel<0, NFV, WUV>), g, block, 0, stream, p, n_slabs, nu); break;  \
    default: hipLaunchKernelGGL((ffn_skinny_kernel<-1, NFV, WUV>), g, block, 0, stream, p, n_slabs, nu); break; \
  }
    if (nf == 4 && wu) {
      MOE_SKINNY_LAUNCH(4, true)
    } else if (nf == 4) {
      MOE_SKINNY_LAUNCH(4, false)
    } else if (wu) {
      MOE_SKINNY_LAUNCH(2, true)
    } else {
      MOE_SKINNY_LAUNCH(2, false)
    }
#undef MOE_SKINNY_LAUNCH
  }
  return hipGetLastError();
}

}  // namespace moe
