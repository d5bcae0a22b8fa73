// Grouped expert GEMM for at most 32 rows per expert (decode- and
// Switch-shaped layers), bf16 MFMA.
//
// With a handful of rows per expert the expert FFN is a stream over the
// expert's weights ("Mixture-of-Experts & Sparse Model Scaling", Computational
// Considerations: MoE layers are more memory-bound than dense ones of equal
// active size), so the kernel is built to keep HBM busy rather than to reuse
// operands: every block owns one expert and a 64-column slab of its weight
// rows, reads that slab exactly once with 16-byte loads, and splits the
// reduction axis over its 4 waves so each wave keeps many independent loads in
// flight.  The expert's <= 32 operand rows ride along as the A operand of
// v_mfma_f32_16x16x32_bf16 (two 16-row fragments; the second is skipped when the
// expert holds 16 rows or fewer).  The 4 partial products are summed in LDS in
// wave order (deterministic) and the activation is applied there.  Experts
// that received no rows read no weights at all.
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int NF = 4;  // 16-column fragments per block: 64 output columns

template <int ACT>
__global__ __launch_bounds__(kThreads) void ffn_skinny_kernel(FfnParams p, int n_slabs) {
  constexpr bool GATED = ACT == 2;
  constexpr int NB = GATED ? 2 : 1;           // weight sets (w1 and w3 when gated)
  constexpr int NFRAG = 2 * NF * NB;          // (row fragment, column fragment, set)
  constexpr int UNR = GATED ? 2 : 4;          // k-steps of 32 loaded ahead
  __shared__ float red[4][NFRAG][4][64];

  const int g = blockIdx.x / n_slabs, slab = blockIdx.x - g * n_slabs;
  const bool routed = g < p.G;
  int rows, a_row0, c_row0;
  if (routed) {
    a_row0 = p.offsets[g];
    rows = p.offsets[g + 1] - a_row0;
    c_row0 = a_row0;
  } else {
    a_row0 = 0;
    rows = p.T;
    c_row0 = (int)(p.rows_bound + (int64_t)(g - p.G) * p.T);
  }
  rows = min(rows, 32);
  if (rows <= 0) return;
  const bool two = rows > 16;
  const int gw = routed ? g : g - p.G;
  const int K = p.K, N = p.N;
  const int64_t wstride = (int64_t)N * K;
  const uint16_t* W = static_cast<const uint16_t*>(routed ? p.w_main : p.w_shared) + gw * wstride;
  const uint16_t* U = W;
  if (GATED) U = static_cast<const uint16_t*>(routed ? p.u_main : p.u_shared) + gw * wstride;
  const uint16_t* A = static_cast<const uint16_t*>(routed ? p.a_main : p.a_shared);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

  uint32_t a_off[2];
  bool a_ok[2];
#pragma unroll
  for (int mf = 0; mf < 2; ++mf) {
    const int r = mf * 16 + (lane & 15);
    a_ok[mf] = r < rows;
    int arow = p.a_from_c ? c_row0 + r : a_row0 + r;
    if (a_ok[mf] && routed && p.gather && !p.a_from_c) arow = p.gather[arow];
    a_off[mf] = (uint32_t)(a_ok[mf] ? arow : 0) * (uint32_t)K;
  }
  uint32_t b_off[NF];
  bool b_ok[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int n = slab * 64 + nf * 16 + (lane & 15);
    b_ok[nf] = n < N;
    b_off[nf] = (uint32_t)(b_ok[nf] ? n : 0) * (uint32_t)K;
  }

  const int kch = (K + 31) / 32, per = (kch + 3) / 4;
  const int kb = min(K, w * per * 32), ke = min(K, (w + 1) * per * 32);
  const int kl = (lane >> 4) * 8;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  f32x4 acc[2][NF][NB];
#pragma unroll
  for (int mf = 0; mf < 2; ++mf)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
#pragma unroll
      for (int s = 0; s < NB; ++s) acc[mf][nf][s] = f32x4{};

  for (int k0 = kb; k0 < ke; k0 += 32 * UNR) {
    u32x4 av[UNR][2], bv[UNR][NF][NB];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kk = k0 + u * 32 + kl;
      const bool k_ok = kk < ke;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
        av[u][mf] = (k_ok && a_ok[mf] && (mf == 0 || two))
                        ? *reinterpret_cast<const u32x4*>(A + a_off[mf] + kk)
                        : z4;
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s)
          bv[u][nf][s] = (k_ok && b_ok[nf])
                             ? *reinterpret_cast<const u32x4*>((s ? U : W) + b_off[nf] + kk)
                             : z4;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, bv[u][nf][s]);
          acc[0][nf][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av[u][0]), b, acc[0][nf][s], 0, 0, 0);
          if (two)
            acc[1][nf][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av[u][1]), b, acc[1][nf][s], 0, 0, 0);
        }
  }

  // 16x16 result layout: lane holds column lane%16, rows 4*(lane/16) + i.
#pragma unroll
  for (int mf = 0; mf < 2; ++mf)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
#pragma unroll
      for (int s = 0; s < NB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][(mf * NF + nf) * NB + s][i][lane] = acc[mf][nf][s][i];
  __syncthreads();

  const float* bias = routed ? p.bias_main : p.bias_shared;
  for (int o = threadIdx.x; o < 2 * NF * 256; o += kThreads) {
    const int mf = o / (NF * 256), rem = o - mf * NF * 256;
    const int nf = rem >> 8, i = (rem >> 6) & 3, l = rem & 63;
    const int row = mf * 16 + (l >> 4) * 4 + i;
    const int col = slab * 64 + nf * 16 + (l & 15);
    if (row >= rows || col >= N) continue;
    const int f0 = (mf * NF + nf) * NB;
    float a = ((red[0][f0][i][l] + red[1][f0][i][l]) + red[2][f0][i][l]) + red[3][f0][i][l];
    if (bias) a += bias[(int64_t)gw * N + col];
    float out;
    if (GATED) {
      const float u = ((red[0][f0 + 1][i][l] + red[1][f0 + 1][i][l]) + red[2][f0 + 1][i][l]) +
                      red[3][f0 + 1][i][l];
      out = silu_f32(a) * u;
    } else if (ACT == 0) {
      out = gelu_f32(a);
    } else if (ACT == 1) {
      out = fmaxf(a, 0.f);
    } else {
      out = a;
    }
    const int64_t idx = (int64_t)(c_row0 + row) * N + col;
    if (p.out_bf16) {
      static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(out);
    } else {
      float* dst = static_cast<float*>(p.out) + idx;
      *dst = p.accumulate ? *dst + out : out;
    }
  }
}

}  // namespace

hipError_t launch_ffn_skinny(const FfnParams& p, hipStream_t stream) {
  const int n_slabs = (p.N + 63) / 64;
  const int64_t blocks = (int64_t)(p.G + p.S) * n_slabs;
  if (blocks > 0) {
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (p.act) {
      case 2: hipLaunchKernelGGL(ffn_skinny_kernel<2>, grid, block, 0, stream, p, n_slabs); break;
      case 1: hipLaunchKernelGGL(ffn_skinny_kernel<1>, grid, block, 0, stream, p, n_slabs); break;
      case 0: hipLaunchKernelGGL(ffn_skinny_kernel<0>, grid, block, 0, stream, p, n_slabs); break;
      default: hipLaunchKernelGGL(ffn_skinny_kernel<-1>, grid, block, 0, stream, p, n_slabs); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
