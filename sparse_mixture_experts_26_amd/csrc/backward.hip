// Backward pass of the layer (token choice, or expert choice): everything
// except the grouped expert GEMMs (which run on the tiled / float32 FFN
// kernels).
//
// The pages train these layers without printing a backward ("Mixture-of-
// Experts & Sparse Model Scaling", Mathematical Formulation: the router learns
// through the gate values and the balancing loss through P_i, f_i being a hard
// count; "Mixture-of-experts Models", Level 2: routing decisions are discrete).
// Gradients flow through the gates (softmax over the selected logits), P_i of
// the load-balancing loss, the log-partition of the z-loss, and softplus of
// the noise; the top-k set, the capacity drops and re-routing carry none.
//
// Every reduction has a fixed order (no atomics), so the gradients are
// deterministic.
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

// ---- per-row gates and gate gradients -------------------------------------------

__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t* dest, const float* gate,
                                                       int64_t n, float* row_gate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = dest[i];
  if (r >= 0) row_gate[r] = gate[i];
}

// dg[t,s] = dy[t] . y_rows[dest[t,s]] (0 for a dropped slot); with expert
// choice dS[t,e] = dy[t] . y_rows[slot[t,e]] (0 where e did not take t).  One
// wave per token, lanes over 4-column chunks, a fixed-order wave reduction.
__global__ __launch_bounds__(256) void gate_grad_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const f32x4* dy = reinterpret_cast<const f32x4*>(p.dy + t * p.d);
  const int n = p.ec ? p.E : p.k;
  for (int s = 0; s < n; ++s) {
    const int r = p.ec ? p.slot[t * p.E + s] : p.dest[t * p.k + s];
    float acc = 0.f;
    if (r >= 0) {
      const f32x4* yr = reinterpret_cast<const f32x4*>(p.y_rows + (int64_t)r * p.d);
      for (int c = lane; c < p.d / 4; c += 64) {
        const f32x4 a = dy[c], b = yr[c];
        acc += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
      }
      acc = wave_sum(acc);
    }
    if (lane == 0) p.dg[t * n + s] = acc;
  }
}

// Expert choice: the gate of row slot[t,e] is scores[t,e].
__global__ __launch_bounds__(256) void ec_row_gate_kernel(const int32_t* slot, const float* scores,
                                                          int64_t n, float* row_gate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = slot[i];
  if (r >= 0) row_gate[r] = scores[i];
}

// dH[t,:] = selected-softmax backward of the gates + g_aux dL_aux/dH +
// g_z dL_z/dH, and for noisy gating dHn = dH * eps * sigmoid(x W_noise^T).
// One wave per token, lane j holds experts j, j+64, j+128, j+192.
__global__ __launch_bounds__(256) void router_bwd_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const float* h = p.logits + t * p.E;
  float v[4], mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < p.E ? h[e] : -INFINITY;
    mx = fmaxf(mx, v[j]);
  }
  mx = wave_max(mx);
  float ex[4], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    ex[j] = e < p.E ? expf(v[j] - mx) : 0.f;
    sum += ex[j];
  }
  sum = wave_sum(sum);
  const float lse = mx + logf(sum);
  const float inv_f = p.inv_f_den;
  float fp = 0.f, pds = 0.f;  // sum_i f_i p_i; expert choice: sum_i p_i dS_i
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < p.E) {
      fp += (float)p.counts[e] * inv_f * (ex[j] / sum);
      if (p.ec) pds += (ex[j] / sum) * p.dg[t * p.E + e];
    }
  }
  fp = wave_sum(fp);
  if (p.ec) pds = wave_sum(pds);
  // gates: sum_m g_m dg_m over the token's slots (k <= 8, every lane)
  float gdg = 0.f;
  if (!p.ec)
    for (int s = 0; s < p.k; ++s) gdg += p.gate[t * p.k + s] * p.dg[t * p.k + s];
  const float c_aux = p.g_aux * (float)p.E / (float)p.T;
  const float c_z = p.g_z * 2.0f * lse / (float)p.T;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e >= p.E) continue;
    const float pe = ex[j] / sum;
    float d = c_aux * pe * ((float)p.counts[e] * inv_f - fp) + c_z * pe;
    if (p.ec) {
      // scores are the full softmax: its backward over all experts
      d += pe * (p.dg[t * p.E + e] - pds);
    } else {
      for (int s = 0; s < p.k; ++s) {
        if (p.idx[t * p.k + s] == e) {
          const float g = p.gate[t * p.k + s];
          d += g * (p.dg[t * p.k + s] - gdg);
        }
      }
    }
    p.dH[t * p.E + e] = d;
    if (p.dHn) {
      const float n = p.noise_pre[t * p.E + e];
      p.dHn[t * p.E + e] = d * p.eps[t * p.E + e] / (1.0f + expf(-n));
    }
  }
}

// ---- router weight gradients: out[e,c] = sum_t G[t,e] x[t,c] --------------------
// Block (column chunk of 256, expert group of 16, token split): every thread
// owns one column and 16 experts; partial[split][e][c] is reduced in split
// order by router_reduce_kernel.
constexpr int kRwExperts = 16;
constexpr int kRwTokens = 64;

template <typename TX>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* G, const TX* x, int T,
                                                           int E, int d, int tokens_per_split,
                                                           float* partial) {
  __shared__ float sg[kRwTokens][kRwExperts];
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * kRwExperts;
  const int t_begin = blockIdx.z * tokens_per_split;
  const int t_end = min(T, t_begin + tokens_per_split);
  float acc[kRwExperts];
#pragma unroll
  for (int j = 0; j < kRwExperts; ++j) acc[j] = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += kRwTokens) {
    __syncthreads();
    for (int i = threadIdx.x; i < kRwTokens * kRwExperts; i += 256) {
      const int tt = i / kRwExperts, j = i % kRwExperts;
      const int t = t0 + tt, e = e0 + j;
      sg[tt][j] = (t < t_end && e < E) ? G[(int64_t)t * E + e] : 0.f;
    }
    __syncthreads();
    if (c < d) {
      const int n = min(kRwTokens, t_end - t0);
      for (int tt = 0; tt < n; ++tt) {
        float xv;
        if constexpr (sizeof(TX) == 2) xv = bf16_to_f32(x[(int64_t)(t0 + tt) * d + c]);
        else xv = x[(int64_t)(t0 + tt) * d + c];
#pragma unroll
        for (int j = 0; j < kRwExperts; ++j) acc[j] = fmaf(sg[tt][j], xv, acc[j]);
      }
    }
  }
  if (c < d) {
#pragma unroll
    for (int j = 0; j < kRwExperts; ++j)
      if (e0 + j < E) partial[((int64_t)blockIdx.z * E + e0 + j) * d + c] = acc[j];
  }
}

__global__ __launch_bounds__(256) void router_reduce_kernel(const float* partial, int nsplit,
                                                            int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float a = 0.f;
  for (int s = 0; s < nsplit; ++s) a += partial[(int64_t)s * n + i];
  out[i] = a;
}

// db_g[e] = sum_t dH[t,e]: one block per expert, strided per-thread sums then
// a fixed-order tree.
__global__ __launch_bounds__(256) void column_sum_kernel(const float* G, int T, int E,
                                                         float* out) {
  __shared__ float s[256];
  const int e = blockIdx.x;
  float a = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) a += G[(int64_t)t * E + e];
  s[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = s[0];
}

// ---- layout kernels --------------------------------------------------------------

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* src, int64_t n,
                                                      uint16_t* dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = f32_to_bf16(src[i]);
}

// dst[g][c][coff + r] = src[g][r][c] for r < R, c < C (64 x 64 tiles via LDS).
// Scalar form, for float32 layers.
template <typename TE>
__global__ __launch_bounds__(256) void transpose_kernel(const TE* src, int R, int C, TE* dst,
                                                        int ld, int coff) {
  __shared__ TE tile[64][65];
  const int g = blockIdx.z;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const TE* s = src + (int64_t)g * R * C;
  TE* o = dst + (int64_t)g * C * ld;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    const int r = r0 + rr, c = c0 + cc;
    if (r < R && c < C) tile[rr][cc] = s[(int64_t)r * C + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    const int r = r0 + rr, c = c0 + cc;
    if (r < R && c < C) o[(int64_t)c * ld + coff + r] = tile[rr][cc];
  }
}

// The same for 16-bit elements with 16-byte accesses (R, C, ld, coff multiples
// of 8): 8 lanes load one 128-byte input row segment and 8 lanes store one
// 128-byte output row segment; rows of the LDS tile are padded to 66 elements
// so the column reads of 8 rows 8 apart hit distinct banks.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* src, int R, int C,
                                                          uint16_t* dst, int ld, int coff) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][66];
  const int g = blockIdx.z;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const uint16_t* s = src + (int64_t)g * R * C;
  uint16_t* o = dst + (int64_t)g * C * ld;
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int rr = i >> 3, ch = i & 7;
    const int r = r0 + rr, c = c0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(s + (int64_t)r * C + c);
    uint32_t* t = reinterpret_cast<uint32_t*>(&tile[rr][ch * 8]);  // 4-byte aligned rows
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = v[q];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int cc = i >> 3, ch = i & 7;
    const int c = c0 + cc, r = r0 + ch * 8;
    if (c >= C || r >= R) continue;
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = (uint32_t)tile[ch * 8 + 2 * q][cc] | ((uint32_t)tile[ch * 8 + 2 * q + 1][cc] << 16);
    *reinterpret_cast<u32x4*>(o + (int64_t)c * ld + coff + r) = v;
  }
}

// Group layout for the weight gradients: kp = rows rounded up to 64, poff the
// exclusive prefix sum of kp over the routed then the shared groups.
__global__ __launch_bounds__(256) void group_desc_kernel(const int32_t* offsets, int G, int S,
                                                         int T, int64_t rows_bound,
                                                         GroupDesc* desc, int32_t* total) {
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  int base = 0;
  for (int g0 = 0; g0 < G + S; g0 += 256) {
    const int g = g0 + tid;
    int rows = 0, row0 = 0;
    if (g < G) {
      row0 = offsets[g];
      rows = offsets[g + 1] - row0;
    } else if (g < G + S) {
      row0 = (int)(rows_bound + (int64_t)(g - G) * T);
      rows = T;
    }
    const int kp = (rows + 63) & ~63;
    scan[tid] = kp;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (g < G + S) {
      GroupDesc d;
      d.poff = base + scan[tid] - kp;
      d.kp = kp;
      d.row0 = row0;
      d.rows = rows;
      desc[g] = d;
    }
    base += scan[255];
    __syncthreads();
  }
  if (tid == 0) *total = base;
}

// Last group whose block starts at or before padded column q (a binary search
// over the ascending poff).
__device__ __forceinline__ int group_of(const GroupDesc* desc, int groups, int q) {
  int lo = 0, hi = groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (desc[mid].poff <= q) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Transposed, zero-padded operand of the weight gradients:
//   dst[C*poff_g + c*kp_g + j] = scale(row) * src[srow(row), coff + c]
// for the group's rows j < rows_g (row = row0_g + j), 0 for rows_g <= j < kp_g.
// srow: the token of the row (gathered sources: x, dy) or the row itself
// (hidden, du, dv); scale: the row's gate for routed rows of dy, else 1.
// Block: 64 padded columns x 64 features.  Sources are read in 16-byte chunks
// along the features, results written in 16-byte chunks along the rows (8
// lanes per 128-byte segment; C, ld and coff are multiples of 8); the float
// tile's rows are padded to 65 words so 8 rows 8 apart hit distinct banks.
template <typename TS, typename TD>
__global__ __launch_bounds__(256) void pack_t_kernel(PackParams p, const TS* src, TD* dst) {
  __shared__ float tile[64][65];
  constexpr int EPC = 16 / sizeof(TS);  // source elements per 16-byte chunk
  const int q0 = blockIdx.x * 64;
  const int f0 = blockIdx.y * 64;
  if (q0 >= *p.total) return;
  const int groups = p.G + p.S;
  const int g = group_of(p.desc, groups, q0);
  const GroupDesc gd = p.desc[g];
  const bool routed = g < p.G;
  const int j0 = q0 - gd.poff;  // first group-local row of the block
  constexpr int CPR = 64 / EPC;  // chunks per tile row
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int jj = i / CPR, ch = i % CPR;
    const int j = j0 + jj, f = f0 + ch * EPC;
    float v[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) v[e] = 0.f;
    if (j < gd.rows && f < p.C) {
      const int64_t row = (int64_t)gd.row0 + j;
      int64_t srow = row;
      if (p.gathered) srow = routed ? p.row_token[row] : j;
      const float sc = (p.row_gate && routed) ? p.row_gate[row] : 1.f;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + srow * p.ld + p.coff + f);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (sizeof(TS) == 2)
          v[e] = bf16_to_f32((uint16_t)(e & 1 ? x[e >> 1] >> 16 : x[e >> 1] & 0xffffu)) * sc;
        else
          v[e] = __uint_as_float(x[e]) * sc;
      }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) tile[jj][ch * EPC + e] = v[e];
  }
  __syncthreads();
  TD* o = dst + (int64_t)p.C * gd.poff;
  constexpr int DPC = 16 / sizeof(TD);  // destination elements per 16-byte chunk
  for (int i = threadIdx.x; i < 64 * (64 / DPC); i += 256) {
    const int ff = i / (64 / DPC), ch = i % (64 / DPC);
    const int f = f0 + ff;
    if (f >= p.C) continue;
    u32x4 w;
    if constexpr (sizeof(TD) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)f32_to_bf16(tile[ch * 8 + 2 * q][ff]) |
               ((uint32_t)f32_to_bf16(tile[ch * 8 + 2 * q + 1][ff]) << 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = __float_as_uint(tile[ch * 4 + q][ff]);
    }
    *reinterpret_cast<u32x4*>(o + (int64_t)f * gd.kp + j0 + ch * DPC) = w;
  }
}

// db[g, c] = sum over the group's rows of scale(row) * src[srow(row), coff + c]
// (same addressing as pack_t_kernel), rows in order.  Routed groups only.
template <typename TS>
__global__ __launch_bounds__(256) void bias_grad_kernel(PackParams p, const TS* src, float* db) {
  const int g = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.C) return;
  const GroupDesc gd = p.desc[g];
  float a = 0.f;
  for (int j = 0; j < gd.rows; ++j) {
    const int64_t row = (int64_t)gd.row0 + j;
    const int64_t srow = p.gathered ? p.row_token[row] : row;
    const float sc = p.row_gate ? p.row_gate[row] : 1.f;
    const TS x = src[srow * p.ld + p.coff + c];
    float v;
    if constexpr (sizeof(TS) == 2) v = bf16_to_f32(x);
    else v = x;
    a = fmaf(sc, v, a);
  }
  db[(int64_t)g * p.C + c] = a;
}

// float32 weight gradient: one thread per output element of C_g = A_g B_g^T
// over the group's zero-padded transposed blocks.
__global__ __launch_bounds__(256) void wgrad_f32_kernel(const float* At, const float* Bt,
                                                        const GroupDesc* desc, int G, int S,
                                                        int M, int N, float* out,
                                                        float* out_shared) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)M * N;
  if (i >= per * (G + S)) return;
  const int g = (int)(i / per);
  const int64_t mn = i - g * per;
  const int m = (int)(mn / N), n = (int)(mn - (int64_t)m * N);
  const GroupDesc gd = desc[g];
  const float* a = At + (int64_t)M * gd.poff + (int64_t)m * gd.kp;
  const float* b = Bt + (int64_t)N * gd.poff + (int64_t)n * gd.kp;
  float acc = 0.f;
  for (int j = 0; j < gd.kp; ++j) acc = fmaf(a[j], b[j], acc);
  if (g < G) out[(int64_t)g * per + mn] = acc;
  else out_shared[(int64_t)(g - G) * per + mn] = acc;
}

// dx[t,:] = sum over the token's kept slots of dx_rows[dest] (slot order) +
// the shared experts' rows + dH[t] W_g + dHn[t] W_noise.  A block takes 8
// tokens; thread j owns columns j, j+256, ...
constexpr int kDxTokens = 8;

template <typename TW>
__global__ __launch_bounds__(256) void dx_kernel(BwdParams p, const TW* w_g, const TW* w_noise) {
  __shared__ float sh[kDxTokens][256], shn[kDxTokens][256];
  const int64_t t0 = (int64_t)blockIdx.x * kDxTokens;
  const int nt = (int)min<int64_t>(kDxTokens, p.T - t0);
  for (int i = threadIdx.x; i < kDxTokens * 256; i += 256) {
    const int tt = i / 256, e = i % 256;
    const bool ok = tt < nt && e < p.E;
    sh[tt][e] = ok ? p.dH[(t0 + tt) * p.E + e] : 0.f;
    shn[tt][e] = ok && p.dHn ? p.dHn[(t0 + tt) * p.E + e] : 0.f;
  }
  __syncthreads();
  // one column per thread: blocks cover 8 tokens x 256 columns, so even a
  // decode batch spreads over many CUs (the per-column order is fixed)
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c < p.d) {
    float acc[kDxTokens];
#pragma unroll
    for (int tt = 0; tt < kDxTokens; ++tt) acc[tt] = 0.f;
    for (int e = 0; e < p.E; ++e) {
      float wg, wn = 0.f;
      if constexpr (sizeof(TW) == 2) {
        wg = bf16_to_f32(w_g[(int64_t)e * p.d + c]);
        if (w_noise) wn = bf16_to_f32(w_noise[(int64_t)e * p.d + c]);
      } else {
        wg = w_g[(int64_t)e * p.d + c];
        if (w_noise) wn = w_noise[(int64_t)e * p.d + c];
      }
#pragma unroll
      for (int tt = 0; tt < kDxTokens; ++tt) acc[tt] = fmaf(sh[tt][e], wg, fmaf(shn[tt][e], wn, acc[tt]));
    }
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t t = t0 + tt;
      float x = 0.f;
      if (p.ec) {
        for (int e = 0; e < p.E; ++e) {  // the experts that took t, in order
          const int r = p.slot[t * p.E + e];
          if (r >= 0) x += p.dx_rows[(int64_t)r * p.d + c];
        }
      } else {
        for (int s = 0; s < p.k; ++s) {
          const int r = p.dest[t * p.k + s];
          if (r >= 0) x += p.dx_rows[(int64_t)r * p.d + c];
        }
      }
      for (int s = 0; s < p.S; ++s) x += p.dx_rows[(p.rows_bound + (int64_t)s * p.T + t) * p.d + c];
      p.dx[t * p.d + c] = x + acc[tt];
    }
  }
}

}  // namespace

hipError_t launch_row_gate(const int32_t* dest, const float* gate, int64_t n, float* row_gate,
                           hipStream_t stream) {
  if (n > 0)
    hipLaunchKernelGGL(row_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       dest, gate, n, row_gate);
  return hipGetLastError();
}

hipError_t launch_ec_row_gate(const int32_t* slot, const float* scores, int64_t n,
                              float* row_gate, hipStream_t stream) {
  if (n > 0)
    hipLaunchKernelGGL(ec_row_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, slot, scores, n, row_gate);
  return hipGetLastError();
}

hipError_t launch_router_backward(const BwdParams& p, hipStream_t stream) {
  const unsigned blocks = (unsigned)((p.T + 3) / 4);
  if (blocks > 0) {
    hipLaunchKernelGGL(gate_grad_kernel, dim3(blocks), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(router_bwd_kernel, dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

int router_wgrad_splits(int64_t T, int64_t E, int64_t d) {
  const int64_t base = ((d + 255) / 256) * ((E + kRwExperts - 1) / kRwExperts);
  int64_t ns = (1024 + base - 1) / base;
  ns = std::min<int64_t>(ns, (T + kRwTokens - 1) / kRwTokens);
  return (int)std::max<int64_t>(ns, 1);
}

hipError_t launch_router_wgrad(const float* G, const void* x, int bf16, int T, int E, int d,
                               float* partial, float* out, hipStream_t stream) {
  const int ns = router_wgrad_splits(T, E, d);
  const int per = (((T + ns - 1) / ns) + kRwTokens - 1) / kRwTokens * kRwTokens;
  const dim3 grid((d + 255) / 256, (E + kRwExperts - 1) / kRwExperts, ns);
  if (bf16)
    hipLaunchKernelGGL(router_wgrad_kernel<uint16_t>, grid, dim3(256), 0, stream, G,
                       static_cast<const uint16_t*>(x), T, E, d, per, partial);
  else
    hipLaunchKernelGGL(router_wgrad_kernel<float>, grid, dim3(256), 0, stream, G,
                       static_cast<const float*>(x), T, E, d, per, partial);
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     partial, ns, n, out);
  return hipGetLastError();
}

hipError_t launch_column_sum(const float* G, int T, int E, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(column_sum_kernel, dim3(E), dim3(256), 0, stream, G, T, E, out);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, int64_t n, uint16_t* dst, hipStream_t stream) {
  if (n > 0)
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       src, n, dst);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int groups, int R, int C, void* dst, int ld,
                            int coff, int esz, hipStream_t stream) {
  const dim3 grid((C + 63) / 64, (R + 63) / 64, groups);
  if (groups <= 0 || R <= 0 || C <= 0) return hipGetLastError();
  if (esz == 2)
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(src), R, C, static_cast<uint16_t*>(dst), ld,
                       coff);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(src), R, C, static_cast<float*>(dst), ld, coff);
  return hipGetLastError();
}

hipError_t launch_group_desc(const int32_t* offsets, int G, int S, int T, int64_t rows_bound,
                             GroupDesc* desc, int32_t* total, hipStream_t stream) {
  hipLaunchKernelGGL(group_desc_kernel, dim3(1), dim3(256), 0, stream, offsets, G, S, T,
                     rows_bound, desc, total);
  return hipGetLastError();
}

hipError_t launch_pack_t(const PackParams& p, const void* src, int src_esz, void* dst,
                         int dst_esz, int64_t padded_bound, hipStream_t stream) {
  const dim3 grid((unsigned)((padded_bound + 63) / 64), (p.C + 63) / 64);
  if (padded_bound <= 0) return hipGetLastError();
  if (src_esz == 4 && dst_esz == 2)
    hipLaunchKernelGGL((pack_t_kernel<float, uint16_t>), grid, dim3(256), 0, stream, p,
                       static_cast<const float*>(src), static_cast<uint16_t*>(dst));
  else if (src_esz == 2 && dst_esz == 2)
    hipLaunchKernelGGL((pack_t_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream, p,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst));
  else
    hipLaunchKernelGGL((pack_t_kernel<float, float>), grid, dim3(256), 0, stream, p,
                       static_cast<const float*>(src), static_cast<float*>(dst));
  return hipGetLastError();
}

hipError_t launch_bias_grad(const PackParams& p, const void* src, int src_esz, float* db,
                            hipStream_t stream) {
  const dim3 grid((p.C + 255) / 256, p.G);
  if (p.G <= 0) return hipGetLastError();
  if (src_esz == 2)
    hipLaunchKernelGGL(bias_grad_kernel<uint16_t>, grid, dim3(256), 0, stream, p,
                       static_cast<const uint16_t*>(src), db);
  else
    hipLaunchKernelGGL(bias_grad_kernel<float>, grid, dim3(256), 0, stream, p,
                       static_cast<const float*>(src), db);
  return hipGetLastError();
}

hipError_t launch_wgrad_f32(const float* At, const float* Bt, const GroupDesc* desc, int G,
                            int S, int M, int N, float* out, float* out_shared,
                            hipStream_t stream) {
  const int64_t n = (int64_t)M * N * (G + S);
  if (n > 0)
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       At, Bt, desc, G, S, M, N, out, out_shared);
  return hipGetLastError();
}

hipError_t launch_dx(const BwdParams& p, const void* w_g, const void* w_noise, int bf16,
                     hipStream_t stream) {
  const unsigned blocks = (unsigned)((p.T + kDxTokens - 1) / kDxTokens);
  const unsigned col_blocks = (unsigned)((p.d + 255) / 256);
  if (blocks == 0 || col_blocks == 0) return hipGetLastError();
  const dim3 g(blocks, col_blocks);
  if (bf16)
    hipLaunchKernelGGL(dx_kernel<uint16_t>, g, dim3(256), 0, stream, p,
                       static_cast<const uint16_t*>(w_g), static_cast<const uint16_t*>(w_noise));
  else
    hipLaunchKernelGGL(dx_kernel<float>, g, dim3(256), 0, stream, p,
                       static_cast<const float*>(w_g), static_cast<const float*>(w_noise));
  return hipGetLastError();
}

}  // namespace moe
