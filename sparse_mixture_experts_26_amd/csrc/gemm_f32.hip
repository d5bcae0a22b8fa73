// Grouped expert FFN halves in float32 (small fp32 layers).
//
// One thread per output element, sequential float32 FMAs along the reduction
// axis; each row finds its expert by binary search over the group offsets.
// Same contract and row layout as the bf16 kernels (routed rows first, then the
// shared groups of T rows), so float32 layers run the identical five steps.
#include "launch.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(64) void ffn_f32_kernel(FfnParams p, int col_blocks) {
  const int64_t r = blockIdx.x / col_blocks;
  const int n = (int)(blockIdx.x - r * col_blocks) * 64 + threadIdx.x;
  if (n >= p.N) return;
  int g;
  int64_t arow;
  const float* A;
  if (r < p.rows_bound) {
    if (r >= p.offsets[p.G]) return;
    int lo = 0, hi = p.G;  // last g with offsets[g] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.offsets[mid] <= r) lo = mid;
      else hi = mid;
    }
    g = lo;
    arow = p.a_from_c ? r : (p.gather ? p.gather[r] : r);
    A = static_cast<const float*>(p.a_main);
  } else {
    const int64_t q = r - p.rows_bound;
    const int s = (int)(q / p.T);
    if (s >= p.S) return;
    g = p.G + s;
    arow = p.a_from_c ? r : q - (int64_t)s * p.T;
    A = static_cast<const float*>(p.a_shared);
  }
  const bool routed = g < p.G;
  const int gw = routed ? g : g - p.G;
  const int64_t wrow = ((int64_t)gw * p.N + n) * p.K;
  const float* W = static_cast<const float*>(routed ? p.w_main : p.w_shared) + wrow;
  const float* a = A + arow * p.K;
  float acc = 0.f, accu = 0.f;
  for (int c = 0; c < p.K; ++c) acc = fmaf(a[c], W[c], acc);
  if (p.act == 2) {  // (the SwiGLU backward form has no second weight set)
    const float* Uw = static_cast<const float*>(routed ? p.u_main : p.u_shared) + wrow;
    for (int c = 0; c < p.K; ++c) accu = fmaf(a[c], Uw[c], accu);
  }
  const float* bias = routed ? p.bias_main : p.bias_shared;
  if (bias) acc += bias[(int64_t)gw * p.N + n];
  if (p.act >= kActBwd) {
    // input gradient of the down projection, scaled by the row's gate, through
    // the activation's backward: du (and dv) from the saved pre-activations
    const bool swi = p.act == kActBwd + 2;
    const int64_t ld = swi ? 2 * (int64_t)p.N : p.N;
    const float g = routed ? p.row_gate[r] : 1.0f;
    const float* pre = static_cast<const float*>(p.pre) + r * ld;
    float du, dv;
    act_backward(p.act - kActBwd, acc * g, pre[n], swi ? pre[p.N + n] : 0.0f, du, dv);
    float* o = static_cast<float*>(p.out) + r * ld;
    o[n] = du;
    if (swi) o[p.N + n] = dv;
    return;
  }
  if (p.act >= 0 && p.pre) {  // pre-activations for the backward
    const int64_t ld = p.act == 2 ? 2 * (int64_t)p.N : p.N;
    float* pre = static_cast<float*>(p.pre) + r * ld;
    pre[n] = acc;
    if (p.act == 2) pre[p.N + n] = accu;
  }
  const float o = p.act >= 0 ? apply_act(p.act, acc, accu) : acc;
  float* dst = static_cast<float*>(p.out) + r * p.N + n;
  *dst = p.accumulate ? *dst + o : o;
}

}  // namespace

hipError_t launch_ffn_f32(const FfnParams& p, hipStream_t stream) {
  const int col_blocks = (p.N + 63) / 64;
  const int64_t rows = p.rows_bound + (int64_t)p.S * p.T;
  const int64_t blocks = rows * col_blocks;
  if (blocks > 0)
    hipLaunchKernelGGL(ffn_f32_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, p,
                       col_blocks);
  return hipGetLastError();
}

}  // namespace moe
