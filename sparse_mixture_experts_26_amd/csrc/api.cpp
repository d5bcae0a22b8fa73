// C ABI of the sparse MoE layer forward: argument validation, workspace
// planning and launch orchestration on the caller's stream.  No allocation,
// no synchronisation; every failure is reported before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "launch.hpp"

namespace moe {
hipError_t launch_ffn_tiled(const FfnParams& p, hipStream_t stream);
hipError_t launch_ffn_skinny(const FfnParams& p, hipStream_t stream);
hipError_t launch_ffn_f32(const FfnParams& p, hipStream_t stream);

// float32 -> plain kernel; <= 32 rows in every group (shared groups hold T
// rows) -> weight-streaming kernel; otherwise the tiled MFMA kernel.
bool ffn_uses_skinny(const FfnParams& p) {
  return p.bf16 && p.group_bound <= 32 && (p.S == 0 || p.T <= 32);
}
hipError_t launch_ffn(const FfnParams& p, hipStream_t stream) {
  if (!p.bf16) return launch_ffn_f32(p, stream);
  return ffn_uses_skinny(p) ? launch_ffn_skinny(p, stream) : launch_ffn_tiled(p, stream);
}
}  // namespace moe

namespace {

using namespace moe;

// Kernels address operands with 31-bit byte offsets (buffer loads): every
// operand must stay below 2^30 two-byte elements.
constexpr int64_t kMaxElems = (int64_t)1 << 30;

struct Cfg {
  int64_t T, d, E, k, h, S;
  int act, bf16;
  bool ec;        // expert-choice routing
  bool rr;        // token choice with overflow re-routing
  int64_t C;      // capacity, clamped to T (no expert can receive more)
  int64_t R;      // routed rows bound: min(T*k, E*C), or E*C for expert choice
  size_t esz;     // bytes per activation / weight element
};

int64_t capacity_of(const moe_config_t* c) {
  if (c->capacity_factor <= 0.0) return c->T;
  const double v = floor(c->capacity_factor * (double)c->T * (double)c->k / (double)c->E);
  if (!(v >= 0.0)) return 0;
  return v > 9.0e18 ? INT64_MAX : (int64_t)v;
}

moe_status_t check_cfg(const moe_config_t* c, Cfg* o) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->T < 0 || c->d <= 0 || c->E <= 0 || c->h <= 0 || c->k < 1 || c->k > c->E ||
      c->n_shared < 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->act < 0 || c->act > 2 || (c->dtype != MOE_F32 && c->dtype != MOE_BF16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (isnan(c->capacity_factor)) return MOE_ERR_INVALID_ARGUMENT;
  if (c->routing != MOE_ROUTE_TOKEN_CHOICE && c->routing != MOE_ROUTE_EXPERT_CHOICE)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->overflow != MOE_OVERFLOW_DROP && c->overflow != MOE_OVERFLOW_REROUTE)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->overflow == MOE_OVERFLOW_REROUTE && c->routing != MOE_ROUTE_TOKEN_CHOICE)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->E > 256 || c->k > 8 || c->d % 8 || c->h % 8) return MOE_ERR_UNSUPPORTED;
  if (c->router_noise && c->E > 128) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 64) return MOE_ERR_UNSUPPORTED;
  o->T = c->T; o->d = c->d; o->E = c->E; o->k = c->k; o->h = c->h; o->S = c->n_shared;
  o->act = c->act;
  o->bf16 = c->dtype == MOE_BF16;
  o->esz = o->bf16 ? 2 : 4;
  o->ec = c->routing == MOE_ROUTE_EXPERT_CHOICE;
  o->rr = c->overflow == MOE_OVERFLOW_REROUTE;
  o->C = std::min<int64_t>(capacity_of(c), c->T);
  o->R = o->ec ? c->E * o->C : std::min<int64_t>(c->T * c->k, c->E * o->C);
  const int64_t rows = o->R + o->S * o->T;
  if (o->T * o->k >= kMaxElems || o->T * o->d >= kMaxElems || o->T * o->E >= kMaxElems ||
      rows * std::max(o->d, o->h) >= kMaxElems || o->d * o->h >= kMaxElems)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Sequential 256-byte-aligned sub-allocation of the caller's workspace; with a
// null base it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

struct RouteWs { float* prob_partial; };
struct DispatchWs { int32_t* local_rank; int32_t* chunk_hist; };
struct FfnWs { TileEntry* entries; int32_t* n_entries; float* split; int split_cap; };
struct DiagWs { double* partial_d; int32_t* partial_i; };
struct RerouteWs {
  uint8_t* fallback; int32_t* list_a; int32_t* list_b; int32_t* fe; int32_t* rin;
  int32_t* off_prim;
  int32_t* chunk_cnt; int32_t* chunk_base; int32_t* chunk_hist; int32_t* chunk_ebase;
  int32_t* local_rank; int32_t* prop; int32_t* pcnt; int32_t* load_g; int32_t* n_g;
};

RouteWs carve_route(Carve& cv, const Cfg& c) {
  return {static_cast<float*>(cv.take((size_t)route_blocks(c.T) * c.E * 4))};
}
DispatchWs carve_dispatch(Carve& cv, const Cfg& c) {
  DispatchWs w;
  w.local_rank = static_cast<int32_t*>(cv.take((size_t)c.T * c.k * 4));
  w.chunk_hist = static_cast<int32_t*>(cv.take((size_t)dispatch_chunks(c.T * c.k) * c.E * 4));
  return w;
}
RerouteWs carve_reroute(Carve& cv, const Cfg& c) {
  RerouteWs w;
  const size_t tk = (size_t)c.T * c.k;
  w.fallback = static_cast<uint8_t*>(cv.take((size_t)c.T * (c.E - c.k)));
  w.list_a = static_cast<int32_t*>(cv.take(2 * tk * 4));
  w.list_b = static_cast<int32_t*>(cv.take(2 * tk * 4));
  w.fe = static_cast<int32_t*>(cv.take(tk * 4));
  w.rin = static_cast<int32_t*>(cv.take(tk * 4));
  w.off_prim = static_cast<int32_t*>(cv.take((size_t)(c.E + 1) * 4));
  const size_t ch = (size_t)std::max(reroute_chunks((int64_t)tk), 1);
  w.chunk_cnt = static_cast<int32_t*>(cv.take(ch * 4));
  w.chunk_base = static_cast<int32_t*>(cv.take(ch * 4));
  w.chunk_hist = static_cast<int32_t*>(cv.take(ch * c.E * 4));
  w.chunk_ebase = static_cast<int32_t*>(cv.take(ch * c.E * 4));
  w.local_rank = static_cast<int32_t*>(cv.take(tk * 4));
  w.prop = static_cast<int32_t*>(cv.take(tk * 4));
  w.pcnt = static_cast<int32_t*>(cv.take(tk * 4));
  w.load_g = static_cast<int32_t*>(cv.take(2 * 256 * 4));
  w.n_g = static_cast<int32_t*>(cv.take(2 * 4));
  return w;
}
DiagWs carve_diag(Carve& cv, const Cfg& c) {
  DiagWs w;
  w.partial_d = static_cast<double*>(cv.take((size_t)diag_blocks(c.T) * 2 * sizeof(double)));
  w.partial_i = static_cast<int32_t*>(cv.take((size_t)diag_blocks(c.T) * 2 * sizeof(int32_t)));
  return w;
}
// Tile schedule of the tiled GEMM, plus the tail-split partials of its
// launches (256 x 256 float32 blocks, `blocks` per split tile: 2, or 3 where
// a down projection with a bf16 output may split).
FfnWs carve_ffn(Carve& cv, int64_t rows_bound, int64_t groups, int64_t S, int64_t T, int64_t d,
                int blocks = 2) {
  FfnWs w;
  const int64_t ent = ffn_max_entries(rows_bound, (int)groups, (int)S, (int)T);
  w.entries = static_cast<TileEntry*>(cv.take((size_t)ent * sizeof(TileEntry)));
  w.n_entries = static_cast<int32_t*>(cv.take(4));
  w.split_cap = (int)ffn_split_cap(ent, d);
  w.split = static_cast<float*>(cv.take((size_t)w.split_cap * blocks * 256 * 256 * 4));
  return w;
}

// A bf16 token-choice layer call keeps its expert rows in bf16 (unless the
// caller wants them, or a top-1 direct store leaves none); where its down
// projection is tiled, that projection's split tiles need a third partial
// block.  The grouped GEMM is tiled unless every group holds at most 32 rows
// (capacity) and there are no shared experts over more than 32 tokens.
bool layer_tiled_bf16_rows(const Cfg& c) {
  return c.bf16 && !c.ec && !(c.C <= 32 && (c.S == 0 || c.T <= 32));
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace of the whole layer: intermediates plus every stage's scratch.
struct LayerWs {
  float* logits; int32_t* idx; float* gate; float* prob_sum;
  int32_t* counts; int32_t* offsets; int32_t* dest; int32_t* row_token;
  float* scores; int32_t* slot;  // expert choice only
  int32_t* final_expert;         // re-routing only
  void* hidden; float* y_rows;
  RouteWs rw; DispatchWs dw; FfnWs fw; DiagWs gw; RerouteWs rrw;
};

LayerWs carve_layer(Carve& cv, const Cfg& c, const moe_aux_t* aux) {
  LayerWs w;
  const size_t tk = (size_t)c.T * c.k;
  auto pick = [&](void* given, size_t bytes) { return given ? given : cv.take(bytes); };
  w.logits = static_cast<float*>(pick(aux ? aux->logits : nullptr, (size_t)c.T * c.E * 4));
  w.idx = static_cast<int32_t*>(pick(aux ? aux->topk_idx : nullptr, tk * 4));
  w.gate = static_cast<float*>(pick(aux ? aux->topk_gate : nullptr, tk * 4));
  w.prob_sum = static_cast<float*>(pick(aux ? aux->prob_sum : nullptr, (size_t)c.E * 4));
  w.counts = static_cast<int32_t*>(pick(aux ? aux->counts : nullptr, (size_t)c.E * 4));
  w.offsets = static_cast<int32_t*>(pick(aux ? aux->offsets : nullptr, (size_t)(c.E + 1) * 4));
  w.dest = static_cast<int32_t*>(pick(aux ? aux->dest : nullptr, tk * 4));
  w.row_token = static_cast<int32_t*>(
      pick(aux ? aux->row_token : nullptr, (size_t)std::max<int64_t>(c.R, (int64_t)tk) * 4));
  w.scores = nullptr;
  w.slot = nullptr;
  w.final_expert = nullptr;
  if (c.rr)
    w.final_expert = static_cast<int32_t*>(pick(aux ? aux->final_expert : nullptr, tk * 4));
  if (c.ec) {
    w.scores = static_cast<float*>(pick(aux ? aux->scores : nullptr, (size_t)c.T * c.E * 4));
    w.slot = static_cast<int32_t*>(pick(aux ? aux->slot : nullptr, (size_t)c.T * c.E * 4));
  }
  const int64_t rows = c.R + c.S * c.T;
  w.hidden = pick(aux ? aux->hidden : nullptr, (size_t)rows * c.h * c.esz);
  w.y_rows = static_cast<float*>(pick(aux ? aux->y_rows : nullptr, (size_t)rows * c.d * 4));
  w.rw = carve_route(cv, c);
  w.dw = carve_dispatch(cv, c);
  w.fw = carve_ffn(cv, c.R, c.E, c.S, c.T, c.d, layer_tiled_bf16_rows(c) ? 3 : 2);
  w.gw = carve_diag(cv, c);
  w.rrw = RerouteWs{};
  if (c.rr) w.rrw = carve_reroute(cv, c);
  return w;
}

size_t layer_ws_bytes(const Cfg& c) {
  Carve cv(nullptr);
  carve_layer(cv, c, nullptr);
  return cv.off + 256;
}

// Expert FFN workspace for a stage call: tile schedule (+ hidden rows).
size_t ffn_ws_bytes(const Cfg& c, int64_t rows_bound, int64_t groups, bool with_hidden) {
  Carve cv(nullptr);
  carve_ffn(cv, rows_bound, groups, 0, c.T, c.d);
  if (with_hidden) cv.take((size_t)rows_bound * c.h * c.esz);
  return cv.off + 256;
}

FfnParams ffn_params(const Cfg& c, int64_t n_groups, const int32_t* offsets, int64_t rows_bound,
                     int64_t group_bound, const FfnWs& fw) {
  FfnParams p;
  memset(&p, 0, sizeof(p));
  p.offsets = offsets;
  p.G = (int)n_groups;
  p.S = 0;
  p.T = (int)c.T;
  p.rows_bound = rows_bound;
  p.group_bound = group_bound;
  p.bf16 = c.bf16;
  p.entries = fw.entries;
  p.n_entries = fw.n_entries;
  p.split = fw.split;
  p.split_cap = fw.split_cap;
  return p;
}

moe_status_t check_ffn_args(const Cfg& c, int64_t n_groups, const int32_t* offsets,
                            int64_t rows_bound, int64_t group_bound) {
  if (n_groups < 0 || n_groups > 256 || rows_bound < 0 || group_bound < 0 || !offsets)
    return MOE_ERR_INVALID_ARGUMENT;
  if (group_bound > rows_bound && n_groups > 0) return MOE_ERR_INVALID_ARGUMENT;
  if (rows_bound * std::max(c.d, c.h) >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if (!aligned(offsets)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t run_up(const Cfg& c, FfnParams p, const void* x_rows, const int32_t* row_token,
                    const void* w1, const void* w3, const float* b1, void* hidden,
                    hipStream_t s) {
  p.a_main = x_rows; p.a_shared = x_rows; p.gather = row_token; p.a_from_c = 0;
  p.w_main = w1; p.u_main = w3; p.bias_main = b1;
  p.out = hidden; p.out_bf16 = c.bf16; p.accumulate = 0;
  p.N = (int)c.h; p.K = (int)c.d; p.act = c.act;
  return hip_status(launch_ffn(p, s));
}

moe_status_t run_down(const Cfg& c, FfnParams p, const void* hidden, const void* w2,
                      const float* b2, float* y_rows, int accumulate, hipStream_t s) {
  p.a_main = hidden; p.a_shared = hidden; p.gather = nullptr; p.a_from_c = 1;
  p.w_main = w2; p.u_main = nullptr; p.bias_main = b2;
  p.out = y_rows; p.out_bf16 = 0; p.accumulate = accumulate;
  p.N = (int)c.d; p.K = (int)c.h; p.act = -1;
  return hip_status(launch_ffn(p, s));
}

// ---- backward workspace ----------------------------------------------------------
struct BwdWs {
  float* row_gate; float* dg; float* dH; float* dHn; float* noise_pre;
  float* r_logits; int32_t* r_idx; float* r_gate; float* r_prob_sum; RouteWs rw;
  float* rpartial;
  void* dy_lp;                   // dy in the config dtype (bf16 layers)
  void* w2t; void* w13t;         // transposed weights, routed then shared groups
  void* duv; float* dxr;         // [rows, Kup] and [rows, d]
  GroupDesc* desc; int32_t* total;
  void* dyT; void* xT; void* hidT; void* duT; void* dvT;
  FfnWs fw;
  int32_t* xcd_bounds;
};

int64_t padded_rows_bound(const Cfg& c) {
  return c.R + 63 * c.E + c.S * ((c.T + 63) / 64 * 64);
}

BwdWs carve_backward(Carve& cv, const Cfg& c, bool noise) {
  BwdWs w;
  memset(&w, 0, sizeof(w));
  const bool swi = c.act == MOE_ACT_SWIGLU;
  const int64_t kup = swi ? 2 * c.h : c.h;
  const int64_t rows = c.R + c.S * c.T;
  const int64_t rp = padded_rows_bound(c);
  const int64_t groups = c.E + c.S;
  const size_t te = (size_t)c.T * c.E * 4, tk = (size_t)c.T * c.k * 4;
  w.row_gate = static_cast<float*>(cv.take((size_t)std::max<int64_t>(c.R, 1) * 4));
  w.dg = static_cast<float*>(cv.take(c.ec ? te : tk));
  w.dH = static_cast<float*>(cv.take(te));
  if (noise) {
    w.dHn = static_cast<float*>(cv.take(te));
    w.noise_pre = static_cast<float*>(cv.take(te));
    w.r_logits = static_cast<float*>(cv.take(te));
    w.r_idx = static_cast<int32_t*>(cv.take(tk));
    w.r_gate = static_cast<float*>(cv.take(tk));
    w.r_prob_sum = static_cast<float*>(cv.take((size_t)c.E * 4));
    w.rw = carve_route(cv, c);
  }
  w.rpartial = static_cast<float*>(
      cv.take((size_t)router_wgrad_splits(c.T, c.E, c.d) * c.E * c.d * 4));
  if (c.bf16) w.dy_lp = cv.take((size_t)c.T * c.d * 2);
  w.w2t = cv.take((size_t)groups * c.h * c.d * c.esz);
  w.w13t = cv.take((size_t)groups * c.d * kup * c.esz);
  w.duv = cv.take((size_t)rows * kup * c.esz);
  w.dxr = static_cast<float*>(cv.take((size_t)rows * c.d * 4));
  w.desc = static_cast<GroupDesc*>(cv.take((size_t)groups * sizeof(GroupDesc)));
  w.total = static_cast<int32_t*>(cv.take(4));
  w.dyT = cv.take((size_t)c.d * rp * c.esz);
  w.xT = cv.take((size_t)c.d * rp * c.esz);
  w.hidT = cv.take((size_t)c.h * rp * c.esz);
  w.duT = cv.take((size_t)c.h * rp * c.esz);
  if (swi) w.dvT = cv.take((size_t)c.h * rp * c.esz);
  const int64_t ent = std::max<int64_t>(ffn_max_entries(c.R, (int)c.E, (int)c.S, (int)c.T),
                                        wgrad_entries((int)groups, (int)std::max(c.d, c.h)));
  w.fw.entries = static_cast<TileEntry*>(cv.take((size_t)ent * sizeof(TileEntry)));
  w.fw.n_entries = static_cast<int32_t*>(cv.take(4));
  w.fw.split_cap = (int)ffn_split_cap(ffn_max_entries(c.R, (int)c.E, (int)c.S, (int)c.T), c.d, true);
  w.fw.split = static_cast<float*>(cv.take((size_t)w.fw.split_cap * 2 * 256 * 256 * 4));
  w.xcd_bounds = static_cast<int32_t*>(cv.take(16 * 4));
  return w;
}

// the bf16 intermediates the kernels address with 31-bit byte offsets
bool backward_fits(const Cfg& c) {
  const int64_t kup = c.act == MOE_ACT_SWIGLU ? 2 * c.h : c.h;
  const int64_t rows = c.R + c.S * c.T;
  const int64_t rp = padded_rows_bound(c);
  return rows * kup < kMaxElems && rows * c.d < kMaxElems && std::max(c.d, c.h) * rp < kMaxElems &&
         c.T * c.d < kMaxElems && c.d * kup < kMaxElems;
}

// Scratch of moe_layer_forward_noalloc: one array per device the library
// runs on, held until the process ends.  Host code must never pass the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is looked up once per device, with that device current,
// and that address is what the launches receive.  No kernel of the layer
// relies on zeroed workspace (every scratch word is written before it is
// read within one call), so nothing is cleared between calls.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t moe_capacity(const moe_config_t* cfg) {
  Cfg c;
  if (check_cfg(cfg, &c) == MOE_ERR_INVALID_ARGUMENT) return -1;
  return capacity_of(cfg);
}

int64_t moe_routed_rows_bound(const moe_config_t* cfg) {
  Cfg c;
  if (check_cfg(cfg, &c) != MOE_OK) return -1;
  return c.R;
}

size_t moe_workspace_bytes(const moe_config_t* cfg) {
  Cfg c;
  if (check_cfg(cfg, &c) != MOE_OK) return 0;
  size_t b = layer_ws_bytes(c);
  b = std::max(b, ffn_ws_bytes(c, std::max(c.R, c.T), c.E, true));
  return b;
}

moe_status_t moe_route_launch_shape(const moe_config_t* cfg, int device_logits, int* waves,
                                    size_t* lds_bytes) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!waves || !lds_bytes) return MOE_ERR_INVALID_ARGUMENT;
  // large bf16 batches compute their logits in a kernel of their own; the
  // router kernel then has its replay shape
  const bool fused = c.bf16 && device_logits && !route_split_logits(c.T, c.E, cfg->router_noise != 0);
  const RoutePlan rp = route_plan((int)c.E, fused && cfg->router_noise != 0, fused);
  *waves = rp.waves;
  *lds_bytes = rp.lds_bytes + rp.static_lds_bytes;
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* w_g,
                       const float* b_g, const void* w_noise, const float* eps,
                       float* logits, int32_t* topk_idx, float* topk_gate, float* prob_sum,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_gate || !prob_sum || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (x) {
    if (!w_g) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->router_bias && !b_g) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->router_noise && (!w_noise || !eps)) return MOE_ERR_INVALID_ARGUMENT;
  }
  const void* ptrs[] = {x, w_g, b_g, w_noise, eps, logits, topk_idx, topk_gate, prob_sum, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  Carve cv(nullptr);
  carve_route(cv, c);
  if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c.T == 0) return MOE_OK;
  Carve wv(ws);
  RouteParams p;
  p.x = x;
  p.w_g = w_g;
  p.b_g = x && cfg->router_bias ? b_g : nullptr;
  p.w_noise = x && cfg->router_noise ? w_noise : nullptr;
  p.eps = x && cfg->router_noise ? eps : nullptr;
  p.logits = logits; p.idx = topk_idx; p.gate = topk_gate;
  p.prob_partial = carve_route(wv, c).prob_partial;
  p.prob_sum = prob_sum;
  p.noise_pre = nullptr;
  p.T = (int)c.T; p.d = (int)c.d; p.E = (int)c.E; p.k = (int)c.k; p.bf16 = c.bf16;
  return hip_status(launch_route(p, stream));
}

moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx, const void* x,
                          int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* row_token,
                          void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !dest || !row_token || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (c.ec || c.rr) return MOE_ERR_INVALID_ARGUMENT;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {topk_idx, x, counts, offsets, dest, row_token, x_perm, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  Carve cv(nullptr);
  carve_dispatch(cv, c);
  if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c.T == 0) return MOE_OK;
  Carve wv(ws);
  DispatchWs dw = carve_dispatch(wv, c);
  DispatchParams p;
  p.idx = topk_idx; p.counts = counts; p.offsets = offsets; p.dest = dest;
  p.row_token = row_token; p.local_rank = dw.local_rank; p.chunk_hist = dw.chunk_hist;
  p.n = (int)(c.T * c.k); p.k = (int)c.k; p.E = (int)c.E; p.C = (int)c.C;
  st = hip_status(launch_dispatch(p, stream));
  if (st != MOE_OK || !x) return st;
  return hip_status(launch_permute(x, row_token, offsets + c.E, x_perm,
                                   (int64_t)c.d * (int64_t)c.esz, c.R, stream));
}

moe_status_t moe_dispatch_reroute(const moe_config_t* cfg, const int32_t* topk_idx,
                                  const float* logits, int32_t* counts, int32_t* offsets,
                                  int32_t* dest, int32_t* row_token, int32_t* final_expert,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!c.rr || !topk_idx || !logits || !counts || !offsets || !dest || !row_token ||
      !final_expert || !ws)
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {topk_idx, logits, counts, offsets, dest, row_token, final_expert, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  Carve cv(nullptr);
  carve_dispatch(cv, c);
  carve_reroute(cv, c);
  if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c.T == 0) return MOE_OK;
  Carve wv(ws);
  DispatchWs dw = carve_dispatch(wv, c);
  RerouteWs rw = carve_reroute(wv, c);
  DispatchParams p;
  p.idx = topk_idx; p.counts = counts; p.offsets = offsets; p.dest = dest;
  p.row_token = row_token; p.local_rank = dw.local_rank; p.chunk_hist = dw.chunk_hist;
  p.n = (int)(c.T * c.k); p.k = (int)c.k; p.E = (int)c.E; p.C = (int)c.C;
  if ((st = hip_status(launch_dispatch(p, stream))) != MOE_OK) return st;
  RerouteParams r;
  r.idx = topk_idx; r.logits = logits; r.counts = counts; r.offsets = offsets;
  r.dest = dest; r.dest_out = dest; r.row_token = row_token; r.final_expert = final_expert;
  r.fallback = rw.fallback; r.list_a = rw.list_a; r.list_b = rw.list_b; r.fe = rw.fe;
  r.rin = rw.rin; r.off_prim = rw.off_prim;
  r.chunk_cnt = rw.chunk_cnt; r.chunk_base = rw.chunk_base; r.chunk_hist = rw.chunk_hist;
  r.chunk_ebase = rw.chunk_ebase; r.local_rank = rw.local_rank; r.prop = rw.prop;
  r.pcnt = rw.pcnt; r.load_g = rw.load_g; r.n_g = rw.n_g;
  r.T = (int)c.T; r.E = (int)c.E; r.k = (int)c.k; r.C = (int)c.C;
  return hip_status(launch_reroute(r, stream));
}

moe_status_t moe_expert_up(const moe_config_t* cfg, int64_t n_groups, const void* x_rows,
                           const int32_t* row_token, const int32_t* offsets, int64_t rows_bound,
                           int64_t group_bound, const void* w1, const void* w3, const float* b1,
                           void* hidden, void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  st = check_ffn_args(c, n_groups, offsets, rows_bound, group_bound);
  if (st != MOE_OK) return st;
  if (!x_rows || !w1 || !hidden || !ws || (c.act == MOE_ACT_SWIGLU && !w3))
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x_rows, row_token, w1, w3, b1, hidden, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ffn_ws_bytes(c, rows_bound, n_groups, false)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (n_groups == 0 || rows_bound == 0) return MOE_OK;
  Carve wv(ws);
  FfnWs fw = carve_ffn(wv, rows_bound, n_groups, 0, c.T, c.d);
  return run_up(c, ffn_params(c, n_groups, offsets, rows_bound, group_bound, fw), x_rows,
                row_token, w1, w3, b1, hidden, stream);
}

moe_status_t moe_expert_down(const moe_config_t* cfg, int64_t n_groups, const void* hidden,
                             const int32_t* offsets, int64_t rows_bound, int64_t group_bound,
                             const void* w2, const float* b2, float* y_rows, int accumulate,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  st = check_ffn_args(c, n_groups, offsets, rows_bound, group_bound);
  if (st != MOE_OK) return st;
  if (!hidden || !w2 || !y_rows || !ws) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {hidden, w2, b2, y_rows, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ffn_ws_bytes(c, rows_bound, n_groups, false)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (n_groups == 0 || rows_bound == 0) return MOE_OK;
  Carve wv(ws);
  FfnWs fw = carve_ffn(wv, rows_bound, n_groups, 0, c.T, c.d);
  return run_down(c, ffn_params(c, n_groups, offsets, rows_bound, group_bound, fw), hidden, w2,
                  b2, y_rows, accumulate, stream);
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t n_groups, const void* x_rows,
                            const int32_t* row_token, const int32_t* offsets, int64_t rows_bound,
                            int64_t group_bound, const void* w1, const void* w3, const void* w2,
                            const float* b1, const float* b2, float* y_rows, int accumulate,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  st = check_ffn_args(c, n_groups, offsets, rows_bound, group_bound);
  if (st != MOE_OK) return st;
  if (!x_rows || !w1 || !w2 || !y_rows || !ws || (c.act == MOE_ACT_SWIGLU && !w3))
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x_rows, row_token, w1, w3, w2, b1, b2, y_rows, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ffn_ws_bytes(c, rows_bound, n_groups, true)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (n_groups == 0 || rows_bound == 0) return MOE_OK;
  Carve wv(ws);
  FfnWs fw = carve_ffn(wv, rows_bound, n_groups, 0, c.T, c.d);
  void* hidden = wv.take((size_t)rows_bound * c.h * c.esz);
  FfnParams p = ffn_params(c, n_groups, offsets, rows_bound, group_bound, fw);
  st = run_up(c, p, x_rows, row_token, w1, w3, b1, hidden, stream);
  if (st != MOE_OK) return st;
  return run_down(c, p, hidden, w2, b2, y_rows, accumulate, stream);
}

moe_status_t moe_combine(const moe_config_t* cfg, const float* y_rows, const int32_t* dest,
                         const float* topk_gate, const float* y_shared, const int32_t* counts,
                         const float* prob_sum, void* y, float* stats, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!y_rows || !dest || !topk_gate || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (c.ec) return MOE_ERR_INVALID_ARGUMENT;
  if (c.S > 0 && !y_shared) return MOE_ERR_INVALID_ARGUMENT;
  if (stats && (!counts || !prob_sum)) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {y_rows, dest, topk_gate, y_shared, counts, prob_sum, y, stats};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  CombineParams p;
  p.y_rows = y_rows; p.dest = dest; p.gate = topk_gate;
  p.y_shared = c.S > 0 ? y_shared : nullptr;
  p.y = y; p.T = (int)c.T; p.d = (int)c.d; p.k = (int)c.k; p.S = (int)c.S; p.out_bf16 = c.bf16;
  st = hip_status(launch_combine(p, stream));
  if (st != MOE_OK || !stats) return st;
  StatsParams sp;
  sp.counts = counts; sp.prob_sum = prob_sum; sp.stats = stats;
  sp.dest = c.rr ? dest : nullptr;
  sp.T = (int)c.T; sp.k = (int)c.k; sp.E = (int)c.E; sp.C = (int)c.C;
  return hip_status(launch_stats(sp, stream));
}

moe_status_t moe_router_diagnostics(const moe_config_t* cfg, const float* logits,
                                    const int32_t* counts, const int32_t* dest, float* diag,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (c.ec || !logits || !counts || !dest || !diag || !ws) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {logits, counts, dest, diag, ws};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  Carve cv(nullptr);
  carve_diag(cv, c);
  if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c.T == 0) return MOE_OK;
  Carve wv(ws);
  DiagWs gw = carve_diag(wv, c);
  DiagParams p;
  p.logits = logits; p.counts = counts; p.dest = dest; p.diag = diag;
  p.partial_d = gw.partial_d; p.partial_i = gw.partial_i;
  p.T = (int)c.T; p.E = (int)c.E; p.k = (int)c.k; p.C = (int)c.C;
  return hip_status(launch_diagnostics(p, stream));
}

moe_status_t moe_expert_choice(const moe_config_t* cfg, const float* logits, float* scores,
                               int32_t* counts, int32_t* offsets, int32_t* row_token,
                               int32_t* slot, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!c.ec || !scores || !counts || !offsets || !row_token || !slot) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {logits, scores, counts, offsets, row_token, slot};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  EcParams p;
  p.scores = scores; p.counts = counts; p.offsets = offsets; p.row_token = row_token;
  p.slot = slot; p.T = (int)c.T; p.E = (int)c.E; p.Cp = (int)c.C;
  return hip_status(launch_expert_choice(p, logits, stream));
}

moe_status_t moe_combine_expert_choice(const moe_config_t* cfg, const float* y_rows,
                                       const int32_t* slot, const float* scores,
                                       const float* y_shared, const int32_t* counts,
                                       const float* prob_sum, void* y, float* stats,
                                       hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!c.ec || !y_rows || !slot || !scores || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (c.S > 0 && !y_shared) return MOE_ERR_INVALID_ARGUMENT;
  if (stats && (!counts || !prob_sum)) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {y_rows, slot, scores, y_shared, counts, prob_sum, y, stats};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  EcCombineParams p;
  p.y_rows = y_rows; p.slot = slot; p.scores = scores;
  p.y_shared = c.S > 0 ? y_shared : nullptr;
  p.y = y; p.T = (int)c.T; p.d = (int)c.d; p.E = (int)c.E; p.S = (int)c.S; p.out_bf16 = c.bf16;
  st = hip_status(launch_combine_ec(p, stream));
  if (st != MOE_OK || !stats) return st;
  EcStatsParams sp;
  sp.counts = counts; sp.prob_sum = prob_sum; sp.slot = slot; sp.stats = stats;
  sp.T = (int)c.T; sp.E = (int)c.E;
  return hip_status(launch_stats_ec(sp, stream));
}

// The whole layer on `ws`; with `noalloc` the caller passes no workspace and
// the layer runs on the current device's static scratch instead.
static moe_status_t layer_forward(const moe_config_t* cfg, const moe_weights_t* w,
                                  const void* x, const float* eps, const float* logits_in,
                                  void* y, const moe_aux_t* aux, void* ws, size_t ws_bytes,
                                  hipStream_t stream, bool noalloc) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  if (!w || !x || !y || (!ws && !noalloc) || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARGUMENT;
  if (c.act == MOE_ACT_SWIGLU && !w->w3) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->ffn_bias && (!w->b1 || !w->b2)) return MOE_ERR_INVALID_ARGUMENT;
  if (!logits_in) {
    if (!w->w_g) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->router_bias && !w->b_g) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->router_noise && (!w->w_noise || !eps)) return MOE_ERR_INVALID_ARGUMENT;
  }
  if (c.S > 0 && (!w->ws1 || !w->ws2 || (c.act == MOE_ACT_SWIGLU && !w->ws3)))
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x, eps, logits_in, y, ws, w->w_g, w->b_g, w->w_noise, w->w1, w->w3,
                        w->w2, w->b1, w->b2, w->ws1, w->ws3, w->ws2};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  if (aux) {
    const void* ap[] = {aux->logits, aux->topk_idx, aux->topk_gate, aux->prob_sum, aux->counts,
                        aux->offsets, aux->dest, aux->row_token, aux->stats, aux->scores,
                        aux->slot, aux->diag, aux->final_expert, aux->hidden, aux->pre,
                        aux->y_rows};
    for (const void* q : ap)
      if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  }
  {
    Carve cv(nullptr);
    carve_layer(cv, c, aux);
    if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  if (c.T == 0) return MOE_OK;
  if (noalloc && (st = static_scratch(&ws)) != MOE_OK) return st;
  Carve wv(ws);
  LayerWs L = carve_layer(wv, c, aux);

  // 1-2. router, top-k, gates, softmax sums
  RouteParams rp;
  rp.x = logits_in ? nullptr : x;
  rp.w_g = w->w_g;
  rp.b_g = cfg->router_bias ? w->b_g : nullptr;
  rp.w_noise = cfg->router_noise ? w->w_noise : nullptr;
  rp.eps = cfg->router_noise ? eps : nullptr;
  rp.logits = logits_in ? const_cast<float*>(logits_in) : L.logits;
  rp.idx = L.idx; rp.gate = L.gate; rp.prob_partial = L.rw.prob_partial; rp.prob_sum = L.prob_sum;
  rp.noise_pre = nullptr;
  rp.T = (int)c.T; rp.d = (int)c.d; rp.E = (int)c.E; rp.k = (int)c.k; rp.bf16 = c.bf16;
  // Top-1 layers without shared experts whose down projection streams the
  // weights: every kept row is its token's only expert output, so that
  // launch stores gate * row straight into the token's output row and there
  // is no combine pass; the router zeroes every output row first, so the
  // dropped tokens' rows stay zero.  Not when the caller wants the float32
  // expert rows.
  FfnParams fp = ffn_params(c, c.E, L.offsets, c.R, c.C, L.fw);
  fp.S = (int)c.S;
  const bool direct = !c.ec && !c.rr && c.k == 1 && c.S == 0 && ffn_uses_skinny(fp) &&
                      !(aux && aux->y_rows);
  if (direct) {
    rp.zero_rows = y;
    rp.row_bytes = (int)(c.d * 2);
  }
  if ((st = hip_status(launch_route(rp, stream))) != MOE_OK) return st;

  // 3. counts, capacity, dispatch tables (expert choice: every expert takes
  //    its best tokens)
  if (c.ec) {
    EcParams ep;
    ep.scores = L.scores; ep.counts = L.counts; ep.offsets = L.offsets;
    ep.row_token = L.row_token; ep.slot = L.slot;
    ep.T = (int)c.T; ep.E = (int)c.E; ep.Cp = (int)c.C;
    if ((st = hip_status(launch_expert_choice(ep, rp.logits, stream))) != MOE_OK) return st;
  } else {
    DispatchParams dp;
    dp.idx = L.idx; dp.counts = L.counts; dp.offsets = L.offsets; dp.dest = L.dest;
    dp.row_token = L.row_token; dp.local_rank = L.dw.local_rank; dp.chunk_hist = L.dw.chunk_hist;
    dp.n = (int)(c.T * c.k); dp.k = (int)c.k; dp.E = (int)c.E; dp.C = (int)c.C;
    if ((st = hip_status(launch_dispatch(dp, stream))) != MOE_OK) return st;
    if (c.rr) {
      RerouteParams r;
      r.idx = L.idx; r.logits = rp.logits; r.counts = L.counts; r.offsets = L.offsets;
      r.dest = L.dest; r.dest_out = L.dest; r.row_token = L.row_token;
      r.final_expert = L.final_expert;
      r.fallback = L.rrw.fallback; r.list_a = L.rrw.list_a; r.list_b = L.rrw.list_b;
      r.fe = L.rrw.fe; r.rin = L.rrw.rin; r.off_prim = L.rrw.off_prim;
      r.chunk_cnt = L.rrw.chunk_cnt; r.chunk_base = L.rrw.chunk_base;
      r.chunk_hist = L.rrw.chunk_hist; r.chunk_ebase = L.rrw.chunk_ebase;
      r.local_rank = L.rrw.local_rank; r.prop = L.rrw.prop; r.pcnt = L.rrw.pcnt;
      r.load_g = L.rrw.load_g; r.n_g = L.rrw.n_g;
      r.T = (int)c.T; r.E = (int)c.E; r.k = (int)c.k; r.C = (int)c.C;
      if ((st = hip_status(launch_reroute(r, stream))) != MOE_OK) return st;
    }
    if (aux && aux->diag) {
      DiagParams gp;
      gp.logits = rp.logits; gp.counts = L.counts; gp.dest = L.dest; gp.diag = aux->diag;
      gp.partial_d = L.gw.partial_d; gp.partial_i = L.gw.partial_i;
      gp.T = (int)c.T; gp.E = (int)c.E; gp.k = (int)c.k; gp.C = (int)c.C;
      if ((st = hip_status(launch_diagnostics(gp, stream))) != MOE_OK) return st;
    }
  }

  // 4. grouped expert FFN: routed groups gathered through row_token, then the
  //    shared experts over all tokens, in one launch per projection
  FfnParams up = fp;
  up.a_main = x; up.a_shared = x; up.gather = L.row_token; up.a_from_c = 0;
  up.w_main = w->w1; up.u_main = w->w3; up.w_shared = w->ws1; up.u_shared = w->ws3;
  up.bias_main = cfg->ffn_bias ? w->b1 : nullptr; up.bias_shared = nullptr;
  up.out = L.hidden; up.out_bf16 = c.bf16; up.accumulate = 0;
  up.N = (int)c.h; up.K = (int)c.d; up.act = c.act;
  up.pre = aux ? aux->pre : nullptr;
  if ((st = hip_status(launch_ffn(up, stream))) != MOE_OK) return st;
  FfnParams dn = fp;
  dn.a_main = L.hidden; dn.a_shared = L.hidden; dn.gather = nullptr; dn.a_from_c = 1;
  dn.w_main = w->w2; dn.u_main = nullptr; dn.w_shared = w->ws2; dn.u_shared = nullptr;
  dn.bias_main = cfg->ffn_bias ? w->b2 : nullptr; dn.bias_shared = nullptr;
  dn.out = L.y_rows; dn.out_bf16 = 0; dn.accumulate = 0;
  dn.N = (int)c.d; dn.K = (int)c.h; dn.act = -1;
  // the two projections pick the same kernel (same dtype, group bound, S
  // and T) over the same groups, so a tiled down projection finds its row
  // tiles already in the schedule scratch the up projection built
  dn.tiles_built = 1;
  if (direct) {
    dn.out = y; dn.out_bf16 = 1;
    dn.direct_token = L.row_token; dn.direct_gate = L.gate;
  }
  // A bf16 layer keeps its own expert rows in bf16, rounded once (bias
  // included) like every other bf16 activation: half the bytes the down
  // projection writes and the combine reads.  Not when the caller wants the
  // float32 rows.  (A tiled down projection's split tiles then sum float32
  // partials in a fixup, in the third scratch block carve_layer gave them.)
  const bool rows_bf16 = c.bf16 && !c.ec && !direct && !(aux && aux->y_rows);
  if (rows_bf16) dn.out_bf16 = 1;
  // Two shared experts on the tiled path run as one group whose reduction
  // covers both in turn (2h deep): one output row per token, the sum of the
  // two, instead of two rows for the combine to add; half the shared tiles,
  // each twice as deep.  Their hidden rows stay where the up projection
  // wrote them (expert s's row t at R + s*T + t); the launch builds its own
  // schedule (one shared group).  Not when the caller wants the rows, and
  // only for h a multiple of the 64-deep stage, so no stage straddles the
  // two experts.
  const bool shared_cat = c.bf16 && !c.ec && c.S == 2 && c.h % 64 == 0 && !ffn_uses_skinny(fp) &&
                          !(aux && aux->y_rows) && !direct;
  if (shared_cat) {
    dn.S = 1;
    dn.shared_cat = 2;
    dn.a_shared = static_cast<const char*>(L.hidden) + (size_t)c.R * c.h * c.esz;
    dn.tiles_built = 0;
    // tiles of two depths: the XCD ranges are cut by depth and the tail is
    // not split
    dn.split = nullptr;
    dn.split_cap = 0;
  }
  if ((st = hip_status(launch_ffn(dn, stream))) != MOE_OK) return st;

  // 5. combine (+ statistics)
  if (c.ec) {
    EcCombineParams cp;
    cp.y_rows = L.y_rows; cp.slot = L.slot; cp.scores = L.scores;
    cp.y_shared = c.S > 0 ? L.y_rows + (size_t)c.R * c.d : nullptr;
    cp.y = y; cp.T = (int)c.T; cp.d = (int)c.d; cp.E = (int)c.E; cp.S = (int)c.S;
    cp.out_bf16 = c.bf16;
    if ((st = hip_status(launch_combine_ec(cp, stream))) != MOE_OK) return st;
    if (aux && aux->stats) {
      EcStatsParams sp;
      sp.counts = L.counts; sp.prob_sum = L.prob_sum; sp.slot = L.slot; sp.stats = aux->stats;
      sp.T = (int)c.T; sp.E = (int)c.E;
      if ((st = hip_status(launch_stats_ec(sp, stream))) != MOE_OK) return st;
    }
    return MOE_OK;
  }
  if (!direct) {
    CombineParams cp;
    cp.y_rows = L.y_rows; cp.dest = L.dest; cp.gate = L.gate;
    cp.y_shared = c.S > 0 ? static_cast<const char*>(static_cast<const void*>(L.y_rows)) +
                                (size_t)c.R * c.d * (rows_bf16 ? 2 : 4)
                          : nullptr;
    cp.y = y; cp.T = (int)c.T; cp.d = (int)c.d; cp.k = (int)c.k; cp.S = shared_cat ? 1 : (int)c.S;
    cp.out_bf16 = c.bf16; cp.rows_bf16 = rows_bf16;
    if ((st = hip_status(launch_combine(cp, stream))) != MOE_OK) return st;
  }
  if (aux && aux->stats) {
    StatsParams sp;
    sp.counts = L.counts; sp.prob_sum = L.prob_sum; sp.stats = aux->stats;
    sp.dest = c.rr ? L.dest : nullptr;
    sp.T = (int)c.T; sp.k = (int)c.k; sp.E = (int)c.E; sp.C = (int)c.C;
    if ((st = hip_status(launch_stats(sp, stream))) != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               const float* eps, const float* logits_in, void* y,
                               const moe_aux_t* aux, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return layer_forward(cfg, w, x, eps, logits_in, y, aux, ws, ws_bytes, stream, false);
}

moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w,
                                       const void* x, const float* eps,
                                       const float* logits_in, void* y, const moe_aux_t* aux,
                                       hipStream_t stream) {
  return layer_forward(cfg, w, x, eps, logits_in, y, aux, nullptr, MOE_NOALLOC_SCRATCH_BYTES,
                       stream, true);
}

size_t moe_backward_workspace_bytes(const moe_config_t* cfg) {
  Cfg c;
  if (check_cfg(cfg, &c) != MOE_OK) return 0;
  Carve cv(nullptr);
  carve_backward(cv, c, cfg->router_noise != 0);
  return cv.off + 256;
}

moe_status_t moe_layer_backward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                const float* eps, const float* dy, float g_aux, float g_z,
                                const moe_aux_t* sv, const moe_grads_t* gr, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  Cfg c;
  moe_status_t st = check_cfg(cfg, &c);
  if (st != MOE_OK) return st;
  const bool swi = c.act == MOE_ACT_SWIGLU, noise = cfg->router_noise != 0;
  if (!w || !x || !dy || !sv || !gr || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!w->w_g || !w->w1 || !w->w2 || (swi && !w->w3)) return MOE_ERR_INVALID_ARGUMENT;
  if (noise && (!w->w_noise || !eps || !gr->dw_noise)) return MOE_ERR_INVALID_ARGUMENT;
  if (c.S > 0 && (!w->ws1 || !w->ws2 || (swi && !w->ws3))) return MOE_ERR_INVALID_ARGUMENT;
  if (!sv->logits || !sv->counts || !sv->offsets || !sv->row_token || !sv->hidden || !sv->pre ||
      !sv->y_rows)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c.ec ? (!sv->scores || !sv->slot) : (!sv->topk_idx || !sv->topk_gate || !sv->dest))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!gr->dx || !gr->dw_g || !gr->dw1 || !gr->dw2 || (swi && !gr->dw3))
    return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->router_bias && !gr->db_g) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->ffn_bias && (!gr->db1 || !gr->db2)) return MOE_ERR_INVALID_ARGUMENT;
  if (c.S > 0 && (!gr->dws1 || !gr->dws2 || (swi && !gr->dws3))) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(g_aux) || !isfinite(g_z)) return MOE_ERR_INVALID_ARGUMENT;
  if (c.d % 8 || c.h % 8) return MOE_ERR_UNSUPPORTED;
  if (!backward_fits(c) || c.E + c.S > 512) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, eps, dy, ws, w->w_g, w->w_noise, w->w1, w->w3, w->w2, w->ws1, w->ws3,
                        w->ws2, sv->logits, sv->topk_idx, sv->topk_gate, sv->counts,
                        sv->offsets, sv->dest, sv->row_token, sv->hidden, sv->pre, sv->y_rows,
                        sv->scores, sv->slot,
                        gr->dx, gr->dw_g, gr->db_g, gr->dw_noise, gr->dw1, gr->dw3, gr->dw2,
                        gr->db1, gr->db2, gr->dws1, gr->dws3, gr->dws2};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_ERR_UNSUPPORTED;
  {
    Carve cv(nullptr);
    carve_backward(cv, c, noise);
    if (ws_bytes < cv.off + 256) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  Carve wv(ws);
  BwdWs B = carve_backward(wv, c, noise);
  const int64_t kup = swi ? 2 * c.h : c.h;
  const int64_t rp = padded_rows_bound(c);
  const int G = (int)c.E, S = (int)c.S;
  hipError_t e;
#define MOE_TRY(call) \
  if ((e = (call)) != hipSuccess) return MOE_ERR_HIP;

  // 1. gates of the routed rows, gate gradients, logit gradients
  if (c.ec) {
    MOE_TRY(launch_ec_row_gate(sv->slot, sv->scores, c.T * c.E, B.row_gate, stream));
  } else {
    MOE_TRY(launch_row_gate(sv->dest, sv->topk_gate, c.T * c.k, B.row_gate, stream));
  }
  if (noise) {
    RouteParams rp0;
    rp0.x = x; rp0.w_g = w->w_g; rp0.b_g = cfg->router_bias ? w->b_g : nullptr;
    rp0.w_noise = w->w_noise; rp0.eps = eps; rp0.logits = B.r_logits; rp0.idx = B.r_idx;
    rp0.gate = B.r_gate; rp0.prob_partial = B.rw.prob_partial; rp0.prob_sum = B.r_prob_sum;
    rp0.noise_pre = B.noise_pre;
    rp0.T = (int)c.T; rp0.d = (int)c.d; rp0.E = (int)c.E; rp0.k = (int)c.k; rp0.bf16 = c.bf16;
    if (c.T > 0) MOE_TRY(launch_route(rp0, stream));
  }
  BwdParams bp;
  bp.dy = dy; bp.y_rows = sv->y_rows; bp.dest = sv->dest; bp.idx = sv->topk_idx;
  bp.gate = sv->topk_gate; bp.logits = sv->logits; bp.counts = sv->counts;
  bp.eps = noise ? eps : nullptr; bp.noise_pre = B.noise_pre;
  bp.dg = B.dg; bp.dH = B.dH; bp.dHn = noise ? B.dHn : nullptr;
  bp.dx_rows = B.dxr; bp.dx = gr->dx; bp.g_aux = g_aux; bp.g_z = g_z;
  bp.rows_bound = c.R; bp.T = (int)c.T; bp.d = (int)c.d; bp.E = (int)c.E; bp.k = (int)c.k;
  bp.S = S;
  // f: routed counts over T*k (token choice), rows over all rows (expert choice)
  const double f_den = c.ec ? (double)c.E * (double)c.C : (double)c.T * (double)c.k;
  bp.inv_f_den = f_den > 0 ? (float)(1.0 / f_den) : 0.f;
  bp.ec = c.ec ? 1 : 0; bp.slot = sv->slot; bp.scores = sv->scores;
  MOE_TRY(launch_router_backward(bp, stream));

  // 2. router weights
  MOE_TRY(launch_router_wgrad(B.dH, x, c.bf16, (int)c.T, G, (int)c.d, B.rpartial, gr->dw_g, stream));
  if (noise)
    MOE_TRY(launch_router_wgrad(B.dHn, x, c.bf16, (int)c.T, G, (int)c.d, B.rpartial,
                                gr->dw_noise, stream));
  if (cfg->router_bias) MOE_TRY(launch_column_sum(B.dH, (int)c.T, G, gr->db_g, stream));

  // 3. transposed weights: w2t[g] = w2[g]^T [h,d]; w13t[g] = [w1[g]^T | w3[g]^T] [d, Kup].
  //    The bf16 tiled GEMMs can read W2, W1 and W3 as stored ([K][N]
  //    weights) instead.  That form runs about 22% slower (two 8-byte LDS
  //    transpose reads per operand fragment instead of one 16-byte read),
  //    while a copy costs both directions of the weight bytes at about
  //    5 TB/s: per group of d x h weights the copy costs as much as the
  //    slowdown on about 2000 rows (2 * 2dh / 5e12 = 0.22 * 2 * rows * d * h /
  //    1.1e15).  Below that many rows per group the stored layout is read.
  const int esz = (int)c.esz;
  const size_t gsz2 = (size_t)c.h * c.d * c.esz, gsz13 = (size_t)c.d * kup * c.esz;
  char* w2t = static_cast<char*>(B.w2t);
  char* w13t = static_cast<char*>(B.w13t);
  FfnParams fp = ffn_params(c, c.E, sv->offsets, c.R, c.C, B.fw);
  fp.S = S;
  const bool few_rows = c.R + c.S * c.T < 2000 * (c.E + c.S);
  const bool bt_down = c.bf16 && few_rows;  // (its input gradient is always tiled)
  // the up projections' input gradient reads W1 (and W3) as stored too, on
  // the kernel the forward's down projection uses (tiled, or weight streaming
  // where every group holds at most 32 rows)
  const bool bt_up = c.bf16 && few_rows && (!swi || c.h % 64 == 0);
  if (!bt_down) {
    MOE_TRY(launch_transpose(w->w2, G, (int)c.d, (int)c.h, w2t, (int)c.d, 0, esz, stream));
    if (S > 0)
      MOE_TRY(launch_transpose(w->ws2, S, (int)c.d, (int)c.h, w2t + G * gsz2, (int)c.d, 0, esz, stream));
  }
  if (!bt_up) {
    MOE_TRY(launch_transpose(w->w1, G, (int)c.h, (int)c.d, w13t, (int)kup, 0, esz, stream));
    if (swi) MOE_TRY(launch_transpose(w->w3, G, (int)c.h, (int)c.d, w13t, (int)kup, (int)c.h, esz, stream));
    if (S > 0) {
      MOE_TRY(launch_transpose(w->ws1, S, (int)c.h, (int)c.d, w13t + G * gsz13, (int)kup, 0, esz, stream));
      if (swi)
        MOE_TRY(launch_transpose(w->ws3, S, (int)c.h, (int)c.d, w13t + G * gsz13, (int)kup, (int)c.h,
                                 esz, stream));
    }
  }

  // 4. input gradient of the down projection with the activation backward:
  //    duv[r] = act'(pre[r]) * gate_r * (dy[token(r)] w2)   (config dtype)
  const void* dy_op = dy;
  if (c.bf16) {
    MOE_TRY(launch_to_bf16(dy, c.T * c.d, static_cast<uint16_t*>(B.dy_lp), stream));
    dy_op = B.dy_lp;
  }
  FfnParams dd = fp;
  dd.a_main = dy_op; dd.a_shared = dy_op; dd.gather = sv->row_token; dd.a_from_c = 0;
  dd.w_main = w2t; dd.w_shared = w2t + G * gsz2; dd.u_main = nullptr; dd.u_shared = nullptr;
  if (bt_down) {  // W2 [d][h] as stored: K = d rows of N = h
    dd.w_main = w->w2; dd.w_shared = w->ws2; dd.bt = 1; dd.kh = 0;
  }
  dd.bias_main = nullptr; dd.bias_shared = nullptr;
  dd.out = B.duv; dd.out_bf16 = c.bf16; dd.accumulate = 0;
  dd.N = (int)c.h; dd.K = (int)c.d; dd.act = kActBwd + c.act;
  dd.pre = sv->pre; dd.row_gate = B.row_gate;
  // (where every group holds at most 32 rows this streams W2 on the
  // weight-streaming kernel, which then reads it as stored)
  MOE_TRY(c.bf16 ? launch_ffn(dd, stream) : launch_ffn_f32(dd, stream));

  // 5. input gradient of the up projection(s): dx_rows = duv [w1 | w3]
  FfnParams du = fp;
  du.a_main = B.duv; du.a_shared = B.duv; du.gather = nullptr; du.a_from_c = 1;
  du.w_main = w13t; du.w_shared = w13t + G * gsz13; du.u_main = nullptr; du.u_shared = nullptr;
  if (bt_up) {  // W1 (and W3) [h][d] as stored: K = h (+ h) rows of N = d
    du.w_main = w->w1; du.w_shared = w->ws1; du.u_main = w->w3; du.u_shared = w->ws3;
    du.bt = 1; du.kh = swi ? (int)c.h : 0;
  }
  du.bias_main = nullptr; du.bias_shared = nullptr;
  du.out = B.dxr; du.out_bf16 = 0; du.accumulate = 0;
  du.N = (int)c.d; du.K = (int)kup; du.act = -1;
  MOE_TRY(launch_ffn(du, stream));

  // 6. dx = expert rows of the token + shared rows + router share
  MOE_TRY(launch_dx(bp, w->w_g, noise ? w->w_noise : nullptr, c.bf16, stream));

  // 7. weight gradients over each group's rows (transposed, zero-padded blocks)
  MOE_TRY(launch_group_desc(sv->offsets, G, S, (int)c.T, c.R, B.desc, B.total, stream));
  PackParams pk;
  pk.desc = B.desc; pk.total = B.total; pk.row_token = sv->row_token; pk.G = G; pk.S = S;
  auto pack = [&](const void* src, int src_esz, int64_t ld, int coff, int C, bool gathered,
                  const float* scale, void* dst) {
    PackParams q = pk;
    q.C = C; q.ld = ld; q.coff = coff; q.gathered = gathered; q.row_gate = scale;
    return launch_pack_t(q, src, src_esz, dst, esz, rp, stream);
  };
  MOE_TRY(pack(dy, 4, c.d, 0, (int)c.d, true, B.row_gate, B.dyT));       // (gate * dy)^T
  MOE_TRY(pack(x, esz, c.d, 0, (int)c.d, true, nullptr, B.xT));          // x^T
  MOE_TRY(pack(sv->hidden, esz, c.h, 0, (int)c.h, false, nullptr, B.hidT));
  MOE_TRY(pack(B.duv, esz, kup, 0, (int)c.h, false, nullptr, B.duT));
  if (swi) MOE_TRY(pack(B.duv, esz, kup, (int)c.h, (int)c.h, false, nullptr, B.dvT));
  auto wgrad = [&](const void* At, const void* Bt, int M, int N, float* out, float* out_s) {
    if (!c.bf16)
      return launch_wgrad_f32(static_cast<const float*>(At), static_cast<const float*>(Bt),
                              B.desc, G, S, M, N, out, out_s, stream);
    FfnParams q = fp;
    q.a_main = At; q.a_shared = At; q.gather = nullptr; q.a_from_c = 0;
    q.w_main = Bt; q.w_shared = Bt; q.u_main = nullptr; q.u_shared = nullptr;
    q.bias_main = nullptr; q.bias_shared = nullptr;
    q.out = out; q.out_shared = out_s; q.out_bf16 = 0; q.accumulate = 0;
    q.M = M; q.N = N; q.K = 0; q.act = kActWgrad; q.gdesc = B.desc; q.xcd_bounds = B.xcd_bounds;
    return launch_ffn_tiled(q, stream);
  };
  MOE_TRY(wgrad(B.dyT, B.hidT, (int)c.d, (int)c.h, gr->dw2, gr->dws2));
  MOE_TRY(wgrad(B.duT, B.xT, (int)c.h, (int)c.d, gr->dw1, gr->dws1));
  if (swi) MOE_TRY(wgrad(B.dvT, B.xT, (int)c.h, (int)c.d, gr->dw3, gr->dws3));
  if (cfg->ffn_bias) {
    PackParams q = pk;
    q.C = (int)c.h; q.ld = kup; q.coff = 0; q.gathered = 0; q.row_gate = nullptr;
    MOE_TRY(launch_bias_grad(q, B.duv, esz, gr->db1, stream));
    q.C = (int)c.d; q.ld = c.d; q.gathered = 1; q.row_gate = B.row_gate;
    MOE_TRY(launch_bias_grad(q, dy, 4, gr->db2, stream));
  }
#undef MOE_TRY
  return MOE_OK;
}

}  // extern "C"
