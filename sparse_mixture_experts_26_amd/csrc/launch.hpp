// Internal launch interface between the C ABI layer (api.cpp) and the HIP
// kernels.  Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

// ---- routing -----------------------------------------------------------------
struct RouteParams {
  const void* x;            // [T,d] bf16 or f32; null = replay `logits`
  const void* w_g;          // [E,d]
  const float* b_g;         // [E] or null
  const void* w_noise;      // [E,d] or null
  const float* eps;         // [T,E] or null
  float* logits;            // [T,E] out (in when replaying)
  int32_t* idx;             // [T,k]
  float* gate;              // [T,k]
  float* prob_partial;      // [route_blocks(T), E]
  float* prob_sum;          // [E]
  float* noise_pre;         // [T,E] out: x W_noise^T before softplus, or null
  int T, d, E, k;
  int bf16;
  // when set, each block also zeroes its tokens' rows (row_bytes bytes, a
  // multiple of 16) of this [T, row_bytes] buffer: the output rows of a
  // top-1 layer whose down projection stores straight into the kept
  // tokens' rows (the dropped tokens' rows stay zero); null = nothing
  void* zero_rows = nullptr;
  int row_bytes = 0;
};
constexpr int kRouteTokens = 16;  // tokens per routing block
inline int route_blocks(int64_t T) { return (int)((T + kRouteTokens - 1) / kRouteTokens); }
hipError_t launch_route(const RouteParams& p, hipStream_t stream);
// bf16 batches of at least this many tokens, with at least 32 logit columns
// (gate plus noise), compute their logits in a kernel of their own (64-token
// blocks, so the router matrix is read from L2 once per 64 tokens instead of
// once per 16) and route_kernel replays them.  A narrower router matrix is
// cheap to re-read, and there the single fused launch is faster.
#ifndef MOE_ROUTE_SPLIT_MIN_T
#define MOE_ROUTE_SPLIT_MIN_T 1024
#endif
inline bool route_split_logits(int64_t T, int64_t E, bool noise) {
  return T >= MOE_ROUTE_SPLIT_MIN_T && E * (noise ? 2 : 1) >= 32;
}
// Launch shape of route_kernel: waves per block, dynamic and static LDS bytes
// (mma: bf16 logits computed on the device; otherwise float32 or replay).
struct RoutePlan { int waves; size_t lds_bytes; size_t static_lds_bytes; };
RoutePlan route_plan(int E, bool noise, bool mma);

// ---- dispatch ----------------------------------------------------------------
struct DispatchParams {
  const int32_t* idx;       // [n] flat assignments, n = T*k
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* dest;            // [n]
  int32_t* row_token;       // [rows]
  int32_t* local_rank;      // [n] scratch
  int32_t* chunk_hist;      // [chunks, E] scratch
  int n, k, E, C;
};
constexpr int kDispatchChunk = 1024;
inline int dispatch_chunks(int64_t n) { return (int)((n + kDispatchChunk - 1) / kDispatchChunk); }
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t stream);

// Overflow re-routing after the primary dispatch (which leaves counts,
// offsets and dest of the arrival-order pass).
struct RerouteParams {
  const int32_t* idx;       // [T,k]
  const float* logits;      // [T,E]
  const int32_t* counts;    // [E] primary counts
  int32_t* offsets;         // [E+1] in: primary, out: over the final placement
  const int32_t* dest;      // [T,k] primary (may be dest_out itself)
  int32_t* dest_out;        // [T,k] final
  int32_t* row_token;       // [T*k]
  int32_t* final_expert;    // [T,k]
  uint8_t* fallback;        // [T, E-k] scratch
  int32_t* list_a;          // [2*T*k] scratch: (assignment, pointer) pairs
  int32_t* list_b;          // [2*T*k] scratch
  int32_t* fe;              // [T*k] scratch
  int32_t* rin;             // [T*k] scratch
  int32_t* off_prim;        // [E+1] scratch: the primary offsets
  int T, E, k, C;
  // multi-block list build and first rounds (scratch; chunks = ceil(T*k/1024))
  int32_t* chunk_cnt;       // [chunks]
  int32_t* chunk_base;      // [chunks]
  int32_t* chunk_hist;      // [chunks, E]
  int32_t* chunk_ebase;     // [chunks, E]
  int32_t* local_rank;      // [T*k]
  int32_t* prop;            // [T*k]
  int32_t* pcnt;            // [T*k]
  int32_t* load_g;          // [2, 256]
  int32_t* n_g;             // [2]
};
constexpr int kRrChunk = 1024;  // list positions per block in the multi-block passes
inline int reroute_chunks(int64_t n) { return (int)((n + kRrChunk - 1) / kRrChunk); }
hipError_t launch_reroute(const RerouteParams& p, hipStream_t stream);

// x_perm[r] = x[row_token[r]] for r < offsets[E]; row_bytes % 16 == 0.
hipError_t launch_permute(const void* x, const int32_t* row_token, const int32_t* total,
                          void* x_perm, int64_t row_bytes, int64_t rows_bound,
                          hipStream_t stream);

// ---- grouped expert GEMMs ------------------------------------------------------
// One launch covers the routed groups (rows given by device offsets) followed by
// n_shared shared groups of T rows each.  Output/hidden row layout: routed rows
// at [0, rows_bound), shared group s at rows_bound + s*T + t.
struct FfnParams {
  const void* a_main;        // routed operand rows (token matrix when gathered)
  const void* a_shared;      // token matrix for the shared groups
  const int32_t* gather;     // routed row r reads a_main row gather[r]; null = r
  int a_from_c;              // operand row index = output row index (down proj)
  const void* w_main;        // [G, N, K]
  const void* w_shared;      // [S, N, K]
  const void* u_main;        // gated second weight set, [G, N, K] (or null)
  const void* u_shared;
  const float* bias_main;    // [G, N] or null
  const float* bias_shared;
  void* out;                 // [rows_bound + S*T, N]
  int out_bf16;
  int accumulate;            // fp32 output only
  const int32_t* offsets;    // [G+1]
  int G, S, T;
  int64_t rows_bound;
  int64_t group_bound;
  int N, K;
  int act;                   // moe_act_t, or -1 for none (down projection); see below
  int bf16;                  // operand dtype
  TileEntry* entries;        // scratch for the tiled path
  int32_t* n_entries;        // scratch
  // nonzero: entries / n_entries already hold this launch's row-tile
  // schedule, built by an earlier tiled launch on the same stream with the
  // same offsets, G, S, T and rows_bound (the forward's down projection
  // reuses the up projection's); the launch then does not rebuild it
  int tiles_built;
  // forward (act 0..2): when set, the pre-activations are stored too: row r
  // holds u = a W^T (+ bias) in [0, N) and, gated, v = a U^T in [N, 2N)
  void* pre;
  // act = kActBwd + a: backward of activation a fused into the epilogue
  // (operand dtype out [rows, 2N when gated else N]: du, then dv), reading
  // `pre` and scaling every routed row by its gate
  const float* row_gate;     // [rows_bound] gate of each routed row
  // act = kActWgrad: per-group weight gradient C_g[M, N] = A_g B_g^T over the
  // group's transposed, zero-padded row block (gdesc); a_main and w_main are
  // the transposed operands, out / out_shared the routed / shared outputs
  int M;
  const GroupDesc* gdesc;    // [G + S]
  void* out_shared;
  int32_t* xcd_bounds;       // [9] scratch: each XCD's tile range
  // tiled path, act -1 and 2: float32 partials of the tiles whose reduction
  // is cut in parts (tail split), blocks of 256 x 256: 2 * split_cap (act -1
  // with a float32 output uses one per later part, the gated up projection,
  // whose epilogue needs the whole sum, one per part of its two), or
  // 3 * split_cap for act -1 with a bf16 output (one per part, summed and
  // rounded by a fixup); null = no split
  float* split;
  int split_cap;
  // tiled path (act -1 or kActBwd + a) and weight-streaming path (act -1):
  // the weights are stored [K][N] per group (output columns contiguous), as
  // W2 and W1 / W3 are for the backward's input gradients; kh > 0: rows
  // k >= kh come from the second set (u_main / u_shared), kh rows per group
  // each (kh % 64 == 0)
  int bt;
  int kh;
  // weight-streaming path, act -1, top-1 layers without shared experts: each
  // routed row r is its token's only expert output, so the epilogue stores
  // direct_gate[t] * row (bias included) as bf16 into row t = direct_token[r]
  // of `out` ([T, N], the layer output) instead of row r; null = row r
  const int32_t* direct_token;
  const float* direct_gate;
  // tiled path, act -1 (a layer call's down projection): nonzero = the
  // launch's one shared group (S = 1) runs over this many (2) shared experts
  // in turn, a reduction of shared_cat * K: expert s's operand row t is row
  // t + s*T of a_shared (rows of K elements) and its weights start s*N*K
  // elements into w_shared; the group's output row t is their sum
  int shared_cat;
};
constexpr int kActBwd = 4;   // act codes 4, 5, 6: GELU, ReLU, SwiGLU backward
constexpr int kActWgrad = 8;
int64_t ffn_max_entries(int64_t rows_bound, int G, int S, int T);
// tiles of a tiled launch with N output columns that its tail split may cut
// (the scratch holds twice as many blocks of 256 x 256 floats); wide: the
// backward's [K][N] input gradients, which may split every tile
int64_t ffn_split_cap(int64_t max_entries, int64_t N, bool wide = false);
hipError_t launch_ffn(const FfnParams& p, hipStream_t stream);
// whether launch_ffn runs p on the weight-streaming kernel
bool ffn_uses_skinny(const FfnParams& p);

// ---- expert-choice routing ---------------------------------------------------------
struct EcParams {
  float* scores;             // [T,E]: written from logits, or given (replay)
  int32_t* counts;           // [E]   = Cp
  int32_t* offsets;          // [E+1] = e * Cp
  int32_t* row_token;        // [E*Cp]
  int32_t* slot;             // [T,E] row of (t, e) or -1
  int T, E, Cp;              // Cp = min(C, T)
};
// logits != null: scores = softmax(logits) first; then the selection.
hipError_t launch_expert_choice(const EcParams& p, const float* logits, hipStream_t stream);

struct EcCombineParams {
  const float* y_rows;       // [E*Cp (+S*T), d]
  const int32_t* slot;       // [T,E]
  const float* scores;       // [T,E]
  const float* y_shared;     // [S,T,d] or null
  void* y;                   // [T,d]
  int T, d, E, S;
  int out_bf16;
};
hipError_t launch_combine_ec(const EcCombineParams& p, hipStream_t stream);

struct EcStatsParams {
  const int32_t* counts;     // [E]
  const float* prob_sum;     // [E]
  const int32_t* slot;       // [T,E]
  float* stats;              // [2E+2]
  int T, E;
};
hipError_t launch_stats_ec(const EcStatsParams& p, hipStream_t stream);

// ---- router z-loss and routing diagnostics ---------------------------------------
struct DiagParams {
  const float* logits;       // [T,E]
  const int32_t* counts;     // [E]
  const int32_t* dest;       // [T,k]
  float* diag;               // [8 + 2E]
  double* partial_d;         // [diag_blocks(T), 2] scratch
  int32_t* partial_i;        // [diag_blocks(T), 2] scratch
  int T, E, k, C;
};
int diag_blocks(int64_t T);
hipError_t launch_diagnostics(const DiagParams& p, hipStream_t stream);

// ---- combine -------------------------------------------------------------------
struct CombineParams {
  const void* y_rows;        // [*, d] float32, or bf16 with rows_bf16
  const int32_t* dest;       // [T,k]
  const float* gate;         // [T,k]
  const void* y_shared;      // [S,T,d] (the dtype of y_rows) or null
  void* y;                   // [T,d]
  int T, d, k, S;
  int out_bf16;
  int rows_bf16 = 0;         // expert rows in bf16 (a bf16 layer call's own rows)
};
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

struct StatsParams {
  const int32_t* counts;     // [E]
  const float* prob_sum;     // [E]
  float* stats;              // [2E+2]
  const int32_t* dest;       // [T,k]: when set, the drop rate counts dest < 0
  int T, k, E, C;
};
hipError_t launch_stats(const StatsParams& p, hipStream_t stream);

// ---- backward --------------------------------------------------------------------
struct BwdParams {
  const float* dy;           // [T,d] upstream gradient of the layer output
  const float* y_rows;       // [rows_bound, d] routed expert outputs (forward)
  const int32_t* dest;       // [T,k]
  const int32_t* idx;        // [T,k]
  const float* gate;         // [T,k]
  const float* logits;       // [T,E]
  const int32_t* counts;     // [E] routed (primary) counts
  const float* eps;          // [T,E] noise, or null
  const float* noise_pre;    // [T,E] x W_noise^T, or null
  float* dg;                 // [T,k] out: gate gradients
  float* dH;                 // [T,E] out: logit gradients
  float* dHn;                // [T,E] out: gradients of x W_noise^T, or null
  const float* dx_rows;      // [rows_bound + S*T, d] expert input gradients
  float* dx;                 // [T,d] out
  float g_aux, g_z;          // weights of L_aux and the z-loss
  float inv_f_den;           // f_e = counts[e] * inv_f_den
  int64_t rows_bound;
  int T, d, E, k, S;
  // expert-choice routing: slot [T,E] (row of (t,e) or -1) and scores [T,E]
  // replace dest / idx / gate, and dg is [T,E] (dS)
  int ec;
  const int32_t* slot;
  const float* scores;
};
hipError_t launch_row_gate(const int32_t* dest, const float* gate, int64_t n, float* row_gate,
                           hipStream_t stream);
hipError_t launch_ec_row_gate(const int32_t* slot, const float* scores, int64_t n,
                              float* row_gate, hipStream_t stream);
// gate gradients, then the logit gradients
hipError_t launch_router_backward(const BwdParams& p, hipStream_t stream);
int router_wgrad_splits(int64_t T, int64_t E, int64_t d);
// out[E,d] = G^T x with G [T,E] float32; partial: [splits, E, d] scratch
hipError_t launch_router_wgrad(const float* G, const void* x, int bf16, int T, int E, int d,
                               float* partial, float* out, hipStream_t stream);
hipError_t launch_column_sum(const float* G, int T, int E, float* out, hipStream_t stream);
hipError_t launch_to_bf16(const float* src, int64_t n, uint16_t* dst, hipStream_t stream);
// dst[g][c][coff + r] = src[g][r][c], elements of esz bytes
hipError_t launch_transpose(const void* src, int groups, int R, int C, void* dst, int ld,
                            int coff, int esz, hipStream_t stream);
hipError_t launch_group_desc(const int32_t* offsets, int G, int S, int T, int64_t rows_bound,
                             GroupDesc* desc, int32_t* total, hipStream_t stream);
// Source addressing of the transposed weight-gradient operands (see GroupDesc).
struct PackParams {
  const GroupDesc* desc;     // [G+S]
  const int32_t* total;      // padded columns in use
  const int32_t* row_token;  // gathered sources: token of each routed row
  const float* row_gate;     // scale of each routed row, or null
  int G, S;
  int C;                     // features (rows of the transposed block)
  int64_t ld;                // source elements per row
  int coff;                  // first source column
  int gathered;              // source rows are tokens (x, dy), else row-space rows
};
hipError_t launch_pack_t(const PackParams& p, const void* src, int src_esz, void* dst,
                         int dst_esz, int64_t padded_bound, hipStream_t stream);
hipError_t launch_bias_grad(const PackParams& p, const void* src, int src_esz, float* db,
                            hipStream_t stream);
hipError_t launch_wgrad_f32(const float* At, const float* Bt, const GroupDesc* desc, int G,
                            int S, int M, int N, float* out, float* out_shared,
                            hipStream_t stream);
hipError_t launch_dx(const BwdParams& p, const void* w_g, const void* w_noise, int bf16,
                     hipStream_t stream);
int64_t wgrad_entries(int groups, int M);

}  // namespace moe
