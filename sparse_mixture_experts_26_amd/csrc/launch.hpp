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
  int T, d, E, k;
  int bf16;
};
constexpr int kRouteTokens = 16;  // tokens per routing block
inline int route_blocks(int64_t T) { return (int)((T + kRouteTokens - 1) / kRouteTokens); }
hipError_t launch_route(const RouteParams& p, hipStream_t stream);

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
};
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
  int act;                   // moe_act_t, or -1 for none (down projection)
  int bf16;                  // operand dtype
  TileEntry* entries;        // scratch for the tiled path
  int32_t* n_entries;        // scratch
};
int64_t ffn_max_entries(int64_t rows_bound, int G, int S, int T);
hipError_t launch_ffn(const FfnParams& p, hipStream_t stream);

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
  const float* y_rows;       // [*, d]
  const int32_t* dest;       // [T,k]
  const float* gate;         // [T,k]
  const float* y_shared;     // [S,T,d] or null
  void* y;                   // [T,d]
  int T, d, k, S;
  int out_bf16;
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

}  // namespace moe
