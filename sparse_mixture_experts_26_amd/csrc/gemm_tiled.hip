// Grouped expert GEMM for many rows per expert (prefill-shaped), bf16 MFMA.
//
// Each expert is an FFN with its own weights that runs once over the tokens
// routed to it ("Mixture-of-Experts & Sparse Model Scaling", Core Concepts;
// "Scaling Capacity via Sparse MoE Architectures", the layer groups tokens by
// expert).  Both operands are contiguous along the reduction axis (C = A B^T).
//
// Tile schedule: a one-block kernel turns the device-side group offsets into a
// list of (group, first row, rows, first output row) entries of at most 256
// rows, so no host synchronisation is needed.  The GEMM is persistent: one
// block per CU walks the tiles; the hardware hands block P to XCD P % 8, and
// XCD x owns an equal, contiguous range of the real tiles (cut by depth
// instead when a down projection's two shared experts run as one 2h-deep
// group), in which groups of 8 row tiles sweep the output columns together so
// the operand slabs of concurrent tiles are shared through that XCD's L2.
// Each round of an XCD's range goes to its blocks with the slot map turned by
// the round, whole tiles of odd rounds walk their reduction from its end (so
// a round begins on the slices of the shared operand rows that the previous
// round ended on, still in the L2 and the MALL), and in a tile of at most 128
// rows the 4 waves of the empty half only keep the barriers.
//
// Block tile: 256 rows x 256 weight rows, 8 waves (2 per SIMD, so one wave's
// stalls are covered by the other's MFMAs) in a 2x4 grid, each wave 128x64 as
// 4x2 tiles of v_mfma_f32_32x32x16_bf16 with float32 accumulators.  For the
// gated (SwiGLU) form the 256 weight rows are 128 rows of w1 and the same 128
// rows of w3, and every wave holds matching gate and up tiles, so
// silu(gate) * up is formed in registers.  Operands travel global -> LDS with
// direct-to-LDS buffer loads (no register staging) in 64-deep stages, so every
// row of a stage is one whole 128-byte line: the vector L1 then issues
// full-line requests, which move about a third more data per clock from L2
// than half-line ones.  A stage is four 16 KiB quarters (B rows 0-127 and
// 128-255, A rows 0-127 and 128-255) and the ring holds ten quarters (the
// whole 160 KiB), i.e. 2.5 stages.  One wave per SIMD (waves 0-3) issues all
// of a block's loads: a wave whose load issue stalls in the memory pipeline
// cannot issue its MFMAs, so the other wave of each SIMD never loads and keeps
// the matrix core fed (about 4% faster than every wave loading its share).
// The loading waves wait for their loads; a plain s_barrier publishes a
// stage.  The 16-byte chunks of every 128-byte LDS row are XOR-swizzled by row
// so the MFMA operand reads are bank-conflict-free.
// Routed rows are gathered from the token matrix through row_token, which
// removes the separate permuted copy from the layer.  The epilogue stages each
// wave's results through LDS and stores 16-byte row chunks.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"

namespace moe {

namespace {

constexpr int BM = 256;      // output rows per tile
constexpr int BR = 256;      // weight rows per tile
constexpr int BK = 64;       // reduction depth per stage (one 128-byte line per row)
constexpr int kThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kGroupM = 8;   // row-tiles that sweep the columns together
constexpr int kQuarter = 128 * BK * 2;  // 128 rows of one operand, 16 KiB
constexpr int kSlots = 10;              // ring of quarters: the whole 160 KiB

// Kept out of line so the fully unrolled epilogue stays small enough to keep
// every accumulator in registers.
__device__ __noinline__ float gelu_outlined(float a) { return gelu_f32(a); }

// Slot of 16-byte chunk kc (0..7) of a 128-byte LDS row: XOR with
// (r ^ r >> 3) & 7 of the row's low 5 bits, so any 8 aligned rows, and the even
// and the odd rows of any 16 aligned rows, hold a given chunk in distinct slots:
// bank-conflict-free operand reads whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle.  Fragment rows are 32-aligned, so the swizzle depends
// on the lane only.
__device__ __forceinline__ int swz(int row) { return (row ^ ((row & 31) >> 3)) & 7; }

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// [K][N] weight quarters: 16-byte chunk c of row k sits at slot
// bt_swz(c) ^ 2 (k mod 4) of its 256-byte row.  A transpose read's 16 lanes
// take 4 rows x 32 bytes (chunks c, c+1, c even): the 2 (k mod 4) term puts
// the 4 rows in distinct 32-byte slots of 128 bytes, and bt_swz (chunk bit 1
// copied into bit 3; an involution) puts the other 16 lanes read with them
// (chunks c+2, c+3, same rows) into the other 128 bytes.
__device__ __forceinline__ int bt_swz(int c) { return c ^ (((c >> 1) & 1) << 3); }

// s_waitcnt with vmcnt = N (gfx9 encoding: vmcnt bits [3:0] and [15:14]) and
// the expcnt / lgkmcnt fields at their maxima, i.e. not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

// Tile t of a launch -> its schedule entry and column block: groups of
// kGroupM row tiles sweep the output columns together.
__device__ __forceinline__ void tile_coords(int t, int n_entries, int n_tiles_n, int& e_idx,
                                            int& n_idx) {
  const int per_group = kGroupM * n_tiles_n;
  const int grp = t / per_group, rem = t - grp * per_group;
  const int gsize = min(kGroupM, n_entries - grp * kGroupM);
  e_idx = grp * kGroupM + rem % gsize;
  n_idx = rem / gsize;
}

// Tail split.  With tiles = w P + r on P persistent blocks, the last round
// holds only r tiles and leaves P - r blocks idle.  When 2r <= P each of those
// tiles is cut into parts (2, or 3 when 3r <= P) of its reduction that run on
// different blocks, so the launch takes w + 1/2 (1/3) tile times instead of
// w + 1.  Tiles [0, full) run whole; unit u (0 <= u < units) is part u % parts
// of tile full + u / parts, part q covering stages [q nk / parts, (q+1) nk /
// parts).  Float32 outputs: part 0 writes the output, the others float32
// partials that split_fixup_kernel adds in part order.  The gated up
// projection (whose epilogue needs the whole sum) uses two parts, both writing
// float32 partials, which split_act_fixup_kernel adds before bias and
// activation.  The scratch holds two partial blocks per split tile.
// The gated form writes and re-reads two float32 partial blocks per split
// tile, four times the bytes of its bf16 output, so it splits only tiles of
// at least 48 reduction stages, where half a tile saves more than that
// traffic costs (a 2048-deep reduction measured 0.6% slower split, a
// 4096-deep one 0.8% faster).
struct SplitPlan {
  int full, units, parts;
};
constexpr int kGatedSplitStages = 48;
__device__ __forceinline__ SplitPlan split_plan(int tiles, int P, int nk, int cap, bool gated) {
  const int w = tiles / P, r = tiles - w * P;
  if (r > 0 && 2 * r <= P && r <= cap && nk >= (gated ? kGatedSplitStages : 2)) {
    const int parts = (!gated && 3 * r <= P && nk >= 3) ? 3 : 2;
    return {w * P, parts * r, parts};
  }
  return {tiles, 0, 1};
}

// ACT: moe_act_t for the up projection (2 = gated SwiGLU), -1 for none
// (float32 output); kActBwd + a: the down projection's input gradient with
// the backward of activation a applied in the epilogue; kActWgrad: the
// per-group weight gradient, whose reduction runs over the group's rows.
//
// Persistent: one block per CU walks tiles.  XCD x (the hardware hands block
// P to XCD P % 8) owns the contiguous tile range [x*per, (x+1)*per) with
// per = ceil(tiles / 8), read from the device-side schedule, so every XCD gets
// an equal share of real tiles and neighbouring tiles share an L2.  Float32
// outputs (act -1) and the gated up projection may split the last round's
// tiles (split_plan): each XCD then also owns a contiguous range of the
// split units, run after its whole tiles, and a fixup kernel finishes them.
//
// BT: the weights are stored [K][N] per group (output columns contiguous:
// w_main / w_shared of group g hold row k at k*N; with p.kh > 0 rows k >= kh
// come from the second set u_main / u_shared, row k - kh), as the backward's
// input gradients find them (W2 for the down projection, W1 and W3 for the up
// projections), so no transposed copy is made.  A weight quarter then holds
// 64 rows of k, each 128 columns (256 bytes) wide, loaded as whole lines; the
// MFMA operand (8 consecutive k of one column per lane) comes from two LDS
// transpose reads (ds_read_b64_tr_b16: within each 16 lanes, lane j gives 4
// consecutive columns of row k0 + j/4 at column 4(j%4), and lane i receives
// column i of rows k0..k0+3).  The 16-byte chunks of row k are XOR-swizzled by
// 2 (k mod 4), so the 4 rows of a read hit distinct banks.
template <int ACT, bool BT = false>
__global__ __launch_bounds__(kThreads, 1) void ffn_tiled_kernel(FfnParams p, int n_tiles_n) {
  constexpr bool GATED = ACT == 2;
  constexpr bool WGRAD = ACT == kActWgrad;
  static_assert(!BT || (!GATED && !WGRAD), "[K][N] weights: plain or backward forms only");
  __shared__ __attribute__((aligned(16))) char L[kSlots * kQuarter];
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform per wave; say so, or LDS-destination and buffer
  // resource operands that depend on it become per-lane (waterfall) loops
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;  // 2 x 4 waves: 128 rows x 64 weight rows each
  const int lr = lane & 31, lh = lane >> 5;
  const int n_entries = *p.n_entries;
  const int tiles = n_entries * n_tiles_n;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3, nq = (gridDim.x + 7 - xcd) >> 3;
  // weight gradients: tiles differ in depth, so the XCD ranges balance work
  // (computed with the schedule); otherwise equal tile counts
  // (the GELU / ReLU forms would spill registers with a split epilogue)
  constexpr bool SPLITS = ACT == -1 || ACT == 2;
  const SplitPlan plan = SPLITS && p.split
                             ? split_plan(tiles, gridDim.x, (p.K + BK - 1) / BK, p.split_cap, GATED)
                             : SplitPlan{tiles, 0, 1};
  const int per = (plan.full + 7) >> 3;
  int t_begin = WGRAD ? p.xcd_bounds[xcd] : xcd * per;
  int t_end = WGRAD ? p.xcd_bounds[xcd + 1] : min(plan.full, (xcd + 1) * per);
  if (ACT == -1 && !BT && p.shared_cat == 2) {
    // the routed tiles come first and the concatenated shared group's last,
    // each of those twice as deep: the XCD ranges are cut by depth, not
    // count (the launch does not split its tail)
    const int ts = ((p.T + BM - 1) / BM) * n_tiles_n, tr = tiles - ts;
    const int64_t ctot = tr + 2 * (int64_t)ts;
    auto at = [&](int x) {
      const int64_t c = ctot * x / 8;
      return (int)(c <= tr ? c : tr + (c - tr + 1) / 2);
    };
    t_begin = at(xcd);
    t_end = at(xcd + 1);
  }
  const int per_h = (plan.units + 7) >> 3;
  const int h_begin = xcd * per_h, h_end = min(plan.units, (xcd + 1) * per_h);
  // Round r of the XCD's range is its tiles [r nq, (r+1) nq); this block
  // takes slot (q + r) mod nq of it.  The slot turns with the round because a
  // row-tile group's tiles cycle through its entries, so a fixed slot would
  // give one block the same entry in every round, and the cheap tiles of a
  // partly filled entry would all land on the same few blocks.
  const int span = max(0, t_end - t_begin), full_r = span / nq, rem_r = span - full_r * nq;
  const int n_whole = full_r + ((q + full_r) % nq < rem_r ? 1 : 0);
  const int N = p.N;
  constexpr uint32_t kOOB = 0x80000000u;

  // Operand reads.  Quarter layout: rows of 128 bytes, chunk c of row r at
  // r*128 + ((c ^ swz(r)) << 4).  Sub-step s (16 deep) reads chunk 2s + lh.
  // the chunk field is bits 4-6 and the row bits 7+, so sub-step s's offset
  // is rd0 ^ (s << 5)
  const int rd0 = lr * 128 + ((lh ^ swz(lr)) << 4);
  // quarter (0 B rows 0-127, 1 B rows 128-255, 2 A rows 0-127, 3 A rows
  // 128-255) and row inside it of this wave's fragments.  The weights come
  // first: they stream from HBM, while the token rows are re-read by every
  // column sweep and mostly hit the MALL, so the weights get the longer
  // lookahead (their quarters are issued two steps ahead, the token rows' one).
  const int qa = 2 + wm;
  int qb[2], rb[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int br = GATED ? ni * 128 + wn * 32 : wn * 64 + ni * 32;
    qb[ni] = br >> 7;
    rb[ni] = br & 127;
  }
  // BT: byte offsets, inside a weight quarter and before the sub-step's
  // 16 rows (s * 4096), of this lane's two transpose reads per fragment
  int tr_off[2][2];
  if constexpr (BT) {
    const int g16 = lane >> 4, j = lane & 15;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k = 8 * (g16 >> 1) + 4 * t + (j >> 2);   // row inside the sub-step
        const int n = rb[ni] + 16 * (g16 & 1) + 4 * (j & 3);  // column inside the quarter
        tr_off[ni][t] = k * 256 + ((bt_swz(n >> 3) ^ (2 * (j >> 2))) << 4) + (n & 7) * 2;
      }
  }

  for (int it = 0;; ++it) {
    // this block's whole tiles, then its split units
    int t, half = -1;  // -1: whole tile; else the part of its reduction
    if (it < n_whole) {
      t = t_begin + it * nq + (q + it) % nq;
    } else {
      const int u = h_begin + q + (it - n_whole) * nq;
      if (u >= h_end) break;
      t = plan.full + u / plan.parts;
      half = u - (t - plan.full) * plan.parts;
    }
    int e_idx, n_idx;
    tile_coords(t, n_entries, n_tiles_n, e_idx, n_idx);
    const TileEntry te = p.entries[e_idx];
    const bool routed = te.group < p.G;
    const int gw = routed ? te.group : te.group - p.G;
    // the shared group of a down projection over 2 shared experts in turn
    const bool cat = ACT == -1 && !BT && !routed && p.shared_cat == 2;
    const int ldk = p.K;                // row stride of both operands
    int K = cat ? 2 * p.K : p.K;        // reduction depth of this tile
    int64_t wstride = (int64_t)N * K;
    const uint16_t* W;
    const uint16_t* U;
    const uint16_t* A;
    if constexpr (WGRAD) {
      // the group's blocks of the transposed operands: M (resp. N) feature
      // rows of kp elements each
      const GroupDesc gd = p.gdesc[te.group];
      K = gd.kp;
      wstride = (int64_t)N * K;
      A = static_cast<const uint16_t*>(p.a_main) + (int64_t)p.M * gd.poff;
      W = static_cast<const uint16_t*>(p.w_main) + (int64_t)N * gd.poff;
      U = W;
    } else {
      // BT with a second weight set: each set holds kh rows of N per group
      const int64_t gstride = (BT && p.kh > 0) ? (int64_t)N * p.kh : wstride;
      W = static_cast<const uint16_t*>(routed ? p.w_main : p.w_shared) + gw * gstride;
      U = W;
      if (GATED || (BT && p.kh > 0))
        U = static_cast<const uint16_t*>(routed ? p.u_main : p.u_shared) + gw * gstride;
      A = static_cast<const uint16_t*>(routed ? p.a_main : p.a_shared);
    }
    const int nk = (K + BK - 1) / BK;
    // stages [kb, kb + nks) of the reduction; chunks at or past k_end read zeros
    const int kb = half < 0 ? 0 : half * nk / plan.parts;
    const int ke = half < 0 ? nk : (half + 1) * nk / plan.parts;
    const int nks = ke - kb;
    const int k_end = ke == nk ? K : ke * BK;
    // whole tiles of odd rounds walk their reduction from the end, so they
    // start on the operand slices the previous round of the XCD ended on,
    // which the L2 and the MALL still hold
    const bool k_rev = half < 0 && (it & 1);
    const int n_out0 = n_idx * (GATED ? BR / 2 : BR);
    // Waves 4-7 compute tile rows 128-255 and issue no loads: in a tile of at
    // most 128 rows (the partly filled last row tile of a group) they only
    // keep the tile's barriers (one before the prologue, one per stage, one
    // before the epilogue), which halves its MFMA work.  (Not in the [K][N]
    // forms, the backward's few-row input gradients, whose registers are full.)
    if (!BT && wm == 1 && te.rows <= 128) {
      for (int st = 0; st < nks + 2; ++st) asm volatile("s_barrier" ::: "memory");
      continue;
    }

    // ---- direct-to-LDS loads.  A quarter is 16 loads of 1 KiB (8 rows x 128
    // bytes, whole cache lines); loading wave w (0-3) fills rows 16w .. 16w+15
    // and 16(w+4) .. 16(w+4)+15 of every quarter with four loads (load j fills
    // the 8-row slot (w + 4 (j/2)) * 2 + j%2).  Lane i fills row i/8, chunk
    // slot i%8 of its load, so it fetches the chunk the swizzle stores there.  Buffer resources return
    // zeros past their end: rows past the tile, weight rows past N and chunks
    // past K need no branches.
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(A), (short)0, 0x7fffffff, 0x00020000);
    // bytes of one group's weight set (BT with a second set: kh rows each)
    const int wbytes = (int)((BT && p.kh > 0 ? (int64_t)N * p.kh : wstride) * 2);
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W), (short)0, wbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t u_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(U), (short)0, wbytes, 0x00020000);
    uint32_t off[4][4];  // [quarter][load]
    int l_kc[4];
    int l_kq[4];  // BT: row (k) inside the stage of this lane's weight loads
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rq = (((wid & 3) + 4 * (j >> 1)) * 2 + (j & 1)) * 8 + (lane >> 3);  // row inside a quarter
      const int kc = (lane & 7) ^ swz(rq);
      l_kc[j] = kc;
      // BT: load j fills rows 4b .. 4b+3 of the stage, 256 bytes each, b the
      // same 1 KiB block index; lane i takes row 4b + i/16 and the chunk that
      // the row's swizzle stores at slot i%16
      const int kq = ((((wid & 3) + 4 * (j >> 1)) * 2 + (j & 1)) << 2) + (lane >> 4);
      const int gc = bt_swz((lane & 15) ^ (2 * (kq & 3)));
      l_kq[j] = kq;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = h * 128 + rq;  // tile row
        const bool ok = row < te.rows;
        int arow = (p.a_from_c && !cat) ? te.c_row0 + row : te.a_row0 + row;
        if (ok && routed && p.gather && !p.a_from_c) arow = p.gather[arow];
        off[2 + h][j] = ok ? ((uint32_t)arow * (uint32_t)(WGRAD ? K : ldk) + kc * 8) * 2u : kOOB;
        if constexpr (BT) {
          const int n = n_out0 + h * 128 + 8 * gc;
          off[h][j] = n < N ? ((uint32_t)kq * (uint32_t)N + n) * 2u : kOOB;
        } else {
          const int n = n_out0 + (GATED ? rq : row);
          off[h][j] = n < N ? ((uint32_t)n * (uint32_t)(WGRAD ? K : ldk) + kc * 8) * 2u : kOOB;
        }
      }
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

    // quarter qq (0..3) of stage kt into ring slot `slot`; stages past the
    // end read zeros
    auto issue = [&](int slot, int qq, int kt) __attribute__((always_inline)) {
      const int k0 = (k_rev && kt < nks ? ke - 1 - kt : kb + kt) * BK;
      __amdgpu_buffer_rsrc_t rs = qq >= 2 ? a_rs : (GATED && qq == 1 ? u_rs : w_rs);
      // BT weight quarters: stage rows k0.. of the set holding them
      int kset = k0;
      if (BT && qq < 2 && p.kh > 0 && k0 >= p.kh) {
        rs = u_rs;
        kset = k0 - p.kh;
      }
      // the second shared expert of a concatenated group: its operand rows
      // are T rows further on, its weights N rows
      uint32_t kbase = (uint32_t)k0 * 2u;
      if (cat && k0 >= ldk)
        kbase = (uint32_t)(k0 - ldk) * 2u + (uint32_t)(qq >= 2 ? p.T : N) * (uint32_t)ldk * 2u;
      if (wid < 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t kadd;
          if (BT && qq < 2)
            kadd = (k0 + l_kq[j] < k_end) ? (uint32_t)kset * (uint32_t)N * 2u : kOOB;
          else
            kadd = (k0 + l_kc[j] * 8 < k_end) ? kbase : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, MOE_LDS(L + slot * kQuarter + ((wid + 4 * (j >> 1)) * 2 + (j & 1)) * 1024), 16,
              off[qq][j] + kadd, 0, 0, 0);
        }
      }
    };
    struct Frags { bf16x8 a[4], b[2]; };
    // sub-step s of the stage whose quarters start at ring slot base
    auto read = [&](Frags& f, int base, int s) __attribute__((always_inline)) {
      // opaque per step, so the slot addresses are formed here (one add per
      // operand) instead of being kept live across the loop for every slot
      int r = rd0;
      asm volatile("" : "+v"(r));
      r ^= s << 5;
      const int sa = base + qa, sb0 = base + qb[0], sb1 = base + qb[1];
      const char* pa = L + (sa >= kSlots ? sa - kSlots : sa) * kQuarter + r;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) f.a[mi] = *reinterpret_cast<const bf16x8*>(pa + mi * 32 * 128);
      if constexpr (BT) {
        // two transpose reads give the 8 consecutive k of one column
        typedef short v4i16 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int sb = ni == 0 ? sb0 : sb1;
          const char* qp = L + (sb >= kSlots ? sb - kSlots : sb) * kQuarter + s * 4096;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)MOE_LDS(qp + tr_off[ni][0]));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)MOE_LDS(qp + tr_off[ni][1]));
          f.b[ni] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      } else {
        f.b[0] = *reinterpret_cast<const bf16x8*>(L + (sb0 >= kSlots ? sb0 - kSlots : sb0) * kQuarter + rb[0] * 128 + r);
        f.b[1] = *reinterpret_cast<const bf16x8*>(L + (sb1 >= kSlots ? sb1 - kSlots : sb1) * kQuarter + rb[1] * 128 + r);
      }
    };
    auto mfma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
    };
    auto barrier = [&]() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };

    // Pipeline.  The ring holds 2.5 stages: quarters are loaded in the order
    // (stage, quarter) and quarter j of that order goes to slot j % 10.  Step
    // kt waits for the loads of stage kt (a loading wave's 8 loads of stage
    // kt+1's first half may stay in flight; the other waves have none); the
    // barrier publishes stage kt and frees the slots of stage kt-1, which take
    // stage kt+1's second half and stage kt+2's first half.  Every wave has completed its reads of stage kt-1
    // before the barrier (lgkmcnt 0): the last 16-deep sub-step of each stage
    // is read before the barrier and multiplied after it, so the MFMAs cover
    // the first read of the next stage.  Every step issues its loads, past the
    // end too (they read zeros), so the wait counts are fixed.
#define MOE_PATTERN()                                                    \
  {                                                                      \
    _Pragma("unroll") for (int i = 0; i < 32; ++i) {                     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 \
      if ((i & 7) < (BT ? 8 : 6)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); \
      if ((i & 3) == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); \
    }                                                                    \
  }
#define MOE_STEP(B, kt)                                        \
  {                                                            \
    wait_vmcnt<8>();                                           \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0) */        \
    barrier();                                                 \
    issue(((B) + 6) % kSlots, 2, (kt) + 1);                    \
    issue(((B) + 7) % kSlots, 3, (kt) + 1);                    \
    issue(((B) + 8) % kSlots, 0, (kt) + 2);                    \
    issue(((B) + 9) % kSlots, 1, (kt) + 2);                    \
    read(f0, (B), 0);                                          \
    mfma(f1);                                                  \
    read(f1, (B), 1);                                          \
    mfma(f0);                                                  \
    read(f0, (B), 2);                                          \
    mfma(f1);                                                  \
    read(f1, (B), 3);                                          \
    mfma(f0);                                                  \
    MOE_PATTERN()                                              \
  }
    Frags f0, f1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) f1.a[mi] = bf16x8{};
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) f1.b[ni] = bf16x8{};
    barrier();  // the previous tile's epilogue is done with the ring
    issue(0, 0, 0);
    issue(1, 1, 0);
    issue(2, 2, 0);
    issue(3, 3, 0);
    issue(4, 0, 1);
    issue(5, 1, 1);
    int kt = 0;
    for (; kt + 5 <= nks; kt += 5) {
      MOE_STEP(0, kt)
      MOE_STEP(4, kt + 1)
      MOE_STEP(8, kt + 2)
      MOE_STEP(2, kt + 3)
      MOE_STEP(6, kt + 4)
    }
    if (kt < nks) MOE_STEP(0, kt)
    if (kt + 1 < nks) MOE_STEP(4, kt + 1)
    if (kt + 2 < nks) MOE_STEP(8, kt + 2)
    if (kt + 3 < nks) MOE_STEP(2, kt + 3)
#undef MOE_STEP
#undef MOE_PATTERN
    mfma(f1);  // the last sub-step
    // loads issued past the end (zeros) land before the LDS is reused
    wait_vmcnt<0>();

    // ---- epilogue.  32x32 result layout: lane holds column lane%32, rows
    // 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15.  Each wave stages its block
    // through a private 16 KiB LDS region (rows padded by 16 bytes so the two
    // lane halves, 4 rows apart, hit different banks) and writes it back as
    // 16-byte row chunks, instead of 2-byte scattered stores.  A wave's LDS
    // operations complete in order, so only the barrier that frees the ring is
    // needed.
    barrier();
    const float* bias = routed ? p.bias_main : p.bias_shared;
    // Up projections write the bf16 hidden layer (and the bf16 pre-activations
    // when asked); every other form stages float32 (the host only selects this
    // kernel for bf16 layers).
    constexpr bool FWD_ACT = ACT >= 0 && ACT <= 2;
    constexpr bool BWD_ACT = ACT >= kActBwd && ACT <= kActBwd + 2;
    constexpr int NJ = GATED ? 1 : 2;            // 32-column blocks per wave
    constexpr int COLS = NJ * 32;                // columns per wave
    char* const region = L + wid * 16384;
    const int col0 = n_out0 + (GATED ? wn * 32 : wn * 64);  // first column of the wave block
    float bcol[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      const int c = col0 + nj * 32 + lr;
      bcol[nj] = (bias && c < N) ? bias[(int64_t)gw * N + c] : 0.f;
    }
    // value(mi, nj, v) of every accumulator -> LDS (bf16 when `bf` holds
    // true, else float32), then store(row, col, chunk) for every 16-byte row
    // chunk inside the tile
    auto emit = [&](auto bf, auto value, auto store) __attribute__((always_inline)) {
      constexpr bool OUT_BF16 = decltype(bf)::value;
      constexpr int esz = OUT_BF16 ? 2 : 4;
      constexpr int row_bytes = COLS * esz + 16;
      constexpr int rows_pass = (128 * row_bytes <= 16384) ? 128 : (64 * row_bytes <= 16384 ? 64 : 32);
      static_assert(rows_pass * row_bytes <= 16384, "staging block exceeds the wave's region");
#pragma unroll
      for (int pass = 0; pass < 128 / rows_pass; ++pass) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          if ((mi * 32) / rows_pass != pass) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = (mi * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) % rows_pass;
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) {
              const float o = value(mi, nj, v);
              char* dst = region + r * row_bytes + (nj * 32 + lr) * esz;
              if (OUT_BF16) *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(o);
              else *reinterpret_cast<float*>(dst) = o;
            }
          }
        }
        // LDS -> global in 16-byte chunks (row-contiguous across lanes)
        constexpr int chunks_row = COLS * esz / 16;
        constexpr int chunks = rows_pass * chunks_row;
        for (int c = lane; c < chunks; c += 64) {
          const int r = c / chunks_row, ch = c - r * chunks_row;
          const int row = wm * 128 + pass * rows_pass + r;
          const int colc = col0 + ch * (16 / esz);
          if (row >= te.rows || colc >= N) continue;
          store(row, colc, *reinterpret_cast<const u32x4*>(region + r * row_bytes + ch * 16));
        }
      }
    };
    const int64_t crow0 = te.c_row0;
    using Bf16 = std::integral_constant<bool, true>;
    using F32 = std::integral_constant<bool, false>;
    if (GATED && half >= 0) {
      // half of a split tile: the raw float32 sums, tile-local rows of BR
      // values (the 128 gate columns, then the 128 up columns)
      float* part = p.split + ((int64_t)(t - plan.full) * 2 + half) * (BM * BR);
#pragma unroll
      for (int set = 0; set < (GATED ? 2 : 1); ++set)
        emit(F32{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][GATED ? set : nj][v]; },
             [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
               *reinterpret_cast<u32x4*>(part + row * BR + set * (BR / 2) + (colc - n_out0)) = ch;
             });
    } else if constexpr (FWD_ACT) {
      uint16_t* out = static_cast<uint16_t*>(p.out);
      emit(Bf16{},
          [&](int mi, int nj, int v) __attribute__((always_inline)) {
            if (GATED) return silu_f32(acc[mi][0][v] + bcol[0]) * acc[mi][1][v];
            float o = acc[mi][nj][v] + bcol[nj];
            if (ACT == 0) o = gelu_outlined(o);
            if (ACT == 1) o = fmaxf(o, 0.f);
            return o;
          },
          [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
            __builtin_nontemporal_store(ch, reinterpret_cast<u32x4*>(out + (crow0 + row) * N + colc));
          });
      if (p.pre) {
        // pre-activations for the backward: u (+ bias), then v when gated
        uint16_t* pre = static_cast<uint16_t*>(p.pre);
        const int64_t ld = GATED ? 2 * (int64_t)N : N;
        emit(Bf16{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v] + bcol[nj]; },
             [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
               *reinterpret_cast<u32x4*>(pre + (crow0 + row) * ld + colc) = ch;
             });
        if (GATED)
          emit(Bf16{}, [&](int mi, int, int v) __attribute__((always_inline)) { return acc[mi][1][v]; },
               [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
                 *reinterpret_cast<u32x4*>(pre + (crow0 + row) * ld + N + colc) = ch;
               });
      }
    } else if constexpr (BWD_ACT) {
      // da = gate * (dy W2) per row; du (and dv) from the saved pre-activations
      constexpr bool SWI = ACT == kActBwd + 2;
      const int64_t ld = SWI ? 2 * (int64_t)N : N;
      const uint16_t* pre = static_cast<const uint16_t*>(p.pre);
      uint16_t* out = static_cast<uint16_t*>(p.out);
      emit(F32{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v]; },
           [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
             const int64_t r = crow0 + row;
             const float g = routed ? p.row_gate[r] : 1.f;
             const f32x4 da = __builtin_bit_cast(f32x4, ch);
             const u32x2 uu = *reinterpret_cast<const u32x2*>(pre + r * ld + colc);
             u32x2 vv = {0u, 0u};
             if (SWI) vv = *reinterpret_cast<const u32x2*>(pre + r * ld + N + colc);
             float du[4], dv[4];
#pragma unroll
             for (int j = 0; j < 4; ++j) {
               const uint32_t wu = uu[j >> 1], wv = vv[j >> 1];
               const float u = bf16_to_f32((uint16_t)(j & 1 ? wu >> 16 : wu & 0xffffu));
               const float v = bf16_to_f32((uint16_t)(j & 1 ? wv >> 16 : wv & 0xffffu));
               act_backward(ACT - kActBwd, da[j] * g, u, v, du[j], dv[j]);
             }
             u32x2 o;
             o[0] = f32_to_bf16(du[0]) | ((uint32_t)f32_to_bf16(du[1]) << 16);
             o[1] = f32_to_bf16(du[2]) | ((uint32_t)f32_to_bf16(du[3]) << 16);
             *reinterpret_cast<u32x2*>(out + r * ld + colc) = o;
             if (SWI) {
               o[0] = f32_to_bf16(dv[0]) | ((uint32_t)f32_to_bf16(dv[1]) << 16);
               o[1] = f32_to_bf16(dv[2]) | ((uint32_t)f32_to_bf16(dv[3]) << 16);
               *reinterpret_cast<u32x2*>(out + r * ld + N + colc) = o;
             }
           });
    } else if (ACT == -1 && !BT && p.out_bf16 && half >= 0) {
      // a part of a split tile with a bf16 output: every part writes its
      // float32 sums (no bias), tile-local rows of BR values, one block per
      // part; split_bf16_fixup_kernel adds them and rounds
      float* part = p.split + ((int64_t)(t - plan.full) * 3 + half) * (BM * BR);
      emit(F32{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v]; },
           [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
             *reinterpret_cast<u32x4*>(part + row * BR + (colc - n_out0)) = ch;
           });
    } else if (SPLITS && half >= 1) {
      // a later part of a split tile: float32 partials (no bias), tile-local
      // rows of BR values
      float* part = p.split + ((int64_t)(t - plan.full) * 2 + half - 1) * (BM * BR);
      emit(F32{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v]; },
           [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
             *reinterpret_cast<u32x4*>(part + row * BR + (colc - n_out0)) = ch;
           });
    } else if (ACT == -1 && !BT && p.out_bf16) {
      // bf16 rows of a down projection (a layer call's expert outputs, read
      // once by its combine), bias added before the one rounding
      uint16_t* out = static_cast<uint16_t*>(p.out);
      emit(Bf16{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v] + bcol[nj]; },
           [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
             __builtin_nontemporal_store(ch, reinterpret_cast<u32x4*>(out + (crow0 + row) * N + colc));
           });
    } else {
      // float32 rows (down projection, input gradients) or weight gradients,
      // all written once for a later launch (or the caller): non-temporal
      float* out = static_cast<float*>(WGRAD && !routed ? p.out_shared : p.out);
      emit(F32{}, [&](int mi, int nj, int v) __attribute__((always_inline)) { return acc[mi][nj][v] + bcol[nj]; },
           [&](int row, int colc, const u32x4& ch) __attribute__((always_inline)) {
             f32x4* dst = reinterpret_cast<f32x4*>(out + (crow0 + row) * N + colc);
             f32x4 val = __builtin_bit_cast(f32x4, ch);
             if (p.accumulate) val += *dst;
             __builtin_nontemporal_store(val, dst);
           });
    }
  }
}

// Weight-gradient schedule: every group (routed, then shared) gets the row
// tiles of its M x N output, whatever its number of rows (a group without
// rows gets zeros).  A tile's depth is its group's padded row count, so the
// 8 XCD ranges are cut where the running work (stages + a fixed per-tile
// cost) crosses each eighth: a heavily loaded expert spreads over several
// XCDs instead of holding one back.  One block.
constexpr int kMaxGroups = 512;  // routed + shared groups a schedule may hold

__global__ __launch_bounds__(256) void build_wgrad_tiles_kernel(int groups, int G, int M,
                                                                int n_tiles_n,
                                                                const GroupDesc* gdesc,
                                                                TileEntry* entries,
                                                                int32_t* n_entries,
                                                                int32_t* xcd_bounds) {
  __shared__ long long scan[256];
  const int tid = threadIdx.x;
  const int mt = (M + BM - 1) / BM;
  const int n = groups * mt;
  for (int i = tid; i < n; i += 256) {
    const int g = i / mt, m0 = (i - g * mt) * BM;
    TileEntry e;
    e.group = g;
    e.a_row0 = m0;
    e.rows = min(BM, M - m0);
    e.c_row0 = (g < G ? g : g - G) * M + m0;
    entries[i] = e;
  }
  const int tiles = n * n_tiles_n;
  __shared__ int s_kp[kMaxGroups];
  for (int g = tid; g < min(groups, kMaxGroups); g += 256) s_kp[g] = gdesc[g].kp / BK + 8;
  __syncthreads();
  // tile t -> its entry, as the GEMM decomposes it
  auto work = [&](int t) {
    int e_idx, n_idx;
    tile_coords(t, n, n_tiles_n, e_idx, n_idx);
    return (long long)s_kp[min(e_idx / mt, kMaxGroups - 1)];
  };
  // each thread a contiguous chunk of tiles: chunk sums, an exclusive scan
  // over the chunks, then every thread cuts inside its own chunk
  const int chunk = (tiles + 255) / 256;
  const int t0 = min(tiles, tid * chunk), t1 = min(tiles, t0 + chunk);
  long long part = 0;
  for (int t = t0; t < t1; ++t) part += work(t);
  scan[tid] = part;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const long long v = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const long long total = scan[255];
  long long run = scan[tid] - part;  // work before this chunk
  // XCD x starts at the first tile whose running work reaches x/8 of the total
  for (int t = t0; t < t1; ++t) {
    const long long before = run;
    run += work(t);
    for (int x = 1; x < 8; ++x)
      if (before * 8 < total * x && run * 8 >= total * x) xcd_bounds[x] = t + 1;
  }
  if (tid == 0) {
    xcd_bounds[0] = 0;
    xcd_bounds[8] = tiles;
    *n_entries = n;
  }
  // every tile weighs at least 8, so with tiles every eighth is crossed
  // exactly once above; without tiles every range is empty
  if (tiles == 0 && tid >= 1 && tid < 8) xcd_bounds[tid] = 0;
}

// Adds the later parts' partials of the split tiles into the float32 output,
// in part order (same plan as the GEMM with P of its blocks).  kFixParts
// blocks per split tile, 16 rows each; every thread issues its 4 chunks'
// loads (partials and output) before adding, so a block waits for memory
// once.  Runs after the GEMM on the same stream.
constexpr int kFixParts = 16;

__global__ __launch_bounds__(256) void split_fixup_kernel(FfnParams p, int n_tiles_n, int P) {
  const int n_entries = *p.n_entries;
  const SplitPlan plan = split_plan(n_entries * n_tiles_n, P, (p.K + BK - 1) / BK, p.split_cap, false);
  const int j = blockIdx.x / kFixParts, r0 = (blockIdx.x % kFixParts) * (BM / kFixParts);
  if (j * plan.parts >= plan.units) return;
  int e_idx, n_idx;
  tile_coords(plan.full + j, n_entries, n_tiles_n, e_idx, n_idx);
  const TileEntry te = p.entries[e_idx];
  const int n_out0 = n_idx * BR;
  float* out = static_cast<float*>(p.out);
  const float* part = p.split + (int64_t)(2 * j) * (BM * BR);
  const bool third = plan.parts == 3;
  constexpr int kChunks = BR / 4;  // float4 chunks per tile row
  constexpr int kPer = (BM / kFixParts) * kChunks / 256;
  f32x4 a[kPer], c3[kPer], b[kPer];
  f32x4* dst[kPer];
  bool ok[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + u * 256;
    const int row = r0 + i / kChunks, c = (i % kChunks) * 4;
    ok[u] = row < te.rows && n_out0 + c < p.N;
    dst[u] = reinterpret_cast<f32x4*>(out + (int64_t)(te.c_row0 + row) * p.N + n_out0 + c);
    if (ok[u]) {
      a[u] = *reinterpret_cast<const f32x4*>(part + row * BR + c);
      if (third) c3[u] = *reinterpret_cast<const f32x4*>(part + BM * BR + row * BR + c);
      b[u] = *dst[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (ok[u]) *dst[u] = third ? (b[u] + a[u]) + c3[u] : b[u] + a[u];
}

// The split tiles of a down projection with a bf16 output: out = ((part0 +
// part1) (+ part2)) + bias, rounded once, in part order (same plan as the
// GEMM with P of its blocks).  kFixParts blocks per split tile, 16 rows each;
// every thread issues its chunks' loads before adding.
__global__ __launch_bounds__(256) void split_bf16_fixup_kernel(FfnParams p, int n_tiles_n, int P) {
  const int n_entries = *p.n_entries;
  const SplitPlan plan = split_plan(n_entries * n_tiles_n, P, (p.K + BK - 1) / BK, p.split_cap, false);
  const int j = blockIdx.x / kFixParts, r0 = (blockIdx.x % kFixParts) * (BM / kFixParts);
  if (j * plan.parts >= plan.units) return;
  int e_idx, n_idx;
  tile_coords(plan.full + j, n_entries, n_tiles_n, e_idx, n_idx);
  const TileEntry te = p.entries[e_idx];
  const bool routed = te.group < p.G;
  const int gw = routed ? te.group : te.group - p.G;
  const float* bias = routed ? p.bias_main : p.bias_shared;
  const int n_out0 = n_idx * BR;
  uint16_t* out = static_cast<uint16_t*>(p.out);
  const float* part = p.split + (int64_t)(3 * j) * (BM * BR);
  const bool third = plan.parts == 3;
  constexpr int kChunks = BR / 4;  // float4 chunks per tile row
  constexpr int kPer = (BM / kFixParts) * kChunks / 256;
  f32x4 a[kPer], b[kPer], c3[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + u * 256;
    const int row = r0 + i / kChunks, c = (i % kChunks) * 4;
    a[u] = *reinterpret_cast<const f32x4*>(part + row * BR + c);
    b[u] = *reinterpret_cast<const f32x4*>(part + BM * BR + row * BR + c);
    if (third) c3[u] = *reinterpret_cast<const f32x4*>(part + 2 * BM * BR + row * BR + c);
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + u * 256;
    const int row = r0 + i / kChunks, c = (i % kChunks) * 4, col = n_out0 + c;
    if (row >= te.rows || col >= p.N) continue;
    f32x4 v = a[u] + b[u];
    if (third) v += c3[u];
    uint32_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float lo = v[2 * q], hi = v[2 * q + 1];
      if (bias) {
        lo += bias[(int64_t)gw * p.N + col + 2 * q];
        hi += bias[(int64_t)gw * p.N + col + 2 * q + 1];
      }
      w[q] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
    }
    u32x2 o;
    o[0] = w[0];
    o[1] = w[1];
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + (int64_t)(te.c_row0 + row) * p.N + col));
  }
}

// The split tiles of the gated up projection: out = silu(gate) * up in bf16
// with gate = part0 + part1 (+ bias) over the first 128 partial columns and
// up the same over the last 128, and the pre-activations when asked.  kFixParts blocks per split tile, 16
// rows each; a thread handles 4 consecutive output columns per row.
template <int ACT>
__global__ __launch_bounds__(256) void split_act_fixup_kernel(FfnParams p, int n_tiles_n, int P) {
  constexpr bool GATED = ACT == 2;
  constexpr int OC = GATED ? BR / 2 : BR;  // output columns of a tile
  const int n_entries = *p.n_entries;
  const SplitPlan plan = split_plan(n_entries * n_tiles_n, P, (p.K + BK - 1) / BK, p.split_cap, true);
  const int j = blockIdx.x / kFixParts, r0 = (blockIdx.x % kFixParts) * (BM / kFixParts);
  if (j * plan.parts >= plan.units) return;
  int e_idx, n_idx;
  tile_coords(plan.full + j, n_entries, n_tiles_n, e_idx, n_idx);
  const TileEntry te = p.entries[e_idx];
  const bool routed = te.group < p.G;
  const int gw = routed ? te.group : te.group - p.G;
  const float* bias = routed ? p.bias_main : p.bias_shared;
  const int n_out0 = n_idx * OC, N = p.N;
  const float* p0 = p.split + (int64_t)(2 * j) * (BM * BR);
  const float* p1 = p0 + BM * BR;
  uint16_t* out = static_cast<uint16_t*>(p.out);
  uint16_t* pre = static_cast<uint16_t*>(p.pre);
  const int64_t ld = GATED ? 2 * (int64_t)N : N;
  constexpr int kChunks = OC / 4;                             // per tile row
  constexpr int kPer = (BM / kFixParts) * kChunks / 256;      // per thread
  f32x4 a0[kPer], a1[kPer], u0[kPer], u1[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + u * 256;
    const int row = r0 + i / kChunks, c = (i % kChunks) * 4;
    a0[u] = *reinterpret_cast<const f32x4*>(p0 + row * BR + c);
    a1[u] = *reinterpret_cast<const f32x4*>(p1 + row * BR + c);
    if (GATED) {
      u0[u] = *reinterpret_cast<const f32x4*>(p0 + row * BR + OC + c);
      u1[u] = *reinterpret_cast<const f32x4*>(p1 + row * BR + OC + c);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + u * 256;
    const int row = r0 + i / kChunks, c = (i % kChunks) * 4, col = n_out0 + c;
    if (row >= te.rows || col >= N) continue;
    const int64_t r = te.c_row0 + row;
    uint16_t o[4], pa[4], pu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = a0[u][q] + a1[u][q];
      if (bias) a += bias[(int64_t)gw * N + col + q];
      float v;
      if (GATED) {
        const float up = u0[u][q] + u1[u][q];
        v = silu_f32(a) * up;
        pu[q] = f32_to_bf16(up);
      } else {
        v = ACT == 0 ? gelu_outlined(a) : fmaxf(a, 0.f);
      }
      pa[q] = f32_to_bf16(a);
      o[q] = f32_to_bf16(v);
    }
    auto pack = [](const uint16_t* h) {
      u32x2 w;
      w[0] = h[0] | ((uint32_t)h[1] << 16);
      w[1] = h[2] | ((uint32_t)h[3] << 16);
      return w;
    };
    __builtin_nontemporal_store(pack(o), reinterpret_cast<u32x2*>(out + r * N + col));
    if (pre) {
      *reinterpret_cast<u32x2*>(pre + r * ld + col) = pack(pa);
      if (GATED) *reinterpret_cast<u32x2*>(pre + r * ld + N + col) = pack(pu);
    }
  }
}

}  // namespace

int64_t ffn_split_cap(int64_t max_entries, int64_t N, bool wide) {
  // never more than half of a 256-block launch; never more than half the
  // tiles, or than all of them for a launch that may run on twice as many
  // blocks as tiles (and so split every tile)
  const int64_t tiles = max_entries * ((N + BR - 1) / BR);
  return std::min<int64_t>(128, wide ? tiles : (tiles + 1) / 2);
}

int64_t ffn_max_entries(int64_t rows_bound, int G, int S, int T) {
  return (rows_bound + BM - 1) / BM + G + (int64_t)S * ((T + BM - 1) / BM);
}

int64_t wgrad_entries(int groups, int M) { return (int64_t)groups * ((M + BM - 1) / BM); }

int device_cus() {
  static int cus = 0;  // CUs of the current device, asked once
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

hipError_t launch_ffn_tiled(const FfnParams& p, hipStream_t stream) {
  const bool wgrad = p.act == kActWgrad;
  const int64_t max_entries =
      wgrad ? wgrad_entries(p.G + p.S, p.M) : ffn_max_entries(p.rows_bound, p.G, p.S, p.T);
  const bool gated = p.act == 2;
  const int cols = gated ? BR / 2 : BR;
  const int n_tiles_n = (p.N + cols - 1) / cols;
  if (wgrad) {
    hipLaunchKernelGGL(build_wgrad_tiles_kernel, dim3(1), dim3(256), 0, stream, p.G + p.S, p.G,
                       p.M, n_tiles_n, p.gdesc, p.entries, p.n_entries, p.xcd_bounds);
  } else if (!p.tiles_built) {
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, stream, p.offsets, p.G, p.S,
                       p.T, p.rows_bound, (int)max_entries, p.entries, p.n_entries);
  }
  // one resident block per CU (160 KiB of LDS each), never more blocks than
  // tiles; the backward's [K][N] input gradients, whose launches at decode
  // and Switch sizes hold fewer tiles than CUs (each a deep reduction), take
  // up to twice that, so the tail split cuts every tile in two on the idle
  // CUs; the weight gradients' work-balanced XCD ranges need a block on every
  // XCD (block P serves XCD P % 8), so at least 8 there
  const bool wide = p.bt && p.act == -1 && p.split && p.split_cap > 0;
  int64_t grid = std::min<int64_t>(device_cus(), max_entries * n_tiles_n * (wide ? 2 : 1));
  if (wgrad) grid = std::max<int64_t>(grid, 8);
  if (grid > 0) {
    const dim3 g((unsigned)grid), block(kThreads);
    if (p.bt) {  // weights stored [K][N] (backward input gradients)
      switch (p.act) {
        case kActBwd + 2:
          hipLaunchKernelGGL((ffn_tiled_kernel<kActBwd + 2, true>), g, block, 0, stream, p, n_tiles_n);
          break;
        case kActBwd + 1:
          hipLaunchKernelGGL((ffn_tiled_kernel<kActBwd + 1, true>), g, block, 0, stream, p, n_tiles_n);
          break;
        case kActBwd:
          hipLaunchKernelGGL((ffn_tiled_kernel<kActBwd, true>), g, block, 0, stream, p, n_tiles_n);
          break;
        default:
          hipLaunchKernelGGL((ffn_tiled_kernel<-1, true>), g, block, 0, stream, p, n_tiles_n);
          break;
      }
    } else switch (p.act) {
      case kActWgrad:
        hipLaunchKernelGGL(ffn_tiled_kernel<kActWgrad>, g, block, 0, stream, p, n_tiles_n);
        break;
      case kActBwd + 2:
        hipLaunchKernelGGL(ffn_tiled_kernel<kActBwd + 2>, g, block, 0, stream, p, n_tiles_n);
        break;
      case kActBwd + 1:
        hipLaunchKernelGGL(ffn_tiled_kernel<kActBwd + 1>, g, block, 0, stream, p, n_tiles_n);
        break;
      case kActBwd:
        hipLaunchKernelGGL(ffn_tiled_kernel<kActBwd>, g, block, 0, stream, p, n_tiles_n);
        break;
      case 2: hipLaunchKernelGGL(ffn_tiled_kernel<2>, g, block, 0, stream, p, n_tiles_n); break;
      case 1: hipLaunchKernelGGL(ffn_tiled_kernel<1>, g, block, 0, stream, p, n_tiles_n); break;
      case 0: hipLaunchKernelGGL(ffn_tiled_kernel<0>, g, block, 0, stream, p, n_tiles_n); break;
      default: hipLaunchKernelGGL(ffn_tiled_kernel<-1>, g, block, 0, stream, p, n_tiles_n); break;
    }
    // the split tiles of a tail split (the plan is made on the device)
    // (a reduction too shallow for the plan ever to split launches no fixup)
    const int nk = (p.K + BK - 1) / BK;
    const bool splits = (p.act == -1 && nk >= 2) || (p.act == 2 && nk >= kGatedSplitStages);
    if (splits && p.split && p.split_cap > 0) {
      const int fix = (int)std::min<int64_t>(p.split_cap, grid / 2);
      const dim3 fg((unsigned)(fix * kFixParts)), fb(256);
      if (fix > 0) {
        if (p.act == 2)
          hipLaunchKernelGGL(split_act_fixup_kernel<2>, fg, fb, 0, stream, p, n_tiles_n, (int)grid);
        else if (p.out_bf16)
          hipLaunchKernelGGL(split_bf16_fixup_kernel, fg, fb, 0, stream, p, n_tiles_n, (int)grid);
        else
          hipLaunchKernelGGL(split_fixup_kernel, fg, fb, 0, stream, p, n_tiles_n, (int)grid);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace moe
