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

#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroups = 8;  // 8-row weight groups per unit: 32 or 64 output columns
constexpr int UNR = 2;     // 32-deep k-steps per pipeline stage
constexpr int kStep = 32 * UNR;  // depth of one pipeline stage
constexpr uint32_t kOOB = 0x80000000u;
// Cache policy of the weight loads: non-temporal.  Every weight byte is read
// exactly once, so keeping it out of the caches' normal replacement lets the
// stream run faster (a pure read stream of this size: 7.0 against 6.3 TB/s);
// the token rows, which every unit of an expert re-reads, keep the default.
constexpr int kNT = 2;
#ifndef MOE_SKINNY_BLOCKS_PER_CU
#define MOE_SKINNY_BLOCKS_PER_CU 2
#endif
constexpr int kBlocksPerCU = MOE_SKINNY_BLOCKS_PER_CU;

// Where a unit's operands live: the load side runs one pipeline step ahead of
// the multiply side, so each keeps its own copy across unit boundaries.
struct UnitDesc {
  int g, rows, c_row0;
  int over;  // rows of a group that exceeds the 32-row limit (0 otherwise)
  uint32_t a_off[2];
  uint32_t b_row[kMaxGroups];  // byte offset of this lane's weight row in group j
  uint32_t b_col;              // BT: byte offset of this lane's 16-byte column chunk
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
// BT: the weights are stored [K][N] per group (output columns contiguous),
// as W1 / W3 are for the backward's input gradient of the up projections;
// with p.kh > 0 rows k >= kh come from the second set (u_main / u_shared),
// kh rows per group each (kh % 64 == 0).  A step's 64 rows of k, each the
// unit's 64 columns (128 bytes), are loaded as whole lines like the stored
// rows are otherwise, and each MFMA operand fragment comes from two LDS
// transpose reads (ds_read_b64_tr_b16: within each 16 lanes, lane j gives 4
// consecutive columns of row k0 + j/4 at column 4(j%4), and lane i receives
// column i of rows k0..k0+3).  Plain (act -1) 64-column units only.
template <int ACT, int NF, bool WU, bool BT = false>
__global__ __launch_bounds__(kThreads) void ffn_skinny_kernel(FfnParams p, int n_slabs,
                                                              int n_units) {
  // act-backward forms (down projection's input gradient): du (dv) from the
  // gated sum and the saved pre-activations, bf16 rows of ld = N (2N SwiGLU)
  constexpr bool BWD = ACT >= kActBwd && ACT <= kActBwd + 2;
  static_assert(!BT || ((ACT == -1 || BWD) && NF == 4), "[K][N] weights: 64-column units only");
  static_assert(!BWD || BT, "act-backward forms read [K][N] weights");
  constexpr int kCols = NF * 16;
  constexpr bool GATED = ACT == 2;
  constexpr int NB = GATED ? 2 : 1;           // weight sets (w1 and w3 when gated)
  constexpr int NFRAG = 2 * NF * NB;          // (row fragment, column fragment, set)
  constexpr int kGroups = kCols / 8;          // 8-row groups of a weight slab
  constexpr int kSlot = NB * kGroups * 1024;  // one step of one wave's weights
  constexpr int kRed = WU ? 0 : NFRAG * 1024; // one wave's partial products
  // output staging: a gated unit's output is the bf16 hidden layer, the
  // others may be float32; whole-unit waves stage one 16-row fragment at a
  // time in a tile of their own, split waves the unit's 32 rows once
  constexpr int kOutB = GATED ? 2 : 4;
  constexpr int kStage = WU ? 4 * 16 * kCols * kOutB : 32 * kCols * kOutB;
  static_assert(kGroups <= kMaxGroups, "weight slab wider than the descriptor");
  // (the gated 64-column split form is never launched: it would hold one block per CU)
  static_assert(4 * (kSlot + kRed) + kStage <= 80 * 1024 || (GATED && NF == 4 && !WU),
                "two blocks per CU");
  __shared__ __attribute__((aligned(16))) char lds[4 * (kSlot + kRed) + kStage];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char* const slot = lds + w * kSlot;
  float* const red = reinterpret_cast<float*>(lds + 4 * kSlot);  // [4][NFRAG][4][64]
  char* const stage = lds + 4 * (kSlot + kRed) + (WU ? w * 16 * kCols * kOutB : 0);
  const int K = p.K, N = p.N;
  // elements of one group's weight set (BT with a second set: kh rows each)
  const int64_t wstride = (BT && p.kh > 0) ? (int64_t)N * p.kh : (int64_t)N * K;
  // a contiguous run of units per block (per wave with WU), the runs in
  // order of XCD first: the hardware hands block P to XCD P % 8, so block
  // P takes run xcd_base + P / 8, and the neighbouring slabs of an expert,
  // which re-read its operand rows, share one XCD's L2
  const int xcd = blockIdx.x & 7, nblk = gridDim.x;
  const int run = (nblk >> 3) * xcd + min(xcd, nblk & 7) + (blockIdx.x >> 3);
  const int64_t workers = WU ? (int64_t)nblk * 4 : nblk;
  const int64_t me = WU ? (int64_t)run * 4 + w : run;
  const int u_begin = (int)(me * n_units / workers);
  const int u_end = (int)((me + 1) * n_units / workers);
  // this wave's contiguous reduction range; every wave runs `per` steps
  // per unit (steps past its range read zeros), so the waves stay in step
  const int kch = (K + kStep - 1) / kStep, per = WU ? kch : (kch + 3) / 4;
  const int kb = WU ? 0 : min(K, w * per * kStep), ke = WU ? K : min(K, (w + 1) * per * kStep);
  const int kl = (lane >> 4) * 8;
  const int total = (u_end - u_begin) * per;
  // Weight loads: one instruction fetches 8 whole rows of a step (8 x 128
  // bytes, whole cache lines): lane l takes row l/8 of the group and the
  // 16-byte chunk (l%8) ^ (l/8), which the load writes to LDS slot l%8 of
  // that row, so the MFMA operand reads below hit distinct banks.
  const int ld_row = lane >> 3, ld_chunk = (lane & 7) ^ ld_row;
  // MFMA operand reads: lane (column n = lane%16, k-slot q = lane/16) of
  // sub-step v reads chunk 4v + q of slab row 16 nf + n from its swizzled slot
  int rd_off[UNR];
#pragma unroll
  for (int v = 0; v < UNR; ++v) {
    const int n = lane & 15, q = lane >> 4;
    rd_off[v] = (n >> 3) * 1024 + (n & 7) * 128 + ((((4 * v + q) ^ (n & 7)) & 7) << 4);
  }
  // BT: transpose reads of sub-step v, half t (rows k0 + 4t ..) for column
  // fragment 0: lane j of 16-lane group q reads row 32v + 8q + 4t + j/4 (row
  // r = 4t + j/4 of 8-row group 4v + q) at column 4(j%4), in 16-byte chunk
  // c = (j/2)%2, which the load's swizzle keeps at slot c ^ r.  Fragment nf
  // adds chunk 2 nf, which xors into the slot bits 1-2 (offset ^ nf << 5).
  int tr_off[UNR][2];
  if constexpr (BT) {
    const int j = lane & 15, q = lane >> 4;
#pragma unroll
    for (int v = 0; v < UNR; ++v)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 4 * t + (j >> 2);
        tr_off[v][t] = (4 * v + q) * 1024 + r * 128 + ((((j >> 1) & 1) ^ r) << 4) + (j & 1) * 8;
      }
  }

  // Unit descriptor.  The expert's row range and gathered rows are re-read
  // only when the expert changes (consecutive units are slabs of one expert):
  // those loads are needed at once, and waiting for them would also wait for
  // the stage in flight.
  int cached_g = -1, cached_rows = 0, cached_r0 = 0, cached_over = 0;
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
      // a group above 32 rows breaks the caller's group_bound promise: its
      // output rows are poisoned with NaN (below) rather than left partly
      // computed
      cached_over = rows > 32 ? rows : 0;
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
    d.over = cached_over;
    d.a_off[0] = cached_a[0];
    d.a_off[1] = cached_a[1];
    d.W = static_cast<const uint16_t*>(routed ? p.w_main : p.w_shared) + gw * wstride;
    d.U = (GATED || (BT && p.kh > 0))
              ? static_cast<const uint16_t*>(routed ? p.u_main : p.u_shared) + gw * wstride
              : d.W;
    d.A = routed ? p.a_main : p.a_shared;
    if constexpr (BT) {
      // the unit's columns are this lane's chunk of each k-row; an expert
      // with no rows reads no weights
      const int n = slab * kCols + ld_chunk * 8;
      d.b_col = (n < N && cached_rows > 0) ? (uint32_t)n * 2u : kOOB;
    } else {
#pragma unroll
      for (int j = 0; j < kGroups; ++j) {
        const int n = slab * kCols + j * 8 + ld_row;
        // an expert with no rows reads no weights: every offset is out of range
        d.b_row[j] = (n < N && cached_rows > 0) ? (uint32_t)n * (uint32_t)K * 2u : kOOB;
      }
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

  // the partial products are the only memory the waves share: a barrier
  // needs this wave's LDS operations done, not its loads in flight (which
  // __syncthreads would drain)
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };

  struct AStage { u32x4 a[UNR][2]; };
  // Loads of step `st` (0..per-1) of the unit described by d: the weights
  // into this wave's LDS slot, the operand rows into registers.  `past` (past
  // the block's last step) turns every offset out of range: the loads read
  // zeros and move no data, and the code stays branch-free.
  auto issue = [&](AStage& sa, const UnitDesc& d, int st, uint32_t past) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.A), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.W), (short)0, (int)(wstride * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t u_rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(d.U), (short)0, (int)(wstride * 2), 0x00020000);
    const int k0 = kb + st * kStep;
    if constexpr (BT) {
      // 64 rows of k, 8 per load; a step lies wholly in one weight set
      // (k0 and kh are multiples of 64)
      const bool second = p.kh > 0 && k0 >= p.kh;
      const int kr0 = second ? k0 - p.kh : k0;
#pragma unroll
      for (int j = 0; j < kGroups; ++j) {
        const int kk = k0 + j * 8 + ld_row;
        const uint32_t off = (kk < ke && d.b_col != kOOB)
                                 ? (uint32_t)(kr0 + j * 8 + ld_row) * (uint32_t)N * 2u + d.b_col
                                 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? u_rs : w_rs,
                                                 MOE_LDS(slot + j * 1024), 16, off | past, 0, 0, kNT);
      }
    } else {
      const uint32_t bk = (k0 + ld_chunk * 8 < ke ? (uint32_t)(k0 + ld_chunk * 8) * 2u : kOOB) | past;
#pragma unroll
      for (int s = 0; s < NB; ++s)
#pragma unroll
        for (int j = 0; j < kGroups; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(s == 0 ? w_rs : u_rs,
                                                   MOE_LDS(slot + (s * kGroups + j) * 1024), 16,
                                                   (d.b_row[j] + bk) | past, 0, 0, kNT);
    }
#pragma unroll
    for (int v = 0; v < UNR; ++v) {
      const int kk = k0 + v * 32 + kl;
      const uint32_t kadd = (kk < ke ? (uint32_t)(k0 + v * 32) * 2u : kOOB) | past;
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
        sa.a[v][mf] = __builtin_amdgcn_raw_buffer_load_b128(a_rs, (d.a_off[mf] + kadd) | past, 0, 0);
    }
  };
  struct BRegs { bf16x8 b[UNR][NF][NB]; };
  // this step's weight fragments, from the wave's slot into registers
  auto fetch = [&](BRegs& br) __attribute__((always_inline)) {
    if constexpr (BT) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int v = 0; v < UNR; ++v)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)MOE_LDS(slot + (tr_off[v][0] ^ (nf << 5))));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)MOE_LDS(slot + (tr_off[v][1] ^ (nf << 5))));
          br.b[v][nf][0] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    } else {
#pragma unroll
      for (int v = 0; v < UNR; ++v)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int s = 0; s < NB; ++s)
            br.b[v][nf][s] = *reinterpret_cast<const bf16x8*>(
                slot + (s * kGroups + 2 * nf) * 1024 + rd_off[v]);
    }
  };
  // Both row fragments are always multiplied: the second reads zeros when the
  // expert holds 16 rows or fewer (MFMA time is negligible here).
  auto compute = [&](const AStage& sa, const BRegs& br) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < UNR; ++v)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int mf = 0; mf < 2; ++mf)
            acc[mf][nf][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, sa.a[v][mf]), br.b[v][nf][s], acc[mf][nf][s], 0, 0, 0);
  };
  // act-backward: du (dv) of one output from its sum a: the row's gate
  // (routed rows; shared rows 1), the saved pre-activations u (v), the
  // activation's backward; staged as bf16 at (r, c) of the du tile and of
  // the dv tile that follows it (tile_rows rows each)
  auto put_bwd = [&](const UnitDesc& d, int r, int c, int row, int col, float a, int tile_rows)
      __attribute__((always_inline)) {
    const bool routed = d.g < p.G;
    const int64_t ra = d.c_row0 + row;
    const int64_t ld = ACT == kActBwd + 2 ? 2 * (int64_t)N : N;
    const uint16_t* pre = static_cast<const uint16_t*>(p.pre);
    const float g = routed ? p.row_gate[ra] : 1.f;
    const float uu = bf16_to_f32(pre[ra * ld + col]);
    const float vv = ACT == kActBwd + 2 ? bf16_to_f32(pre[ra * ld + N + col]) : 0.f;
    float du, dv;
    act_backward(ACT - kActBwd, a * g, uu, vv, du, dv);
    uint16_t* st = reinterpret_cast<uint16_t*>(stage);
    st[r * kCols + c] = f32_to_bf16(du);
    if (ACT == kActBwd + 2) st[(tile_rows + r) * kCols + c] = f32_to_bf16(dv);
  };
  // act-backward: tile rows [0, nrows) of the du tile (and the dv tile after
  // it) to output rows row0 + r, columns col (du) and N + col (dv) of rows
  // of ld bf16 elements, as 16-byte non-temporal stores; thread i of n
  auto drain_bwd = [&](const UnitDesc& d, int u, int row0, int nrows, int tile_rows, int i, int n)
      __attribute__((always_inline)) {
    const int slab = u - d.g * n_slabs;
    const int64_t ld = ACT == kActBwd + 2 ? 2 * (int64_t)N : N;
    constexpr int per_row = kCols * 2 / 16;
    constexpr int sets = ACT == kActBwd + 2 ? 2 : 1;
    for (int c = i; c < sets * nrows * per_row; c += n) {
      const int set = c / (nrows * per_row), cc = c - set * nrows * per_row;
      const int r = cc / per_row, q = cc - r * per_row;
      const int col = slab * kCols + q * 8;
      if (row0 + r >= d.rows || col >= N) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) +
                                            (d.c_row0 + row0 + r) * ld + set * N + col);
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(stage + ((set * tile_rows + r) * per_row + q) * 16), dst);
    }
  };
  // one output value of the unit: bias, pre-activations, activation
  auto value = [&](const UnitDesc& d, int row, int col, float a, float up)
      __attribute__((always_inline)) -> float {
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
    if (GATED) return silu_f32(a) * up;
    if (ACT == 0) return gelu_f32(a);
    if (ACT == 1) return fmaxf(a, 0.f);
    // top-1 direct store: the gate times the row, formed as the combine
    // forms it (fma onto zero), so the stored bf16 value is the same
    if constexpr (ACT == -1 && !BT)
      if (p.direct_token) a = fmaf(p.direct_gate[p.direct_token[d.c_row0 + row]], a, 0.f);
    return a;
  };
  // output row of unit row `row` (the token's row for a top-1 direct store)
  auto out_row = [&](const UnitDesc& d, int row) __attribute__((always_inline)) -> int64_t {
    if constexpr (ACT == -1 && !BT)
      if (p.direct_token) return p.direct_token[d.c_row0 + row];
    return (int64_t)d.c_row0 + row;
  };
  // Outputs leave through LDS as 16-byte non-temporal stores, whole 64- or
  // 128-byte row segments per 4 or 8 lanes: the unit's output rows are
  // written while the weight stream runs, and scattered 2- or 4-byte stores
  // of the same bytes cost that stream about a sixth of its time (the next
  // kernel reads them once, so they need not stay in the caches either).
  // put(): one value into the staging tile (tile row r, unit column c)
  auto put = [&](int r, int c, float v) __attribute__((always_inline)) {
    if (GATED || p.out_bf16)
      reinterpret_cast<uint16_t*>(stage)[r * kCols + c] = f32_to_bf16(v);
    else
      reinterpret_cast<float*>(stage)[r * kCols + c] = v;
  };
  // drain(): tile rows [0, nrows) to output rows row0 + r (r < rows), by
  // thread i of n; every 16-byte chunk lies wholly inside or outside N
  // columns since N is a multiple of 8
  auto drain = [&](const UnitDesc& d, int u, int row0, int nrows, int i, int n)
      __attribute__((always_inline)) {
    const int slab = u - d.g * n_slabs;
    const bool b16 = GATED || p.out_bf16;
    const int per_row = kCols * (b16 ? 2 : 4) / 16;
    for (int c = i; c < nrows * per_row; c += n) {
      const int r = c / per_row, q = c - r * per_row;
      const int col = slab * kCols + q * (b16 ? 8 : 4);
      if (row0 + r >= d.rows || col >= N) continue;
      // 16-byte aligned: the output is, and N is a multiple of 8
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(p.out) +
                                            (out_row(d, row0 + r) * N + col) * (b16 ? 2 : 4));
      u32x4 v = *reinterpret_cast<const u32x4*>(stage + c * 16);
      if (!b16 && p.accumulate)
        v = __builtin_bit_cast(u32x4, __builtin_bit_cast(f32x4, v) + __builtin_bit_cast(f32x4, *dst));
      __builtin_nontemporal_store(v, dst);
    }
  };
  // a group over the limit: NaN in every output row of the group (within
  // rows_bound) and column of the unit's slab; thread i of n strides
  auto poison = [&](const UnitDesc& d, int u, int i, int n) __attribute__((always_inline)) {
    const int slab = u - d.g * n_slabs;
    const int64_t lim = p.rows_bound - d.c_row0;
    const int rows = (int)min((int64_t)d.over, lim > 0 ? lim : 0);
    for (int o = i; o < rows * kCols; o += n) {
      const int row = o / kCols, col = slab * kCols + (o - row * kCols);
      if (col >= N) continue;
      if constexpr (BWD) {  // du (and dv) rows of ld elements
        const int64_t ld = ACT == kActBwd + 2 ? 2 * (int64_t)N : N;
        uint16_t* o16 = static_cast<uint16_t*>(p.out) + (d.c_row0 + row) * ld + col;
        o16[0] = 0x7fc0u;
        if (ACT == kActBwd + 2) o16[N] = 0x7fc0u;
        continue;
      }
      const int64_t idx = out_row(d, row) * N + col;
      if (p.out_bf16) static_cast<uint16_t*>(p.out)[idx] = 0x7fc0u;
      else static_cast<float*>(p.out)[idx] = __builtin_nanf("");
    }
  };
  // sum the 4 waves' partial products in wave order, activation, store (with
  // WU the wave's own products, straight from the 16x16 result layout: lane
  // holds column lane%16 of rows 4*(lane/16) + i)
  auto finish = [&](const UnitDesc& d, int u) __attribute__((always_inline)) {
    if constexpr (WU) {
      const int slab = u - d.g * n_slabs;
      if (d.over) {
        poison(d, u, lane, 64);
        return;
      }
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        if (mf * 16 >= d.rows) break;
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = (lane >> 4) * 4 + i, row = mf * 16 + r;
            const int c = nf * 16 + (lane & 15), col = slab * kCols + c;
            if (row < d.rows && col < N) {
              if constexpr (BWD) put_bwd(d, r, c, row, col, acc[mf][nf][0][i], 16);
              else put(r, c, value(d, row, col, acc[mf][nf][0][i], GATED ? acc[mf][nf][NB - 1][i] : 0.f));
            }
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's tile written
        if constexpr (BWD) drain_bwd(d, u, mf * 16, 16, 16, lane, 64);
        else drain(d, u, mf * 16, 16, lane, 64);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // and read, before it is reused
      }
      return;
    }
    auto R = [&](int wv, int f, int i, int l) -> float& {
      return red[((wv * NFRAG + f) * 4 + i) * 64 + l];
    };
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) R(w, (mf * NF + nf) * NB + s, i, lane) = acc[mf][nf][s][i];
    lds_barrier();
    const int slab = u - d.g * n_slabs;
    for (int o = threadIdx.x; o < 2 * NF * 256; o += kThreads) {
      const int mf = o / (NF * 256), rem = o - mf * NF * 256;
      const int nf = rem >> 8, i = (rem >> 6) & 3, l = rem & 63;
      const int row = mf * 16 + (l >> 4) * 4 + i;
      const int c = nf * 16 + (l & 15), col = slab * kCols + c;
      if (row >= d.rows || col >= N || d.over) continue;
      const int f0 = (mf * NF + nf) * NB;
      const float a = ((R(0, f0, i, l) + R(1, f0, i, l)) + R(2, f0, i, l)) + R(3, f0, i, l);
      float up = 0.f;
      if (GATED)
        up = ((R(0, f0 + 1, i, l) + R(1, f0 + 1, i, l)) + R(2, f0 + 1, i, l)) + R(3, f0 + 1, i, l);
      if constexpr (BWD) put_bwd(d, row, c, row, col, a, 32);
      else put(row, c, value(d, row, col, a, up));
    }
    if (d.over) {
      poison(d, u, threadIdx.x, kThreads);
    } else {
      lds_barrier();  // the staged tile is complete
      if constexpr (BWD) drain_bwd(d, u, 0, 32, 32, threadIdx.x, kThreads);
      else drain(d, u, 0, 32, threadIdx.x, kThreads);
    }
    lds_barrier();  // the partial products and the tile are reused by the next unit
  };

  // One continuous pipeline over the block's units.  Step i: wait for its
  // loads (weights in the slot, operand rows in registers), copy its weight
  // fragments out of the slot, issue step i+1's loads (of this unit or the
  // next) into the same slot, then multiply; so one step's loads are always
  // in flight while the previous one is multiplied, and a unit's reduction
  // and stores overlap the next unit's first loads.
  if (total <= 0) return;
  UnitDesc ld, cd;  // load side, multiply side
  describe(u_begin, ld);
  cd = ld;
  zero_acc();
  AStage s0, s1;
  issue(s0, ld, 0, 0u);
#define MOE_SKINNY_STEP(Acur, Anext, i)                                    \
  {                                                                        \
    __builtin_amdgcn_s_waitcnt(0x0f70); /* vmcnt(0) */                     \
    BRegs br;                                                              \
    fetch(br);                                                             \
    __builtin_amdgcn_s_waitcnt(0xc07f); /* lgkmcnt(0): slot free */         \
    asm volatile("" ::: "memory");                                         \
    const int nl = (i) + 1;                                                \
    const int nq = nl < total ? nl : total - 1;                            \
    describe(u_begin + nq / per, ld);                                      \
    issue(Anext, ld, nq % per, nl < total ? 0u : kOOB);                    \
    compute(Acur, br);                                                     \
    if ((i) % per == per - 1) {                                            \
      finish(cd, u_begin + (i) / per);                                     \
      zero_acc();                                                          \
      cd = ld;                                                             \
    }                                                                      \
  }
  // the loop body has no exit of its own: an exit between the two steps
  // would join the loop's back edge with loads still in flight
  int i = 0;
  for (; i + 1 < total; i += 2) {
    MOE_SKINNY_STEP(s0, s1, i)
    MOE_SKINNY_STEP(s1, s0, i + 1)
  }
  if (i < total) MOE_SKINNY_STEP(s0, s1, i)
#undef MOE_SKINNY_STEP
  // loads issued past the end (zeros) land before the block's LDS is freed
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

}  // namespace

int device_cus();

hipError_t launch_ffn_skinny(const FfnParams& p, hipStream_t stream) {
  // the gated form stages the bf16 hidden layer (the only output it has:
  // the kernel serves bf16 layers)
  if (p.act == 2 && !p.out_bf16) return hipErrorInvalidValue;
  // Unit width and work split from a cost model in wave-steps of one
  // 16-column fragment: the busiest worker's units times their steps (the
  // K-split pays about 3 more steps per unit for its LDS reduction), times
  // the width.  The cheaper estimate wins, with no margin for either form
  // (the Mixtral decode batch's gated up projection: 64-column whole units
  // 282 us against 32-column split units 286 us, where a 15% margin for the
  // split had kept the latter); ties go to the form and the width tried first
  // (the wider unit, the K-split).
  const int64_t groups = p.G + p.S;
  const int64_t cap = (int64_t)device_cus() * kBlocksPerCU;
  const int64_t kch = (p.K + kStep - 1) / kStep;
  int nf = 2;
  bool wu = false;
  double best = 1e300;
  // [K][N] weights: the plain and the act-backward forms only; the
  // act-backward forms only with [K][N] weights
  const bool bwd = p.act >= kActBwd && p.act <= kActBwd + 2;
  if (p.bt ? !(p.act == -1 || bwd) : bwd) return hipErrorInvalidValue;
  for (int cand = 4; cand >= (p.bt ? 4 : 2); cand -= 2) {
    const int64_t units = groups * ((p.N + cand * 16 - 1) / (cand * 16));
    if (units == 0) continue;
    const int64_t blocks = std::min<int64_t>(units, cap);
    const double ksplit = (double)((units + blocks - 1) / blocks) * ((kch + 3) / 4 + 3) * cand;
    const int64_t wblocks = std::min<int64_t>((units + 3) / 4, cap);
    const double whole = (double)((units + 4 * wblocks - 1) / (4 * wblocks)) * kch * cand;
    // a gated 64-column unit split over the waves would need 128 KiB of LDS
    // (weight slots and partial products), leaving one block per CU
    if (ksplit < best && !(p.act == 2 && cand == 4)) { best = ksplit; nf = cand; wu = false; }
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
    if (p.bt) {
#define MOE_SKINNY_BT(A)                                                                          \
  if (wu) hipLaunchKernelGGL((ffn_skinny_kernel<A, 4, true, true>), g, block, 0, stream, p, n_slabs, nu); \
  else hipLaunchKernelGGL((ffn_skinny_kernel<A, 4, false, true>), g, block, 0, stream, p, n_slabs, nu);
      switch (p.act) {
        case kActBwd + 2: MOE_SKINNY_BT(kActBwd + 2) break;
        case kActBwd + 1: MOE_SKINNY_BT(kActBwd + 1) break;
        case kActBwd: MOE_SKINNY_BT(kActBwd) break;
        default: MOE_SKINNY_BT(-1) break;
      }
#undef MOE_SKINNY_BT
    } else if (nf == 4 && wu) {
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
