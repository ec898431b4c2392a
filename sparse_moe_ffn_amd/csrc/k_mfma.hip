// W4A8 grouped products on the int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// MobileMoE close reading, section "Custom MoE kernel": after the count sort
// each expert runs one batched product over its contiguous rows (fused gate/up
// with SwiGLU, then down).  INT4 weights follow eq. (6) (section
// "Quantisation-aware training"): one FP32 scale per 32 weights along the
// reduction dimension.  The MFMA's K of 32 is exactly one quantisation group,
// so every MFMA (started from a zero accumulator) yields the exact int32 group
// sum, which is then scaled in FP32:
//     acc = fma(s_w[col][g], (float) isum_g, acc)   for g ascending
// -- the same order the row-tile kernels and the CPU oracle use, so results
// agree bit for bit.
//
// Tiling.  A workgroup is one wave.  It owns kMT x 32 rows of one expert
// (kMT = 1 or 2 MFMA row tiles) and two 32-column tiles of the output (gate/up:
// the gate tile and the matching up tile of the same 32 hidden columns, so
// SwiGLU is applied in registers).  Activation fragments (one 16-byte load
// per lane per group) and weight fragments (one 8-byte load per lane per
// group, straight from the prepacked INT4 layout of csrc/common.h, which is in
// MFMA operand order) go from global memory to registers two groups at a
// time, one stage ahead of the math.  There is no LDS and no barrier, so
// waves never wait for each other and about 140 (kMT = 1) or 200 (kMT = 2)
// VGPRs leave 3 or 2 waves per SIMD to hide the load latency.  kMT = 2 halves
// the weight traffic per MFMA and is used once the problem has enough tiles
// to fill the chip with it.  Nibbles are unpacked in registers to int8 (times
// 16; the scales are pre-divided by 16).  Workgroup ids are remapped so that
// consecutive tiles (same expert, neighbouring column slices) land on the same
// XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kXcd = 8;
constexpr int kRingWide = 3;  // register-ring depth of the four-column-tile waves
constexpr int kRingDeep = 8;  // register-ring depth of the small-launch waves

__device__ __forceinline__ v4i unpack16(uint2 w) {
  uint32_t q0, q1, q2, q3;
  unpack8(w.x, q0, q1);
  unpack8(w.y, q2, q3);
  return v4i{(int)q0, (int)q1, (int)q2, (int)q3};
}

// Capture of the exact group sums (test twins only).
struct Capture {
  int32_t* isum;
  int64_t wrows;
  int G, p0, n;
};

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) v4i gint4;
typedef const __attribute__((address_space(1))) v2u guint2;
typedef const __attribute__((address_space(1))) float gfloat;

// One group's registers: activation fragments, packed weight fragments and
// scales.  Global-address-space views: loads through them are global_load
// (not flat), which keeps the memory counter in order and lets the
// prefetches stay in flight across the math.
template <int kMT, int kNT>
struct WSlot {
  v4i a[kMT];
  v2u b[kNT];
  float s[kNT];
};

// One group: per (row tile, column tile) one MFMA from a zero accumulator
// (the exact int32 group sum), then acc = fma(scale, sum, acc).  Each
// tile's weights are unpacked just before their first MFMA, and the
// epilogue of one product is issued after the next product's MFMA, so the
// matrix core and the vector ALU work at the same time with two MFMA
// results live.
template <int kMT, int kNT, bool kCapture>
__device__ __forceinline__ void wcompute1(v16f (&acc)[kMT][kNT], const WSlot<kMT, kNT>& st, int g,
                                          int lane, const int (&rb)[kNT], const Capture& cap) {
  v4i bv[kNT];
  v16i Rp;
  int pm = 0, pj = 0;
  auto epi = [&](const v16i& R, int m, int j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][j][r] = fmaf(st.s[j], (float)R[r], acc[m][j][r]);
    if (kCapture) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < cap.n) {
          const int64_t col = (int64_t)rb[j] * 32 + (lane & 31);
          cap.isum[(((int64_t)(cap.p0 + row)) * cap.wrows + col) * cap.G + g] = R[r] >> 4;
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kNT; ++j)
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      if (m == 0) bv[j] = unpack16(make_uint2(st.b[j].x, st.b[j].y));
      const v16i R = __builtin_amdgcn_mfma_i32_32x32x32_i8(st.a[m], bv[j], v16i{}, 0, 0, 0);
      if (j + m > 0) epi(Rp, pm, pj);
      Rp = R;
      pm = m;
      pj = j;
    }
  epi(Rp, pm, pj);
#pragma unroll
  for (int j = 0; j < kNT; ++j)
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      if (m == 0) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU: unpack tile j
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      if (j + m > 0) __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // VALU: previous epilogue
    }
  __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
}

// Arguments of one W4A8 product; a launch carries one, or two (the routed
// experts and the shared expert) in the merged form.
struct W4A8Prob {
  ExpertArgs a;
  int nsplit, K, N;
  const int8_t* act;
  const float* act_scale;
  const uint8_t* wq;
  const float* wsc;
  float* out;
  int32_t* isum;
};

// The weighted combine done in the shared down's epilogue (down problems
// with the shared expert's rows, one per token): instead of writing ys, the
// tile writes y[t][c] = fma(w[t][k-1], f[inv[t*k+k-1]][c], ... fma(w[t][0],
// f[inv[t*k]][c], 0)) + ys[t][c], the combine kernel's arithmetic in its
// order (positions outside [0, Tk) add nothing), with ys[t][c] the value
// the shared down would have stored.  The routed outputs f must be complete
// (an earlier launch).
struct CombineArgs {
  const float* f;      // [Tk][N] routed outputs, expert-sorted
  const int32_t* inv;  // [Tk] position of slot t*k+j in f
  const float* w;      // [Tk] gate weights
  float* y;            // [T][N]
  int64_t Tk;
  int k;               // 1..kMaxCmbK
};
constexpr int kMaxCmbK = 8;

// Workgroup b runs on XCD b % 8 as that XCD's slot b / 8.  Each XCD works
// through a contiguous range of logical tile ids (the same expert's weights
// stay in its L2): slot i of XCD x takes logical id x * per + i, with per the
// problem's tile count over 8.  A routed problem's real tile count is only
// known from the offsets, so it is counted in the kernel (the grid is sized
// for the worst case) and the spare slots exit; the empty tail is thereby
// spread over the XCDs instead of idling the last ones.
//
// The combine in the shared down's epilogue (CombineArgs), for k <= kK:
// the tile's positions and gate weights go to workgroup memory, then the
// rows are taken kRB at a time, every gather of those rows issued before
// the sums.
template <int kNT, int kK>
__device__ __forceinline__ void combine_epilogue(const v16f (&acc)[kNT], float srow,
                                                 const int (&cpos)[kK / 2],
                                                 const float (&cwt)[kK / 2], const CombineArgs& C,
                                                 int p0, int n, int col0, int N, int lane) {
  constexpr int kRB = 32 / (kK * kNT);  // rows per batch: 32 gathers in flight per lane
  static_assert(kRB >= 1 && 16 % kRB == 0, "rows per batch");
  __shared__ int s_pos[32][kK];
  __shared__ float s_w[32][kK];
#pragma unroll
  for (int q = 0; q < kK / 2; ++q) {
    const int jj = (lane >> 5) * (kK / 2) + q;
    s_pos[lane & 31][jj] = cpos[q];
    s_w[lane & 31][jj] = cwt[q];
  }
  __syncthreads();  // one wave per workgroup: its stores are visible to its own loads
  const int c = lane & 31;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += kRB) {
    float v[kRB][kK][kNT], wj[kRB][kK], sc[kRB];
    int pj[kRB][kK], rl[kRB];
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int r = r0 + u;
      rl[u] = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      sc[u] = __shfl(srow, rl[u]);  // every lane takes part (before any divergence)
#pragma unroll
      for (int jj = 0; jj < kK; ++jj) {
        const int p = s_pos[rl[u]][jj];
        // slots past k and positions outside [0, Tk) add nothing; they read
        // row 0 (a valid address) and are never used
        pj[u][jj] = (jj < C.k && rl[u] < n && p >= 0 && (int64_t)p < C.Tk) ? p : -1;
        wj[u][jj] = s_w[rl[u]][jj];
        const int pr = pj[u][jj] >= 0 ? pj[u][jj] : 0;
#pragma unroll
        for (int j = 0; j < kNT; ++j) v[u][jj][j] = C.f[(int64_t)pr * N + col0 + j * 32 + c];
      }
    }
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kK; ++jj)
          if (pj[u][jj] >= 0) a = fmaf(wj[u][jj], v[u][jj][j], a);
        if (rl[u] < n) C.y[(int64_t)(p0 + rl[u]) * N + col0 + j * 32 + c] = a + acc[j][r0 + u] * sc[u];
      }
    }
  }
}

// One tile (kMT row tiles x kNT column tiles) of problem P for XCD x, slot
// i; logical id = mt * nsplit + split.  kDense: rows are the tokens in order
// (shared expert), per_dense its slots per XCD; otherwise routed
// (expert-sorted rows, tiles found from the offsets).  kGM: the activations
// are group-major (act_offset in common.h), so a tile's 32 rows of one group
// are read from one contiguous kilobyte when the rows are consecutive.
// K % 128 == 0.  Called by one whole wave.
template <int kMT, int kNT, bool kGateUp, bool kCapture, bool kDense, bool kGM = false,
          bool kDeep = false, int kCmbK = 0>
__device__ __forceinline__ void w4a8w_tile(const W4A8Prob& P, int x, int i, int per_dense,
                                           const CombineArgs* cmb = nullptr) {
  // kCmbK > 0: the combine in the epilogue for k <= kCmbK (shared down only)
  constexpr bool kCmb = kCmbK > 0;
  static_assert(!kCmb || (kDense && !kGateUp && kMT == 1), "combine: shared down, one row tile");
  static_assert(!kGateUp || kNT % 2 == 0, "gate/up tiles come in (gate, up) pairs");
  constexpr int kP = kNT / 2;  // gate/up: column pairs per wave
  constexpr int kBM = 32 * kMT;
  const ExpertArgs& a = P.a;
  const int nsplit = P.nsplit, K = P.K, N = P.N;
  const int8_t* __restrict__ act = P.act;
  const float* __restrict__ act_scale = P.act_scale;
  const uint8_t* __restrict__ wq = P.wq;
  const float* __restrict__ wsc = P.wsc;
  float* __restrict__ out = P.out;
  int32_t* __restrict__ isum = P.isum;
  const int lane = threadIdx.x;
  const int rows = (int)a.rows;
  int mt, split, p0, n, e;
  if constexpr (kDense) {
    const int logical = x * per_dense + i;
    mt = logical / nsplit;
    split = logical % nsplit;
    p0 = mt * kBM;
    n = min(kBM, rows - p0);
    e = 0;
  } else {
    const RoutedTiles rt = routed_tiles(a.offsets, a.E, rows, kBM);
    const int per = (rt.total * nsplit + kXcd - 1) / kXcd;
    if (i >= per) return;
    const int logical = x * per + i;
    mt = logical / nsplit;
    split = logical % nsplit;
    routed_pick(rt, kBM, mt, p0, n, e);
  }
  if (n <= 0) return;
  const int G = K / kGroup, h = a.h;
  int col0, rb[kNT];
  if constexpr (kGateUp) {  // tiles 0..kP-1: gate; kP..2kP-1: the matching up tiles
    col0 = split * kP * 32;
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      rb[p] = split * kP + p;
      rb[kP + p] = h / 32 + split * kP + p;
    }
  } else {
    col0 = split * kNT * 32;
#pragma unroll
    for (int j = 0; j < kNT; ++j) rb[j] = split * kNT + j;
  }
  // source row of this lane's A rows (padding rows read the tile's first row;
  // their results are never stored) and its activation scale
  // (byte offsets from the activation base fit 32 bits: rows * K < 2^31)
  uint32_t aoff[kMT];
  float srow[kMT];
#pragma unroll
  for (int m = 0; m < kMT; ++m) {
    const int r = m * 32 + (lane & 31);
    const int rr = r < n ? r : 0;
    int src = p0 + rr;
    if constexpr (kGateUp && !kDense) {
      src = a.perm[p0 + rr] / a.k;
      if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
    }
    aoff[m] = (uint32_t)src * (uint32_t)(kGM ? 32 : K) + 16u * (uint32_t)(lane >> 5);
    srow[m] = act_scale[src];
  }
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : N;
  const uint8_t* we = wq + (int64_t)e * (wrows / 32) * G * kChunkBytes;
  const float* se = wsc + (int64_t)e * (wrows / 32) * G * 32;
  const uint8_t* pb[kNT];  // wave-uniform bases (scalar registers)
  const uint8_t* ps[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    pb[j] = we + (int64_t)rb[j] * G * kChunkBytes;
    ps[j] = (const uint8_t*)(se + (int64_t)rb[j] * G * 32);
  }
  const Capture cap{isum, wrows, G, p0, n};
  // bytes from one group of an activation row to the next (x_q has T rows,
  // the hidden rows `rows`)
  const uint32_t astride = kGM ? 32u * (uint32_t)(kGateUp ? a.T : a.rows) : 32u;

  v16f acc[kMT][kNT];
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[m][j] = v16f{};

  // Combine: the positions and gate weights of the tile's 32 tokens are
  // requested now, so they arrive under the products; lane l holds slots
  // (l >> 5) kCmbK / 2 .. + kCmbK / 2 - 1 of row l & 31.
  constexpr int kCmbPer = kCmb ? kCmbK / 2 : 1;
  int cpos[kCmbPer];
  float cwt[kCmbPer];
  if constexpr (kCmb) {
    const int rr = (lane & 31) < n ? (lane & 31) : 0;
    const int64_t t = p0 + rr;
#pragma unroll
    for (int q = 0; q < kCmbPer; ++q) {
      const int jj = (lane >> 5) * kCmbPer + q;
      const int jc = jj < cmb->k ? jj : 0;
      cpos[q] = cmb->inv[t * cmb->k + jc];
      cwt[q] = cmb->w[t * cmb->k + jc];
    }
  }

  // Register ring of kD single-group slots: slot i % kD holds group i,
  // loaded kD - 1 groups before its products (the last groups re-load group
  // G - 1: valid addresses, results unused).  Every load is a scalar base
  // plus a 32-bit lane offset.  Four column tiles or two row tiles per wave
  // keep three slots (registers for three waves per SIMD instead of two:
  // M prefill 459 -> 436 us, L 609 -> 583 us per step).  kDeep (launches of
  // fewer waves than the chip has SIMDs, as in decode batches): eight slots,
  // so that each wave keeps seven groups of weights in flight.
  constexpr int kD = kDeep ? kRingDeep : (kNT >= 4 || kMT >= 2) ? kRingWide : 4;
  WSlot<kMT, kNT> sl[kD];
  auto load = [&](WSlot<kMT, kNT>& st, int g) {
#pragma unroll
    for (int m = 0; m < kMT; ++m) st.a[m] = *(gint4*)(act + (aoff[m] + (uint32_t)g * astride));
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      st.b[j] = *(guint2*)(pb[j] + (uint32_t)(g * kChunkBytes + lane * 8));
      st.s[j] = *(gfloat*)(ps[j] + (uint32_t)(g * 128 + (lane & 31) * 4));
    }
  };
  // the first slots in slot order (the counter wait at the loop head must
  // find slot 0 oldest, as it is on every later iteration)
#pragma unroll
  for (int i = 0; i < kD - 1; ++i) {
    load(sl[i], min(i, G - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int g = 0; g < G; g += kD) {
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      load(sl[(i + kD - 1) % kD], min(g + i + kD - 1, G - 1));
      if (G % kD == 0 || g + i < G) wcompute1<kMT, kNT, kCapture>(acc, sl[i], g + i, lane, rb, cap);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const float s = __shfl(srow[m], rl);
      const int row = m * 32 + rl;
      if (row >= n) continue;
      if constexpr (kGateUp) {
#pragma unroll
        for (int p = 0; p < kP; ++p)
          out[(int64_t)(p0 + row) * h + col0 + p * 32 + (lane & 31)] =
              silu(acc[m][p][r] * s) * (acc[m][kP + p][r] * s);
      } else if constexpr (!kCmb) {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          out[(int64_t)(p0 + row) * N + col0 + j * 32 + (lane & 31)] = acc[m][j][r] * s;
      }
    }
  if constexpr (kCmb) combine_epilogue<kNT, kCmbK>(acc[0], srow[0], cpos, cwt, *cmb, p0, n, col0, N, lane);
}

template <int kMT, bool kGateUp, bool kCapture, bool kDense>
__global__ __launch_bounds__(64) void k_w4a8w(W4A8Prob P) {
  const int b = (int)blockIdx.x;
  w4a8w_tile<kMT, 2, kGateUp, kCapture, kDense>(P, b % kXcd, b / kXcd, (int)gridDim.x / kXcd);
}

// Routed (P0) and shared (P1) products of the same kind in one launch, both
// with group-major activations (the one-call layer writes them so).  Every
// XCD gets its share of both: its first per1 slots take shared tiles, the
// rest routed tiles.  Workgroups start in slot order, so the shared tiles
// (as long as or, for down with h_s = 4h, four times as long as a routed
// tile) go first and the short routed ones fill in behind them.  kNT1: the
// shared problem's 32-column tiles per wave (down with few tokens: 1, so
// that twice as many waves share its long reduction).
template <int kMT0, int kMT1, bool kGateUp, int kNT1 = 2, int kNT0 = 2, bool kDeep = false>
__global__ __launch_bounds__(64) void k_w4a8w_pair(W4A8Prob P0, W4A8Prob P1, int per1) {
  const int b = (int)blockIdx.x, x = b % kXcd, i = b / kXcd;
  if (i < per1)
    w4a8w_tile<kMT1, kNT1, kGateUp, false, true, true, kDeep>(P1, x, i, per1);
  else
    w4a8w_tile<kMT0, kNT0, kGateUp, false, false, true, kDeep>(P0, x, i - per1, 0);
}

// The shared down with the combine in its epilogue (CombineArgs), launched
// after the routed down: one row tile and kNT column tiles per wave.
template <int kNT, int kK>
__global__ __launch_bounds__(64) void k_w4a8w_shared_cmb(W4A8Prob P, CombineArgs C, int per) {
  const int b = (int)blockIdx.x;
  w4a8w_tile<1, kNT, false, false, true, true, false, kK>(P, b % kXcd, b / kXcd, per, &C);
}

// Launches of at most this many waves (decode batches) take the deep
// register ring: the chip then holds every wave at once with spare
// registers, and the weight stream, not the products, sets the pace.
constexpr int64_t kDeepRingWaves = 2048;

// The merged gate/up takes two column pairs per wave, and the merged down
// four column tiles per routed wave, from this many two-tile waves on.
constexpr int64_t kWideGateUpWaves = 4096;

// The shared down takes one 32-column tile per wave up to this many tokens.
constexpr int64_t kNarrowSharedDownRows = 256;

// Two row tiles per wave once that still gives at least 4 waves per SIMD
// (256 CUs x 4 SIMDs): half the weight traffic per MFMA, fewer waves.
bool two_row_tiles(const ExpertArgs& a, int nsplit) {
  const int64_t tiles64 = tile_bound(a, 64);
  return tiles64 * nsplit >= 4096;
}

// Logical tiles of a problem with bm-row tiles (routed: worst case).
int64_t n_tiles(const ExpertArgs& a, int bm, int nsplit) {
  return tile_bound(a, bm) * nsplit;
}

unsigned grid_of(int64_t n) { return (unsigned)(kXcd * ((n + kXcd - 1) / kXcd)); }

W4A8Prob gateup_prob(const ExpertArgs& a, const int8_t* xq, const float* sx, const uint8_t* wq,
                     const float* ws, float* a_buf, int32_t* isum) {
  return W4A8Prob{a, a.h / 32, a.d, 2 * a.h, xq, sx, wq, ws, a_buf, isum};
}

W4A8Prob down_prob(const ExpertArgs& a, const int8_t* hq, const float* hs, const uint8_t* wq,
                   const float* ws, float* f, int32_t* isum) {
  ExpertArgs b = a;
  b.perm = nullptr;
  return W4A8Prob{b, a.d / 64, a.h, a.d, hq, hs, wq, ws, f, isum};
}

template <bool kGateUp>
hipError_t launch_prob(const W4A8Prob& P, hipStream_t st) {
  const dim3 block(64);
  const ExpertArgs& a = P.a;
  const bool dense = a.offsets == nullptr;
  if (P.isum) {  // test twin (routed only): one row tile per wave
    hipLaunchKernelGGL((k_w4a8w<1, kGateUp, true, false>), dim3(grid_of(n_tiles(a, 32, P.nsplit))),
                       block, 0, st, P);
  } else if (two_row_tiles(a, P.nsplit)) {
    const dim3 grid(grid_of(n_tiles(a, 64, P.nsplit)));
    if (dense)
      hipLaunchKernelGGL((k_w4a8w<2, kGateUp, false, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((k_w4a8w<2, kGateUp, false, false>), grid, block, 0, st, P);
  } else {
    const dim3 grid(grid_of(n_tiles(a, 32, P.nsplit)));
    if (dense)
      hipLaunchKernelGGL((k_w4a8w<1, kGateUp, false, true>), grid, block, 0, st, P);
    else
      hipLaunchKernelGGL((k_w4a8w<1, kGateUp, false, false>), grid, block, 0, st, P);
  }
  return hipGetLastError();
}

// Routed problem R and dense problem D in one launch; each keeps the row
// tiles it would get on its own.
template <bool kGateUp>
hipError_t launch_pair(const W4A8Prob& R, const W4A8Prob& D0, hipStream_t st) {
  const dim3 block(64);
  // down of few tokens: the shared down's tiles would be few waves each
  // running the long h_s reduction; one 32-column tile per wave doubles them
  const bool narrow = !kGateUp && D0.a.rows <= kNarrowSharedDownRows;
  W4A8Prob D = D0;
  if (narrow) D.nsplit = D0.N / 32;
  const bool r2 = two_row_tiles(R.a, R.nsplit), d2 = two_row_tiles(D.a, D.nsplit);
  const int64_t n0 = n_tiles(R.a, r2 ? 64 : 32, R.nsplit);
  const int64_t n1 = n_tiles(D.a, d2 ? 64 : 32, D.nsplit);
  const int per1 = (int)(grid_of(n1) / kXcd);
  const dim3 grid(grid_of(n0) + grid_of(n1));
  if constexpr (kGateUp) {
    // two (gate, up) column pairs per wave when the one-pair form would have
    // more waves than the chip holds at once: each activation fragment feeds
    // four products instead of two, and the launch is closer to one wave
    // per slot (S prefill: 44.5 against 46.1 us; with fewer tiles, as in
    // decode batches, the one-pair form is faster)
    if (!r2 && !d2 && n0 + n1 >= kWideGateUpWaves && R.a.h % 64 == 0 && D.a.h % 64 == 0) {
      // (half the column splits: still one row tile per wave)
      W4A8Prob R2 = R, D2 = D;
      R2.nsplit = R.a.h / 64;
      D2.nsplit = D.a.h / 64;
      const int64_t m0 = n_tiles(R2.a, 32, R2.nsplit), m1 = n_tiles(D2.a, 32, D2.nsplit);
      const int q1 = (int)(grid_of(m1) / kXcd);
      hipLaunchKernelGGL((k_w4a8w_pair<1, 1, true, 4, 4>), dim3(grid_of(m0) + grid_of(m1)), block, 0,
                         st, R2, D2, q1);
      return hipGetLastError();
    }
  }
  if constexpr (!kGateUp) {
    // the routed down with four 32-column tiles per wave on a large launch:
    // its reduction is short (h), so each wave's first loads weigh on it
    // (S prefill: 23.1 against 24.1 us; the shared down, with its long h_s
    // reduction, keeps two: with four, 27.4 us)
    if (!narrow && !r2 && !d2 && n0 + n1 >= kWideGateUpWaves && R.N % 128 == 0) {
      W4A8Prob R2 = R;
      R2.nsplit = R.N / 128;
      const int64_t m0 = n_tiles(R2.a, 32, R2.nsplit);
      hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false, 2, 4>), dim3(grid_of(m0) + grid_of(n1)), block, 0,
                         st, R2, D, per1);
      return hipGetLastError();
    }
    if (narrow) {
      if (r2)
        hipLaunchKernelGGL((k_w4a8w_pair<2, 1, false, 1>), grid, block, 0, st, R, D, per1);
      else if (n0 + n1 <= kDeepRingWaves)
        hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false, 1, 2, true>), grid, block, 0, st, R, D, per1);
      else
        hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false, 1>), grid, block, 0, st, R, D, per1);
      return hipGetLastError();
    }
  }
  if (r2 && d2)
    hipLaunchKernelGGL((k_w4a8w_pair<2, 2, kGateUp>), grid, block, 0, st, R, D, per1);
  else if (r2)
    hipLaunchKernelGGL((k_w4a8w_pair<2, 1, kGateUp>), grid, block, 0, st, R, D, per1);
  else if (d2)
    hipLaunchKernelGGL((k_w4a8w_pair<1, 2, kGateUp>), grid, block, 0, st, R, D, per1);
  else if (n0 + n1 <= kDeepRingWaves)
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, kGateUp, 2, 2, true>), grid, block, 0, st, R, D, per1);
  else
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, kGateUp>), grid, block, 0, st, R, D, per1);
  return hipGetLastError();
}

// Routed down, then the shared down with the combine in its epilogue
// (y written, no ys).  The routed launch keeps the tile forms of the merged
// launch; the shared launch takes two 32-column tiles per wave.  Used from
// kCmbMinTokens tokens on: there the combine launch it replaces (which
// reads every routed and shared output row once more) costs more than the
// second launch and the gathers in the epilogue (M prefill: routed down
// 69 + shared down with the combine 70 us, against 108 us for the merged
// down and 39 us for the combine; S prefill, 2048 tokens: 17 + 18 against
// 23 + 8 us).
constexpr int64_t kCmbMinTokens = 4096;

hipError_t launch_down_cmb(const W4A8Prob& R, const W4A8Prob& D0, const CombineArgs& C,
                           hipStream_t st) {
  const dim3 block(64);
  const bool r2 = two_row_tiles(R.a, R.nsplit);
  const int64_t n0 = n_tiles(R.a, r2 ? 64 : 32, R.nsplit);
  if (!r2 && n0 >= kWideGateUpWaves && R.N % 128 == 0) {
    W4A8Prob R2 = R;
    R2.nsplit = R.N / 128;
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false, 2, 4>), dim3(grid_of(n_tiles(R2.a, 32, R2.nsplit))),
                       block, 0, st, R2, D0, 0);
  } else if (r2) {
    hipLaunchKernelGGL((k_w4a8w_pair<2, 1, false>), dim3(grid_of(n0)), block, 0, st, R, D0, 0);
  } else if (n0 <= kDeepRingWaves) {
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false, 2, 2, true>), dim3(grid_of(n0)), block, 0, st, R, D0,
                       0);
  } else {
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, false>), dim3(grid_of(n0)), block, 0, st, R, D0, 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  W4A8Prob D = D0;
  D.nsplit = D0.N / 64;
  const unsigned g1 = grid_of(n_tiles(D.a, 32, D.nsplit));
  const int per = (int)(g1 / kXcd);
  if (C.k <= 4)
    hipLaunchKernelGGL((k_w4a8w_shared_cmb<2, 4>), dim3(g1), block, 0, st, D, C, per);
  else
    hipLaunchKernelGGL((k_w4a8w_shared_cmb<2, 8>), dim3(g1), block, 0, st, D, C, per);
  return hipGetLastError();
}

}  // namespace

bool down_cmb_fits(const ExpertArgs& ar, const ExpertArgs& as) {
  return ar.k >= 1 && ar.k <= kMaxCmbK && as.rows == ar.T && ar.d % 64 == 0 &&
         ar.T >= kCmbMinTokens;
}

hipError_t launch_down_i4_mfma_cmb(const ExpertArgs& ar, const ExpertArgs& as, const int8_t* hq_r,
                                   const float* hs_r, const int8_t* hq_s, const float* hs_s,
                                   const uint8_t* wq_r, const float* ws_r, const uint8_t* wq_s,
                                   const float* ws_s, float* f, const int32_t* inv_perm,
                                   const float* topk_w, float* y, hipStream_t st) {
  if (!down_cmb_fits(ar, as)) return hipErrorInvalidValue;
  const CombineArgs C{f, inv_perm, topk_w, y, ar.rows, ar.k};
  return launch_down_cmb(down_prob(ar, hq_r, hs_r, wq_r, ws_r, f, nullptr),
                         down_prob(as, hq_s, hs_s, wq_s, ws_s, nullptr, nullptr), C, st);
}

hipError_t launch_gateup_i4_mfma(const ExpertArgs& a, const int8_t* xq, const float* sx,
                                 const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum,
                                 hipStream_t st) {
  return launch_prob<true>(gateup_prob(a, xq, sx, wq, ws, a_buf, isum), st);
}

hipError_t launch_down_i4_mfma(const ExpertArgs& a, const int8_t* hq, const float* hs,
                               const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                               hipStream_t st) {
  return launch_prob<false>(down_prob(a, hq, hs, wq, ws, f, isum), st);
}

hipError_t launch_gateup_i4_mfma_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                      const int8_t* xq, const float* sx, const uint8_t* wq_r,
                                      const float* ws_r, const uint8_t* wq_s, const float* ws_s,
                                      float* abuf_r, float* abuf_s, hipStream_t st) {
  return launch_pair<true>(gateup_prob(ar, xq, sx, wq_r, ws_r, abuf_r, nullptr),
                           gateup_prob(as, xq, sx, wq_s, ws_s, abuf_s, nullptr), st);
}

hipError_t launch_down_i4_mfma_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                    const int8_t* hq_r, const float* hs_r, const int8_t* hq_s,
                                    const float* hs_s, const uint8_t* wq_r, const float* ws_r,
                                    const uint8_t* wq_s, const float* ws_s, float* f, float* ys,
                                    hipStream_t st) {
  return launch_pair<false>(down_prob(ar, hq_r, hs_r, wq_r, ws_r, f, nullptr),
                            down_prob(as, hq_s, hs_s, wq_s, ws_s, ys, nullptr), st);
}

}  // namespace mm
