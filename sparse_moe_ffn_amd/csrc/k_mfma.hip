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

// One wave's registers for two groups: activation fragments, packed weight
// fragments and scales.
// Global-address-space views: loads through them are global_load (not flat),
// which keeps the memory counter in order and lets the prefetch stay in
// flight across the math.
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) v4i gint4;
typedef const __attribute__((address_space(1))) v2u guint2;
typedef const __attribute__((address_space(1))) float gfloat;

template <int kMT, int kNT>
struct WStage {
  v4i a[2][kMT];
  v2u b[2][kNT];
  float s[2][kNT];
};

// Loads groups g0 and g0 + 1 relative to the current pointers (row-major
// activations: the offsets are compile-time constants and fold into the load
// instructions; group-major: astride, the 16-byte units from one group to
// the next, is the row count times 2).  pb / ps are wave-uniform (the lane
// offset is added here), so the loads take a scalar base and a small
// per-lane offset.
template <int kMT, int kNT>
__device__ __forceinline__ void wload(WStage<kMT, kNT>& st, gint4* const (&pa)[kMT],
                                      guint2* const (&pb)[kNT], gfloat* const (&ps)[kNT],
                                      int g0, int lane, int astride) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int m = 0; m < kMT; ++m) st.a[i][m] = pa[m][(g0 + i) * astride];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      st.b[i][j] = pb[j][(g0 + i) * 64 + lane];
      st.s[i][j] = ps[j][(g0 + i) * 32 + (lane & 31)];
    }
  }
}

// Two groups: per group one MFMA per (row tile, column tile) from a zero
// accumulator (the exact int32 group sum), then acc = fma(scale, sum, acc).
// The epilogue of one tile is placed after the next tile's MFMA so that the
// matrix core and the vector ALU work at the same time.
template <int kMT, int kNT, bool kCapture>
__device__ __forceinline__ void wcompute(v16f (&acc)[kMT][kNT], const WStage<kMT, kNT>& st,
                                         int g0, int lane, const int (&rb)[kNT],
                                         const Capture& cap) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v4i bv[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) bv[j] = unpack16(make_uint2(st.b[i][j].x, st.b[i][j].y));
    v16i R[kMT][kNT];
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
      for (int j = 0; j < kNT; ++j)
        R[m][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(st.a[i][m], bv[j], v16i{}, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][j][r] = fmaf(st.s[i][j], (float)R[m][j][r], acc[m][j][r]);
        if (kCapture) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < cap.n) {
              const int64_t col = (int64_t)rb[j] * 32 + (lane & 31);
              cap.isum[(((int64_t)(cap.p0 + row)) * cap.wrows + col) * cap.G + g0 + i] =
                  R[m][j][r] >> 4;
            }
          }
        }
      }
  }
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

// Workgroup b runs on XCD b % 8 as that XCD's slot b / 8.  Each XCD works
// through a contiguous range of logical tile ids (the same expert's weights
// stay in its L2): slot i of XCD x takes logical id x * per + i, with per the
// problem's tile count over 8.  A routed problem's real tile count is only
// known from the offsets, so it is counted in the kernel (the grid is sized
// for the worst case) and the spare slots exit; the empty tail is thereby
// spread over the XCDs instead of idling the last ones.
//
// One tile (kMT row tiles x kNT column tiles) of problem P for XCD x, slot
// i; logical id = mt * nsplit + split.  kDense: rows are the tokens in order
// (shared expert), per_dense its slots per XCD; otherwise routed
// (expert-sorted rows, tiles found from the offsets).  kGM: the activations
// are group-major (act_offset in common.h), so a tile's 32 rows of one group
// are read from one contiguous kilobyte when the rows are consecutive.
// K % 128 == 0.  Called by one whole wave.
template <int kMT, int kNT, bool kGateUp, bool kCapture, bool kDense, bool kGM = false>
__device__ __forceinline__ void w4a8w_tile(const W4A8Prob& P, int x, int i, int per_dense) {
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
  gint4* pa[kMT];
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
    pa[m] = (gint4*)(act + (int64_t)src * (kGM ? 32 : K) + 16 * (lane >> 5));
    srow[m] = act_scale[src];
  }
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : N;
  const uint8_t* we = wq + (int64_t)e * (wrows / 32) * G * kChunkBytes;
  const float* se = wsc + (int64_t)e * (wrows / 32) * G * 32;
  guint2* pb[kNT];
  gfloat* ps[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    pb[j] = (guint2*)(we + (int64_t)rb[j] * G * kChunkBytes);
    ps[j] = (gfloat*)(se + (int64_t)rb[j] * G * 32);
  }
  const Capture cap{isum, wrows, G, p0, n};
  // activation rows: x_q has T, the hidden rows have `rows`
  const int astride = kGM ? 2 * (int)(kGateUp ? a.T : a.rows) : kGroup / 16;

  v16f acc[kMT][kNT];
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[m][j] = v16f{};

  // Two register stages in ping-pong, each two groups; the pointers advance
  // four groups per iteration.  The last iteration's prefetch re-reads its
  // own second stage (valid addresses, result unused).  G % 4 == 0.
  WStage<kMT, kNT> s0, s1;
  wload(s0, pa, pb, ps, 0, lane, astride);
  for (int g = 0; g < G; g += 4) {
    wload(s1, pa, pb, ps, 2, lane, astride);
    __builtin_amdgcn_sched_barrier(0);
    wcompute<kMT, kNT, kCapture>(acc, s0, g, lane, rb, cap);
    __builtin_amdgcn_sched_barrier(0);
    const int adv = g + 4 < G ? 4 : 2;
#pragma unroll
    for (int m = 0; m < kMT; ++m) pa[m] += adv * astride;
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      pb[j] += adv * 64;
      ps[j] += adv * 32;
    }
    wload(s0, pa, pb, ps, 0, lane, astride);
    __builtin_amdgcn_sched_barrier(0);
    wcompute<kMT, kNT, kCapture>(acc, s1, g + 2, lane, rb, cap);
    __builtin_amdgcn_sched_barrier(0);
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
      } else {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          out[(int64_t)(p0 + row) * N + col0 + j * 32 + (lane & 31)] = acc[m][j][r] * s;
      }
    }
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
// tile) go first and the short routed ones fill in behind them.
template <int kMT0, int kMT1, bool kGateUp>
__global__ __launch_bounds__(64) void k_w4a8w_pair(W4A8Prob P0, W4A8Prob P1, int per1) {
  const int b = (int)blockIdx.x, x = b % kXcd, i = b / kXcd;
  if (i < per1)
    w4a8w_tile<kMT1, 2, kGateUp, false, true, true>(P1, x, i, per1);
  else
    w4a8w_tile<kMT0, 2, kGateUp, false, false, true>(P0, x, i - per1, 0);
}

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
hipError_t launch_pair(const W4A8Prob& R, const W4A8Prob& D, hipStream_t st) {
  const dim3 block(64);
  const bool r2 = two_row_tiles(R.a, R.nsplit), d2 = two_row_tiles(D.a, D.nsplit);
  const int64_t n0 = n_tiles(R.a, r2 ? 64 : 32, R.nsplit);
  const int64_t n1 = n_tiles(D.a, d2 ? 64 : 32, D.nsplit);
  const int per1 = (int)(grid_of(n1) / kXcd);
  const dim3 grid(grid_of(n0) + grid_of(n1));
  if (r2 && d2)
    hipLaunchKernelGGL((k_w4a8w_pair<2, 2, kGateUp>), grid, block, 0, st, R, D, per1);
  else if (r2)
    hipLaunchKernelGGL((k_w4a8w_pair<2, 1, kGateUp>), grid, block, 0, st, R, D, per1);
  else if (d2)
    hipLaunchKernelGGL((k_w4a8w_pair<1, 2, kGateUp>), grid, block, 0, st, R, D, per1);
  else
    hipLaunchKernelGGL((k_w4a8w_pair<1, 1, kGateUp>), grid, block, 0, st, R, D, per1);
  return hipGetLastError();
}

}  // namespace

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
