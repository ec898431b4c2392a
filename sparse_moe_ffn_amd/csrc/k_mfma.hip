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
// Tiling.  A workgroup (4 waves) owns 64 rows of one expert (two 32-row MFMA
// tiles) and one slice of the output columns.  The activation rows are staged
// through LDS in 128-column chunks (row stride padded by 16 bytes against bank
// conflicts) and shared by the 4 waves; each wave reads its weight fragments
// straight from the prepacked INT4 layout (csrc/common.h), which is already in
// MFMA operand order, so one 8-byte load per lane per 32x32 group is fully
// coalesced.  Nibbles are unpacked in registers to int8 (times 16; the scales
// are pre-divided by 16).  Workgroup ids are remapped so that consecutive
// tiles (same expert, neighbouring column slices) land on the same XCD and
// share its L2.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));



constexpr int kKC = 128;                 // activation columns per LDS chunk (4 groups)
constexpr int kGPC = kKC / kGroup;       // groups per chunk
constexpr int kStride16 = kKC / 16 + 1;  // LDS row stride in 16-byte units (padded)
constexpr int kXcd = 8;

struct Tile {
  int p0, n, e, split, mt;
};

// Logical tile of this workgroup.  Tiles are numbered (expert, row tile,
// column slice) with the slice fastest; workgroup b runs on XCD b % 8 and gets
// logical id (b % 8) * per + b / 8, so each XCD works on a contiguous range of
// tiles (same expert's weights in its L2).  Returns false if there is none.
template <int kBM, bool kDense>
__device__ bool map_tile(const ExpertArgs& a, int nsplit, Tile& t) {
  __shared__ int s_p0, s_n, s_e, s_split;
  const int per = (int)gridDim.x / kXcd;
  const int logical = ((int)blockIdx.x % kXcd) * per + (int)blockIdx.x / kXcd;
  const int mt = logical / nsplit;
  if (threadIdx.x < 64) {
    if constexpr (kDense) {
      if (threadIdx.x == 0) {
        s_p0 = mt * kBM;
        s_n = max(0, min(kBM, (int)a.rows - s_p0));
        s_e = 0;
      }
    } else {
      routed_tile(a.offsets, a.E, (int)a.rows, kBM, mt, &s_p0, &s_n, &s_e);
    }
    if (threadIdx.x == 0) s_split = logical % nsplit;
  }
  __syncthreads();
  t.p0 = s_p0;
  t.n = s_n;
  t.e = s_e;
  t.split = s_split;
  t.mt = mt;
  return t.n > 0;
}

__device__ __forceinline__ v4i unpack16(uint2 w) {
  uint32_t q0, q1, q2, q3;
  unpack8(w.x, q0, q1);
  unpack8(w.y, q2, q3);
  return v4i{(int)q0, (int)q1, (int)q2, (int)q3};
}

// Per-wave state of one 128-column chunk: the activation pieces this thread
// stages into LDS, and the wave's weight fragments and scales for the chunk's
// 4 groups.
template <int kLoads, int kNT>
struct Chunk {
  int4 a[kLoads];
  uint2 b[kGPC][kNT];
  float s[kGPC][kNT];
};

// Issues the global loads of chunk k0 (no value is inspected afterwards, so
// they stay in flight until the LDS store / MFMA that consumes them).
// Padding rows read row 0: their results are never stored, and each output
// row depends only on its own activation row.
template <int kBM, int kLoads, int kNT>
__device__ __forceinline__ void load_chunk(Chunk<kLoads, kNT>& c, const int8_t* __restrict__ act,
                                           const int* s_off, int K, int k0,
                                           const uint2* const (&Bp)[kNT],
                                           const float* const (&Sp)[kNT]) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int r = idx / (kKC / 16), cc = idx % (kKC / 16);
    const int src = max(s_off[r], 0);
    c.a[i] = *reinterpret_cast<const int4*>(act + (int64_t)src * K + k0 + cc * 16);
  }
#pragma unroll
  for (int gl = 0; gl < kGPC; ++gl) {
    const int g = k0 / kGroup + gl;
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      c.b[gl][j] = Bp[j][g * 64];
      c.s[gl][j] = Sp[j][g * 32];
    }
  }
}

template <int kLoads, int kNT>
__device__ __forceinline__ void store_chunk(int4* __restrict__ As, const Chunk<kLoads, kNT>& c) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = threadIdx.x + 256 * i;
    As[(idx / (kKC / 16)) * kStride16 + idx % (kKC / 16)] = c.a[i];
  }
}

// Capture of the exact group sums (test twins only).
struct Capture {
  int32_t* isum;
  int64_t wrows;
  int G, p0, n;
};

// The chunk's 4 groups for this wave: per group, one MFMA per (row tile,
// column tile) started from zero (the exact int32 group sum), then the FP32
// epilogue acc = fma(scale, (float) isum, acc).  The epilogue of group gl-1
// is placed before the MFMA of group gl on the same tile, and the scheduler
// is asked to alternate one MFMA with one tile epilogue, so matrix and vector
// work overlap within the wave.
template <int kMT, int kNT, bool kCapture, int kLoads>
__device__ __forceinline__ void compute_chunk(v16f (&acc)[kMT][kNT], const int4* __restrict__ As,
                                              const Chunk<kLoads, kNT>& c, int g0, int lane,
                                              const int (&rb)[kNT], const Capture& cap) {
  auto epi = [&](const v16i& is, float sc, v16f& ac, int m, int j, int g) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ac[r] = fmaf(sc, (float)is[r], ac[r]);
    if (kCapture) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < cap.n) {
          const int64_t col = (int64_t)rb[j] * 32 + (lane & 31);
          cap.isum[(((int64_t)(cap.p0 + row)) * cap.wrows + col) * cap.G + g] = is[r] >> 4;
        }
      }
    }
  };
  v16i R[kMT][kNT];
#pragma unroll
  for (int gl = 0; gl < kGPC; ++gl) {
    v4i bv[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) bv[j] = unpack16(c.b[gl][j]);
    v4i av[kMT];
#pragma unroll
    for (int m = 0; m < kMT; ++m) {
      const int4 a4 = As[(m * 32 + (lane & 31)) * kStride16 + gl * 2 + (lane >> 5)];
      av[m] = v4i{a4.x, a4.y, a4.z, a4.w};
    }
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (gl > 0) epi(R[m][j], c.s[gl - 1][j], acc[m][j], m, j, g0 + gl - 1);
        R[m][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[m], bv[j], v16i{}, 0, 0, 0);
      }
  }
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) epi(R[m][j], c.s[kGPC - 1][j], acc[m][j], m, j, g0 + kGPC - 1);
#pragma unroll
  for (int i = 0; i < kGPC * kMT * kNT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // one tile epilogue
  }
}

// One W4A8 product tile.  kGateUp: the wave's two column tiles are the gate
// tile and the matching up tile of 32 hidden columns (slice = 128 hidden
// columns per workgroup); output a = SiLU(g*s) * (u*s) to out [rows][h].
// Otherwise: the wave's kNT tiles are consecutive output columns (slice =
// 4 * kNT * 32 columns); output f = acc * s_row to out [rows][N].
// kMT row tiles of 32 (kBM = 32 * kMT rows per workgroup).  K % 128 == 0.
// kDense: rows are the tokens in order (shared expert); otherwise routed
// (expert-sorted rows, tiles found from the offsets).
template <int kMT, int kNT, bool kGateUp, bool kCapture, bool kDense>
__global__ __launch_bounds__(256) void k_w4a8(ExpertArgs a, int nsplit, int K, int N,
                                              const int8_t* __restrict__ act,
                                              const float* __restrict__ act_scale,
                                              const uint8_t* __restrict__ wq,
                                              const float* __restrict__ wsc,
                                              float* __restrict__ out,
                                              int32_t* __restrict__ isum) {
  constexpr int kBM = 32 * kMT;
  constexpr int kLoads = kBM * kKC / 16 / 256;  // 16-byte pieces per thread per chunk
  static_assert(kLoads * 256 == kBM * kKC / 16, "chunk must split evenly over 256 threads");
  __shared__ int4 As[2][kBM * kStride16];
  __shared__ float s_scale[kBM];
  __shared__ int s_off[kBM];  // source row of each tile row in `act`, -1 for padding
  Tile t;
  if (!map_tile<kBM, kDense>(a, nsplit, t)) return;
  const int G = K / kGroup;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = a.h;
  if (threadIdx.x < kBM) {
    const int r = threadIdx.x;
    int off = -1;
    float s = 0.0f;
    if (r < t.n) {
      int src = t.p0 + r;
      if (kGateUp && !kDense) {
        src = a.perm[t.p0 + r] / a.k;
        if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
      }
      off = src;
      s = act_scale[src];
    }
    s_off[r] = off;
    s_scale[r] = s;
  }
  // this wave's column tiles (32-row blocks of the weight matrix)
  int col0, rb[kNT];
  if (kGateUp) {
    col0 = t.split * 128 + wave * 32;
    rb[0] = col0 / 32;
    rb[1] = (h + col0) / 32;
  } else {
    col0 = t.split * (4 * kNT * 32) + wave * kNT * 32;
#pragma unroll
    for (int j = 0; j < kNT; ++j) rb[j] = col0 / 32 + j;
  }
  // Waves whose columns lie past the end compute on a valid block (0) and
  // store nothing.
  const bool active = col0 < (kGateUp ? h : N);
  const int64_t wrows = kGateUp ? 2 * h : N;
  const uint8_t* we = wq + (int64_t)t.e * (wrows / 32) * G * kChunkBytes;
  const float* se = wsc + (int64_t)t.e * (wrows / 32) * G * 32;
  const uint2* Bp[kNT];
  const float* Sp[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int rbj = active ? rb[j] : 0;
    Bp[j] = reinterpret_cast<const uint2*>(we + (int64_t)rbj * G * kChunkBytes) + lane;
    Sp[j] = se + (int64_t)rbj * G * 32 + (lane & 31);
  }
  const Capture cap{active ? isum : nullptr, wrows, G, t.p0, active ? t.n : 0};
  __syncthreads();  // s_off / s_scale ready

  v16f acc[kMT][kNT];
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[m][j] = v16f{};

  // Two register sets and two LDS buffers in ping-pong: while chunk c is
  // multiplied, chunk c+1 is in flight.  The last chunk's prefetch re-reads
  // it (valid addresses, result unused).
  Chunk<kLoads, kNT> c0, c1;
  load_chunk<kBM>(c0, act, s_off, K, 0, Bp, Sp);
  store_chunk(As[0], c0);
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += 2 * kKC) {
    {
      const int k1 = k0 + kKC < K ? k0 + kKC : k0;
      load_chunk<kBM>(c1, act, s_off, K, k1, Bp, Sp);
      __builtin_amdgcn_sched_barrier(0);  // prefetch issued before the math
      compute_chunk<kMT, kNT, kCapture>(acc, As[0], c0, k0 / kGroup, lane, rb, cap);
      __builtin_amdgcn_sched_barrier(0);  // LDS store (waits for the prefetch) after it
      store_chunk(As[1], c1);
      __syncthreads();
      if (k0 + kKC >= K) break;
    }
    {
      const int k2 = k0 + 2 * kKC < K ? k0 + 2 * kKC : k0 + kKC;
      load_chunk<kBM>(c0, act, s_off, K, k2, Bp, Sp);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk<kMT, kNT, kCapture>(acc, As[1], c1, (k0 + kKC) / kGroup, lane, rb, cap);
      __builtin_amdgcn_sched_barrier(0);
      store_chunk(As[0], c0);
      __syncthreads();
    }
  }
  if (!active) return;
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= t.n) continue;
      const float s = s_scale[row];
      if (kGateUp) {
        out[(int64_t)(t.p0 + row) * h + col0 + (lane & 31)] =
            silu(acc[m][0][r] * s) * (acc[m][1][r] * s);
      } else {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          out[(int64_t)(t.p0 + row) * N + col0 + j * 32 + (lane & 31)] = acc[m][j][r] * s;
      }
    }
}

// Grid: 8 * ceil(tiles * nsplit / 8) workgroups, tiles = worst case.
unsigned grid_for(const ExpertArgs& a, int bm, int nsplit) {
  const int64_t mt = (a.rows + bm - 1) / bm + (a.offsets ? a.E : 0);
  const int64_t n = mt * nsplit;
  return (unsigned)(kXcd * ((n + kXcd - 1) / kXcd));
}

}  // namespace

hipError_t launch_gateup_i4_mfma(const ExpertArgs& a, const int8_t* xq, const float* sx,
                                 const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum,
                                 hipStream_t st) {
  const int nsplit = (a.h + 127) / 128;
  const dim3 grid(grid_for(a, 64, nsplit));
  if (!a.offsets)
    hipLaunchKernelGGL((k_w4a8<2, 2, true, false, true>), grid, dim3(256), 0, st, a, nsplit, a.d,
                       2 * a.h, xq, sx, wq, ws, a_buf, nullptr);
  else if (isum)
    hipLaunchKernelGGL((k_w4a8<2, 2, true, true, false>), grid, dim3(256), 0, st, a, nsplit, a.d,
                       2 * a.h, xq, sx, wq, ws, a_buf, isum);
  else
    hipLaunchKernelGGL((k_w4a8<2, 2, true, false, false>), grid, dim3(256), 0, st, a, nsplit, a.d,
                       2 * a.h, xq, sx, wq, ws, a_buf, isum);
  return hipGetLastError();
}

hipError_t launch_down_i4_mfma(const ExpertArgs& a, const int8_t* hq, const float* hs,
                               const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                               hipStream_t st) {
  // routed rows (sorted order, contiguous): 64-row tiles, 256-column slices;
  // dense rows (shared expert, few row tiles): 32-row tiles, 128-column slices
  ExpertArgs b = a;
  b.perm = nullptr;
  if (a.offsets) {
    const int nsplit = (a.d + 255) / 256;
    const dim3 grid(grid_for(b, 64, nsplit));
    if (isum)
      hipLaunchKernelGGL((k_w4a8<2, 2, false, true, false>), grid, dim3(256), 0, st, b, nsplit, a.h, a.d,
                         hq, hs, wq, ws, f, isum);
    else
      hipLaunchKernelGGL((k_w4a8<2, 2, false, false, false>), grid, dim3(256), 0, st, b, nsplit, a.h, a.d,
                         hq, hs, wq, ws, f, isum);
  } else {
    const int nsplit = (a.d + 127) / 128;
    const dim3 grid(grid_for(b, 32, nsplit));
    if (isum)
      hipLaunchKernelGGL((k_w4a8<1, 1, false, true, true>), grid, dim3(256), 0, st, b, nsplit, a.h, a.d,
                         hq, hs, wq, ws, f, isum);
    else
      hipLaunchKernelGGL((k_w4a8<1, 1, false, false, true>), grid, dim3(256), 0, st, b, nsplit, a.h, a.d,
                         hq, hs, wq, ws, f, isum);
  }
  return hipGetLastError();
}

}  // namespace mm
