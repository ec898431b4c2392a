// BF16-weight expert products on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, FP32 accumulation).
//
// MobileMoE close reading, section "Custom MoE kernel": per expert, one fused
// gate/up product over its contiguous (expert-sorted) rows with SwiGLU, then
// the down product.  In the BF16-weight format the token rows, the weights and
// the hidden rows are BF16 (round to nearest even) and products accumulate in
// FP32; no quantisation scales are involved, so the MFMA accumulates straight
// into the output registers.
//
// Three forms, chosen by row count (launch_*_bf16_mfma below):
//  - k_bf16_lds, 128 rows and more: four waves share a 128-row x 128-weight-row
//    tile staged through LDS in double-buffered K blocks of 32 (each global
//    byte feeds two waves' matrix-core products);
//  - k_bf16w, fewer rows: a workgroup is one wave that owns kMT x 32 rows of
//    one expert and two 32-column tiles (gate/up: the gate tile and the
//    matching up tile of the same 32 hidden columns, so SwiGLU is applied in
//    registers); each lane loads 16 bytes (8 BF16 values) of its row per
//    operand and K step of 16, two K steps at a time, one stage ahead of the
//    math; no LDS, no barriers; tiles are ordered row tile fastest, so the
//    waves working on one column slice of an expert share it in L2;
//  - k_bf16_gemv, decode batches (a few rows per expert): weight streaming,
//    each wave one weight row pair with all of its 16-byte loads issued before
//    the math, FP32 dot products reduced across the wave.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef const __attribute__((address_space(1))) v4i gv4i;

constexpr int kXcd = 8;

template <int kMT>
struct BStage {
  v4i a[2][kMT];
  v4i b[2][2];
};

template <int kMT>
__device__ __forceinline__ void bload(BStage<kMT>& st, gv4i* const (&pa)[kMT],
                                      gv4i* const (&pb)[2], int s0) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int m = 0; m < kMT; ++m) st.a[i][m] = pa[m][2 * (s0 + i)];
#pragma unroll
    for (int j = 0; j < 2; ++j) st.b[i][j] = pb[j][2 * (s0 + i)];
  }
}

template <int kMT>
__device__ __forceinline__ void bcompute(v16f (&acc)[kMT][2], const BStage<kMT>& st) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int m = 0; m < kMT; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(v8bf, st.a[i][m]), __builtin_bit_cast(v8bf, st.b[i][j]),
            acc[m][j], 0, 0, 0);
}

// act: BF16 rows [.][K] (gate/up: the token rows, gathered through perm;
// down: the sorted hidden rows); w: BF16 [E][wrows][K].  out: gate/up -> BF16
// hidden rows [rows][h]; down -> FP32 [rows][N].  K % 32 == 0.
template <int kMT, bool kGateUp, bool kDense>
__global__ __launch_bounds__(64) void k_bf16w(ExpertArgs a, int nsplit, int n_mt, int K, int N,
                                              const uint16_t* __restrict__ act,
                                              const uint16_t* __restrict__ w,
                                              void* __restrict__ out) {
  constexpr int kBM = 32 * kMT;
  const int lane = threadIdx.x;
  const int per = (int)gridDim.x / kXcd;
  const int logical = ((int)blockIdx.x % kXcd) * per + (int)blockIdx.x / kXcd;
  const int mt = logical % n_mt, split = logical / n_mt;
  if (split >= nsplit) return;
  const int rows = (int)a.rows;
  int p0, n, e;
  if constexpr (kDense) {
    p0 = mt * kBM;
    n = min(kBM, rows - p0);
    e = 0;
  } else {
    routed_tile_wave(a.offsets, a.E, rows, kBM, mt, p0, n, e);
  }
  if (n <= 0) return;
  const int h = a.h;
  int col0, rb[2];
  if constexpr (kGateUp) {
    col0 = split * 32;
    rb[0] = split;
    rb[1] = h / 32 + split;
  } else {
    col0 = split * 64;
    rb[0] = 2 * split;
    rb[1] = 2 * split + 1;
  }
  // this lane's activation rows (padding rows read the tile's first row;
  // their results are never stored)
  gv4i* pa[kMT];
#pragma unroll
  for (int m = 0; m < kMT; ++m) {
    const int r = m * 32 + (lane & 31);
    const int rr = r < n ? r : 0;
    int src = p0 + rr;
    if constexpr (kGateUp && !kDense) {
      src = a.perm[p0 + rr] / a.k;
      if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
    }
    pa[m] = (gv4i*)(act + (int64_t)src * K + 8 * (lane >> 5));
  }
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : N;
  gv4i* pb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    pb[j] = (gv4i*)(w + ((int64_t)e * wrows + rb[j] * 32 + (lane & 31)) * K + 8 * (lane >> 5));

  v16f acc[kMT][2];
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = v16f{};

  // Stages of two K steps (32 columns); the pointers advance 64 columns per
  // iteration; the last iteration's prefetch re-reads its own second stage.
  const int S = K / 16;  // K steps
  BStage<kMT> s0, s1;
  bload(s0, pa, pb, 0);
  for (int s = 0; s < S; s += 4) {
    if (s + 2 >= S) {  // K % 64 == 32: a last single stage
      __builtin_amdgcn_sched_barrier(0);
      bcompute(acc, s0);
      break;
    }
    bload(s1, pa, pb, 2);
    __builtin_amdgcn_sched_barrier(0);
    bcompute(acc, s0);
    __builtin_amdgcn_sched_barrier(0);
    const int adv = s + 4 < S ? 4 : 2;
#pragma unroll
    for (int m = 0; m < kMT; ++m) pa[m] += adv * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) pb[j] += adv * 2;
    if (s + 4 < S) bload(s0, pa, pb, 0);
    __builtin_amdgcn_sched_barrier(0);
    bcompute(acc, s1);
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= n) continue;
      if constexpr (kGateUp) {
        const float v = silu(acc[m][0][r]) * acc[m][1][r];
        reinterpret_cast<uint16_t*>(out)[(int64_t)(p0 + row) * h + col0 + (lane & 31)] =
            f32_to_bf16(v);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          reinterpret_cast<float*>(out)[(int64_t)(p0 + row) * N + col0 + j * 32 + (lane & 31)] =
              acc[m][j][r];
      }
    }
}

// Workgroup-tiled form for shapes with enough rows: 4 waves share one tile of
// 128 rows of one expert and 128 weight rows (gate/up: the 64 gate rows and
// the 64 matching up rows of 64 hidden columns; down: 128 output columns),
// staged through LDS in K blocks of 32 (double-buffered; the global loads of
// block kb + 1 are in flight during the math of block kb).  Wave (wm, wn)
// computes rows wm*64 .. +63 against weight rows wn*32 .. +31 and 64 + wn*32
// .. +31 (gate/up) or wn*64 .. +63 (down), 2 x 2 MFMA tiles, so each operand
// byte read from global memory feeds two waves' MFMAs.  LDS rows are padded
// to 80 bytes, which keeps the 16-byte fragment reads of 8 consecutive lanes
// on distinct banks.
constexpr int kLBM = 128;   // rows (and weight rows) per workgroup
constexpr int kLBK = 32;    // K block
constexpr int kLRow = 40;   // LDS row stride in BF16 elements (80 bytes)

template <bool kGateUp, bool kDense>
__global__ __launch_bounds__(256) void k_bf16_lds(ExpertArgs a, int nsplit, int n_mt, int K,
                                                  int N, const uint16_t* __restrict__ act,
                                                  const uint16_t* __restrict__ w,
                                                  void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kLBM * kLRow];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kLBM * kLRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int per = (int)gridDim.x / kXcd;
  const int logical = ((int)blockIdx.x % kXcd) * per + (int)blockIdx.x / kXcd;
  const int mt = logical % n_mt, split = logical / n_mt;
  if (split >= nsplit) return;  // the whole workgroup
  const int rows = (int)a.rows;
  int p0, n, e;
  if constexpr (kDense) {
    p0 = mt * kLBM;
    n = min(kLBM, rows - p0);
    e = 0;
  } else {
    routed_tile_wave(a.offsets, a.E, rows, kLBM, mt, p0, n, e);  // every wave: same tile
  }
  if (n <= 0) return;  // the whole workgroup
  const int h = a.h;
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : N;

  // Global -> LDS: thread t moves 16 bytes (8 values) of rows t/4 and t/4 + 64
  // of both operands per K block (chunk t % 4 of the block's 32 values).
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  const uint16_t* ga[2];
  const uint16_t* gb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = lr + 64 * i;
    const int rr = r < n ? r : 0;  // padding rows read the tile's first row (never stored)
    int src = p0 + rr;
    if constexpr (kGateUp && !kDense) {
      src = a.perm[p0 + rr] / a.k;
      if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
    }
    ga[i] = act + (int64_t)src * K + lc;
    // weight row r of the tile
    int64_t wr;
    if constexpr (kGateUp) wr = r < 64 ? split * 64 + r : h + split * 64 + (r - 64);
    else wr = (int64_t)split * kLBM + r;
    gb[i] = w + ((int64_t)e * wrows + wr) * K + lc;
  }
  v4i ra0, ra1, rb0, rb1;  // one K block of both operands in flight
  // this lane's fragment rows in the tile
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  int arow[2], brow[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) arow[m] = wm * 64 + m * 32 + fr;
  if constexpr (kGateUp) {
    brow[0] = wn * 32 + fr;
    brow[1] = 64 + wn * 32 + fr;
  } else {
    brow[0] = wn * 64 + fr;
    brow[1] = wn * 64 + 32 + fr;
  }

  v16f acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = v16f{};

  const int KB = K / kLBK;
  uint16_t* const sa0 = &sA[0][lr * kLRow + lc];
  uint16_t* const sb0 = &sB[0][lr * kLRow + lc];
  constexpr int kBuf = kLBM * kLRow, kHalf = 64 * kLRow;
  ra0 = *reinterpret_cast<const v4i*>(ga[0]);
  ra1 = *reinterpret_cast<const v4i*>(ga[1]);
  rb0 = *reinterpret_cast<const v4i*>(gb[0]);
  rb1 = *reinterpret_cast<const v4i*>(gb[1]);
  *reinterpret_cast<v4i*>(sa0) = ra0;
  *reinterpret_cast<v4i*>(sa0 + kHalf) = ra1;
  *reinterpret_cast<v4i*>(sb0) = rb0;
  *reinterpret_cast<v4i*>(sb0 + kHalf) = rb1;
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < KB) {
      const int o = (kb + 1) * kLBK;
      ra0 = *reinterpret_cast<const v4i*>(ga[0] + o);
      ra1 = *reinterpret_cast<const v4i*>(ga[1] + o);
      rb0 = *reinterpret_cast<const v4i*>(gb[0] + o);
      rb1 = *reinterpret_cast<const v4i*>(gb[1] + o);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i fa[2], fb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        fa[m] = *reinterpret_cast<const v4i*>(&sA[cur][arow[m] * kLRow + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const v4i*>(&sB[cur][brow[j] * kLRow + ks * 16 + fk]);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(v8bf, fa[m]), __builtin_bit_cast(v8bf, fb[j]), acc[m][j], 0, 0, 0);
    }
    if (kb + 1 < KB) {
      const int nb = (cur ^ 1) * kBuf;
      *reinterpret_cast<v4i*>(sa0 + nb) = ra0;
      *reinterpret_cast<v4i*>(sa0 + nb + kHalf) = ra1;
      *reinterpret_cast<v4i*>(sb0 + nb) = rb0;
      *reinterpret_cast<v4i*>(sb0 + nb + kHalf) = rb1;
    }
    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= n) continue;
      if constexpr (kGateUp) {
        const float v = silu(acc[m][0][r]) * acc[m][1][r];
        reinterpret_cast<uint16_t*>(out)[(int64_t)(p0 + row) * h + split * 64 + wn * 32 + fr] =
            f32_to_bf16(v);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          reinterpret_cast<float*>(out)[(int64_t)(p0 + row) * N + split * kLBM + wn * 64 + j * 32 +
                                        fr] = acc[m][j][r];
      }
    }
}

// Few rows (decode batches): weight-streaming form.  A workgroup of 4 waves
// owns one tile of up to kGR rows of one expert (routed: found from the
// offsets, so only experts that own rows are read; dense: rows in order) and
// 4 outputs: gate/up -- wave w takes hidden column j = 4 * block + w, i.e.
// gate row j and up row h + j, and applies SwiGLU; down -- wave w takes
// output rows 8 * block + 2w and + 1.  Lane l holds the 8-value chunks l,
// l + 64, ... of K of its two weight rows and of the tile's activation rows
// (16-byte loads, all issued before the math), forms FP32 partial dot
// products of the BF16 values and the wave adds them up.
constexpr int kGR = 4;     // rows per tile
constexpr int kGMaxC = 5;  // 8-value chunks per lane: K <= 64 * 8 * 5 = 2560

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float dot8(const uint4& wv, const uint4& xv, float acc) {
  acc = fmaf(bf_lo(wv.x), bf_lo(xv.x), acc);
  acc = fmaf(bf_hi(wv.x), bf_hi(xv.x), acc);
  acc = fmaf(bf_lo(wv.y), bf_lo(xv.y), acc);
  acc = fmaf(bf_hi(wv.y), bf_hi(xv.y), acc);
  acc = fmaf(bf_lo(wv.z), bf_lo(xv.z), acc);
  acc = fmaf(bf_hi(wv.z), bf_hi(xv.z), acc);
  acc = fmaf(bf_lo(wv.w), bf_lo(xv.w), acc);
  return fmaf(bf_hi(wv.w), bf_hi(xv.w), acc);
}

template <bool kGateUp, bool kDense>
__global__ __launch_bounds__(256) void k_bf16_gemv(ExpertArgs a, int K, int N, int nblk,
                                                   const uint16_t* __restrict__ act,
                                                   const uint16_t* __restrict__ w,
                                                   void* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = (int)blockIdx.x / nblk, blk = (int)blockIdx.x % nblk;
  const int rows = (int)a.rows;
  int p0, n, e;
  if constexpr (kDense) {
    p0 = tile * kGR;
    n = min(kGR, rows - p0);
    e = 0;
  } else {
    routed_tile_wave(a.offsets, a.E, rows, kGR, tile, p0, n, e);  // every wave: same tile
  }
  if (n <= 0) return;
  const int h = a.h;
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : N;
  int r0, r1;
  if constexpr (kGateUp) {
    r0 = blk * 4 + wave;
    r1 = h + r0;
  } else {
    r0 = blk * 8 + 2 * wave;
    r1 = r0 + 1;
  }
  const uint4* w0 = reinterpret_cast<const uint4*>(w + ((int64_t)e * wrows + r0) * K);
  const uint4* w1 = reinterpret_cast<const uint4*>(w + ((int64_t)e * wrows + r1) * K);
  const int nc = K / 8;
  uint4 wv0[kGMaxC], wv1[kGMaxC], xv[kGR][kGMaxC];
#pragma unroll
  for (int c = 0; c < kGMaxC; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nc) {
      wv0[c] = w0[ch];
      wv1[c] = w1[ch];
    }
  }
#pragma unroll
  for (int r = 0; r < kGR; ++r) {
    if (r >= n) break;
    int src = p0 + r;
    if constexpr (kGateUp && !kDense) {
      src = a.perm[p0 + r] / a.k;
      if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
    }
    const uint4* xr = reinterpret_cast<const uint4*>(act + (int64_t)src * K);
#pragma unroll
    for (int c = 0; c < kGMaxC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) xv[r][c] = xr[ch];
    }
  }
  float acc0[kGR], acc1[kGR];
#pragma unroll
  for (int r = 0; r < kGR; ++r) {
    acc0[r] = 0.0f;
    acc1[r] = 0.0f;
    if (r >= n) continue;
#pragma unroll
    for (int c = 0; c < kGMaxC; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nc) {
        acc0[r] = dot8(wv0[c], xv[r][c], acc0[r]);
        acc1[r] = dot8(wv1[c], xv[r][c], acc1[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kGR; ++r) {
    if (r >= n) break;
    const float g = wave_sum(acc0[r]), u = wave_sum(acc1[r]);
    if (lane == 0) {
      if constexpr (kGateUp) {
        reinterpret_cast<uint16_t*>(out)[(int64_t)(p0 + r) * h + r0] = f32_to_bf16(silu(g) * u);
      } else {
        float* o = reinterpret_cast<float*>(out) + (int64_t)(p0 + r) * N;
        o[r0] = g;
        o[r1] = u;
      }
    }
  }
}

// The weight-streaming form applies: few rows (a decode batch), K a multiple
// of 8 up to 2560, and whole groups of outputs (gate/up: h % 4, down: N % 8).
bool bf16_gemv_fits(const ExpertArgs& a, int K, bool gateup, int N) {
  const bool few = a.offsets ? a.rows <= 64 : a.rows <= 16;
  return few && K % 8 == 0 && K <= 64 * 8 * kGMaxC && (gateup ? a.h % 4 == 0 : N % 8 == 0);
}

unsigned gemv_tiles_bf16(const ExpertArgs& a) { return (unsigned)tile_bound(a, kGR); }

unsigned grid_bf16(int n_mt, int nsplit) {
  const int64_t n = (int64_t)n_mt * nsplit;
  return (unsigned)(kXcd * ((n + kXcd - 1) / kXcd));
}

int n_row_tiles(const ExpertArgs& a, int bm) {
  return (int)tile_bound(a, bm);
}

}  // namespace

hipError_t launch_gateup_bf16_mfma(const ExpertArgs& a, const uint16_t* xb, const uint16_t* w,
                                   uint16_t* h_out, hipStream_t st) {
  if (bf16_gemv_fits(a, a.d, true, 2 * a.h)) {
    const int nblk = a.h / 4;
    const dim3 grid(gemv_tiles_bf16(a) * nblk), block(256);
    if (!a.offsets)
      hipLaunchKernelGGL((k_bf16_gemv<true, true>), grid, block, 0, st, a, a.d, 2 * a.h, nblk, xb,
                         w, h_out);
    else
      hipLaunchKernelGGL((k_bf16_gemv<true, false>), grid, block, 0, st, a, a.d, 2 * a.h, nblk, xb,
                         w, h_out);
    return hipGetLastError();
  }
  if (a.h % 64 == 0 && a.d % kLBK == 0 && a.rows >= kLBM) {
    const int nsplit = a.h / 64, n_mt = n_row_tiles(a, kLBM);
    const dim3 grid(grid_bf16(n_mt, nsplit)), block(256);
    if (!a.offsets)
      hipLaunchKernelGGL((k_bf16_lds<true, true>), grid, block, 0, st, a, nsplit, n_mt, a.d,
                         2 * a.h, xb, w, h_out);
    else
      hipLaunchKernelGGL((k_bf16_lds<true, false>), grid, block, 0, st, a, nsplit, n_mt, a.d,
                         2 * a.h, xb, w, h_out);
    return hipGetLastError();
  }
  const int nsplit = a.h / 32, n_mt = n_row_tiles(a, 64);
  const dim3 grid(grid_bf16(n_mt, nsplit)), block(64);
  if (!a.offsets)
    hipLaunchKernelGGL((k_bf16w<2, true, true>), grid, block, 0, st, a, nsplit, n_mt, a.d, 2 * a.h,
                       xb, w, h_out);
  else
    hipLaunchKernelGGL((k_bf16w<2, true, false>), grid, block, 0, st, a, nsplit, n_mt, a.d,
                       2 * a.h, xb, w, h_out);
  return hipGetLastError();
}

hipError_t launch_down_bf16_mfma(const ExpertArgs& a, const uint16_t* hb, const uint16_t* w,
                                 float* f, hipStream_t st) {
  ExpertArgs b = a;
  b.perm = nullptr;
  if (bf16_gemv_fits(b, a.h, false, a.d)) {
    const int nblk = a.d / 8;
    const dim3 grid(gemv_tiles_bf16(b) * nblk), block(256);
    if (!b.offsets)
      hipLaunchKernelGGL((k_bf16_gemv<false, true>), grid, block, 0, st, b, a.h, a.d, nblk, hb, w,
                         f);
    else
      hipLaunchKernelGGL((k_bf16_gemv<false, false>), grid, block, 0, st, b, a.h, a.d, nblk, hb, w,
                         f);
    return hipGetLastError();
  }
  if (a.d % kLBM == 0 && a.h % kLBK == 0 && a.rows >= kLBM) {
    const int nsplit = a.d / kLBM, n_mt = n_row_tiles(b, kLBM);
    const dim3 grid(grid_bf16(n_mt, nsplit)), block(256);
    if (!b.offsets)
      hipLaunchKernelGGL((k_bf16_lds<false, true>), grid, block, 0, st, b, nsplit, n_mt, a.h, a.d,
                         hb, w, f);
    else
      hipLaunchKernelGGL((k_bf16_lds<false, false>), grid, block, 0, st, b, nsplit, n_mt, a.h,
                         a.d, hb, w, f);
    return hipGetLastError();
  }
  const int nsplit = a.d / 64, n_mt = n_row_tiles(b, 64);
  const dim3 grid(grid_bf16(n_mt, nsplit)), block(64);
  if (!b.offsets)
    hipLaunchKernelGGL((k_bf16w<2, false, true>), grid, block, 0, st, b, nsplit, n_mt, a.h, a.d,
                       hb, w, f);
  else
    hipLaunchKernelGGL((k_bf16w<2, false, false>), grid, block, 0, st, b, nsplit, n_mt, a.h, a.d,
                       hb, w, f);
  return hipGetLastError();
}

}  // namespace mm
