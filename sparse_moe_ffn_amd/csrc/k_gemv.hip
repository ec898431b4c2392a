// W4A8 products for a few rows per expert (decode batches): the weight
// stream is the whole cost, so the work is spread over the weight matrix
// rather than over the rows.
//
// MobileMoE close reading, sections "Custom MoE kernel" (per-expert product
// over the expert's contiguous rows, fused gate/up with SwiGLU, then down)
// and "Runtime latency" (decode is bound by the bytes of the selected
// experts' weights).  INT4 weights per eq. (6) (section "Quantisation-aware
// training"): output = s_act * sum_g s_w[g] * isum_g with exact int32 group
// sums isum_g, applied as the FMA chain over g ascending -- the order of the
// matrix-core and row-tile kernels and of the CPU oracle, so all agree bit for
// bit.
//
// A workgroup owns one tile of up to kR rows of one expert and one 32-row
// block of the weight matrix (for gate/up: the gate block and the matching up
// block).  Its 4 waves split the quantisation groups.  Each lane reads 16
// bytes of a pair of adjacent 512-byte chunks (groups g, g+1 of the block,
// layout in common.h), so every wave load is one fully coalesced 1 KB access
// and all of a workgroup's weight bytes are in flight before the first use.
// The exact int32 group sums go to LDS; then one thread per (row, output)
// applies the scales in group order.  Only experts that own rows have tiles,
// so only the selected experts' weights are read.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace mm {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxPairs = 10;  // group pairs per wave: K <= 2 * 32 * 4 * 10 = 2560

// First row, row count and expert of tile `tile` (routed: expert-sorted rows,
// tiles numbered expert by expert; dense: rows in order).  All threads call.
template <int kR, bool kDense>
__device__ void gemv_tile(const ExpertArgs& a, int tile, int& p0, int& n, int& e) {
  __shared__ int s_p0, s_n, s_e;
  if constexpr (kDense) {
    p0 = tile * kR;
    n = (int)min((int64_t)kR, a.rows - p0);
    e = 0;
    return;
  }
  if (threadIdx.x < 64) routed_tile(a.offsets, a.E, (int)a.rows, kR, tile, &s_p0, &s_n, &s_e);
  __syncthreads();
  p0 = s_p0;
  n = s_n;
  e = s_e;
}

// Partial group sums of one lane for one activation row: the lane holds 16
// weights (x16) of each of rows rho and rho+1, for one half of a group.
__device__ __forceinline__ void dot16x2(const uint4& w, const int4& x, int& p0, int& p1) {
  uint32_t l0, h0, l1, h1, l2, h2, l3, h3;
  unpack8(w.x, l0, h0);
  unpack8(w.y, l1, h1);
  unpack8(w.z, l2, h2);
  unpack8(w.w, l3, h3);
  int s = __builtin_amdgcn_sdot4((int)l0, x.x, 0, false);
  s = __builtin_amdgcn_sdot4((int)h0, x.y, s, false);
  s = __builtin_amdgcn_sdot4((int)l1, x.z, s, false);
  p0 = __builtin_amdgcn_sdot4((int)h1, x.w, s, false);
  s = __builtin_amdgcn_sdot4((int)l2, x.x, 0, false);
  s = __builtin_amdgcn_sdot4((int)h2, x.y, s, false);
  s = __builtin_amdgcn_sdot4((int)l3, x.z, s, false);
  p1 = __builtin_amdgcn_sdot4((int)h3, x.w, s, false);
}

// Arguments of one weight-streaming product (a launch carries one, or the
// routed and the shared problem together).
struct GemvProb {
  ExpertArgs a;
  int K, N, RB;
  const int8_t* act;
  const float* act_scale;
  const uint8_t* wq;
  const float* wsc;
  float* out;
  int32_t* isum;
  // down only, instead of act/act_scale: FP32 hidden rows [rows][K] that the
  // workgroup quantises itself (K % 128 == 0)
  const float* actf;
};

constexpr int kMaxQV = 20;  // float2 per lane of a quantised row: K <= 128 * 20

// Wave-level INT8 quantisation of one FP32 row (K % 128 == 0, K <= 128 *
// kMaxQV) into LDS: the same rule and arithmetic as the standalone quantiser
// (exact max|v| over the row, s = 2*amax/255, codes clamp(rint(v/s))), so
// its codes and scale are bit-identical.  Returns s on every lane.
__device__ __forceinline__ void load_row_regs(const float* __restrict__ x, int K, float2 (&v)[kMaxQV],
                                              int lane) {
  const int nv = K / 128;
  const float2* xr = reinterpret_cast<const float2*>(x);
#pragma unroll
  for (int i = 0; i < kMaxQV; ++i)
    if (i < nv) v[i] = xr[lane + 64 * i];
}

// The quantisation of a row already held in registers (load_row_regs).
__device__ __forceinline__ float quant_regs_lds(const float2 (&v)[kMaxQV], int K,
                                                int8_t* __restrict__ dst, int lane) {
  const int nv = K / 128;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxQV; ++i)
    if (i < nv) amax = fmaxf(amax, fmaxf(fabsf(v[i].x), fabsf(v[i].y)));
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  uint16_t* q = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
  for (int i = 0; i < kMaxQV; ++i)
    if (i < nv) {
      int8_t c0 = 0, c1 = 0;
      if (sr != 0.0f) {
        c0 = quant_i8(v[i].x, sr, yr);
        c1 = quant_i8(v[i].y, sr, yr);
      }
      q[lane + 64 * i] = (uint16_t)((uint8_t)c0 | ((uint16_t)(uint8_t)c1 << 8));
    }
  return sr;
}

__device__ __forceinline__ float quant_row_lds(const float* __restrict__ x, int K,
                                               int8_t* __restrict__ dst, int lane) {
  float2 v[kMaxQV];
  load_row_regs(x, K, v, lane);
  return quant_regs_lds(v, K, dst, lane);
}

// Block `blk` of problem P.  out: gate/up -> a = SiLU(g * s) * (u * s) into
// out [rows][h]; down -> f = acc * s into out [rows][N].  K: reduction length
// (multiple of 64, <= 2560); RB: 32-row weight blocks per output (gate/up:
// h / 32, down: N / 32).  kDense: rows are the tokens in order (shared
// expert); otherwise routed.  Called by the whole workgroup.
template <int kR, bool kGateUp, bool kCapture, bool kDense, bool kQIn = false>
__device__ __forceinline__ void gemv_block(const GemvProb& P, int blk) {
  static_assert(!kQIn || (!kGateUp && kR == 4), "in-kernel quantisation: down, one row per wave");
  const ExpertArgs& a = P.a;
  const int K = P.K, N = P.N, RB = P.RB;
  const int8_t* __restrict__ act = P.act;
  const float* __restrict__ act_scale = P.act_scale;
  const uint8_t* __restrict__ wq = P.wq;
  const float* __restrict__ wsc = P.wsc;
  float* __restrict__ out = P.out;
  int32_t* __restrict__ isum = P.isum;
  constexpr int kM = kGateUp ? 2 : 1;  // weight blocks per workgroup
  const int G = K / kGroup, GP = G / 2;
  extern __shared__ int4 smem4[];
  int32_t* s_is = reinterpret_cast<int32_t*>(smem4);              // [kM][kR][G][32]
  float* s_sc = reinterpret_cast<float*>(s_is + kM * kR * G * 32);  // [kM][G][32]
  int4* s_act = reinterpret_cast<int4*>(s_sc + kM * G * 32);        // [kR][K/16]
  __shared__ int s_src[kR];
  __shared__ float s_as[kR];
  __shared__ float s_tsc[kR];
  const int c16 = K / 16;

  // Routed gate/up of at most kR tokens: every token row (and its scale) is
  // staged before the tile is known (its rows are some of these tokens), so
  // the activation loads do not wait for the offsets and the permutation.
  const bool pre = kGateUp && !kDense && a.T <= kR;
  if (pre) {
    for (int i = threadIdx.x; i < (int)a.T * c16; i += blockDim.x)
      s_act[i] = reinterpret_cast<const int4*>(act)[i];  // rows 0..T-1 of x_q [T][K]
    if ((int)threadIdx.x < (int)a.T) s_tsc[threadIdx.x] = act_scale[threadIdx.x];
  }
  // In-kernel quantisation of a routed problem of at most kR rows: wave w
  // reads hidden row w before the tile is known (the tile's rows are some
  // of these), so those loads do not wait for the offsets either.
  const bool preq = kQIn && !kDense && a.rows <= kR;
  float2 qv[kMaxQV];
  if constexpr (kQIn) {
    const int w = (int)(threadIdx.x >> 6);
    if (preq && w < (int)a.rows) load_row_regs(P.actf + (int64_t)w * K, K, qv, threadIdx.x & 63);
  }
  const int tile = blk / RB, rbo = blk % RB;
  int p0, n, e;
  gemv_tile<kR, kDense>(a, tile, p0, n, e);  // (routed: a barrier, after which the above is visible)
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wrows = kGateUp ? 2 * (int64_t)a.h : N;
  int rbm[kM];
  rbm[0] = rbo;
  if (kGateUp) rbm[kM - 1] = rbo + a.h / 32;

  // Weight loads first: pair i of this wave is groups 2*(wave + 4i) and +1
  // (pairs past the end are neither loaded nor used).
  const uint8_t* we = wq + (int64_t)e * (wrows / 32) * G * kChunkBytes;
  uint4 wv[kMaxPairs][kM];
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int gp = wave + kWaves * i;
    if (gp < GP) {
#pragma unroll
      for (int m = 0; m < kM; ++m)
        wv[i][m] = reinterpret_cast<const uint4*>(
            we + ((int64_t)rbm[m] * G + 2 * gp) * kChunkBytes)[lane];
    }
  }

  if constexpr (kQIn) {
    // slot r of the staged rows holds hidden row p0 + r (padding slots stay
    // zero): quantised by wave r, or with pre-read rows by the wave holding
    // that row (wave p0 + r); wave r clears slot r when r >= n
    const int r = wave;
    int8_t* dst = reinterpret_cast<int8_t*>(s_act) + (int64_t)r * K;
    if (r >= n) {
      for (int c = lane; c < K / 16; c += 64) reinterpret_cast<int4*>(dst)[c] = make_int4(0, 0, 0, 0);
      if (lane == 0) s_as[r] = 0.0f;
    }
    if (preq) {
      const int slot = wave - p0;
      if (slot >= 0 && slot < n) {
        const float sr = quant_regs_lds(qv, K, reinterpret_cast<int8_t*>(s_act) + (int64_t)slot * K, lane);
        if (lane == 0) s_as[slot] = sr;
      }
    } else if (r < n) {
      const float sr = quant_row_lds(P.actf + (int64_t)(p0 + r) * K, K, dst, lane);
      if (lane == 0) s_as[r] = sr;
    }
  } else if (threadIdx.x < kR) {
    const int r = threadIdx.x;
    int src = -1;
    float s = 0.0f;
    if (r < n) {
      src = p0 + r;
      if (kGateUp && !kDense) {
        src = a.T == 1 ? 0 : a.perm[p0 + r] / a.k;
        if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
      }
      s = pre ? s_tsc[src] : act_scale[src];
    }
    s_src[r] = src;
    s_as[r] = s;
  }
  // scales of the workgroup's blocks: G * 32 contiguous floats per block
  const float* se = wsc + (int64_t)e * (wrows / 32) * G * 32;
  for (int i = threadIdx.x; i < kM * G * 32; i += blockDim.x) {
    const int m = i / (G * 32), j = i % (G * 32);
    s_sc[i] = se[(int64_t)rbm[m] * G * 32 + j];
  }
  __syncthreads();  // s_src ready (in-kernel quantisation: activations staged)
  if (!kQIn && !pre) {
    for (int i = threadIdx.x; i < kR * c16; i += blockDim.x) {
      const int r = i / c16, c = i % c16;
      int4 v = make_int4(0, 0, 0, 0);
      if (r < n) v = reinterpret_cast<const int4*>(act + (int64_t)s_src[r] * K)[c];
      s_act[i] = v;
    }
    __syncthreads();  // activations and scales staged
  }

  // Lane geometry inside a pair: lanes 0..31 hold group 2gp, 32..63 group
  // 2gp+1; within a group, lane l (= lane % 32) holds rows 2*(l % 16) and
  // 2*(l % 16) + 1, columns 16 * (l / 16) .. +15.  Lanes l and l ^ 16 hold the
  // two column halves of the same rows: each keeps one row and hands the
  // other row's partial to its partner.
  const int gsel = lane >> 5, half = (lane >> 4) & 1;
  const int row = 2 * (lane & 15) + half;
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int gp = wave + kWaves * i;
    if (gp >= GP) break;
    const int g = 2 * gp + gsel;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (r >= n) break;
        const int4 x = s_act[(pre ? s_src[r] : r) * c16 + g * 2 + half];
        int q0, q1;
        dot16x2(wv[i][m], x, q0, q1);
        const int send = half ? q0 : q1;
        const int keep = half ? q1 : q0;
        const int full = keep + __shfl_xor(send, 16);
        s_is[((m * kR + r) * G + g) * 32 + row] = full;
      }
    }
  }
  __syncthreads();

  // One thread per (row r, output column o of the block).
  for (int t = threadIdx.x; t < n * 32; t += blockDim.x) {
    const int r = t / 32, o = t % 32;
    float acc[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      float ac = 0.0f;
      const int32_t* is = s_is + (m * kR + r) * G * 32 + o;
      const float* sc = s_sc + m * G * 32 + o;
      for (int g = 0; g < G; ++g) ac = fmaf(sc[g * 32], (float)is[g * 32], ac);
      acc[m] = ac;
      if (kCapture) {
        const int64_t col = (int64_t)rbm[m] * 32 + o;
        for (int g = 0; g < G; ++g)
          isum[((int64_t)(p0 + r) * wrows + col) * G + g] = is[g * 32] >> 4;
      }
    }
    const float s = s_as[r];
    if (kGateUp)
      out[(int64_t)(p0 + r) * a.h + rbo * 32 + o] = silu(acc[0] * s) * (acc[kM - 1] * s);
    else
      out[(int64_t)(p0 + r) * N + rbo * 32 + o] = acc[0] * s;
  }
}

template <int kR, bool kGateUp, bool kCapture, bool kDense>
__global__ __launch_bounds__(256) void k_gemv_i4(GemvProb P) {
  gemv_block<kR, kGateUp, kCapture, kDense>(P, (int)blockIdx.x);
}

// Routed (P0, the first n0 blocks) and shared (P1) products in one launch.
template <int kR, bool kGateUp, bool kQIn = false>
__global__ __launch_bounds__(256) void k_gemv_i4_pair(GemvProb P0, GemvProb P1, int n0) {
  if ((int)blockIdx.x < n0)
    gemv_block<kR, kGateUp, false, false, kQIn>(P0, (int)blockIdx.x);
  else
    gemv_block<kR, kGateUp, false, true, kQIn>(P1, (int)blockIdx.x - n0);
}

constexpr int kRGemv = 4;

size_t gemv_lds(int K, bool gateup) {
  const int G = K / kGroup, m = gateup ? 2 : 1;
  return (size_t)m * kRGemv * G * 32 * 4 + (size_t)m * G * 32 * 4 + (size_t)kRGemv * K;
}

unsigned gemv_tiles(const ExpertArgs& a) { return (unsigned)tile_bound(a, kRGemv); }

GemvProb gemv_gateup_prob(const ExpertArgs& a, const int8_t* xq, const float* sx,
                          const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum) {
  return GemvProb{a, a.d, 2 * a.h, a.h / 32, xq, sx, wq, ws, a_buf, isum, nullptr};
}

GemvProb gemv_down_prob(const ExpertArgs& a, const int8_t* hq, const float* hs,
                        const uint8_t* wq, const float* ws, float* f, int32_t* isum) {
  ExpertArgs b = a;
  b.perm = nullptr;
  return GemvProb{b, a.h, a.d, a.d / 32, hq, hs, wq, ws, f, isum, nullptr};
}

template <bool kGateUp>
hipError_t launch_gemv(const GemvProb& P, hipStream_t st) {
  const dim3 grid(gemv_tiles(P.a) * P.RB);
  const size_t lds = gemv_lds(P.K, kGateUp);
  if (!P.a.offsets)
    hipLaunchKernelGGL((k_gemv_i4<kRGemv, kGateUp, false, true>), grid, dim3(256), lds, st, P);
  else if (P.isum)
    hipLaunchKernelGGL((k_gemv_i4<kRGemv, kGateUp, true, false>), grid, dim3(256), lds, st, P);
  else
    hipLaunchKernelGGL((k_gemv_i4<kRGemv, kGateUp, false, false>), grid, dim3(256), lds, st, P);
  return hipGetLastError();
}

template <bool kGateUp, bool kQIn = false>
hipError_t launch_gemv_pair(const GemvProb& R, const GemvProb& D, hipStream_t st) {
  const unsigned n0 = gemv_tiles(R.a) * R.RB, n1 = gemv_tiles(D.a) * D.RB;
  const size_t lds = std::max(gemv_lds(R.K, kGateUp), gemv_lds(D.K, kGateUp));
  hipLaunchKernelGGL((k_gemv_i4_pair<kRGemv, kGateUp, kQIn>), dim3(n0 + n1), dim3(256), lds, st, R,
                     D, (int)n0);
  return hipGetLastError();
}

}  // namespace

bool gemv_i4_fits(int K, bool gateup) {
  return K % 64 == 0 && K <= 2 * kGroup * kWaves * kMaxPairs && gemv_lds(K, gateup) <= 65536;
}

hipError_t launch_gateup_i4_gemv(const ExpertArgs& a, const int8_t* xq, const float* sx,
                                 const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum,
                                 hipStream_t st) {
  return launch_gemv<true>(gemv_gateup_prob(a, xq, sx, wq, ws, a_buf, isum), st);
}

hipError_t launch_down_i4_gemv(const ExpertArgs& a, const int8_t* hq, const float* hs,
                               const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                               hipStream_t st) {
  return launch_gemv<false>(gemv_down_prob(a, hq, hs, wq, ws, f, isum), st);
}

hipError_t launch_gateup_i4_gemv_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                      const int8_t* xq, const float* sx, const uint8_t* wq_r,
                                      const float* ws_r, const uint8_t* wq_s, const float* ws_s,
                                      float* abuf_r, float* abuf_s, hipStream_t st) {
  return launch_gemv_pair<true>(gemv_gateup_prob(ar, xq, sx, wq_r, ws_r, abuf_r, nullptr),
                                gemv_gateup_prob(as, xq, sx, wq_s, ws_s, abuf_s, nullptr), st);
}

hipError_t launch_down_i4_gemv_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                    const int8_t* hq_r, const float* hs_r, const int8_t* hq_s,
                                    const float* hs_s, const uint8_t* wq_r, const float* ws_r,
                                    const uint8_t* wq_s, const float* ws_s, float* f, float* ys,
                                    hipStream_t st) {
  return launch_gemv_pair<false>(gemv_down_prob(ar, hq_r, hs_r, wq_r, ws_r, f, nullptr),
                                 gemv_down_prob(as, hq_s, hs_s, wq_s, ws_s, ys, nullptr), st);
}

bool gemv_i4_qin_fits(int K) { return gemv_i4_fits(K, false) && K % 128 == 0 && K <= 128 * kMaxQV; }

hipError_t launch_down_i4_gemv_pair_f32in(const ExpertArgs& ar, const ExpertArgs& as,
                                          const float* a_r, const float* a_s, const uint8_t* wq_r,
                                          const float* ws_r, const uint8_t* wq_s,
                                          const float* ws_s, float* f, float* ys, hipStream_t st) {
  GemvProb R = gemv_down_prob(ar, nullptr, nullptr, wq_r, ws_r, f, nullptr);
  GemvProb D = gemv_down_prob(as, nullptr, nullptr, wq_s, ws_s, ys, nullptr);
  R.actf = a_r;
  D.actf = a_s;
  return launch_gemv_pair<false, true>(R, D, st);
}

}  // namespace mm
