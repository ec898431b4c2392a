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
// layout in common.h; the pieces permuted among the lanes of a group), so
// every wave load is one fully coalesced 1 KB access
// and all of a workgroup's weight bytes are in flight before the first use.
// The exact int32 group sums go to LDS; then one thread per (row, output)
// applies the scales in group order.  Only experts that own rows have tiles,
// so only the selected experts' weights are read.
#pragma once

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

// Flag-in-word hand-off between the workgroups of one launch (the one-launch
// decode layer): every FP32 value travels as a 64-bit word, tag << 32 | bits,
// written and read with device-scope atomic accesses (a naturally aligned
// 64-bit access is single-copy atomic), so a reader knows a value belongs to
// this call when its tag matches and needs no counter and no fence.  The
// values are the FP32 bits unchanged.  A reader polls; a wait gives up after
// `spin` polls and bumps *status, so a kernel always ends.
struct LLWait {
  uint32_t tag, spin;
  uint32_t* status;
};

__device__ __forceinline__ void ll_put(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_get(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ll_ready(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
__device__ __forceinline__ float ll_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// End of one poll round of a wave: true when every lane's words were ready
// (or the wait gives up: then the status word counts it); else it sleeps.
__device__ __forceinline__ bool ll_settle(bool lane_ok, uint32_t& n, const LLWait& L) {
  if (__ballot(!lane_ok) == 0) return true;
  if (++n >= L.spin) {
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(L.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
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
  // one-launch layer (kFused): actf rows and out are flag-in-word buffers;
  // routed: the tile table in workgroup memory (FusedTiles)
  LLWait ll;
  const int32_t* tiles;
};

// Tile table of the one-launch layer's routing (every expert of the call
// owns one tile, experts in index order): [0] tile count, then first row,
// row count and expert of each tile.
constexpr int kFusedTiles = 32;
enum : int { kTileCount = 0, kTileP0 = 1, kTileN = 1 + kFusedTiles, kTileE = 1 + 2 * kFusedTiles,
             kTileWords = 1 + 3 * kFusedTiles };

constexpr int kMaxQV = 20;  // float2 per lane of a quantised row: K <= 128 * 20

// Wave-level INT8 quantisation of one FP32 row (K % 128 == 0, K <= 128 *
// kMaxQV) into LDS: the same rule and arithmetic as the standalone quantiser
// (exact max|v| over the row, s = 2*amax/255, codes clamp(rint(v/s))), so
// its codes and scale are bit-identical.  Returns s on every lane.
template <int kNQ = kMaxQV>
__device__ __forceinline__ void load_row_regs(const float* __restrict__ x, int K, float2 (&v)[kNQ],
                                              int lane) {
  const int nv = K / 128;
  const float2* xr = reinterpret_cast<const float2*>(x);
#pragma unroll
  for (int i = 0; i < kNQ; ++i)
    if (i < nv) v[i] = xr[lane + 64 * i];
}

// The quantisation of a row already held in registers (load_row_regs).
template <int kNQ = kMaxQV>
__device__ __forceinline__ float quant_regs_lds(const float2 (&v)[kNQ], int K,
                                                int8_t* __restrict__ dst, int lane) {
  const int nv = K / 128;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kNQ; ++i)
    if (i < nv) amax = fmaxf(amax, fmaxf(fabsf(v[i].x), fabsf(v[i].y)));
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  uint16_t* q = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
  for (int i = 0; i < kNQ; ++i)
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

template <int kNQ = kMaxQV>
__device__ __forceinline__ float quant_row_lds(const float* __restrict__ x, int K,
                                               int8_t* __restrict__ dst, int lane) {
  float2 v[kNQ];
  load_row_regs<kNQ>(x, K, v, lane);
  return quant_regs_lds<kNQ>(v, K, dst, lane);
}

// The row quantiser over the whole workgroup: rows r < n (n <= 4) of src
// (workgroup memory, floats, row stride K, K % 128 == 0) into INT8 rows of
// dst (row stride K) and their scales into scale[r]; wave w takes the
// 128-column chunks w, w+4, ... of every row.  The rule, codes and scales of
// the row quantiser (quant_regs_lds): max|v| over the row, s = 2 max / 255,
// codes clamp(rint(v / s)) by quant_i8's fast path, and by quant_i8 itself
// for a chunk in which any element needs its exact division.  Called by the
// whole workgroup; ends with a barrier.
__device__ __forceinline__ void quant_rows_wg(const float* src, int n, int K, int8_t* dst,
                                              float* scale, int tid) {
  __shared__ float s_amax[4][kWaves];
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = K / 128;
  const float2* s2 = reinterpret_cast<const float2*>(src);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= n) break;
    float m = 0.0f;
    for (int c = wave; c < nch; c += kWaves) {
      const float2 v = s2[r * (K / 2) + c * 64 + lane];
      m = fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y)));
    }
    m = max64(m);
    if (lane == 0) s_amax[r][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= n) break;
    float amax = s_amax[r][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, s_amax[r][w]);
    const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
    if (tid == 0) scale[r] = sr;
    uint16_t* q = reinterpret_cast<uint16_t*>(dst + (int64_t)r * K);
    for (int c = wave; c < nch; c += kWaves) {
      const int p = c * 64 + lane;
      const float2 v = s2[r * (K / 2) + p];
      int c0 = 0, c1 = 0;
      if (sr != 0.0f) {
        bool slow = false;
        c0 = quant_code_fast(v.x, yr, slow);
        c1 = quant_code_fast(v.y, yr, slow);
        if (__ballot(slow) != 0) {
          c0 = quant_i8(v.x, sr, yr);
          c1 = quant_i8(v.y, sr, yr);
        }
      }
      q[p] = (uint16_t)((uint8_t)(int8_t)c0 | ((uint16_t)(uint8_t)(int8_t)c1 << 8));
    }
  }
  __syncthreads();
}

// The workgroup form of ll_settle: true for every thread once every
// thread's words were ready in the same poll round, so the whole workgroup
// leaves the wait together (two barriers per round).
__device__ __forceinline__ bool ll_settle_wg(bool lane_ok, uint32_t& n, const LLWait& L) {
  __shared__ int s_vote[kWaves];
  const int w = (int)(threadIdx.x >> 6);
  const bool wave_ok = __ballot(!lane_ok) == 0;
  if ((threadIdx.x & 63) == 0) s_vote[w] = wave_ok ? 1 : 0;
  __syncthreads();
  bool all = true;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) all = all && s_vote[i] != 0;
  __syncthreads();
  if (all) return true;
  if (++n >= L.spin) {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(L.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
}

// nw consecutive flag-in-word values from src into workgroup memory stg
// (floats), spread over the workgroup's 256 threads (word base + tid +
// 256 i); the workgroup waits until all of them are this call's.  Up to
// 256 * kStageW words per pass (one pass for every routed row set of up to
// 2560 values and for one token's shared rows).  Called by the whole
// workgroup.
constexpr int kStageW = 10;
__device__ __forceinline__ void stage_words_ll(const uint64_t* src, int nw, float* stg, int tid,
                                               const LLWait& L) {
  for (int base = 0; base < nw; base += 256 * kStageW) {
    float val[kStageW];
    uint32_t n = 0;
    for (;;) {
      // every load of the round is issued before any is looked at (words
      // past the end re-read the last one and are ignored)
      uint64_t w[kStageW];
#pragma unroll
      for (int i = 0; i < kStageW; ++i) w[i] = ll_get(src + min(base + tid + 256 * i, nw - 1));
      bool ok = true;
#pragma unroll
      for (int i = 0; i < kStageW; ++i) {
        ok = ok & (base + tid + 256 * i >= nw || ll_ready(w[i], L.tag));
        val[i] = ll_value(w[i]);
      }
      if (ll_settle_wg(ok, n, L)) break;
    }
#pragma unroll
    for (int i = 0; i < kStageW; ++i) {
      const int j = base + tid + 256 * i;
      if (j < nw) stg[j] = val[i];
    }
  }
}

// Block `blk` of problem P.  out: gate/up -> a = SiLU(g * s) * (u * s) into
// out [rows][h]; down -> f = acc * s into out [rows][N].  K: reduction length
// (multiple of 64, <= 2560); RB: 32-row weight blocks per output (gate/up:
// h / 32, down: N / 32).  kDense: rows are the tokens in order (shared
// expert); otherwise routed.  Called by the whole workgroup.
//
// The one-launch decode layer (k_decode.hip) runs this block with kFused,
// where the rows' producers are other workgroups of the same launch:
// `pre_tile()` runs before the tile lookup (it may build the routing in
// workgroup memory, a.offsets / a.perm pointing there), and `hook()` runs
// once the block's weight and scale loads are issued and before any
// activation is read.  Both are called by every thread.  The hidden rows a
// down block reads (actf) and every output are flag-in-word buffers (LLWait
// below): a wave waits for its row's values themselves, after its weight
// loads are issued.  With kQX (gate/up, T <= kR) the token rows are
// quantised from FP32 (P.actf [T][K], plain memory) in the workgroup with
// the row quantiser's rule, before `pre_tile()`, instead of being read as
// x_q.
struct NoHook {
  __device__ void operator()() const {}
};

template <int kR, bool kGateUp, bool kCapture, bool kDense, bool kQIn = false, bool kFused = false,
          bool kQX = false, class PreHook = NoHook, class Hook = NoHook>
__device__ __forceinline__ void gemv_block(const GemvProb& P, int blk,
                                           const PreHook& pre_tile = PreHook(),
                                           const Hook& hook = Hook()) {
  static_assert(!kQIn || (!kGateUp && kR == 4), "in-kernel quantisation: down, one row per wave");
  static_assert(!kQX || (kGateUp && kFused && kR == 4), "in-kernel x quantisation: fused gate/up");
  const ExpertArgs& a = P.a;
  int K = P.K, N = P.N, RB = P.RB;
  int tid = (int)threadIdx.x;
  if constexpr (kFused) {
    // the fused kernel may run several blocks in a loop: these values are
    // made opaque so that what derives from them is recomputed per block
    // instead of being kept live across the loop
    __asm__ volatile("" : "+s"(K), "+s"(N), "+s"(RB));
    __asm__ volatile("" : "+v"(tid));
  }
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
  const bool pre = kGateUp && !kDense && a.T <= kR && !kFused;
  if (pre) {
    for (int i = tid; i < (int)a.T * c16; i += blockDim.x)
      s_act[i] = reinterpret_cast<const int4*>(act)[i];  // rows 0..T-1 of x_q [T][K]
    if (tid < (int)a.T) s_tsc[tid] = act_scale[tid];
  }
  // In-kernel quantisation of a routed problem of at most kR rows: wave w
  // reads hidden row w before the tile is known (the tile's rows are some
  // of these), so those loads do not wait for the offsets either.
  const bool preq = kQIn && !kDense && a.rows <= kR && !kFused;
  float2 qv[kMaxQV];
  if constexpr (kQIn) {
    const int w = (int)(tid >> 6);
    if (preq && w < (int)a.rows) load_row_regs(P.actf + (int64_t)w * K, K, qv, tid & 63);
  }
  // token row t quantised by wave t into LDS row t (as the pre-staged x_q
  // rows above); routed: before the routing (it overlaps the wait for the
  // logits), dense: once the weight loads are issued
  auto quant_x = [&]() {
    // the T token rows land in the s_is region first (written only by the
    // products, later), then the whole workgroup quantises them
    float* xs = reinterpret_cast<float*>(s_is);
    const int nq = (int)a.T * K / 4;
    for (int i = tid; i < nq; i += kWaves * 64)
      reinterpret_cast<float4*>(xs)[i] = reinterpret_cast<const float4*>(P.actf)[i];
    __syncthreads();
    quant_rows_wg(xs, (int)a.T, K, reinterpret_cast<int8_t*>(s_act), s_tsc, tid);
  };
  if constexpr (kQX && !kDense) quant_x();
  pre_tile();
  const int tile = blk / RB, rbo = blk % RB;
  int p0, n, e;
  if constexpr (kFused && !kDense) {
    // the routing's tile table (built, and made visible, by pre_tile)
    n = 0;
    p0 = e = 0;
    if (tile < P.tiles[kTileCount]) {
      p0 = P.tiles[kTileP0 + tile];
      n = P.tiles[kTileN + tile];
      e = P.tiles[kTileE + tile];
    }
  } else {
    gemv_tile<kR, kDense>(a, tile, p0, n, e);  // (routed: a barrier, after which the above is visible)
  }
  if (n <= 0) return;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t wrows = kGateUp ? 2 * (int64_t)a.h : N;
  int rbm[kM];
  rbm[0] = rbo;
  if (kGateUp) rbm[kM - 1] = rbo + a.h / 32;

  // Weight loads first: pair i of this wave is groups 2*(wave + 4i) and +1
  // (pairs past the end are neither loaded nor used).  Lane l of a group
  // (l = lane % 32) reads the chunk's 16-byte piece (l % 2) * 16 + l / 2:
  // rows 2 * (l / 2) and 2 * (l / 2) + 1, column half l % 2, so the two
  // halves of the same rows sit in adjacent lanes.
  const int piece = (lane & 32) + (lane & 1) * 16 + ((lane & 31) >> 1);
  const uint8_t* we = wq + (int64_t)e * (wrows / 32) * G * kChunkBytes;
  uint4 wv[kMaxPairs][kM];
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int gp = wave + kWaves * i;
    if (gp < GP) {
#pragma unroll
      for (int m = 0; m < kM; ++m)
        wv[i][m] = reinterpret_cast<const uint4*>(
            we + ((int64_t)rbm[m] * G + 2 * gp) * kChunkBytes)[piece];
    }
  }

  // scales of the workgroup's blocks: G * 32 contiguous floats per block;
  // the first kScR per thread are loaded now, with the weights, so that
  // their latency does not add to the activations' (the rest, if any,
  // later)
  const float* se = wsc + (int64_t)e * (wrows / 32) * G * 32;
  const int nsc = kM * G * 32;
  constexpr int kScR = (kGateUp || kDense) ? 10 : 3;  // routed down: h <= 768 in the preload
  float scr[kScR];
#pragma unroll
  for (int i = 0; i < kScR; ++i) {
    const int j = tid + kWaves * 64 * i;
    if (j < nsc) scr[i] = se[(int64_t)rbm[j / (G * 32)] * G * 32 + j % (G * 32)];
  }
  // Routed gate/up whose token rows are not pre-staged: every thread finds
  // the source token of the rows it stages itself and loads them at once
  // (no barrier between the permutation and the activation loads); the
  // first thread of each row also takes the row's scale.
  const bool direct = !kQIn && !pre && !kQX;
  if constexpr (kQX && kDense) quant_x();
  hook();
  if constexpr (kQIn && kFused) {
    // the tile's n hidden rows (contiguous) land in the s_is region first
    // (it is written only after the quantisation), then wave r quantises row
    // r from there; wave r clears slot r when r >= n
    float* stg = reinterpret_cast<float*>(s_is);
    stage_words_ll(reinterpret_cast<const uint64_t*>(P.actf) + (int64_t)p0 * K, n * K, stg, tid, P.ll);
    __syncthreads();
    quant_rows_wg(stg, n, K, reinterpret_cast<int8_t*>(s_act), s_as, tid);
  } else if constexpr (kQIn) {
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
  } else if (direct) {
    for (int i = tid; i < kR * c16; i += blockDim.x) {
      const int r = i / c16, c = i % c16;
      int4 v = make_int4(0, 0, 0, 0);
      if (r < n) {
        int src = p0 + r;
        if (kGateUp && !kDense) {
          src = a.T == 1 ? 0 : a.perm[p0 + r] / a.k;
          if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
        }
        v = reinterpret_cast<const int4*>(act + (int64_t)src * K)[c];
        if (c == 0) s_as[r] = act_scale[src];
      } else if (c == 0) {
        s_as[r] = 0.0f;
      }
      s_act[i] = v;
    }
  } else if (tid < kR) {
    const int r = tid;
    int src = -1;
    float s = 0.0f;
    if (r < n) {
      src = p0 + r;
      if (kGateUp && !kDense) {
        src = a.T == 1 ? 0 : a.perm[p0 + r] / a.k;
        if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
      }
      s = (pre || kQX) ? s_tsc[src] : act_scale[src];
    }
    s_src[r] = src;
    s_as[r] = s;
  }
#pragma unroll
  for (int i = 0; i < kScR; ++i) {
    const int j = tid + kWaves * 64 * i;
    if (j < nsc) s_sc[j] = scr[i];
  }
  for (int j = tid + kWaves * 64 * kScR; j < nsc; j += kWaves * 64)
    s_sc[j] = se[(int64_t)rbm[j / (G * 32)] * G * 32 + j % (G * 32)];
  __syncthreads();  // scales, activations (or, in-kernel quantisation, the codes) staged

  // Lane geometry inside a pair: lanes 0..31 hold group 2gp, 32..63 group
  // 2gp+1; within a group, lane l (= lane % 32) holds rows 2*(l / 2) and
  // 2*(l / 2) + 1, columns 16 * (l % 2) .. +15.  Lanes l and l ^ 1 hold the
  // two column halves of the same rows: each keeps row l and takes its
  // partner's partial for it (one DPP move).
  const int gsel = lane >> 5, half = lane & 1;
  const int row = lane & 31;
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
        const int4 x = s_act[((pre || kQX) ? s_src[r] : r) * c16 + g * 2 + half];
        int q0, q1;
        dot16x2(wv[i][m], x, q0, q1);
        const int send = half ? q0 : q1;
        const int keep = half ? q1 : q0;
        const int full = keep + __builtin_amdgcn_mov_dpp(send, kDppXor1, 0xF, 0xF, true);
        s_is[((m * kR + r) * G + g) * 32 + row] = full;
      }
    }
  }
  __syncthreads();

  // Gate/up: the gate and the up chains of output (r, o) are taken by
  // threads r*32+o and 128+r*32+o (other waves, so the two run side by side),
  // then joined through workgroup memory (n * 32 <= 128).
  if constexpr (kGateUp && kR * 32 <= 128) {
    __shared__ float s_up[kR * 32];
    const int m = tid >> 7, t = tid & 127;
    const int r = t / 32, o = t % 32;
    float ac = 0.0f;
    if (t < n * 32) {
      const int32_t* is = s_is + (m * kR + r) * G * 32 + o;
      const float* sc = s_sc + m * G * 32 + o;
      int g = 0;
      for (; g + 8 <= G; g += 8) {
        float sv[8];
        int iv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sv[j] = sc[(g + j) * 32];
          iv[j] = is[(g + j) * 32];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ac = fmaf(sv[j], (float)iv[j], ac);
      }
      for (; g < G; ++g) ac = fmaf(sc[g * 32], (float)is[g * 32], ac);
      if (kCapture) {
        const int64_t col = (int64_t)rbm[m] * 32 + o;
        for (int g2 = 0; g2 < G; ++g2)
          isum[((int64_t)(p0 + r) * wrows + col) * G + g2] = is[g2 * 32] >> 4;
      }
      if (m == 1) s_up[t] = ac;
    }
    __syncthreads();
    if (m == 0 && t < n * 32) {
      const float s = s_as[r];
      const int64_t at = (int64_t)(p0 + r) * a.h + rbo * 32 + o;
      const float v = silu(ac * s) * (s_up[t] * s);
      if constexpr (kFused)
        ll_put(reinterpret_cast<uint64_t*>(out) + at, v, P.ll.tag);
      else
        out[at] = v;
    }
    return;
  }
  // One thread per (row r, output column o of the block).
  for (int t = tid; t < n * 32; t += blockDim.x) {
    const int r = t / 32, o = t % 32;
    float acc[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      float ac = 0.0f;
      const int32_t* is = s_is + (m * kR + r) * G * 32 + o;
      const float* sc = s_sc + m * G * 32 + o;
      // the chain over g in order; its operands read 8 groups at a time
      int g = 0;
      for (; g + 8 <= G; g += 8) {
        float sv[8];
        int iv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sv[j] = sc[(g + j) * 32];
          iv[j] = is[(g + j) * 32];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ac = fmaf(sv[j], (float)iv[j], ac);
      }
      for (; g < G; ++g) ac = fmaf(sc[g * 32], (float)is[g * 32], ac);
      acc[m] = ac;
      if (kCapture) {
        const int64_t col = (int64_t)rbm[m] * 32 + o;
        for (int g = 0; g < G; ++g)
          isum[((int64_t)(p0 + r) * wrows + col) * G + g] = is[g * 32] >> 4;
      }
    }
    const float s = s_as[r];
    const int64_t at = kGateUp ? (int64_t)(p0 + r) * a.h + rbo * 32 + o : (int64_t)(p0 + r) * N + rbo * 32 + o;
    const float v = kGateUp ? silu(acc[0] * s) * (acc[kM - 1] * s) : acc[0] * s;
    if constexpr (kFused)
      ll_put(reinterpret_cast<uint64_t*>(out) + at, v, P.ll.tag);
    else
      out[at] = v;
  }
}

constexpr int kRGemv = 4;  // rows per tile of the launched blocks

// Dynamic workgroup memory of one block (s_is, s_sc and s_act above).
inline size_t gemv_lds(int K, bool gateup) {
  const int G = K / kGroup, m = gateup ? 2 : 1;
  return (size_t)m * kRGemv * G * 32 * 4 + (size_t)m * G * 32 * 4 + (size_t)kRGemv * K;
}

}  // namespace
}  // namespace mm
