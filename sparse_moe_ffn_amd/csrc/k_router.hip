// FP32 router: logits, top-k selection and gate weights.
//
// The router stays in FP32 (MobileMoE close reading, section "Pre-training",
// MoE stability list); eq. (*) weights each selected expert's output by
// router_i(x).  The logit of (token t, expert e) is computed in one fixed
// order so that the selection is reproducible bit for bit:
//   lane l of a wave accumulates x[t][j] * w[e][j] for j = l, l+64, ... with
//   fused multiply-adds, then the 64 partials are added as a balanced binary
//   tree over lane indices (pairs at distance 1, 2, 4, ..., 32), then bias[e]
//   is added.  Experts are ranked by (logit descending, index ascending).
#include "common.h"
#include "launch.h"
#include "router_topk.h"

namespace mm {
namespace {

constexpr int kTok = 4;     // tokens per workgroup (one per wave for the top-k)
constexpr int kRowStride = 17;  // LDS stride of one row of 16 quad sums (padded)
constexpr int64_t kSmallRouterT = 64;  // up to this many tokens: the one-token-per-workgroup form

// Top-k and gate weights of one token; lane e holds the logit of expert e
// (-inf for e >= E).  k rounds of a wave arg-max under the total order (value
// descending, index ascending): the round's maximum, then the lowest lane
// holding it; lane j keeps the winner of round j (select_topk_lanes).  Writes
// idx[0..k) and w[0..k).  Called by a whole wave.
template <int kGating>
__device__ __forceinline__ void select_topk(float mine, float gl, int lane, int E, int k,
                                            int32_t* __restrict__ idx, float* __restrict__ w) {
  int sel;
  float wv;
  select_topk_lanes<kGating>(mine, gl, lane, E, k, sel, wv);
  if (lane < k) {
    idx[lane] = sel;
    w[lane] = wv;
  }
}

// The first two levels of the 64-lane tree (pairs at distance 1, then 2) in
// registers: every lane of a quad ends with its quad's sum.
__device__ __forceinline__ float quad_sum(float p) {
  p = p + dpp<kDppXor1>(p);
  return p + dpp<kDppXor2>(p);
}

// Workgroup = 4 waves and 4 tokens.  Phase 1: wave w takes experts w, w+4,
// w+8, ... (at most 16); for each one, lane l forms the 4 tokens' partial sums
// over columns j = l, l+64, ... (fused multiply-adds, ascending j), adds them
// within its quad (the tree's first two levels) and one lane per quad stores
// the quad sum to LDS.  Phase 2: lane r of the wave finishes the tree over the
// 16 quad sums of row r (one (token, expert) pair), adds the bias and writes
// the logit.  Phase 3: wave w takes token w, lane e holding the logit of
// expert e, and does the top-k and the gate weights.
// kNX = d / 64 (0: any d, row read from memory in the loop).  kQuant (kNX > 0
// only): also writes the tokens' INT8 rows xq and scales sx.  hist (may be
// NULL): the workgroup's count of each expert over its kTok tokens' k picks,
// one byte at hist[e * hist_stride + blockIdx.x] for e < E (the count sort
// reads it instead of counting the ids again).
template <int kGating, int kNX, bool kQuant = false>
__global__ __launch_bounds__(256) void k_router(int64_t T, int d, int E, int k,
                                                const float* __restrict__ x,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias,
                                                int32_t* __restrict__ idx,
                                                float* __restrict__ w,
                                                int8_t* __restrict__ xq = nullptr,
                                                float* __restrict__ sx = nullptr,
                                                int64_t gm_rows = 0,
                                                uint8_t* __restrict__ hist = nullptr,
                                                int64_t hist_stride = 0) {
  __shared__ float s_part[4][16 * kTok][kRowStride];
  __shared__ float s_logit[kTok][64];
  __shared__ int s_hist[64];
  // the wave index is made wave-uniform (a scalar), so the expert loop
  // branches on scalars and each expert row is read from a scalar base
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (hist != nullptr && threadIdx.x < 64) s_hist[threadIdx.x] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int nt = (int)min((int64_t)kTok, T - t0);
  const int ne = (E - wave + 3) / 4;  // experts of this wave

  if constexpr (kNX > 0) {
    float xv[kTok][kNX];
#pragma unroll
    for (int q = 0; q < kTok; ++q)
#pragma unroll
      for (int i = 0; i < kNX; ++i) xv[q][i] = q < nt ? x[(t0 + q) * d + lane + kWave * i] : 0.0f;
    // expert rows read kRing ahead (a ring of register sets: 4 for narrow
    // rows, 2 for wide ones to keep registers for occupancy); rows past this
    // wave's last expert re-read expert E-1 (valid, unused)
    constexpr int kRing = kNX <= 12 ? 4 : 2;
    float wv[kRing][kNX];
    auto load_row = [&](int i, float (&dst)[kNX]) {
      const float* we = wr + (int64_t)min(wave + 4 * i, E - 1) * d;
#pragma unroll
      for (int c = 0; c < kNX; ++c) dst[c] = we[lane + kWave * c];
    };
#pragma unroll
    for (int i = 0; i < kRing; ++i) load_row(i, wv[i]);
    // wave w quantises token w (every wave holds all kTok rows), while the
    // first expert rows are in flight
    if constexpr (kQuant) {
      // one copy of the quantiser on the selected row (four inlined copies
      // kept 185 VGPRs live: two waves per SIMD instead of four)
      const int wq = __builtin_amdgcn_readfirstlane(wave);
      if (wq < nt) {
        float sel[kNX];
#pragma unroll
        for (int c = 0; c < kNX; ++c) {
          float v = xv[0][c];
#pragma unroll
          for (int q = 1; q < kTok; ++q) v = wq == q ? xv[q][c] : v;
          sel[c] = v;
        }
        quant_row_regs(sel, lane, t0 + wq, d, xq, sx, gm_rows);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < ne) {
#pragma unroll
        for (int q = 0; q < kTok; ++q) {
          float p = 0.0f;
#pragma unroll
          for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[q][c], wv[i % kRing][c], p);
          p = quad_sum(p);
          // the four lanes of a quad store the same sum to the same word
          // (no lane mask around the store)
          s_part[wave][i * kTok + q][lane >> 2] = p;
        }
      }
      if (i + kRing < 16) load_row(i + kRing, wv[i % kRing]);
    }
  } else {
    for (int i = 0; i < ne; ++i) {
      const float* we = wr + (int64_t)(wave + 4 * i) * d;
      for (int q = 0; q < kTok; ++q) {
        float p = 0.0f;
        if (q < nt)
          for (int j = lane; j < d; j += kWave) p = __builtin_fmaf(x[(t0 + q) * d + j], we[j], p);
        p = quad_sum(p);
        if ((lane & 3) == 0) s_part[wave][i * kTok + q][lane >> 2] = p;
      }
    }
  }
  __syncthreads();
  // Phase 2: lane r reduces row r = (expert slot i, token q) of its wave.
  if (lane < ne * kTok) {
    const float* row = s_part[wave][lane];
    float p[16];
#pragma unroll
    for (int l = 0; l < 16; ++l) p[l] = row[l];
#pragma unroll
    for (int s2 = 1; s2 < 16; s2 <<= 1)
#pragma unroll
      for (int l = 0; l < 16; l += 2 * s2) p[l] = p[l] + p[l + s2];
    const int i = lane / kTok, q = lane % kTok;
    const int e = wave + 4 * i;
    s_logit[q][e] = p[0];  // the bias is added at the selection
  }
  __syncthreads();
  if (wave < nt) {
    const int64_t t = t0 + wave;
    float mine, gl;
    biased_logit<kGating>(s_logit[wave], bias, lane, E, mine, gl);
    int sel;
    float wv;
    select_topk_lanes<kGating>(mine, gl, lane, E, k, sel, wv);
    if (lane < k) {
      idx[t * k + lane] = sel;
      w[t * k + lane] = wv;
      if (hist != nullptr) atomicAdd(&s_hist[sel], 1);  // a count: order does not matter
    }
  }
  if (hist != nullptr) {
    __syncthreads();
    if ((int)threadIdx.x < E)
      hist[threadIdx.x * hist_stride + blockIdx.x] = (uint8_t)s_hist[threadIdx.x];
  }
}

// Few tokens (decode): one token per workgroup of 16 waves; wave w takes
// experts w, w+16, w+32, w+48 and reads all of their rows at once, so the
// router costs about one memory round trip.  Each logit is the 64-lane tree
// sum of its partials (the same order as above) plus the bias.
constexpr int kSmallWaves = 16;
constexpr int kSmallPer = 4;  // experts per wave (E <= 64)

template <int kGating, int kNX, bool kQuant = false>
__global__ __launch_bounds__(64 * kSmallWaves) void k_router_small(
    int64_t T, int d, int E, int k, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, int32_t* __restrict__ idx, float* __restrict__ w,
    int8_t* __restrict__ xq = nullptr, float* __restrict__ sx = nullptr, int64_t gm_rows = 0) {
  __shared__ float s_logit[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  float xv[kNX], wv[kSmallPer][kNX];
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const float* we = wr + (int64_t)min(wave + kSmallWaves * i, E - 1) * d;
#pragma unroll
    for (int c = 0; c < kNX; ++c) wv[i][c] = we[lane + kWave * c];
  }
#pragma unroll
  for (int c = 0; c < kNX; ++c) xv[c] = x[t * d + lane + kWave * c];
  if constexpr (kQuant) {
    if (wave == 0) quant_row_regs(xv, lane, t, d, xq, sx, gm_rows);
  }
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const int e = wave + kSmallWaves * i;
    if (e >= E) break;
    float p = 0.0f;
#pragma unroll
    for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[c], wv[i][c], p);
    const float l = tree_sum64(p);  // the bias is added at the selection
    if (lane == 0) s_logit[e] = l;
  }
  __syncthreads();
  if (wave != 0) return;
  float mine, gl;
  biased_logit<kGating>(s_logit, bias, lane, E, mine, gl);
  select_topk<kGating>(mine, gl, lane, E, k, idx + t * k, w + t * k);
}

// Few tokens (T <= 2), the whole front of the layer in one workgroup: the
// router logits of every token (wave w keeps the rows of experts w, w+16,
// w+32, w+48 in registers and runs through the tokens), the per-token INT8
// quantisation of x, the top-k and gate weights, and the stable count sort of
// the T*k assignments (expert offsets by a wave scan, each slot's rank among
// the earlier slots with the same expert), written exactly as mm_route_permute
// writes them.
constexpr int kFrontMaxT = 16;  // LDS sizing; used up to kFrontUseT tokens
constexpr int kFrontUseT = 2;    // beyond this the per-token router workgroups are faster

template <int kGating, int kNX>
__global__ __launch_bounds__(64 * kSmallWaves) void k_front_small(
    int64_t T, int d, int E, int k, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, int32_t* __restrict__ idx, float* __restrict__ w,
    int8_t* __restrict__ xq, float* __restrict__ sx, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  __shared__ float s_logit[kFrontMaxT][64];
  __shared__ int s_id[kFrontMaxT * 8];
  __shared__ int s_cnt[64];
  __shared__ int s_off[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = (int)T;
  float wv[kSmallPer][kNX];
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const float* we = wr + (int64_t)min(wave + kSmallWaves * i, E - 1) * d;
#pragma unroll
    for (int c = 0; c < kNX; ++c) wv[i][c] = we[lane + kWave * c];
  }
  if (threadIdx.x < 64) s_cnt[threadIdx.x] = 0;
  for (int t = 0; t < nt; ++t) {
    float xv[kNX];
#pragma unroll
    for (int c = 0; c < kNX; ++c) xv[c] = x[(int64_t)t * d + lane + kWave * c];
    if (wave == (t & (kSmallWaves - 1))) quant_row_regs(xv, lane, t, d, xq, sx, 0);
#pragma unroll
    for (int i = 0; i < kSmallPer; ++i) {
      const int e = wave + kSmallWaves * i;
      if (e >= E) break;
      float p = 0.0f;
#pragma unroll
      for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[c], wv[i][c], p);
      const float l = tree_sum64(p);  // the bias is added at the selection
      if (lane == 0) s_logit[t][e] = l;
    }
  }
  __syncthreads();
  if (wave < nt) {  // wave t: top-k of token t
    const int t = wave;
    float mine, gl;
    biased_logit<kGating>(s_logit[t], bias, lane, E, mine, gl);
    int sel;
    float wgt;
    select_topk_lanes<kGating>(mine, gl, lane, E, k, sel, wgt);
    if (lane < k) {
      idx[t * k + lane] = sel;
      w[t * k + lane] = wgt;
      s_id[t * k + lane] = sel;
      atomicAdd(&s_cnt[sel], 1);
    }
  }
  __syncthreads();
  if (wave == 0) {  // expert offsets: exclusive scan of the counts
    const int c = lane < E ? s_cnt[lane] : 0;
    int inc = c;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int v = __shfl_up(inc, s);
      if (lane >= s) inc += v;
    }
    if (lane < E) {
      s_off[lane] = inc - c;
      offsets[lane] = inc - c;
      if (lane == E - 1) offsets[E] = inc;
    }
  }
  __syncthreads();
  const int tk = nt * k;
  if ((int)threadIdx.x < tk) {  // stable rank among the earlier slots of the same expert
    const int slot = threadIdx.x, e = s_id[slot];
    int rank = 0;
    for (int q = 0; q < slot; ++q) rank += s_id[q] == e;
    const int pos = s_off[e] + rank;
    perm[pos] = slot;
    inv_perm[slot] = pos;
  }
}

template <int kG, int kNX, bool kQ>
void launch_router_nx(bool small, int64_t T, int d, int E, int k, const float* x, const float* wr,
                      const float* bias, int32_t* idx, float* w, int8_t* xq, float* sx,
                      int64_t gm, uint8_t* g_hist, int64_t g_hist_stride, hipStream_t st) {
  if constexpr (kNX > 0 && kNX <= 20) {
    if (small) {
      hipLaunchKernelGGL((k_router_small<kG, kNX, kQ>), dim3((unsigned)T), dim3(64 * kSmallWaves),
                         0, st, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm);
      return;
    }
  }
  hipLaunchKernelGGL((k_router<kG, kNX, kQ>), dim3((unsigned)((T + kTok - 1) / kTok)), dim3(256), 0,
                     st, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, g_hist, g_hist_stride);
}

// Widths with a register form (d / 64 in the list below) can also quantise
// x in the same pass (kQ); other widths never get kQ = true.
template <int kG, bool kQ>
void launch_router_g(bool small, int64_t T, int d, int E, int k, const float* x, const float* wr,
                     const float* bias, int32_t* idx, float* w, int8_t* xq, float* sx, int64_t gm,
                     uint8_t* hist, int64_t hist_stride, hipStream_t st) {
  switch (d % kWave == 0 ? d / kWave : 0) {
    case 4: launch_router_nx<kG, 4, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 8: launch_router_nx<kG, 8, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 12: launch_router_nx<kG, 12, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 16: launch_router_nx<kG, 16, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 20: launch_router_nx<kG, 20, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 24: launch_router_nx<kG, 24, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    case 32: launch_router_nx<kG, 32, kQ>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); break;
    default: launch_router_nx<kG, 0, false>(small, T, d, E, k, x, wr, bias, idx, w, nullptr, nullptr, 0, hist, hist_stride, st); break;
  }
}

bool router_quant_fused(int d) {
  const int nx = d % kWave == 0 ? d / kWave : 0;
  return nx == 4 || nx == 8 || nx == 12 || nx == 16 || nx == 20 || nx == 24 || nx == 32;
}

template <int kG>
bool launch_front_g(int64_t T, int d, int E, int k, const float* x, const float* wr,
                    const float* bias, int32_t* idx, float* w, int8_t* xq, float* sx,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm, hipStream_t st) {
  const dim3 grid(1), block(64 * kSmallWaves);
#define MM_FRONT(NX)                                                                               \
  hipLaunchKernelGGL((k_front_small<kG, NX>), grid, block, 0, st, T, d, E, k, x, wr, bias, idx, w, \
                     xq, sx, offsets, perm, inv_perm)
  switch (d % kWave == 0 ? d / kWave : 0) {
    case 4: MM_FRONT(4); return true;
    case 8: MM_FRONT(8); return true;
    case 12: MM_FRONT(12); return true;
    case 16: MM_FRONT(16); return true;
    case 20: MM_FRONT(20); return true;
    default: return false;
  }
#undef MM_FRONT
}

}  // namespace

bool launch_front_small(int64_t T, int d, int E, int k, int gating, const float* x,
                        const float* wr, const float* bias, int32_t* idx, float* w, int8_t* xq,
                        float* sx, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        hipStream_t st) {
  if (T < 1 || T > kFrontUseT || k > 8) return false;
  switch (gating) {
    case 0: return launch_front_g<0>(T, d, E, k, x, wr, bias, idx, w, xq, sx, offsets, perm, inv_perm, st);
    case 1: return launch_front_g<1>(T, d, E, k, x, wr, bias, idx, w, xq, sx, offsets, perm, inv_perm, st);
    case 2: return launch_front_g<2>(T, d, E, k, x, wr, bias, idx, w, xq, sx, offsets, perm, inv_perm, st);
    default: return launch_front_g<3>(T, d, E, k, x, wr, bias, idx, w, xq, sx, offsets, perm, inv_perm, st);
  }
}

hipError_t launch_router(int64_t T, int d, int E, int k, int gating, const float* x,
                         const float* wr, const float* bias, int32_t* idx, float* w,
                         int8_t* xq, float* sx, hipStream_t st, int xq_layout,
                         uint8_t* hist, int64_t hist_stride) {
  const int64_t gm = act_gm_rows(xq_layout, T);
  // few tokens: one 16-wave workgroup per token (widths with a register form up to 1280)
  const bool small = T <= kSmallRouterT;
  if (hist != nullptr && small) return hipErrorInvalidValue;  // the per-token form counts nothing
  const bool q = xq != nullptr && router_quant_fused(d);
#define MM_ROUTER_G(G)                                                                            \
  if (q) launch_router_g<G, true>(small, T, d, E, k, x, wr, bias, idx, w, xq, sx, gm, hist, hist_stride, st); \
  else launch_router_g<G, false>(small, T, d, E, k, x, wr, bias, idx, w, nullptr, nullptr, 0, hist, hist_stride, st)
  switch (gating) {
    case 0: MM_ROUTER_G(0); break;
    case 1: MM_ROUTER_G(1); break;
    case 2: MM_ROUTER_G(2); break;
    default: MM_ROUTER_G(3); break;
  }
#undef MM_ROUTER_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || xq == nullptr || q) return e;
  return launch_act_quant_i8(T, d, x, xq, sx, st, xq_layout);  // widths without the fused form
}

}  // namespace mm
