// The whole MoE layer of a decode step (1 to 4 tokens) in one kernel launch.
//
// MobileMoE close reading, section "Runtime latency": decoding a few tokens is
// bound by reading the selected experts' weights, and section "Custom MoE
// kernel", principle (2): the layer's steps are fused so that the
// intermediates never take a round trip through separate launches.  At a few
// tokens the layer moves about 3 MB of INT4 weights (a fraction of a
// microsecond of HBM time), so what is left to save is the chain of launches
// and their dependency gaps.  This kernel computes exactly what mm_moe_forward
// computes for the same inputs (eq. (*), with the same arithmetic in the same
// order: the router, top-k and count sort of the router kernels, the
// weight-streaming gate/up and down blocks of gemv_block.h, the combine of
// combine_row.h), so the outputs agree bit for bit.
//
// Workgroups take roles by index, in dependency order, and a consumer only
// waits for producers with lower indices:
//   router        ceil(E/4) groups, one wave per expert: the logits of every
//                 token into the state's logit table
//   shared g/u    hs/32 blocks of the shared expert's gate/up (+ SwiGLU),
//                 quantising x in the workgroup (no waits)
//   routed g/u    Umax * h/32 blocks (Umax = min(T*k, E) experts at most, one
//                 4-row tile each since every expert has at most T <= 4 rows):
//                 wait for the logits, redo the top-k and the count sort in
//                 workgroup memory, then the tile's product
//   shared down   d/32 blocks: weights issued, then wait for the shared
//                 hidden rows, quantise them, product into ys
//   routed down   Umax * d/32 blocks: routing as above, weights issued, wait
//                 for the tile's hidden rows, product into f
//   combine       one workgroup: topk_idx / topk_w, then (as the expert
//                 outputs arrive) the weighted combine, optional RMSNorm
// Every value handed from one workgroup to another (logits, hidden rows,
// expert outputs) is a flag-in-word: the FP32 bits with this call's tag in
// the upper half of one 64-bit word, stored and polled with device-scope
// atomic accesses (LLWait in gemv_block.h), so a consumer waits for the data
// itself, with no counter, no fence and no cache invalidation.  The tag is
// the state's call count + 1, read at the start; the last workgroup to finish
// (counted on the exit counter) bumps the call count and clears the exit
// counter, so each call leaves the state ready for the next.  Polls are
// bounded: a wait that gives up bumps the status word and goes on, so the
// kernel always ends.
#include <algorithm>
#include <mutex>

#include "combine_row.h"
#include "common.h"
#include "gemv_block.h"
#include "launch.h"
#include "router_topk.h"

namespace mm {
namespace {

constexpr int kDecMaxT = 4;
constexpr int kDecMaxSlots = kDecMaxT * 8;  // T * k, k <= 8
constexpr int kRouterNX = 20;               // d / 64 <= 20
constexpr int kLogitStride = 64;            // logit table [T][64]
// The logit table is written in kLogitCopies copies, kLogitCopyStride words
// apart (so they sit in different memory channels); a consumer reads copy
// blockIdx % kLogitCopies, which spreads the polls of every routed
// workgroup.
constexpr int kLogitCopies = 8;
constexpr int kLogitCopyStride = kDecMaxT * kLogitStride + 32;

// State words: the call count (word 0), the give-up count (word 4), and the
// exit counter on a line of its own; then the logit copies (64-bit words).
enum : int { kCallCount = 0, kStatus = 4, kExit = 64, kStateWords = 128 };

struct DecodeArgs {
  int T, d, E, k, h, hs;
  const float* x;
  const float* wr;
  const float* bias;
  const uint8_t* gq;  // routed gate/up, prepacked INT4 + scales
  const float* gs;
  const uint8_t* dq;  // routed down
  const float* dsc;
  const uint8_t* sgq;  // shared gate/up / down
  const float* sgs;
  const uint8_t* sdq;
  const float* sds;
  int32_t* topk_idx;
  float* topk_w;
  void* y;
  float* y_norm;
  float eps;
  int out_bf16;
  uint32_t* state;   // kStateWords words
  uint64_t* logits;  // kLogitCopies copies of [T][kLogitStride], flag-in-word
  uint64_t* a_r;     // [T*k][h] routed hidden rows, expert-sorted, flag-in-word
  uint64_t* a_s;     // [T][hs]
  uint64_t* f;       // [T*k][d] routed outputs, expert-sorted
  uint64_t* ys;      // [T][d]
  uint32_t spin_limit;
};

// Routing of the call in workgroup memory, identical to the router kernels'
// top-k and mm_route_permute's stable count sort.
struct RouteTab {
  int32_t off[65];
  int32_t perm[kDecMaxSlots];
  int32_t inv[kDecMaxSlots];
  int32_t idx[kDecMaxSlots];
  float w[kDecMaxSlots];
  int32_t tiles[kTileWords];  // every expert of the call owns one tile (FusedTiles)
};
static_assert(kFusedTiles >= kDecMaxSlots, "one tile per slot at most");

template <int kGating>
__device__ __forceinline__ void build_routing(const DecodeArgs& A, const LLWait& L, RouteTab& R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = A.E, k = A.k, Tk = A.T * A.k;
  if (wave < A.T) {  // wave t: top-k of token t, once its logits have arrived
    const uint64_t* row =
        A.logits + (blockIdx.x % kLogitCopies) * kLogitCopyStride + wave * kLogitStride;
    float raw = 0.0f;
    uint32_t n = 0;
    for (;;) {
      bool ok = true;
      if (lane < E) {
        const uint64_t w = ll_get(row + lane);
        ok = ll_ready(w, L.tag);
        raw = ll_value(w);
      }
      if (ll_settle(ok, n, L)) break;
    }
    float mine, gl;
    biased_value<kGating>(raw, A.bias, lane, E, mine, gl);
    int sel;
    float wgt;
    select_topk_lanes<kGating>(mine, gl, lane, E, k, sel, wgt);
    if (lane < k) {
      R.idx[wave * k + lane] = sel;
      R.w[wave * k + lane] = wgt;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane e: its count and its offset (the slots with a lower expert: the
    // exclusive scan of the counts), and, for experts with rows, its tile
    // (one per expert, T <= 4 rows) numbered in expert order
    int c = 0, below = 0;
    for (int s = 0; s < Tk; ++s) {
      const int v = R.idx[s];
      c += v == lane;
      below += v < lane;
    }
    const bool has = lane < E && c > 0;
    const uint64_t used = __ballot(has);
    if (lane < E) R.off[lane] = below;
    if (lane == 0) {
      R.off[E] = Tk;
      R.tiles[kTileCount] = __popcll(used);
    }
    if (has) {
      // experts with rows below this lane (mbcnt: set bits of `used` under the lane)
      const int u = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(used >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)used, 0u));
      R.tiles[kTileP0 + u] = below;
      R.tiles[kTileN + u] = c;
      R.tiles[kTileE + u] = lane;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < Tk) {  // stable rank among the earlier slots of the same expert
    const int s = threadIdx.x, e = R.idx[s];
    int rank = 0;
    for (int q = 0; q < s; ++q) rank += R.idx[q] == e;
    const int pos = R.off[e] + rank;
    R.perm[pos] = s;
    R.inv[s] = pos;
  }
  __syncthreads();
}

// Router workgroup g: wave w computes the logits of expert 4g + w for every
// token (the router kernels' order: lane partials over columns l, l+64, ...
// with fused multiply-adds, then the 64-lane tree).  The token rows are
// staged in workgroup memory (xs: T*d floats) so that all of them are read
// at once; every logit goes to each of the kLogitCopies copies of the table.
__device__ __forceinline__ void router_role(const DecodeArgs& A, const LLWait& L, int g, float* xs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = 4 * g + wave, nx = A.d / kWave;
  float wv[kRouterNX];
  if (e < A.E) {
    const float* we = A.wr + (int64_t)e * A.d;
#pragma unroll
    for (int c = 0; c < kRouterNX; ++c)
      if (c < nx) wv[c] = we[lane + kWave * c];
  }
  for (int i = threadIdx.x; i < A.T * A.d / 4; i += 256)
    reinterpret_cast<float4*>(xs)[i] = reinterpret_cast<const float4*>(A.x)[i];
  __syncthreads();
  if (e < A.E) {
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      if (t >= A.T) break;
      float p = 0.0f;
#pragma unroll
      for (int c = 0; c < kRouterNX; ++c)
        if (c < nx) p = __builtin_fmaf(xs[t * A.d + lane + kWave * c], wv[c], p);
      const float l = tree_sum64(p);  // the bias is added at the selection
      if (lane < kLogitCopies) ll_put(A.logits + lane * kLogitCopyStride + t * kLogitStride + e, l, L.tag);
    }
  }
}

// Combine of token t (one workgroup per token), the arithmetic of
// combine_token: per output column the gate-weighted FMA chain over the
// token's k expert rows (j ascending, from 0), then + ys; then RMSNorm from
// the per-lane sum of squares over the lane's columns l, l+64, ... of float4
// (x, y, z, w in order) and the wave butterfly sum.  Thread tid takes the
// columns tid + 256 m of every row: it waits for its words of the k expert
// rows and the ys row (one wait for k = 4 with ys and d <= 1024, two for
// d = 1280) and forms y for those columns itself; for the norm, wave 0 forms
// the sum of squares in combine_token's order from the y row in workgroup
// memory.
template <bool kBF16Out, bool kNorm>
__device__ __forceinline__ void combine_token_ll(const DecodeArgs& A, const LLWait& L,
                                                 const RouteTab& R, int t, float* lds) {
  __shared__ float s_inv_rms;
  const int k = A.k, d = A.d;
  const bool shared = A.hs > 0;
  const int nrows = k + (shared ? 1 : 0);
  constexpr int kRows = 5, kCols = 4;  // per wait: 5 rows x 1024 columns
  float* yrow = lds;                   // [d], for the norm
  for (int c0 = 0; c0 < d; c0 += 256 * kCols) {
    float acc[kCols];
#pragma unroll
    for (int m = 0; m < kCols; ++m) acc[m] = 0.0f;
    for (int r0 = 0; r0 < nrows; r0 += kRows) {
      const uint64_t* rp[kRows];
      float wr[kRows];
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) {
        const int j = min(r0 + jj, nrows - 1);
        rp[jj] = j < k ? A.f + (int64_t)__builtin_amdgcn_readfirstlane(R.inv[t * k + j]) * d
                       : A.ys + (int64_t)t * d;
        wr[jj] = j < k ? R.w[t * k + j] : 0.0f;
      }
      uint64_t w[kRows][kCols];
      uint32_t n = 0;
      for (;;) {
        // every load of the round is issued before any is looked at
        // (positions past the row or the row count re-read a valid word
        // and are ignored)
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
          for (int m = 0; m < kCols; ++m)
            w[jj][m] = ll_get(rp[jj] + min(c0 + (int)threadIdx.x + 256 * m, d - 1));
        bool ok = true;
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
          for (int m = 0; m < kCols; ++m) {
            const bool used = r0 + jj < nrows && c0 + (int)threadIdx.x + 256 * m < d;
            ok = ok & (!used || ll_ready(w[jj][m], L.tag));
          }
        if (ll_settle_wg(ok, n, L)) break;
      }
      // rows in order: the expert rows into the FMA chain, the ys row added
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) {
        const int j = r0 + jj;
        if (j >= nrows) break;
#pragma unroll
        for (int m = 0; m < kCols; ++m) {
          const float v = ll_value(w[jj][m]);
          acc[m] = j < k ? fmaf(wr[jj], v, acc[m]) : acc[m] + v;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kCols; ++m) {
      const int c = c0 + (int)threadIdx.x + 256 * m;
      if (c < d) {
        if (kBF16Out)
          reinterpret_cast<uint16_t*>(A.y)[(int64_t)t * d + c] = f32_to_bf16(acc[m]);
        else
          reinterpret_cast<float*>(A.y)[(int64_t)t * d + c] = acc[m];
        if (kNorm) yrow[c] = acc[m];
      }
    }
  }
  if constexpr (kNorm) {
    __syncthreads();
    if (threadIdx.x < 64) {
      const float4* y4 = reinterpret_cast<const float4*>(yrow);
      float ss = 0.0f;
      for (int c4 = threadIdx.x; c4 < d / 4; c4 += 64) {
        const float4 a = y4[c4];
        ss = fmaf(a.x, a.x, ss);
        ss = fmaf(a.y, a.y, ss);
        ss = fmaf(a.z, a.z, ss);
        ss = fmaf(a.w, a.w, ss);
      }
      ss = wave_sum(ss);
      if (threadIdx.x == 0) s_inv_rms = 1.0f / sqrtf(ss / (float)d + A.eps);
    }
    __syncthreads();
    const float inv_rms = s_inv_rms;
    for (int c = threadIdx.x; c < d; c += 256) A.y_norm[(int64_t)t * d + c] = yrow[c] * inv_rms;
  }
}

// Launch shape: workgroups per role (each loops over its role's blocks with
// that stride) and the blocks per role.
struct DecodeGrid {
  int router, sgu_b, rgu_b, sdn_b, rdn_b;  // blocks (router: workgroups)
  int sgu_w, rgu_w, sdn_w, rdn_w;          // workgroups
};

template <int kGating>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fused(
    DecodeArgs A, DecodeGrid G) {
  __shared__ RouteTab R;
  extern __shared__ int4 smem4[];
  const uint32_t count = __hip_atomic_load(A.state + kCallCount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const LLWait L{__builtin_amdgcn_readfirstlane(count) + 1u, A.spin_limit, A.state + kStatus};
  const int T = A.T, d = A.d, h = A.h, hs = A.hs, Tk = A.T * A.k;
  int b = (int)blockIdx.x;
  bool routed = false;  // routing table built (uniform over the workgroup)
  auto routing = [&]() {
    if (routed) return;
    build_routing<kGating>(A, L, R);
    routed = true;
  };

  if (b < G.router) {
    router_role(A, L, b, reinterpret_cast<float*>(smem4));
  } else if ((b -= G.router) < G.sgu_w) {
    const ExpertArgs as{T, T, d, hs, 1, 1, nullptr, nullptr};
    const GemvProb P{as, d, 2 * hs, hs / 32, nullptr, nullptr, A.sgq, A.sgs,
                     reinterpret_cast<float*>(A.a_s), nullptr, A.x, L};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.sgu_b; blk += G.sgu_w) {
      gemv_block<kRGemv, true, false, true, false, true, true>(P, blk);
      __syncthreads();
    }
  } else if ((b -= G.sgu_w) < G.rgu_w) {
    const ExpertArgs ar{Tk, T, d, h, A.E, A.k, R.perm, R.off};
    const GemvProb P{ar, d, 2 * h, h / 32, nullptr, nullptr, A.gq, A.gs,
                     reinterpret_cast<float*>(A.a_r), nullptr, A.x, L, R.tiles};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.rgu_b; blk += G.rgu_w) {
      gemv_block<kRGemv, true, false, false, false, true, true>(P, blk, routing);
      __syncthreads();
    }
  } else if ((b -= G.rgu_w) < G.sdn_w) {
    const ExpertArgs as{T, T, d, hs, 1, 1, nullptr, nullptr};
    const GemvProb P{as, hs, d, d / 32, nullptr, nullptr, A.sdq, A.sds,
                     reinterpret_cast<float*>(A.ys), nullptr, reinterpret_cast<const float*>(A.a_s), L};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.sdn_b; blk += G.sdn_w) {
      gemv_block<kRGemv, false, false, true, true, true, false>(P, blk);
      __syncthreads();
    }
  } else if ((b -= G.sdn_w) < G.rdn_w) {
    const ExpertArgs ar{Tk, T, d, h, A.E, A.k, nullptr, R.off};
    const GemvProb P{ar, h, d, d / 32, nullptr, nullptr, A.dq, A.dsc,
                     reinterpret_cast<float*>(A.f), nullptr, reinterpret_cast<const float*>(A.a_r), L,
                     R.tiles};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.rdn_b; blk += G.rdn_w) {
      gemv_block<kRGemv, false, false, false, true, true, false>(P, blk, routing);
      __syncthreads();
    }
  } else {
    // combine workgroup of token t = b
    const int t = b - G.rdn_w;
    routing();
    if ((int)threadIdx.x < A.k) {
      A.topk_idx[t * A.k + threadIdx.x] = R.idx[t * A.k + threadIdx.x];
      A.topk_w[t * A.k + threadIdx.x] = R.w[t * A.k + threadIdx.x];
    }
    float* lds = reinterpret_cast<float*>(smem4);
    if (A.y_norm)
      combine_token_ll<false, true>(A, L, R, t, lds);
    else if (A.out_bf16)
      combine_token_ll<true, false>(A, L, R, t, lds);
    else
      combine_token_ll<false, false>(A, L, R, t, lds);
  }

  // The last workgroup out (every other one has finished all of its waits
  // when it counts itself out) moves the call count on and clears the exit
  // counter.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(A.state + kExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == gridDim.x - 1) {
      __hip_atomic_store(A.state + kCallCount, L.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(A.state + kExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

// Scratch of the no-allocation entry point (mm_moe_decode_noalloc): the
// state block and intermediates of mm_moe_decode in a fixed device array,
// for callers that cannot allocate.  Each device holds its own copy at its
// own address (hipGetSymbolAddress once per device); in host code the name
// is only a handle for that lookup.  Zero at load; cleared once more when a
// device's address is first taken; every call leaves the state ready for the
// next (see the call count above).
constexpr size_t kDecodeScratchBytes = size_t(512) << 10;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

__global__ void k_clear_words(uint32_t* p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

}  // namespace

size_t decode_scratch_capacity() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void** out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the state block starts at zero (a kernel, not a memset node: the call
    // may be under stream capture)
    const int words = (int)(decode_fused_state_bytes() / 4);
    hipLaunchKernelGGL(k_clear_words, dim3((words + 255) / 256), dim3(256), 0, st,
                       static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

bool decode_fused_fits(int64_t T, int d, int E, int k, int h, int hs) {
  return T >= 1 && T <= kDecMaxT && k >= 1 && k <= 8 && E >= 1 && E <= 64 && d % 128 == 0 &&
         d <= kWave * kRouterNX && h % 64 == 0 && hs % 64 == 0 && gemv_i4_fits(d, true) &&
         gemv_i4_qin_fits(h) && (hs == 0 || gemv_i4_qin_fits(hs));
}

size_t decode_fused_state_bytes() {
  return (size_t)kStateWords * 4 + (size_t)kLogitCopies * kLogitCopyStride * 8;
}

namespace {

// Resident workgroups per CU of one instantiation and LDS size, and the CU
// count, per device (asked once: the launch sits on the decode path).
struct OccEntry {
  int dev, gating;
  size_t lds;
  int per_cu, cus;
};
std::mutex g_occ_mu;
OccEntry g_occ[32];
int g_occ_n = 0;

hipError_t occupancy(const void* fn, int gating, size_t lds, int& per_cu, int& cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_occ_mu);
  for (int i = 0; i < g_occ_n; ++i)
    if (g_occ[i].dev == dev && g_occ[i].gating == gating && g_occ[i].lds == lds) {
      per_cu = g_occ[i].per_cu;
      cus = g_occ[i].cus;
      return hipSuccess;
    }
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
  if (e != hipSuccess) return e;
  g_occ[g_occ_n % 32] = OccEntry{dev, gating, lds, per_cu, cus};
  ++g_occ_n;
  if (g_occ_n > 32) g_occ_n = 32;
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode_fused(const DecodeFusedArgs& a, hipStream_t st, int* grid_out) {
  DecodeArgs A{};
  A.T = (int)a.T;
  A.d = a.d;
  A.E = a.E;
  A.k = a.k;
  A.h = a.h;
  A.hs = a.hs;
  A.x = a.x;
  A.wr = a.wr;
  A.bias = a.bias;
  A.gq = a.gq;
  A.gs = a.gs;
  A.dq = a.dq;
  A.dsc = a.ds;
  A.sgq = a.sgq;
  A.sgs = a.sgs;
  A.sdq = a.sdq;
  A.sds = a.sds;
  A.topk_idx = a.topk_idx;
  A.topk_w = a.topk_w;
  A.y = a.y;
  A.y_norm = a.y_norm;
  A.eps = a.eps;
  A.out_bf16 = a.out_bf16 ? 1 : 0;
  A.state = static_cast<uint32_t*>(a.state);
  A.logits = reinterpret_cast<uint64_t*>(static_cast<char*>(a.state) + kStateWords * 4);
  A.a_r = static_cast<uint64_t*>(a.a_r);
  A.a_s = static_cast<uint64_t*>(a.a_s);
  A.f = static_cast<uint64_t*>(a.f);
  A.ys = static_cast<uint64_t*>(a.ys);
  A.spin_limit = a.spin_limit;
  // Blocks per role: every expert of the call owns one 4-row tile (at most
  // min(T*k, E) of them); tiles that turn out unused return at once.
  const int umax = (int)std::min<int64_t>(a.T * a.k, a.E);
  DecodeGrid G{};
  G.router = (a.E + 3) / 4;
  G.sgu_b = a.hs / 32;
  G.rgu_b = umax * (a.h / 32);
  G.sdn_b = a.hs > 0 ? a.d / 32 : 0;
  G.rdn_b = umax * (a.d / 32);
  const size_t lds = std::max(gemv_lds(a.d, true),
                              std::max(gemv_lds(a.h, false), gemv_lds(a.hs > 0 ? a.hs : 64, false)));
  const void* fn = nullptr;
  switch (a.gating) {
    case 0: fn = reinterpret_cast<const void*>(&k_decode_fused<0>); break;
    case 1: fn = reinterpret_cast<const void*>(&k_decode_fused<1>); break;
    case 2: fn = reinterpret_cast<const void*>(&k_decode_fused<2>); break;
    default: fn = reinterpret_cast<const void*>(&k_decode_fused<3>); break;
  }
  // Every workgroup must be resident at once (a consumer waits for
  // producers launched before it): with more blocks than fit, each
  // workgroup of a role takes every m-th block of it.
  int per_cu = 0, cus = 0;
  hipError_t e = occupancy(fn, a.gating, lds, per_cu, cus);
  if (e != hipSuccess) return e;
  const int64_t cap = (int64_t)per_cu * cus;
  int grid = 0;
  for (int m = 1;; ++m) {
    auto wg = [&](int blocks) { return (blocks + m - 1) / m; };
    G.sgu_w = wg(G.sgu_b);
    G.rgu_w = wg(G.rgu_b);
    G.sdn_w = wg(G.sdn_b);
    G.rdn_w = wg(G.rdn_b);
    grid = G.router + G.sgu_w + G.rgu_w + G.sdn_w + G.rdn_w + (int)a.T;
    if (grid <= cap) break;
    if (G.sgu_w <= 1 && G.rgu_w <= 1 && G.sdn_w <= 1 && G.rdn_w <= 1) return hipErrorInvalidConfiguration;
  }
  if (grid_out) *grid_out = grid;
  void* args[] = {&A, &G};
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, lds, st);
}

}  // namespace mm
