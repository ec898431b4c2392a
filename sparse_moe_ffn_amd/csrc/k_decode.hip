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
//                 gate/up, quantise the hidden rows, product into ys
//   routed down   Umax * d/32 blocks: routing as above, weights issued, wait
//                 for the tile's gate/up, product into f
//   combine       one workgroup: topk_idx / topk_w, then (after every down
//                 block) the weighted combine, optional RMSNorm
// A producer makes its stores visible at device scope (a workgroup barrier,
// then one device-scope release increment of the stage's counter); a consumer
// polls the counter (bounded: a wait that gives up bumps the status word and
// goes on, so the kernel always ends), fences with device-scope acquire, then
// a barrier (the pattern of a grid-wide barrier, across the XCDs' L2s).  The
// last workgroup to finish resets the counters, so each call leaves the state
// as it found it.
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

// Counter words at the start of the state.
enum : int {
  kCtrRouter = 0,    // router workgroups done
  kCtrSharedGU = 1,  // shared gate/up blocks done
  kCtrDown = 2,      // down blocks (both kinds) done
  kCtrExit = 3,      // workgroups finished
  kCtrStatus = 4,    // waits that gave up (never reset here)
  kCtrTile = 8,      // routed gate/up blocks done, one word per tile
  kCtrWords = 64
};
static_assert(kCtrTile + kDecMaxSlots <= kCtrWords, "tile counters fit the counter block");

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
  uint32_t* ctr;  // kCtrWords counters
  float* logits;  // [T][kLogitStride]
  float* a_r;     // [T*k][h] routed hidden rows, expert-sorted
  float* a_s;     // [T][hs]
  float* f;       // [T*k][d] routed outputs, expert-sorted
  float* ys;      // [T][d]
  uint32_t spin_limit;
};

// The workgroup's stores are ordered before one device-scope release
// increment of the stage's counter.
__device__ __forceinline__ void signal_done(uint32_t* c) {
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *c >= target (thread 0 polls, at most spin_limit times; giving
// up bumps the status word), then fences so that the producers' stores are
// seen by the whole workgroup.
__device__ __forceinline__ void wait_count(uint32_t* c, uint32_t target, uint32_t* status,
                                           uint32_t spin_limit) {
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++n >= spin_limit) {
        __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Routing of the call in workgroup memory, identical to the router kernels'
// top-k and mm_route_permute's stable count sort.
struct RouteTab {
  int32_t off[65];
  int32_t perm[kDecMaxSlots];
  int32_t inv[kDecMaxSlots];
  int32_t idx[kDecMaxSlots];
  float w[kDecMaxSlots];
};

template <int kGating>
__device__ __forceinline__ void build_routing(const DecodeArgs& A, RouteTab& R) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = A.E, k = A.k, Tk = A.T * A.k;
  if (wave < A.T) {  // wave t: top-k of token t
    float mine, gl;
    biased_logit<kGating>(A.logits + wave * kLogitStride, A.bias, lane, E, mine, gl);
    int sel;
    float wgt;
    select_topk_lanes<kGating>(mine, gl, lane, E, k, sel, wgt);
    if (lane < k) {
      R.idx[wave * k + lane] = sel;
      R.w[wave * k + lane] = wgt;
    }
  }
  __syncthreads();
  if (wave == 0) {  // expert offsets: exclusive scan of the counts
    int c = 0;
    for (int s = 0; s < Tk; ++s) c += R.idx[s] == lane;
    if (lane >= E) c = 0;
    int inc = c;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int v = __shfl_up(inc, s);
      if (lane >= s) inc += v;
    }
    if (lane < E) {
      R.off[lane] = inc - c;
      if (lane == E - 1) R.off[E] = inc;
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
// with fused multiply-adds, then the 64-lane tree).
__device__ __forceinline__ void router_role(const DecodeArgs& A, int g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = 4 * g + wave, nx = A.d / kWave;
  if (e < A.E) {
    float wv[kRouterNX];
    const float* we = A.wr + (int64_t)e * A.d;
#pragma unroll
    for (int c = 0; c < kRouterNX; ++c)
      if (c < nx) wv[c] = we[lane + kWave * c];
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      if (t >= A.T) break;
      float p = 0.0f;
#pragma unroll
      for (int c = 0; c < kRouterNX; ++c)
        if (c < nx) p = __builtin_fmaf(A.x[(int64_t)t * A.d + lane + kWave * c], wv[c], p);
      const float l = tree_sum64(p);  // the bias is added at the selection
      if (lane == 0) A.logits[t * kLogitStride + e] = l;
    }
  }
  signal_done(A.ctr + kCtrRouter);
}

// Combine of token t by wave t, the arithmetic of combine_token: per output
// column the gate-weighted FMA chain over the token's k expert rows (j
// ascending, from 0), then + ys; with norm_lds, RMSNorm from the per-lane sum
// of squares over the lane's columns l, l+64, ... (x, y, z, w in order) and
// the wave butterfly sum.  norm_lds: [d] floats of workgroup memory.
constexpr int kMaxChunks = 5;  // float4 columns per lane: d <= 1280

template <bool kBF16Out, bool kNorm>
__device__ __forceinline__ void combine_small(const DecodeArgs& A, const RouteTab& R, int t,
                                              float4* norm_lds) {
  const int lane = threadIdx.x & 63, k = A.k, q = A.d / 4;
  int pj[8];
  float wj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pj[j] = j < k ? R.inv[t * k + j] : 0;
    wj[j] = j < k ? R.w[t * k + j] : 0.0f;
  }
  const float4* f4 = reinterpret_cast<const float4*>(A.f);
  const float4* ys4 = A.hs > 0 ? reinterpret_cast<const float4*>(A.ys) + (int64_t)t * q : nullptr;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c4 = lane + 64 * i;
    if (c4 >= q) break;
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) v[j] = f4[(int64_t)pj[j] * q + c4];
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ys4) sv = ys4[c4];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        a.x = fmaf(wj[j], v[j].x, a.x);
        a.y = fmaf(wj[j], v[j].y, a.y);
        a.z = fmaf(wj[j], v[j].z, a.z);
        a.w = fmaf(wj[j], v[j].w, a.w);
      }
    if (ys4) {
      a.x += sv.x;
      a.y += sv.y;
      a.z += sv.z;
      a.w += sv.w;
    }
    if (kBF16Out) {
      ushort4 o;
      o.x = f32_to_bf16(a.x);
      o.y = f32_to_bf16(a.y);
      o.z = f32_to_bf16(a.z);
      o.w = f32_to_bf16(a.w);
      reinterpret_cast<ushort4*>(A.y)[(int64_t)t * q + c4] = o;
    } else {
      reinterpret_cast<float4*>(A.y)[(int64_t)t * q + c4] = a;
    }
    if (kNorm) {
      ss = fmaf(a.x, a.x, ss);
      ss = fmaf(a.y, a.y, ss);
      ss = fmaf(a.z, a.z, ss);
      ss = fmaf(a.w, a.w, ss);
      norm_lds[c4] = a;
    }
  }
  if constexpr (kNorm) {
    ss = wave_sum(ss);
    const float inv_rms = 1.0f / sqrtf(ss / (float)A.d + A.eps);
    for (int c4 = lane; c4 < q; c4 += 64) {
      const float4 a = norm_lds[c4];
      reinterpret_cast<float4*>(A.y_norm)[(int64_t)t * q + c4] =
          make_float4(a.x * inv_rms, a.y * inv_rms, a.z * inv_rms, a.w * inv_rms);
    }
  }
}

// Launch shape: workgroups per role (each loops over its role's blocks with
// that stride) and the blocks per role.
struct DecodeGrid {
  int router, sgu_b, rgu_b, sdn_b, rdn_b;  // blocks
  int sgu_w, rgu_w, sdn_w, rdn_w;          // workgroups
};

template <int kGating>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fused(
    DecodeArgs A, DecodeGrid G) {
  __shared__ RouteTab R;
  extern __shared__ int4 smem4[];
  uint32_t* ctr = A.ctr;
  uint32_t* status = ctr + kCtrStatus;
  const int T = A.T, d = A.d, h = A.h, hs = A.hs, Tk = A.T * A.k;
  int b = (int)blockIdx.x;
  bool routed = false;  // routing table built (uniform over the workgroup)
  auto routing = [&]() {
    if (routed) return;
    wait_count(ctr + kCtrRouter, (uint32_t)G.router, status, A.spin_limit);
    build_routing<kGating>(A, R);
    routed = true;
  };

  if (b < G.router) {
    router_role(A, b);
  } else if ((b -= G.router) < G.sgu_w) {
    const ExpertArgs as{T, T, d, hs, 1, 1, nullptr, nullptr};
    const GemvProb P{as, d, 2 * hs, hs / 32, nullptr, nullptr, A.sgq, A.sgs, A.a_s, nullptr, A.x};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.sgu_b; blk += G.sgu_w) {
      gemv_block<kRGemv, true, false, true, false, true, true>(P, blk);
      signal_done(ctr + kCtrSharedGU);
    }
  } else if ((b -= G.sgu_w) < G.rgu_w) {
    const ExpertArgs ar{Tk, T, d, h, A.E, A.k, R.perm, R.off};
    const GemvProb P{ar, d, 2 * h, h / 32, nullptr, nullptr, A.gq, A.gs, A.a_r, nullptr, A.x};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.rgu_b; blk += G.rgu_w) {
      gemv_block<kRGemv, true, false, false, false, true, true>(P, blk, routing);
      signal_done(ctr + kCtrTile + blk / (h / 32));
    }
  } else if ((b -= G.rgu_w) < G.sdn_w) {
    const ExpertArgs as{T, T, d, hs, 1, 1, nullptr, nullptr};
    const GemvProb P{as, hs, d, d / 32, nullptr, nullptr, A.sdq, A.sds, A.ys, nullptr, A.a_s};
    auto ready = [&]() { wait_count(ctr + kCtrSharedGU, (uint32_t)G.sgu_b, status, A.spin_limit); };
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.sdn_b; blk += G.sdn_w) {
      gemv_block<kRGemv, false, false, true, true, true, false>(P, blk, NoHook(), ready);
      signal_done(ctr + kCtrDown);
    }
  } else if ((b -= G.sdn_w) < G.rdn_w) {
    const ExpertArgs ar{Tk, T, d, h, A.E, A.k, nullptr, R.off};
    const GemvProb P{ar, h, d, d / 32, nullptr, nullptr, A.dq, A.dsc, A.f, nullptr, A.a_r};
#pragma clang loop unroll(disable)
    for (int blk = b; blk < G.rdn_b; blk += G.rdn_w) {
      const int u = blk / (d / 32);
      auto ready = [&]() { wait_count(ctr + kCtrTile + u, (uint32_t)(h / 32), status, A.spin_limit); };
      gemv_block<kRGemv, false, false, false, true, true, false>(P, blk, routing, ready);
      signal_done(ctr + kCtrDown);
    }
  } else {
    routing();
    if ((int)threadIdx.x < Tk) {
      A.topk_idx[threadIdx.x] = R.idx[threadIdx.x];
      A.topk_w[threadIdx.x] = R.w[threadIdx.x];
    }
    wait_count(ctr + kCtrDown, (uint32_t)(G.sdn_b + G.rdn_b), status, A.spin_limit);
    const int t = threadIdx.x >> 6;
    float4* nbuf = reinterpret_cast<float4*>(smem4) + (int64_t)t * (d / 4);
    if (t < T) {
      if (A.y_norm)
        combine_small<false, true>(A, R, t, nbuf);
      else if (A.out_bf16)
        combine_small<true, false>(A, R, t, nullptr);
      else
        combine_small<false, false>(A, R, t, nullptr);
    }
  }

  // The last workgroup out resets the counters: every other workgroup has
  // passed all of its waits by the time it counts itself out.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(ctr + kCtrExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == gridDim.x - 1) {
      for (int i = 0; i < kCtrWords; ++i)
        if (i != kCtrStatus) __hip_atomic_store(ctr + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

// Scratch of the no-allocation entry point (mm_moe_decode_noalloc): the
// state block and intermediates of mm_moe_decode in a fixed device array,
// for callers that cannot allocate.  Each device holds its own copy at its
// own address (hipGetSymbolAddress once per device); in host code the name
// is only a handle for that lookup.  Zero at load; cleared once more when a
// device's address is first taken; every call leaves the counters zero.
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

size_t decode_fused_state_bytes() { return (size_t)kCtrWords * 4 + (size_t)kDecMaxT * kLogitStride * 4; }

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
  A.ctr = static_cast<uint32_t*>(a.state);
  A.logits = reinterpret_cast<float*>(static_cast<char*>(a.state) + kCtrWords * 4);
  A.a_r = a.a_r;
  A.a_s = a.a_s;
  A.f = a.f;
  A.ys = a.ys;
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
    grid = G.router + G.sgu_w + G.rgu_w + G.sdn_w + G.rdn_w + 1;
    if (grid <= cap) break;
    if (G.sgu_w <= 1 && G.rgu_w <= 1 && G.sdn_w <= 1 && G.rdn_w <= 1) return hipErrorInvalidConfiguration;
  }
  if (grid_out) *grid_out = grid;
  void* args[] = {&A, &G};
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, lds, st);
}

}  // namespace mm
