// Training-side pieces of the MoE layer (MobileMoE close reading, section
// "Pre-training": the aux-loss-free expert-bias update of the stability list
// and the drop-and-pad dispatch of the efficiency list; section
// "Quantisation-aware training": eq. (6) applied as fake quantisation).
#include "common.h"
#include "launch_train.h"

#include <algorithm>

namespace mm {
namespace {

// One workgroup: histogram of the T*k expert ids in LDS, then every bias
// steps by lambda towards balance, the direction taken exactly in integers
// (T*k against E*load_e).  Ids outside [0, E) are not counted.
__global__ __launch_bounds__(1024) void k_bias_update(int64_t Tk, int E, const int32_t* __restrict__ idx,
                                                      float lambda, float* __restrict__ bias,
                                                      int32_t* __restrict__ load) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < Tk; i += blockDim.x) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = hist[e];
    const int64_t below = Tk - (int64_t)E * c;
    const float b = bias[e];
    bias[e] = below > 0 ? b + lambda : (below < 0 ? b - lambda : b);
    if (load) load[e] = c;
  }
}

// One wave: offsets_c = exclusive prefix sum of min(count_e, C) over the
// experts, count_e from the count sort's offsets.
__global__ __launch_bounds__(64) void k_drop_pad_scan(int E, int64_t C, const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ offsets_c) {
  const int lane = threadIdx.x;
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int kept = e < E ? (int)min((int64_t)(offsets[e + 1] - offsets[e]), C) : 0;
    int incl = kept;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int v = __shfl_up(incl, s);
      if (lane >= s) incl += v;
    }
    if (e < E) offsets_c[e] = run + incl - kept;
    run += __shfl(incl, 63);
  }
  if (lane == 0) offsets_c[E] = run;
}

// Thread i: padded-table entry i (i < E*C) and assignment i (i < T*k).  An
// assignment's rank within its expert is its count-sort row minus the
// expert's offset; ranks below C are kept.
__global__ __launch_bounds__(256) void k_drop_pad_fill(int64_t Tk, int E, int64_t C,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ inv,
                                                       const int32_t* __restrict__ offsets_c,
                                                       int32_t* __restrict__ buf,
                                                       int32_t* __restrict__ perm_c,
                                                       int32_t* __restrict__ inv_c) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)E * C) {
    const int e = (int)(i / C);
    const int64_t p = i - (int64_t)e * C;
    const int64_t cnt = offsets[e + 1] - offsets[e];
    buf[i] = p < cnt ? perm[offsets[e] + p] : -1;
  }
  if (i < Tk) {
    const int e = idx[i];
    int32_t row = -1;
    if (e >= 0 && e < E) {
      const int64_t r = (int64_t)inv[i] - offsets[e];
      if (r >= 0 && r < C && r < (int64_t)(offsets[e + 1] - offsets[e]))
        row = (int32_t)(offsets_c[e] + r);
    }
    inv_c[i] = row;
    if (row >= 0) perm_c[row] = (int32_t)i;
    if (i >= offsets_c[E]) perm_c[i] = -1;
  }
}

template <int kBits>
__device__ __forceinline__ float fq_levels() { return kBits == 4 ? 15.0f : 255.0f; }

// eq. (6) code of one value and its straight-through pass flag.
template <int kBits>
__device__ __forceinline__ float fq_one(float x, float s, bool& pass) {
  constexpr float qmin = kBits == 4 ? -8.0f : -128.0f, qmax = kBits == 4 ? 7.0f : 127.0f;
  if (s == 0.0f) {
    pass = true;
    return 0.0f;
  }
  const float u = rintf(x / s);  // IEEE quotient, round half to even
  pass = u >= qmin && u <= qmax;
  return s * fminf(fmaxf(u, qmin), qmax);
}

// Groups of 32 consecutive elements: 8 lanes per group, 4 elements per lane.
template <int kBits>
__global__ __launch_bounds__(256) void k_fake_quant_g32(int64_t n4, const float4* __restrict__ x,
                                                        float4* __restrict__ xbar,
                                                        const float4* __restrict__ gout,
                                                        float4* __restrict__ gin) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < n4;  // n4 is a multiple of 8: whole groups only
  const float4 v = live ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live && gin) g = gout[i];
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  if (!live) return;
  const float s = (2.0f * amax) / fq_levels<kBits>();
  bool p0, p1, p2, p3;
  const float4 o = make_float4(fq_one<kBits>(v.x, s, p0), fq_one<kBits>(v.y, s, p1),
                               fq_one<kBits>(v.z, s, p2), fq_one<kBits>(v.w, s, p3));
  if (xbar) xbar[i] = o;
  if (gin) gin[i] = make_float4(p0 ? g.x : 0.0f, p1 ? g.y : 0.0f, p2 ? g.z : 0.0f, p3 ? g.w : 0.0f);
}

// One group per row: one wave per row, the row read twice (maximum, then
// the codes; the second read hits the caches for rows up to tens of KB).
template <int kBits>
__global__ __launch_bounds__(256) void k_fake_quant_row(int64_t rows, int64_t q4, const float4* __restrict__ x,
                                                        float4* __restrict__ xbar,
                                                        const float4* __restrict__ gout,
                                                        float4* __restrict__ gin) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float4* xr = x + r * q4;
  float amax = 0.0f;
  for (int64_t c = lane; c < q4; c += 64) {
    const float4 v = xr[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = max64(amax);
  const float s = (2.0f * amax) / fq_levels<kBits>();
  for (int64_t c = lane; c < q4; c += 64) {
    const float4 v = xr[c];
    bool p0, p1, p2, p3;
    const float4 o = make_float4(fq_one<kBits>(v.x, s, p0), fq_one<kBits>(v.y, s, p1),
                                 fq_one<kBits>(v.z, s, p2), fq_one<kBits>(v.w, s, p3));
    if (xbar) xbar[r * q4 + c] = o;
    if (gin) {
      const float4 g = gout[r * q4 + c];
      gin[r * q4 + c] = make_float4(p0 ? g.x : 0.0f, p1 ? g.y : 0.0f, p2 ? g.z : 0.0f, p3 ? g.w : 0.0f);
    }
  }
}

}  // namespace

hipError_t launch_bias_update(int64_t Tk, int E, const int32_t* idx, float lambda, float* bias,
                              int32_t* load, hipStream_t st) {
  hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(1024), (size_t)E * sizeof(int), st, Tk, E, idx,
                     lambda, bias, load);
  return hipGetLastError();
}

hipError_t launch_drop_pad(int64_t Tk, int E, int64_t C, const int32_t* idx, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv, int32_t* buf, int32_t* offsets_c,
                           int32_t* perm_c, int32_t* inv_c, hipStream_t st) {
  hipLaunchKernelGGL(k_drop_pad_scan, dim3(1), dim3(64), 0, st, E, C, offsets, offsets_c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = std::max<int64_t>(Tk, (int64_t)E * C);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_drop_pad_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Tk, E, C,
                     idx, offsets, perm, inv, offsets_c, buf, perm_c, inv_c);
  return hipGetLastError();
}

hipError_t launch_fake_quant(int64_t rows, int64_t cols, int bits, bool row_group, const float* x,
                             float* xbar, const float* gout, float* gin, hipStream_t st) {
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float4* xb4 = reinterpret_cast<float4*>(xbar);
  const float4* go4 = reinterpret_cast<const float4*>(gout);
  float4* gi4 = reinterpret_cast<float4*>(gin);
  if (row_group) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (bits == 4)
      hipLaunchKernelGGL(k_fake_quant_row<4>, grid, dim3(256), 0, st, rows, cols / 4, x4, xb4, go4, gi4);
    else
      hipLaunchKernelGGL(k_fake_quant_row<8>, grid, dim3(256), 0, st, rows, cols / 4, x4, xb4, go4, gi4);
  } else {
    const int64_t n4 = rows * cols / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    if (bits == 4)
      hipLaunchKernelGGL(k_fake_quant_g32<4>, grid, dim3(256), 0, st, n4, x4, xb4, go4, gi4);
    else
      hipLaunchKernelGGL(k_fake_quant_g32<8>, grid, dim3(256), 0, st, n4, x4, xb4, go4, gi4);
  }
  return hipGetLastError();
}

}  // namespace mm
