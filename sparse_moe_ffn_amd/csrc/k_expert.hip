// Expert products, row-tile (SIMT) form: used for small row counts (decode),
// for the FP32 and BF16 formats, and for the debug twins that expose the exact
// int32 group sums.
//
// MobileMoE close reading, section "Custom MoE kernel": after the count sort
// each expert multiplies its contiguous slice of tokens by its fused gate/up
// weight, applies SwiGLU, then the down weight.  INT4 weights use eq. (6)
// (section "Quantisation-aware training"): every output is
//   s_act * sum_g s_w[g] * isum_g,  isum_g = exact int32 sum over group g.
//
// A workgroup owns one tile of up to kRows rows of one expert.  The routed
// grid is sized for the worst case (ceil(rows/kRows) + min(E, rows) tiles); each
// workgroup derives its (expert, tile) from expert_offsets on the device and
// exits if it has none.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

// Resolves this workgroup's tile: first sorted row p0, row count n, expert e.
// Routed form: experts' tiles are numbered expert by expert.  All threads of
// the block must call it.
template <int kRows>
__device__ void find_tile(const ExpertArgs& a, int& p0, int& n, int& e) {
  __shared__ int s_p0, s_n, s_e;
  if (a.offsets == nullptr) {
    p0 = (int)blockIdx.x * kRows;
    n = (int)min((int64_t)kRows, a.rows - p0);
    e = 0;
    return;
  }
  if (threadIdx.x < 64)
    routed_tile(a.offsets, a.E, (int)a.rows, kRows, (int)blockIdx.x, &s_p0, &s_n, &s_e);
  __syncthreads();
  p0 = s_p0;
  n = s_n;
  e = s_e;
}

// Loads the 32 prepacked INT4 weights of (row o, group g) as eight words of
// four int8 values (x16), in column order.
__device__ __forceinline__ void load_w32(const uint8_t* __restrict__ w, int G, int o, int g,
                                         uint32_t (&q)[8]) {
  const uint2* c = reinterpret_cast<const uint2*>(w + ((int64_t)(o >> 5) * G + g) * kChunkBytes);
  const uint2 a = c[o & 31], b = c[(o & 31) + 32];
  unpack8(a.x, q[0], q[1]);
  unpack8(a.y, q[2], q[3]);
  unpack8(b.x, q[4], q[5]);
  unpack8(b.y, q[6], q[7]);
}

__device__ __forceinline__ int dot32(const uint32_t (&q)[8], const int* __restrict__ act) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = __builtin_amdgcn_sdot4((int)q[i], act[i], s, false);
  return s;
}

constexpr int kRowsI4 = 16;
constexpr int kRowsFp = 8;

// INT4 gate/up + SwiGLU + per-row INT8 re-quantisation of the hidden row
// (skipped when hq is null: the FP32 rows in aout are then the output).
// A rows (INT8) are staged in LDS; thread o computes gate o and up o for every
// row of the tile and writes a = SiLU(g) * u (FP32) to the staging buffer
// `abuf`; the block then reduces max|a| per row, and every thread quantises
// the values it wrote itself into hq with the row scale hs.
template <bool kCapture>
__global__ __launch_bounds__(256) void k_gateup_i4(ExpertArgs a, const int8_t* __restrict__ xq,
                                                   const float* __restrict__ sx,
                                                   const uint8_t* __restrict__ wq,
                                                   const float* __restrict__ wsc,
                                                   float* __restrict__ aout,
                                                   int8_t* __restrict__ hq,
                                                   float* __restrict__ hs,
                                                   int32_t* __restrict__ isum) {
  extern __shared__ int4 smem4[];
  int8_t* As = reinterpret_cast<int8_t*>(smem4);
  __shared__ int s_tok[kRowsI4];
  int p0, n, e;
  find_tile<kRowsI4>(a, p0, n, e);
  if (n <= 0) return;
  const int d = a.d, h = a.h, G = d / kGroup, N2 = 2 * h;
  if (threadIdx.x < kRowsI4) {
    int tok = (int)threadIdx.x < n ? (a.perm ? a.perm[p0 + threadIdx.x] / a.k : p0 + threadIdx.x) : 0;
    if ((unsigned)tok >= (unsigned)a.T) tok = 0;  // stays in bounds for a corrupt perm
    s_tok[threadIdx.x] = tok;
  }
  __syncthreads();
  const int c16 = d / 16;
  for (int i = threadIdx.x; i < kRowsI4 * c16; i += blockDim.x) {
    const int r = i / c16, c = i % c16;
    int4 v = make_int4(0, 0, 0, 0);
    if (r < n) v = reinterpret_cast<const int4*>(xq + (int64_t)s_tok[r] * d)[c];
    smem4[r * c16 + c] = v;
  }
  __syncthreads();
  const uint8_t* we = wq + (int64_t)e * (N2 / 32) * G * kChunkBytes;
  const float* se = wsc + (int64_t)e * (N2 / 32) * G * 32;
  float amax[kRowsI4];
#pragma unroll
  for (int r = 0; r < kRowsI4; ++r) amax[r] = 0.0f;
  for (int o = threadIdx.x; o < h; o += blockDim.x) {
    float ag[kRowsI4], au[kRowsI4];
#pragma unroll
    for (int r = 0; r < kRowsI4; ++r) ag[r] = au[r] = 0.0f;
    for (int g = 0; g < G; ++g) {
      uint32_t qg[8], qu[8];
      load_w32(we, G, o, g, qg);
      load_w32(we, G, o + h, g, qu);
      const float sg = se[((int64_t)(o >> 5) * G + g) * 32 + (o & 31)];
      const float su = se[((int64_t)((o + h) >> 5) * G + g) * 32 + (o & 31)];
#pragma unroll
      for (int r = 0; r < kRowsI4; ++r) {
        const int* ar = reinterpret_cast<const int*>(As + r * d + g * kGroup);
        const int ig = dot32(qg, ar), iu = dot32(qu, ar);
        ag[r] = fmaf(sg, (float)ig, ag[r]);
        au[r] = fmaf(su, (float)iu, au[r]);
        if (kCapture && r < n) {
          isum[((int64_t)(p0 + r) * N2 + o) * G + g] = ig >> 4;
          isum[((int64_t)(p0 + r) * N2 + o + h) * G + g] = iu >> 4;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsI4; ++r)
      if (r < n) {
        const float s = sx[s_tok[r]];
        const float v = silu(ag[r] * s) * (au[r] * s);
        aout[(int64_t)(p0 + r) * h + o] = v;
        amax[r] = fmaxf(amax[r], fabsf(v));
      }
  }
  if (hq == nullptr) return;  // FP32 rows only
  // per-row max|a| over the block (exact, order-free), then the row scale
  __shared__ float red[4][kRowsI4];
  __shared__ float srow[kRowsI4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < kRowsI4; ++r) {
    const float m = wave_max(amax[r]);
    if (lane == 0) red[wv][r] = m;
  }
  __syncthreads();
  if (threadIdx.x < kRowsI4) {
    const int r = threadIdx.x;
    const float m = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
    const float s = (2.0f * m) / 255.0f;
    srow[r] = s;
    if (r < n) hs[p0 + r] = s;
  }
  __syncthreads();
  for (int o = threadIdx.x; o < h; o += blockDim.x) {
#pragma unroll
    for (int r = 0; r < kRowsI4; ++r)
      if (r < n) {
        const int64_t i = (int64_t)(p0 + r) * h + o;
        hq[i] = srow[r] != 0.0f ? quant_i8(aout[i], srow[r]) : (int8_t)0;
      }
  }
}

// INT4 down: f = s_h * sum_g s_w * isum_g over the hidden row.
template <bool kCapture>
__global__ __launch_bounds__(256) void k_down_i4(ExpertArgs a, const int8_t* __restrict__ hq,
                                                 const float* __restrict__ hs,
                                                 const uint8_t* __restrict__ wq,
                                                 const float* __restrict__ wsc,
                                                 float* __restrict__ f,
                                                 int32_t* __restrict__ isum) {
  extern __shared__ int4 smem4[];
  int8_t* As = reinterpret_cast<int8_t*>(smem4);
  int p0, n, e;
  find_tile<kRowsI4>(a, p0, n, e);
  if (n <= 0) return;
  const int d = a.d, h = a.h, G = h / kGroup;
  const int c16 = h / 16;
  for (int i = threadIdx.x; i < kRowsI4 * c16; i += blockDim.x) {
    const int r = i / c16, c = i % c16;
    int4 v = make_int4(0, 0, 0, 0);
    if (r < n) v = reinterpret_cast<const int4*>(hq + (int64_t)(p0 + r) * h)[c];
    smem4[r * c16 + c] = v;
  }
  __syncthreads();
  const uint8_t* we = wq + (int64_t)e * (d / 32) * G * kChunkBytes;
  const float* se = wsc + (int64_t)e * (d / 32) * G * 32;
  for (int o = threadIdx.x; o < d; o += blockDim.x) {
    float acc[kRowsI4];
#pragma unroll
    for (int r = 0; r < kRowsI4; ++r) acc[r] = 0.0f;
    for (int g = 0; g < G; ++g) {
      uint32_t q[8];
      load_w32(we, G, o, g, q);
      const float s = se[((int64_t)(o >> 5) * G + g) * 32 + (o & 31)];
#pragma unroll
      for (int r = 0; r < kRowsI4; ++r) {
        const int is = dot32(q, reinterpret_cast<const int*>(As + r * h + g * kGroup));
        acc[r] = fmaf(s, (float)is, acc[r]);
        if (kCapture && r < n) isum[((int64_t)(p0 + r) * d + o) * G + g] = is >> 4;
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsI4; ++r)
      if (r < n) f[(int64_t)(p0 + r) * d + o] = acc[r] * hs[p0 + r];
  }
}

template <bool kBF16>
__device__ __forceinline__ float ldw(const void* w, int64_t i) {
  if (kBF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(w)[i]);
  return reinterpret_cast<const float*>(w)[i];
}

// FP32 / BF16 gate/up + SwiGLU.  BF16: x is rounded to BF16 on load and the
// hidden row is written as BF16.
template <bool kBF16>
__global__ __launch_bounds__(256) void k_gateup_fp(ExpertArgs a, const float* __restrict__ x,
                                                   const void* __restrict__ w,
                                                   void* __restrict__ hout) {
  extern __shared__ int4 smem4[];
  float* As = reinterpret_cast<float*>(smem4);
  int p0, n, e;
  find_tile<kRowsFp>(a, p0, n, e);
  if (n <= 0) return;
  const int d = a.d, h = a.h;
  for (int i = threadIdx.x; i < kRowsFp * d; i += blockDim.x) {
    const int r = i / d, c = i % d;
    float v = 0.0f;
    if (r < n) {
      int64_t tok = a.perm ? a.perm[p0 + r] / a.k : p0 + r;
      if (tok < 0 || tok >= a.T) tok = 0;  // stays in bounds for a corrupt perm
      v = x[tok * d + c];
      if (kBF16) v = bf16_to_f32(f32_to_bf16(v));
    }
    As[i] = v;
  }
  __syncthreads();
  const int64_t wbase = (int64_t)e * 2 * h * d;
  for (int o = threadIdx.x; o < h; o += blockDim.x) {
    float ag[kRowsFp], au[kRowsFp];
#pragma unroll
    for (int r = 0; r < kRowsFp; ++r) ag[r] = au[r] = 0.0f;
    for (int c = 0; c < d; ++c) {
      const float wg = ldw<kBF16>(w, wbase + (int64_t)o * d + c);
      const float wu = ldw<kBF16>(w, wbase + (int64_t)(o + h) * d + c);
#pragma unroll
      for (int r = 0; r < kRowsFp; ++r) {
        ag[r] = fmaf(As[r * d + c], wg, ag[r]);
        au[r] = fmaf(As[r * d + c], wu, au[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsFp; ++r)
      if (r < n) {
        const float v = silu(ag[r]) * au[r];
        const int64_t i = (int64_t)(p0 + r) * h + o;
        if (kBF16)
          reinterpret_cast<uint16_t*>(hout)[i] = f32_to_bf16(v);
        else
          reinterpret_cast<float*>(hout)[i] = v;
      }
  }
}

template <bool kBF16>
__global__ __launch_bounds__(256) void k_down_fp(ExpertArgs a, const void* __restrict__ hin,
                                                 const void* __restrict__ w,
                                                 float* __restrict__ f) {
  extern __shared__ int4 smem4[];
  float* As = reinterpret_cast<float*>(smem4);
  int p0, n, e;
  find_tile<kRowsFp>(a, p0, n, e);
  if (n <= 0) return;
  const int d = a.d, h = a.h;
  for (int i = threadIdx.x; i < kRowsFp * h; i += blockDim.x) {
    const int r = i / h, c = i % h;
    As[i] = r < n ? ldw<kBF16>(hin, (int64_t)(p0 + r) * h + c) : 0.0f;
  }
  __syncthreads();
  const int64_t wbase = (int64_t)e * d * h;
  for (int o = threadIdx.x; o < d; o += blockDim.x) {
    float acc[kRowsFp];
#pragma unroll
    for (int r = 0; r < kRowsFp; ++r) acc[r] = 0.0f;
    for (int c = 0; c < h; ++c) {
      const float wv = ldw<kBF16>(w, wbase + (int64_t)o * h + c);
#pragma unroll
      for (int r = 0; r < kRowsFp; ++r) acc[r] = fmaf(As[r * h + c], wv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kRowsFp; ++r)
      if (r < n) f[(int64_t)(p0 + r) * d + o] = acc[r];
  }
}

unsigned tiles_for(const ExpertArgs& a, int rows_per_tile) {
  return (unsigned)tile_bound(a, rows_per_tile);
}

}  // namespace

hipError_t launch_gateup_i4(const ExpertArgs& a, const int8_t* xq, const float* sx,
                            const uint8_t* wq, const float* ws, float* a_buf, int8_t* hq,
                            float* hs, int32_t* isum, hipStream_t st) {
  const size_t lds = (size_t)kRowsI4 * a.d;
  if (isum)
    hipLaunchKernelGGL(k_gateup_i4<true>, dim3(tiles_for(a, kRowsI4)), dim3(256), lds, st, a, xq,
                       sx, wq, ws, a_buf, hq, hs, isum);
  else
    hipLaunchKernelGGL(k_gateup_i4<false>, dim3(tiles_for(a, kRowsI4)), dim3(256), lds, st, a, xq,
                       sx, wq, ws, a_buf, hq, hs, isum);
  return hipGetLastError();
}

hipError_t launch_down_i4(const ExpertArgs& a, const int8_t* hq, const float* hs,
                          const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                          hipStream_t st) {
  const size_t lds = (size_t)kRowsI4 * a.h;
  if (isum)
    hipLaunchKernelGGL(k_down_i4<true>, dim3(tiles_for(a, kRowsI4)), dim3(256), lds, st, a, hq, hs,
                       wq, ws, f, isum);
  else
    hipLaunchKernelGGL(k_down_i4<false>, dim3(tiles_for(a, kRowsI4)), dim3(256), lds, st, a, hq, hs,
                       wq, ws, f, isum);
  return hipGetLastError();
}

hipError_t launch_gateup_fp(const ExpertArgs& a, bool bf16, const void* x, const void* w,
                            void* h_out, hipStream_t st) {
  const size_t lds = (size_t)kRowsFp * a.d * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL(k_gateup_fp<true>, dim3(tiles_for(a, kRowsFp)), dim3(256), lds, st, a,
                       (const float*)x, w, h_out);
  else
    hipLaunchKernelGGL(k_gateup_fp<false>, dim3(tiles_for(a, kRowsFp)), dim3(256), lds, st, a,
                       (const float*)x, w, h_out);
  return hipGetLastError();
}

hipError_t launch_down_fp(const ExpertArgs& a, bool bf16, const void* hrow, const void* w,
                          float* f, hipStream_t st) {
  const size_t lds = (size_t)kRowsFp * a.h * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL(k_down_fp<true>, dim3(tiles_for(a, kRowsFp)), dim3(256), lds, st, a, hrow, w,
                       f);
  else
    hipLaunchKernelGGL(k_down_fp<false>, dim3(tiles_for(a, kRowsFp)), dim3(256), lds, st, a, hrow,
                       w, f);
  return hipGetLastError();
}

}  // namespace mm
