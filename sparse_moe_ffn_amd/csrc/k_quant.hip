// Weight quantisation (eq. (6), b = 4, group 32), prepacking, per-row INT8
// activation quantisation, BF16 conversion and RMSNorm.
//
// eq. (6) and the INT8 activation rule are from the section "Quantisation-
// aware training" of the MobileMoE close reading (paper-archivist.com).
#include <utility>

#include "common.h"
#include "launch.h"

namespace mm {
namespace {

// One thread per (row, group of 32 columns).
__global__ __launch_bounds__(256) void k_quantize_int4g32(int64_t rows, int64_t cols,
                                                          const float* __restrict__ w,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ s) {
  const int64_t G = cols / kGroup;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * G) return;
  const int64_t r = i / G, g = i % G;
  const float* wg = w + r * cols + g * kGroup;
  float v[kGroup];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kGroup; ++c) {
    v[c] = wg[c];
    amax = fmaxf(amax, fabsf(v[c]));
  }
  const float sg = (2.0f * amax) / 15.0f;
  s[i] = sg;
  uint8_t* qg = q + r * (cols / 2) + g * (kGroup / 2);
#pragma unroll
  for (int b = 0; b < kGroup / 2; ++b) {
    int lo = 0, hi = 0;
    if (sg != 0.0f) {
      lo = (int)fminf(fmaxf(rintf(v[2 * b] / sg), -8.0f), 7.0f);
      hi = (int)fminf(fmaxf(rintf(v[2 * b + 1] / sg), -8.0f), 7.0f);
    }
    qg[b] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
  }
}

// One thread per (matrix, 32-row block, group, lane of the chunk): writes the
// 8 bytes of that lane (layout in common.h) and, for lanes 0..31, the scale.
__global__ __launch_bounds__(256) void k_prepack_int4g32(int64_t n_mat, int64_t rows,
                                                         int64_t cols,
                                                         const uint8_t* __restrict__ qc,
                                                         const float* __restrict__ sc,
                                                         uint8_t* __restrict__ qo,
                                                         float* __restrict__ so) {
  const int64_t G = cols / kGroup, RB = rows / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_mat * RB * G * 64) return;
  const int L = (int)(i % 64);
  const int64_t chunk = i / 64;  // ((m * RB + rb) * G + g)
  const int64_t g = chunk % G;
  const int64_t mrb = chunk / G;  // m * RB + rb
  const int64_t row = mrb * 32 + (L % 32);  // global row over all matrices
  const uint8_t* src = qc + row * (cols / 2);
  const int64_t base = g * kGroup + 16 * (L / 32);
  auto nib = [&](int64_t c) -> uint32_t { return (src[c / 2] >> (4 * (c & 1))) & 0xFu; };
  uint32_t word[2];
#pragma unroll
  for (int wi = 0; wi < 2; ++wi) {
    uint32_t acc = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t lo = nib(base + 8 * wi + b), hi = nib(base + 8 * wi + b + 4);
      acc |= (lo | (hi << 4)) << (8 * b);
    }
    word[wi] = acc;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(qo + chunk * kChunkBytes + L * 8);
  dst[0] = word[0];
  dst[1] = word[1];
  if (L < 32) so[chunk * 32 + L] = sc[row * G + g] * 0.0625f;
}

// One wave per row: exact max|v|, s = 2*amax/255, q = clamp(rint(v/s)).
__global__ __launch_bounds__(256) void k_act_quant_i8(int64_t rows, int64_t cols,
                                                      const float* __restrict__ x,
                                                      int8_t* __restrict__ q,
                                                      float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + r * cols;
  float amax = 0.0f;
  for (int64_t c = lane; c < cols; c += kWave) amax = fmaxf(amax, fabsf(xr[c]));
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f;
  if (lane == 0) s[r] = sr;
  int8_t* qr = q + r * cols;
  for (int64_t c = lane; c < cols; c += kWave) qr[c] = sr != 0.0f ? quant_i8(xr[c], sr) : (int8_t)0;
}

// Same quantiser, rows with cols % 128 == 0: the row is read once as float2
// per lane, kept in registers, and written as 2 codes per lane.  One wave per
// row r (r < rows).  gm_rows: 0 row-major codes, else group-major with that
// many rows.
template <int kMaxV>
__device__ __forceinline__ void quant_row_v2(int64_t r, int64_t cols, const float* __restrict__ x,
                                             int8_t* __restrict__ q, float* __restrict__ s,
                                             int64_t gm_rows) {
  const int lane = threadIdx.x & 63;
  const int nv = (int)(cols / 128);
  const float2* xr = reinterpret_cast<const float2*>(x + r * cols);
  float2 v[kMaxV];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxV; ++i)
    if (i < nv) {
      v[i] = xr[lane + 64 * i];
      amax = fmaxf(amax, fmaxf(fabsf(v[i].x), fabsf(v[i].y)));
    }
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  if (lane == 0) s[r] = sr;
#pragma unroll
  for (int i = 0; i < kMaxV; ++i)
    if (i < nv) {
      int8_t a = 0, b = 0;
      if (sr != 0.0f) {
        a = quant_i8(v[i].x, sr, yr);
        b = quant_i8(v[i].y, sr, yr);
      }
      *reinterpret_cast<uint16_t*>(q + act_offset(r, 2 * (lane + 64 * i), cols, gm_rows)) =
          (uint16_t)((uint8_t)a | ((uint16_t)(uint8_t)b << 8));
    }
}

// Same quantiser with 16-byte loads: lane l holds the float4 columns
// 4 j .. 4 j + 3, j = l + 64 i (cols % 4 == 0, cols <= 256 * kMaxF4); its four
// codes are one 4-byte store in either layout (they share a quantisation
// group).  Every load of the row is issued before the first use.
template <int kMaxF4>
__device__ __forceinline__ void quant_row_v4(int64_t r, int64_t cols, const float* __restrict__ x,
                                             int8_t* __restrict__ q, float* __restrict__ s,
                                             int64_t gm_rows) {
  const int lane = threadIdx.x & 63;
  const int n4 = (int)(cols / 4);
  const float4* xr = reinterpret_cast<const float4*>(x + r * cols);
  float4 v[kMaxF4];
#pragma unroll
  for (int i = 0; i < kMaxF4; ++i)
    if (lane + 64 * i < n4) v[i] = xr[lane + 64 * i];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxF4; ++i)
    if (lane + 64 * i < n4)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  if (lane == 0) s[r] = sr;
#pragma unroll
  for (int i = 0; i < kMaxF4; ++i) {
    const int j = lane + 64 * i;
    if (j >= n4) continue;
    uint32_t word = 0;
    if (sr != 0.0f) {
      word = (uint32_t)(uint8_t)quant_i8(v[i].x, sr, yr) |
             (uint32_t)(uint8_t)quant_i8(v[i].y, sr, yr) << 8 |
             (uint32_t)(uint8_t)quant_i8(v[i].z, sr, yr) << 16 |
             (uint32_t)(uint8_t)quant_i8(v[i].w, sr, yr) << 24;
    }
    *reinterpret_cast<uint32_t*>(q + act_offset(r, 4 * j, cols, gm_rows)) = word;
  }
}

// The same quantiser for two short rows per wave (cols % 4 == 0, cols <=
// 128 * kMaxH): lanes 0..31 take row r0, lanes 32..63 row r0 + 1 (if it is
// below `rows`), half-lane l the float4 columns l + 32 i.  Halves the waves
// of a launch of short rows, so all of them are resident at once.
template <int kMaxH>
__device__ __forceinline__ void quant_rows2_v4(int64_t r0, int64_t rows, int64_t cols,
                                               const float* __restrict__ x, int8_t* __restrict__ q,
                                               float* __restrict__ s, int64_t gm_rows) {
  const int lane = threadIdx.x & 63, hl = lane & 31;
  const int64_t r = r0 + (lane >> 5);
  const bool live = r < rows;
  const int n4 = (int)(cols / 4);
  const float4* xr = reinterpret_cast<const float4*>(x + (live ? r : r0) * cols);
  float4 v[kMaxH];
#pragma unroll
  for (int i = 0; i < kMaxH; ++i)
    if (live && hl + 32 * i < n4) v[i] = xr[hl + 32 * i];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxH; ++i)
    if (live && hl + 32 * i < n4)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  // maximum over each 32-lane half: within the 16-lane rows, then the half's two rows
  m = fmaxf(m, dpp<kDppXor1>(m));
  m = fmaxf(m, dpp<kDppXor2>(m));
  m = fmaxf(m, dpp<kDppHalfMirror>(m));
  m = fmaxf(m, dpp<kDppMirror>(m));
  const float m0 = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16)));
  const float m1 = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48)));
  const float amax = lane < 32 ? m0 : m1;
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  if (!live) return;
  if (hl == 0) s[r] = sr;
#pragma unroll
  for (int i = 0; i < kMaxH; ++i) {
    const int j = hl + 32 * i;
    if (j >= n4) continue;
    uint32_t word = 0;
    if (sr != 0.0f) {
      word = (uint32_t)(uint8_t)quant_i8(v[i].x, sr, yr) |
             (uint32_t)(uint8_t)quant_i8(v[i].y, sr, yr) << 8 |
             (uint32_t)(uint8_t)quant_i8(v[i].z, sr, yr) << 16 |
             (uint32_t)(uint8_t)quant_i8(v[i].w, sr, yr) << 24;
    }
    *reinterpret_cast<uint32_t*>(q + act_offset(r, 4 * j, cols, gm_rows)) = word;
  }
}

// Same quantiser writing f16 paired codes (common.h): lane l holds columns
// 4 j .. 4 j + 3, j = l + 64 i, read as float4; those are columns 0..3 (j
// even) or 4..7 (j odd) of an 8-column block, which land in slots 0, 4, 1, 5
// (as the codes) or 2, 6, 3, 7 (the codes divided by 16): two 4-byte stores.
// cols % 128 == 0.
template <int kMaxV4>
__device__ __forceinline__ void quant_row_f16p(int64_t r, int64_t cols,
                                               const float* __restrict__ x,
                                               uint16_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int n4 = (int)(cols / 4);
  const float4* xr = reinterpret_cast<const float4*>(x + r * cols);
  float4 v[kMaxV4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxV4; ++i) {
    const int j = lane + 64 * i;
    if (j < n4) {
      v[i] = xr[j];
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
  }
  amax = max64(amax);
  const float sr = (2.0f * amax) / 255.0f, yr = quant_recip(sr);
  if (lane == 0) s[r] = sr;
#pragma unroll
  for (int i = 0; i < kMaxV4; ++i) {
    const int j = lane + 64 * i;
    if (j < n4) {
      int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
      if (sr != 0.0f) {
        c0 = quant_i8(v[i].x, sr, yr);
        c1 = quant_i8(v[i].y, sr, yr);
        c2 = quant_i8(v[i].z, sr, yr);
        c3 = quant_i8(v[i].w, sr, yr);
      }
      const int hi = j & 1;  // columns 4..7 of the block
      const float m = hi ? 0.0625f : 1.0f;
      auto h = [&](int c) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)((float)c * m)); };
      uint32_t* row = reinterpret_cast<uint32_t*>(q + r * cols + 8 * (j >> 1));
      row[hi] = h(c0) | (h(c2) << 16);
      row[2 + hi] = h(c1) | (h(c3) << 16);
    }
  }
}

template <int kMaxV>
__global__ __launch_bounds__(256) void k_act_quant_i8_v2(int64_t rows, int64_t cols,
                                                         const float* __restrict__ x,
                                                         int8_t* __restrict__ q,
                                                         float* __restrict__ s, int64_t gm_rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r < rows) quant_row_v2<kMaxV>(r, cols, x, q, s, gm_rows);
}

template <int kMaxV4>
__global__ __launch_bounds__(256) void k_act_quant_f16p(int64_t rows, int64_t cols,
                                                        const float* __restrict__ x,
                                                        uint16_t* __restrict__ q,
                                                        float* __restrict__ s) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r < rows) quant_row_f16p<kMaxV4>(r, cols, x, q, s);
}

// Two row sets in one launch: blocks [0, nb0) cover set 0, the rest set 1
// (the launcher puts the set with the longer rows first, so that its waves,
// the longest, start first and the short ones fill in behind them).
constexpr int kMaxH2 = 5;  // two rows per wave up to 640 columns

struct QuantRows {
  int64_t rows, cols;
  const float* x;
  int8_t* q;
  float* s;
  int64_t gm_rows;
};

// kRows2: set B (the shorter rows) two rows per wave.
template <int kMaxV, bool kRows2>
__global__ __launch_bounds__(256) void k_act_quant_i8_pair(QuantRows A, QuantRows B, int nb0) {
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nb0) {
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r < A.rows) quant_row_v4<kMaxV / 2>(r, A.cols, A.x, A.q, A.s, A.gm_rows);
  } else if constexpr (kRows2) {
    const int64_t r = ((int64_t)(blockIdx.x - nb0) * 4 + wave) * 2;
    if (r < B.rows) quant_rows2_v4<kMaxH2>(r, B.rows, B.cols, B.x, B.q, B.s, B.gm_rows);
  } else {
    const int64_t r = (int64_t)(blockIdx.x - nb0) * 4 + wave;
    if (r < B.rows) quant_row_v4<kMaxV / 2>(r, B.cols, B.x, B.q, B.s, B.gm_rows);
  }
}

template <int kMaxV4>
__global__ __launch_bounds__(256) void k_act_quant_f16p_pair(QuantRows A, QuantRows B, int nb0) {
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nb0) {
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r < A.rows) quant_row_f16p<kMaxV4>(r, A.cols, A.x, reinterpret_cast<uint16_t*>(A.q), A.s);
  } else {
    const int64_t r = (int64_t)(blockIdx.x - nb0) * 4 + wave;
    if (r < B.rows) quant_row_f16p<kMaxV4>(r, B.cols, B.x, reinterpret_cast<uint16_t*>(B.q), B.s);
  }
}

__global__ __launch_bounds__(256) void k_convert_bf16(int64_t n, const float* __restrict__ x,
                                                      uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = f32_to_bf16(x[i]);
}

__global__ __launch_bounds__(256) void k_rmsnorm(int64_t rows, int64_t cols, float eps,
                                                 const float* __restrict__ x,
                                                 float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + r * cols;
  float ss = 0.0f;
  for (int64_t c = lane; c < cols; c += kWave) ss = fmaf(xr[c], xr[c], ss);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)cols + eps);
  for (int64_t c = lane; c < cols; c += kWave) y[r * cols + c] = xr[c] * inv;
}

// Residual add and (optionally) the RMSNorm of the sum, one wave per row:
// sum = x + r (FP32), norm = sum / sqrt(mean(sum^2) + eps) with the sum of
// squares accumulated as k_rmsnorm does.  The join of a decoder block's
// sub-layers (the residual stream and the next sub-layer's normalised input).
__global__ __launch_bounds__(256) void k_add_rmsnorm(int64_t rows, int64_t cols, float eps,
                                                     const float* __restrict__ x,
                                                     const float* __restrict__ r,
                                                     float* __restrict__ sum,
                                                     float* __restrict__ norm) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * cols;
  const float* rr = r + row * cols;
  float* sr = sum + row * cols;
  float ss = 0.0f;
  for (int64_t c = lane; c < cols; c += kWave) {
    const float v = xr[c] + rr[c];
    sr[c] = v;
    ss = fmaf(v, v, ss);
  }
  if (norm == nullptr) return;
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)cols + eps);
  for (int64_t c = lane; c < cols; c += kWave) norm[row * cols + c] = (xr[c] + rr[c]) * inv;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_quantize_int4g32(int64_t rows, int64_t cols, const float* w, uint8_t* q,
                                   float* s, hipStream_t st) {
  const int64_t n = rows * (cols / kGroup);
  hipLaunchKernelGGL(k_quantize_int4g32, dim3(blocks_for(n, 256)), dim3(256), 0, st, rows, cols,
                     w, q, s);
  return hipGetLastError();
}

hipError_t launch_prepack_int4g32(int64_t n_mat, int64_t rows, int64_t cols, const uint8_t* qc,
                                  const float* sc, uint8_t* qo, float* so, hipStream_t st) {
  const int64_t n = n_mat * (rows / 32) * (cols / kGroup) * 64;
  hipLaunchKernelGGL(k_prepack_int4g32, dim3(blocks_for(n, 256)), dim3(256), 0, st, n_mat, rows,
                     cols, qc, sc, qo, so);
  return hipGetLastError();
}

hipError_t launch_act_quant_i8(int64_t rows, int64_t cols, const float* x, int8_t* q, float* s,
                               hipStream_t st, int layout) {
  if (layout == kActF16Paired) {
    if (cols % 128 != 0 || cols > 256 * 12) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_act_quant_f16p<12>, dim3(blocks_for(rows, 4)), dim3(256), 0, st, rows,
                       cols, x, reinterpret_cast<uint16_t*>(q), s);
    return hipGetLastError();
  }
  if (cols % 128 == 0 && cols <= 128 * 24)
    hipLaunchKernelGGL(k_act_quant_i8_v2<24>, dim3(blocks_for(rows, 4)), dim3(256), 0, st, rows,
                       cols, x, q, s, act_gm_rows(layout, rows));
  else if (layout != kActRowMajor)
    return hipErrorInvalidValue;  // other layouts only for cols % 128 == 0
  else
    hipLaunchKernelGGL(k_act_quant_i8, dim3(blocks_for(rows, 4)), dim3(256), 0, st, rows, cols, x,
                       q, s);
  return hipGetLastError();
}

hipError_t launch_act_quant_i8_pair(int64_t rows0, int64_t cols0, const float* x0, int8_t* q0,
                                    float* s0, int64_t rows1, int64_t cols1, const float* x1,
                                    int8_t* q1, float* s1, hipStream_t st, int layout) {
  auto fits = [](int64_t c) { return c % 128 == 0 && c <= 128 * 24; };
  if (!fits(cols0) || !fits(cols1)) {
    hipError_t e = launch_act_quant_i8(rows0, cols0, x0, q0, s0, st, layout);
    if (e != hipSuccess) return e;
    return launch_act_quant_i8(rows1, cols1, x1, q1, s1, st, layout);
  }
  QuantRows A{rows0, cols0, x0, q0, s0, act_gm_rows(layout, rows0)};
  QuantRows B{rows1, cols1, x1, q1, s1, act_gm_rows(layout, rows1)};
  if (B.cols > A.cols) std::swap(A, B);
  const int nbA = (int)blocks_for(A.rows, 4);
  const bool rows2 = layout != kActF16Paired && B.cols <= 128 * kMaxH2;
  const int nbB = (int)blocks_for(rows2 ? (B.rows + 1) / 2 : B.rows, 4);
  if (layout == kActF16Paired)
    hipLaunchKernelGGL(k_act_quant_f16p_pair<12>, dim3(nbA + nbB), dim3(256), 0, st, A, B, nbA);
  else if (rows2)
    hipLaunchKernelGGL((k_act_quant_i8_pair<24, true>), dim3(nbA + nbB), dim3(256), 0, st, A, B, nbA);
  else
    hipLaunchKernelGGL((k_act_quant_i8_pair<24, false>), dim3(nbA + nbB), dim3(256), 0, st, A, B, nbA);
  return hipGetLastError();
}

hipError_t launch_convert_bf16(int64_t n, const float* x, uint16_t* y, hipStream_t st) {
  hipLaunchKernelGGL(k_convert_bf16, dim3(blocks_for(n, 256)), dim3(256), 0, st, n, x, y);
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(int64_t rows, int64_t cols, float eps, const float* x,
                              const float* r, float* sum, float* norm, hipStream_t st) {
  hipLaunchKernelGGL(k_add_rmsnorm, dim3(blocks_for(rows, 4)), dim3(256), 0, st, rows, cols, eps,
                     x, r, sum, norm);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int64_t rows, int64_t cols, float eps, const float* x, float* y,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(blocks_for(rows, 4)), dim3(256), 0, st, rows, cols, eps, x,
                     y);
  return hipGetLastError();
}

}  // namespace mm
