// Training passes of the routed experts (MobileMoE close reading, section
// "Pre-training": the experts' FFNs batched into grouped matrix products;
// section "Quantisation-aware training": weights and activations fake-
// quantised by eq. (6), gradients passed straight through the rounding).
//
// Grouped FP32 products on the FP32 matrix cores (v_mfma_f32_16x16x4_f32:
// FP32 products, FP32 sums; this form issues at close to the chip's FP32
// matrix rate, the 32 x 32 x 2 form at about 85 % of it): C[m][n] = sum over k of A(m, k) B(k, n) with
//   A(m, k) = A[m * lda + k]  (kAK)   or  A[k * lda + m]
//   B(k, n) = B[n * ldb + k]  (kBK)   or  B[k * ldb + n].
// Grouped by rows (!kGroupK): group e owns rows [off[e], off[e+1]) of A and
// C and multiplies them by its own B (B + e * strideB); K is fixed.
// Grouped by the reduction (kGroupK): group e sums k over [off[e], off[e+1])
// into its own C (C + e * strideC); M and N are fixed.
// K slices of 16 are staged through LDS, the next slice's loads issued
// before the current slice's matrix instructions.
#include "common.h"
#include "launch_train.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 16;

// Workgroup tile (32 kWM kTM) x (32 (4 / kWM) kTN): four waves in a kWM x
// (4 / kWM) grid, each holding 2 kTM x 2 kTN blocks of 16 x 16 accumulators
// (independent chains).  Two LDS buffers of K slices (k-major rows of the
// tile width + 16 floats, so the four k rows one fragment read touches fall
// in disjoint bank halves): slice i + 1 is stored while slice i is
// multiplied, one barrier per slice.
template <bool kAK, bool kBK_, bool kGroupK, int kWM, int kTM, int kTN>
__global__ __launch_bounds__(256) void k_gemm_f32(int E, int64_t M, int64_t N, int64_t K,
                                                  const int32_t* __restrict__ off,
                                                  const float* __restrict__ A, int64_t lda,
                                                  const float* __restrict__ B, int64_t ldb,
                                                  int64_t strideB, float* __restrict__ C,
                                                  int64_t ldc, int64_t strideC) {
  constexpr int kWN = 4 / kWM;
  constexpr int kBM = 32 * kWM * kTM, kBN = 32 * kWN * kTN, kLdA = kBM + 16, kLdB = kBN + 16;
  constexpr int kNA = (kBM * 4 + 255) / 256, kNB = (kBN * 4 + 255) / 256;  // float4 per thread
  __shared__ float sA[2][kBK][kLdA];
  __shared__ float sB[2][kBK][kLdB];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave % kWM, wn = wave / kWM;
  int e;
  int64_t m0, mEnd, n0, k0, kEnd;
  if constexpr (kGroupK) {
    const int64_t ntn = (N + kBN - 1) / kBN;
    e = blockIdx.y;
    m0 = (int64_t)(blockIdx.x / ntn) * kBM;
    n0 = (int64_t)(blockIdx.x % ntn) * kBN;
    mEnd = M;
    k0 = off ? off[e] : 0;  // no offsets: one group over [0, K)
    kEnd = off ? off[e + 1] : K;
    C += (int64_t)e * strideC;
  } else {
    // find this workgroup's group and row tile: groups hold ceil(rows / kBM) tiles each
    int64_t bx = blockIdx.x;
    e = -1;
    for (int g = 0; g < E; ++g) {
      const int64_t tiles = (off[g + 1] - off[g] + kBM - 1) / kBM;
      if (bx < tiles) {
        e = g;
        break;
      }
      bx -= tiles;
    }
    if (e < 0) return;  // past the last tile (the grid is an upper bound)
    m0 = off[e] + bx * kBM;
    mEnd = off[e + 1];
    n0 = (int64_t)blockIdx.y * kBN;
    k0 = 0;
    kEnd = K;
    B += (int64_t)e * strideB;
  }

  // this thread's share of a K slice: kNA float4 of A and kNB of B.  The
  // loads are unconditional from addresses clamped into the operands (out-of-
  // range elements are zeroed on the way into LDS): a predicated load would
  // split the code into branches, and the compiler then waits for each load
  // before issuing the next.
  float4 ra[kNA], rb[kNB];
  bool va[kNA], vb[kNB];
  auto load = [&](int64_t k) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int u = t + 256 * i;
      if ((kBM * 4) % 256 != 0 && u >= kBM * 4) break;
      if constexpr (kAK) {
        const int64_t m = m0 + (u >> 2), kk = k + (u & 3) * 4;
        va[i] = m < mEnd;
        ra[i] = *reinterpret_cast<const float4*>(A + min(m, mEnd - 1) * lda + kk);
      } else {
        const int64_t kk = k + u / (kBM / 4), m = m0 + (u % (kBM / 4)) * 4;
        va[i] = kk < kEnd && m < mEnd;
        ra[i] = *reinterpret_cast<const float4*>(A + min(kk, kEnd - 1) * lda + min(m, mEnd - 4));
      }
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int u = t + 256 * i;
      if ((kBN * 4) % 256 != 0 && u >= kBN * 4) break;
      if constexpr (kBK_) {
        const int64_t n = n0 + (u >> 2), kk = k + (u & 3) * 4;
        vb[i] = n < N;
        rb[i] = *reinterpret_cast<const float4*>(B + min(n, N - 1) * ldb + kk);
      } else {
        const int64_t kk = k + u / (kBN / 4), n = n0 + (u % (kBN / 4)) * 4;
        vb[i] = kk < kEnd && n < N;
        rb[i] = *reinterpret_cast<const float4*>(B + min(kk, kEnd - 1) * ldb + min(n, N - 4));
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
      const int u = t + 256 * i;
      if ((kBM * 4) % 256 != 0 && u >= kBM * 4) break;
      if (!va[i]) ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kAK) {
        const int mi = u >> 2, k4 = (u & 3) * 4;
        sA[buf][k4][mi] = ra[i].x;
        sA[buf][k4 + 1][mi] = ra[i].y;
        sA[buf][k4 + 2][mi] = ra[i].z;
        sA[buf][k4 + 3][mi] = ra[i].w;
      } else {
        *reinterpret_cast<float4*>(&sA[buf][u / (kBM / 4)][(u % (kBM / 4)) * 4]) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int u = t + 256 * i;
      if ((kBN * 4) % 256 != 0 && u >= kBN * 4) break;
      if (!vb[i]) rb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kBK_) {
        const int ni = u >> 2, k4 = (u & 3) * 4;
        sB[buf][k4][ni] = rb[i].x;
        sB[buf][k4 + 1][ni] = rb[i].y;
        sB[buf][k4 + 2][ni] = rb[i].z;
        sB[buf][k4 + 3][ni] = rb[i].w;
      } else {
        *reinterpret_cast<float4*>(&sB[buf][u / (kBN / 4)][(u % (kBN / 4)) * 4]) = rb[i];
      }
    }
  };

  f32x4 acc[2 * kTM][2 * kTN];
#pragma unroll
  for (int i = 0; i < 2 * kTM; ++i)
#pragma unroll
    for (int j = 0; j < 2 * kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  const int quad = lane >> 4, li = lane & 15;
  if (k0 < kEnd) {
    load(k0);
    store(0);
  }
  __syncthreads();
  int cur = 0;
  for (int64_t k = k0; k < kEnd; k += kBK) {
    const bool more = k + kBK < kEnd;
    if (more) load(k + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 4) {
      // fragments: A[i][k] and B[k][j] with i, j = lane % 16, k = kk + lane / 16
      float a[2 * kTM], b[2 * kTN];
#pragma unroll
      for (int i = 0; i < 2 * kTM; ++i) a[i] = sA[cur][kk + quad][wm * 32 * kTM + 16 * i + li];
#pragma unroll
      for (int j = 0; j < 2 * kTN; ++j) b[j] = sB[cur][kk + quad][wn * 32 * kTN + 16 * j + li];
#pragma unroll
      for (int i = 0; i < 2 * kTM; ++i)
#pragma unroll
        for (int j = 0; j < 2 * kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(cur ^ 1);  // its last readers finished before the previous barrier
    __syncthreads();
    cur ^= 1;
  }
  // acc[i][j][r] holds row 4 (lane / 16) + r, column lane % 16 of block (i, j)
#pragma unroll
  for (int i = 0; i < 2 * kTM; ++i)
#pragma unroll
    for (int j = 0; j < 2 * kTN; ++j) {
      const int64_t col = n0 + wn * 32 * kTN + 16 * j + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 32 * kTM + 16 * i + 4 * quad + r;
        if (row < mEnd && col < N) C[row * ldc + col] = acc[i][j][r];
      }
    }
}

// Forward activation of one expert row (one wave per row): a = silu(g) * u
// (FP32), then abar = eq. (6) fake quantisation of a with b = 8, one group
// per row.  a is written to abar first and read back by the same lane.
__global__ __launch_bounds__(256) void k_train_act(int64_t R, int h, const float* __restrict__ gu,
                                                   float* __restrict__ abar) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float* g = gu + r * 2 * h;
  float* o = abar + r * h;
  float amax = 0.0f;
  for (int j = lane; j < h; j += 64) {
    const float a = silu(g[j]) * g[h + j];
    o[j] = a;
    amax = fmaxf(amax, fabsf(a));
  }
  amax = max64(amax);
  const float s = (2.0f * amax) / 255.0f;
  for (int j = lane; j < h; j += 64) {
    const float a = o[j];
    o[j] = s == 0.0f ? 0.0f : s * fminf(fmaxf(rintf(a / s), -128.0f), 127.0f);
  }
}

// Backward of the activation (one wave per row): the quantiser's pass flag
// from a recomputed bit for bit, then
//   da = dabar * pass, dg = da u sig(g) (1 + g (1 - sig(g))), du = da g sig(g).
__global__ __launch_bounds__(256) void k_train_act_bwd(int64_t R, int h, const float* __restrict__ gu,
                                                       const float* __restrict__ dabar,
                                                       float* __restrict__ dgu) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float* g = gu + r * 2 * h;
  float amax = 0.0f;
  for (int j = lane; j < h; j += 64) amax = fmaxf(amax, fabsf(silu(g[j]) * g[h + j]));
  amax = max64(amax);
  const float s = (2.0f * amax) / 255.0f;
  for (int j = lane; j < h; j += 64) {
    const float gj = g[j], uj = g[h + j];
    const float a = silu(gj) * uj;
    bool pass = true;
    if (s != 0.0f) {
      const float q = rintf(a / s);
      pass = q >= -128.0f && q <= 127.0f;
    }
    const float da = pass ? dabar[r * h + j] : 0.0f;
    const float sig = 1.0f / (1.0f + expf(-gj));
    dgu[r * 2 * h + j] = da * uj * sig * (1.0f + gj * (1.0f - sig));
    dgu[r * 2 * h + h + j] = da * gj * sig;
  }
}

// dst[r] = scale[perm[r]] * src[perm[r] / k] (scale NULL: 1), zero rows for
// negative entries; one wave per row.
__global__ __launch_bounds__(256) void k_gather_rows(int64_t R, int64_t q4, int k,
                                                     const int32_t* __restrict__ perm,
                                                     const float* __restrict__ scale,
                                                     const float4* __restrict__ src,
                                                     float4* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int32_t a = perm[r];
  const float w = a < 0 ? 0.0f : (scale ? scale[a] : 1.0f);
  const int64_t t = a < 0 ? 0 : a / k;
  for (int64_t c = lane; c < q4; c += 64) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a >= 0) {
      v = src[t * q4 + c];
      v.x *= w;
      v.y *= w;
      v.z *= w;
      v.w *= w;
    }
    dst[r * q4 + c] = v;
  }
}

// 64 x 64 tiles for every form (measured on the S expert shapes: as fast
// as or faster than 32 x 128, 64 x 128 and 128 x 128).
// Router backward, one wave per token: lane e < E holds the logit z_e the
// gate reads (FP32, x_t . Wr_e (+ bias)), the wave the gate-weight
// gradients g_j = dy_t . f_inv(t,j); then dz_e of the softmax (or
// sigmoid-renormalised) gate plus the z-loss term, written to dz [T][E], and
// dx_t += sum_e dz_e Wr_e with lanes over the columns.
__global__ __launch_bounds__(256) void k_router_bwd(int64_t T, int d, int E, int k, int gating,
                                                    const float* __restrict__ x,
                                                    const float* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    const int32_t* __restrict__ idx,
                                                    const float* __restrict__ f,
                                                    const int32_t* __restrict__ inv,
                                                    const float* __restrict__ dy, float zscale,
                                                    float* __restrict__ dz, float* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int q = d / 4;
  const float4* x4 = reinterpret_cast<const float4*>(x + t * d);
  const bool live = lane < E;
  float z = 0.0f;
  if (live) {
    const float4* w4 = reinterpret_cast<const float4*>(wr + (int64_t)lane * d);
    for (int c = 0; c < q; ++c) {
      const float4 a = x4[c], b = w4[c];
      z = fmaf(a.x, b.x, z);
      z = fmaf(a.y, b.y, z);
      z = fmaf(a.z, b.z, z);
      z = fmaf(a.w, b.w, z);
    }
    if (bias && !(gating & 2)) z += bias[lane];
  }
  // gradient of each gate weight: G_e = g_j where e = idx(j)
  float G = 0.0f;
  bool sel = false;
  const float4* dy4 = reinterpret_cast<const float4*>(dy + t * d);
  for (int j = 0; j < k; ++j) {
    const int32_t r = inv[t * k + j];
    float part = 0.0f;
    if (r >= 0) {
      const float4* f4 = reinterpret_cast<const float4*>(f + (int64_t)r * d);
      for (int c = lane; c < q; c += 64) {
        const float4 a = dy4[c], b = f4[c];
        part = fmaf(a.x, b.x, part);
        part = fmaf(a.y, b.y, part);
        part = fmaf(a.z, b.z, part);
        part = fmaf(a.w, b.w, part);
      }
    }
    const float gj = wave_sum(part);
    if (lane == idx[t * k + j]) {
      G = gj;
      sel = true;
    }
  }
  const float m = max64(live ? z : -INFINITY);
  const float ex = live ? expf(z - m) : 0.0f;
  const float S = wave_sum(ex);
  const float p = ex / S;
  float dze = live ? zscale * (m + logf(S)) * p : 0.0f;
  if (!(gating & 1)) {
    const float pg = wave_sum(sel ? p * G : 0.0f);
    dze += live ? p * (G - pg) : 0.0f;
  } else {
    const float sg = sel ? 1.0f / (1.0f + expf(-z)) : 0.0f;
    const float Ss = wave_sum(sg);
    const float wg = wave_sum(sel ? sg / Ss * G : 0.0f);
    if (sel) dze += sg * (1.0f - sg) / Ss * (G - wg);
  }
  if (live) dz[t * E + lane] = dze;
  for (int c = lane; c < q; c += 64) {
    float4 acc = reinterpret_cast<float4*>(dx + t * d)[c];
    for (int e = 0; e < E; ++e) {
      const float de = __shfl(dze, e);
      const float4 w = reinterpret_cast<const float4*>(wr + (int64_t)e * d)[c];
      acc.x = fmaf(de, w.x, acc.x);
      acc.y = fmaf(de, w.y, acc.y);
      acc.z = fmaf(de, w.z, acc.z);
      acc.w = fmaf(de, w.w, acc.w);
    }
    reinterpret_cast<float4*>(dx + t * d)[c] = acc;
  }
}

template <bool kAK, bool kBK_, bool kGroupK>
hipError_t gemm(int E, int64_t R, int64_t M, int64_t N, int64_t K, const int32_t* off, const float* A,
                int64_t lda, const float* B, int64_t ldb, int64_t strideB, float* C, int64_t ldc,
                int64_t strideC, hipStream_t st) {
  constexpr int kWM = 2, kTM = 1, kTN = 1;
  constexpr int kBM = 32 * kWM * kTM, kBN = 32 * (4 / kWM) * kTN;
  dim3 grid;
  if (kGroupK)
    grid = dim3((unsigned)(((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN)), (unsigned)E);
  else
    grid = dim3((unsigned)((R + kBM - 1) / kBM + E), (unsigned)((N + kBN - 1) / kBN));
  hipLaunchKernelGGL((k_gemm_f32<kAK, kBK_, kGroupK, kWM, kTM, kTN>), grid, dim3(256), 0, st, E, M, N, K,
                     off, A, lda, B, ldb, strideB, C, ldc, strideC);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_backward(int64_t T, int d, int E, int k, int gating, const float* x,
                                  const float* wr, const float* bias, const int32_t* idx,
                                  const float* f, const int32_t* inv, const float* dy, float lambda_z,
                                  float* dz, float* dwr, float* dx, hipStream_t st) {
  hipLaunchKernelGGL(k_router_bwd, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, T, d, E, k, gating,
                     x, wr, bias, idx, f, inv, dy, (float)(2.0 * lambda_z / (double)T), dz, dx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dWr = dz^T x: one group over the T tokens
  return gemm<false, false, true>(1, T, E, d, T, nullptr, dz, E, x, d, 0, dwr, d, 0, st);
}

hipError_t launch_gather_rows(int64_t R, int64_t d, int k, const int32_t* perm, const float* scale,
                              const float* src, float* dst, hipStream_t st) {
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, R, d / 4, k, perm,
                     scale, reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst));
  return hipGetLastError();
}

hipError_t launch_expert_train_forward(int E, int d, int h, int64_t R, const int32_t* off,
                                       const float* xs, const float* wgu, const float* wd, float* gu,
                                       float* abar, float* f, hipStream_t st) {
  hipError_t e = gemm<true, true, false>(E, R, R, 2 * h, d, off, xs, d, wgu, d, (int64_t)2 * h * d, gu,
                                         2 * h, 0, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_train_act, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, R, h, gu, abar);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return gemm<true, true, false>(E, R, R, d, h, off, abar, h, wd, h, (int64_t)d * h, f, d, 0, st);
}

hipError_t launch_expert_backward(int E, int d, int h, int64_t R, const int32_t* off, const float* xs,
                                  const float* wgu, const float* wd, const float* gu,
                                  const float* abar, const float* df, float* dxs, float* dwgu,
                                  float* dwd, float* dabar, float* dgu, hipStream_t st) {
  hipError_t e;
  if (R > 0) {  // no kept rows: no row products, but the weight gradients below are still zeroed
    // dabar = df wd_e  [R][h]
    e = gemm<true, false, false>(E, R, R, h, d, off, df, d, wd, h, (int64_t)d * h, dabar, h, 0, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_train_act_bwd, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, R, h, gu,
                       dabar, dgu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dxs = dgu wgu_e  [R][d]
    if ((e = gemm<true, false, false>(E, R, R, d, 2 * h, off, dgu, 2 * h, wgu, d, (int64_t)2 * h * d,
                                      dxs, d, 0, st)) != hipSuccess)
      return e;
  }
  // dwd_e = df^T abar over the expert's rows  [d][h]
  if ((e = gemm<false, false, true>(E, R, d, h, 0, off, df, d, abar, h, 0, dwd, h, (int64_t)d * h,
                                    st)) != hipSuccess)
    return e;
  // dwgu_e = dgu^T xs  [2h][d]
  return gemm<false, false, true>(E, R, 2 * h, d, 0, off, dgu, 2 * h, xs, d, 0, dwgu, d,
                                  (int64_t)2 * h * d, st);
}

}  // namespace mm
