// Launchers of the weight-streaming products (the block routine and its
// layout are described in gemv_block.h).
#include <algorithm>

#include "gemv_block.h"
#include "launch.h"

namespace mm {
namespace {

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
