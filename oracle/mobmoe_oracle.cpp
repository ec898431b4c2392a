// MobileMoE MoE-FFN layer: CPU oracle.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
// HIP library is checked against.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may load it.  It shares no code, header, table
// or helper with the HIP library under sparse_moe_ffn_amd/, and it includes
// nothing from there.
//
// Sources (page titles as published; sections named on those pages):
//   [P1] "MobileMoE: Scaling On-Device Mixture of Experts" close reading,
//        paper-archivist.com.
//        - section "MoE preliminaries and three design factors", eq. (*):
//          y = sum over the top-k routed experts of router_i(x) * FFN_i(x),
//          plus the always-on shared expert FFN^(s)(x).
//        - section "Pre-training", MoE stability list: the router runs in FP32.
//        - section "Quantisation-aware training", eq. (6): symmetric group
//          quantiser, group size 32, b = 4 for weights; activations are
//          quantised to INT8 on the fly; router stays FP32.
//        - section "Pre-training", MoE stability and efficiency lists: the
//          aux-loss-free expert-bias update and drop-and-pad dispatch with
//          capacity factor 1.5 (training side).
//        - section "Custom MoE kernel": count-sort of tokens by expert id,
//          one fused gate/up product per expert, SwiGLU, down product,
//          weighted scatter back through the inverse permutation.
//
// Precision policy.  In the INT4/INT8 path every floating-point result can
// decide an integer downstream (the top-k choice, the INT8 code of the hidden
// row), so that path is evaluated in FP32 with the operation order stated at
// each function: scale application as an fma chain over groups, SwiGLU with
// the exponential exp_ref below, softmax with a fixed summation tree, combine
// as an fma chain over slots.  The device follows the same order and must
// match bit for bit.  The FP32-weight and BF16-weight paths and RMSNorm have
// no such decisions and are evaluated in double precision (the plain
// definition); the device is compared to them within a tolerance.
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared -fopenmp
// (no fast-math: every FMA below is written out as std::fma).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

constexpr int kGroup = 32;  // eq. (6) group size

int8_t clamp_i(float v, int lo, int hi) {
  if (v < (float)lo) return (int8_t)lo;
  if (v > (float)hi) return (int8_t)hi;
  return (int8_t)(int)v;
}

// Round-to-nearest-even of an FP32 value to BF16, returned as FP32.
float round_bf16(float v) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  u &= 0xFFFF0000u;
  float r;
  std::memcpy(&r, &u, 4);
  return r;
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// e^x in FP32 by Cody-Waite range reduction and a Taylor polynomial (a
// textbook method; constants are the exact values of ln 2 and 1/n!):
//   n = round_half_even(x * log2(e)),  r = x - n*ln2 with ln2 split in a part
//   whose product with n is exact (ln2_hi, 15 significant bits) and the rest;
//   p(r) = sum_{i=0..7} r^i / i! in Horner form with fused multiply-adds;
//   e^x = p(r) * 2^n.  x >= 88.72 gives +inf, x <= -87.33 gives 0.
constexpr double kLn2 = 0.69314718055994530942;
constexpr float kLn2Hi = 0.693145751953125f;                 // 11357 / 2^14
constexpr float kLn2Lo = (float)(kLn2 - 0.693145751953125);
constexpr float kLog2e = (float)(1.0 / kLn2);

float exp_ref(float x) {
  if (x >= 88.72f) return INFINITY;
  if (x <= -87.33f) return 0.0f;
  const float n = std::nearbyint(x * kLog2e);
  float r = std::fma(n, -kLn2Hi, x);
  r = std::fma(n, -kLn2Lo, r);
  float p = 1.0f / 5040.0f;
  p = std::fma(p, r, 1.0f / 720.0f);
  p = std::fma(p, r, 1.0f / 120.0f);
  p = std::fma(p, r, 1.0f / 24.0f);
  p = std::fma(p, r, 1.0f / 6.0f);
  p = std::fma(p, r, 0.5f);
  p = std::fma(p, r, 1.0f);
  p = std::fma(p, r, 1.0f);
  return std::ldexp(p, (int)n);
}

float silu32(float z) { return z / (1.0f + exp_ref(-z)); }

// Balanced pairwise sum of 64 values: pairs at distance 1, then 2, 4, ..., 32.
float tree64(float* p) {
  for (int s = 1; s < 64; s *= 2)
    for (int l = 0; l < 64; l += 2 * s) p[l] = p[l] + p[l + s];
  return p[0];
}

}  // namespace

extern "C" {

const char* ora_version() { return "mobmoe-oracle 1"; }

// ---------------------------------------------------------------------------
// eq. (6) with b = 4, group 32 along the input (reduction) dimension.
//   s_g = (2 * max|W_g|) / 15                      (FP32, IEEE division)
//   q   = clamp(round_half_even(W / s_g), -8, 7)   (FP32 division)
//   an all-zero group gives s_g = 0 and q = 0.
// w: [rows][cols] FP32, q: [rows][cols] int8 (one value per element),
// s: [rows][cols/32] FP32.  Returns 0, or -1 if cols is not a multiple of 32.
int ora_quant_w4g32(int64_t rows, int64_t cols, const float* w, int8_t* q, float* s) {
  if (cols % kGroup) return -1;
  const int64_t G = cols / kGroup;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      const float* wg = w + r * cols + g * kGroup;
      float amax = 0.0f;
      for (int c = 0; c < kGroup; ++c) amax = std::max(amax, std::fabs(wg[c]));
      float sg = (2.0f * amax) / 15.0f;
      s[r * G + g] = sg;
      for (int c = 0; c < kGroup; ++c) {
        int8_t v = 0;
        if (sg != 0.0f) v = clamp_i(std::nearbyint(wg[c] / sg), -8, 7);
        q[r * cols + g * kGroup + c] = v;
      }
    }
  }
  return 0;
}

// Dynamic INT8 quantisation of activations, one scale per row: eq. (6) read
// with b = 8 and the whole row as the group.
//   s = (2 * max|v|) / 255,  q = clamp(round_half_even(v / s), -128, 127)
//   an all-zero row gives s = 0 and q = 0.
int ora_quant_act_i8(int64_t rows, int64_t cols, const float* x, int8_t* q, float* s) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * cols;
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) amax = std::max(amax, std::fabs(xr[c]));
    float sr = (2.0f * amax) / 255.0f;
    s[r] = sr;
    for (int64_t c = 0; c < cols; ++c) {
      int8_t v = 0;
      if (sr != 0.0f) v = clamp_i(std::nearbyint(xr[c] / sr), -128, 127);
      q[r * cols + c] = v;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// FP32 router logit for one (token, expert), in the fixed order the device
// uses (needed because the top-k choice must agree bit for bit):
//   64 partial sums p[l], l = 0..63; p[l] = 0, then for j = l, l+64, l+128, ...
//   in ascending order p[l] = fma(x[j], w[j], p[l]);
//   then a balanced pairwise tree: for s = 1, 2, 4, 8, 16, 32 in turn, every
//   p[l] with l a multiple of 2s becomes p[l] + p[l+s];  logit = p[0] + bias.
// Requires d % 64 == 0.
static float router_logit(const float* x, const float* w, int d, float bias) {
  float p[64];
  for (int l = 0; l < 64; ++l) p[l] = 0.0f;
  for (int j = 0; j < d; ++j) p[j % 64] = std::fma(x[j], w[j], p[j % 64]);
  return tree64(p) + bias;
}

// Router: FP32 logits (plus an optional per-expert bias added to every
// logit), top-k selection, softmax gate weights.
//   selection: experts ordered by (logit descending, index ascending); the
//     first k are idx[t][0..k-1].  Selecting on the logits is the same as
//     selecting on the softmax, which is monotone in the logit.
//   gate weights: softmax over ALL E logits, not renormalised over the k, in
//     FP32: m = max_e l_e, z_e = exp_ref(l_e - m), S = tree64 of z_0..z_{E-1}
//     padded with zeros to 64 entries, w[t][j] = z_idx / S.
// With select_only_bias the bias takes part in the selection only (the
// load-balancing bias of the "Pre-training" section, which steers routing but
// not the gate values): experts are ranked by (logit + bias) and the gate
// weights are computed from the logits without the bias, m then being the
// maximum of those.
// logits_out [T][E] FP32 is optional (the ranked values).  Returns -1 on bad shapes.
int ora_router(int64_t T, int d, int E, int k, const float* x, const float* wr,
               const float* bias, float* logits_out, int32_t* idx, double* w,
               int select_only_bias) {
  if (d % 64 || E < 1 || k < 1 || k > E) return -1;
  std::vector<float> lg(E), gl(E);
  std::vector<int> order(E);
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      if (select_only_bias) {
        gl[e] = router_logit(x + t * d, wr + (int64_t)e * d, d, 0.0f);
        lg[e] = gl[e] + (bias ? bias[e] : 0.0f);
      } else {
        lg[e] = router_logit(x + t * d, wr + (int64_t)e * d, d, bias ? bias[e] : 0.0f);
        gl[e] = lg[e];
      }
    }
    if (logits_out)
      for (int e = 0; e < E; ++e) logits_out[t * E + e] = lg[e];
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return lg[a] > lg[b]; });
    float m = gl[0];
    for (int e = 1; e < E; ++e) m = std::max(m, gl[e]);
    float z[64], zs[64];
    for (int e = 0; e < 64; ++e) z[e] = e < E ? exp_ref(gl[e] - m) : 0.0f;
    std::copy(z, z + 64, zs);
    const float S = tree64(zs);
    for (int j = 0; j < k; ++j) {
      int e = order[j];
      idx[t * k + j] = e;
      w[t * k + j] = z[e] / S;
    }
  }
  return 0;
}

// Sigmoid gating with per-token renormalisation over the selected k
// (the training-time gate of the "Pre-training" section): selection as above
// on the (biased) logits, FP32: g_j = 1 / (1 + exp_ref(-l_j)) for the k
// selected, S = tree64 of g_0..g_{k-1} padded with zeros, w_j = g_j / S.
// With select_only_bias, l_j in g_j is the logit without the bias.
int ora_router_sigmoid(int64_t T, int d, int E, int k, const float* x, const float* wr,
                       const float* bias, int32_t* idx, double* w, int select_only_bias) {
  if (d % 64 || E < 1 || k < 1 || k > E) return -1;
  std::vector<float> lg(E), gl(E);
  std::vector<int> order(E);
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      if (select_only_bias) {
        gl[e] = router_logit(x + t * d, wr + (int64_t)e * d, d, 0.0f);
        lg[e] = gl[e] + (bias ? bias[e] : 0.0f);
      } else {
        lg[e] = router_logit(x + t * d, wr + (int64_t)e * d, d, bias ? bias[e] : 0.0f);
        gl[e] = lg[e];
      }
    }
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return lg[a] > lg[b]; });
    float g[64], gs[64];
    for (int j = 0; j < 64; ++j) g[j] = j < k ? 1.0f / (1.0f + exp_ref(-gl[order[j]])) : 0.0f;
    std::copy(g, g + 64, gs);
    const float S = tree64(gs);
    for (int j = 0; j < k; ++j) {
      idx[t * k + j] = order[j];
      w[t * k + j] = g[j] / S;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Count sort of the T*k (token, slot) assignments by expert id ("Custom MoE
// kernel" section): tokens routed to one expert become one contiguous run.
//   count[e]   = number of (t, j) with idx[t][j] == e
//   offsets    = exclusive prefix sum of count, offsets[E] = T*k
//   walking t ascending, then j ascending: p = cursor[e]++,
//   perm[p] = t*k + j, inv_perm[t*k + j] = p.
// Returns -1 if an id is out of range.
int ora_route(int64_t T, int E, int k, const int32_t* idx, int32_t* offsets,
              int32_t* perm, int32_t* inv_perm) {
  std::vector<int64_t> count(E, 0);
  for (int64_t i = 0; i < T * k; ++i) {
    if (idx[i] < 0 || idx[i] >= E) return -1;
    count[idx[i]]++;
  }
  int64_t run = 0;
  std::vector<int64_t> cursor(E);
  for (int e = 0; e < E; ++e) {
    offsets[e] = (int32_t)run;
    cursor[e] = run;
    run += count[e];
  }
  offsets[E] = (int32_t)run;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int64_t slot = t * k + j;
      int64_t p = cursor[idx[slot]]++;
      perm[p] = (int32_t)slot;
      inv_perm[slot] = (int32_t)p;
    }
  return 0;
}

// ---------------------------------------------------------------------------
// W4A8 linear on one row: out[o] = s_a * sum_g s_w[o][g] * isum[o][g], with
//   isum[o][g] = sum_{c in group g} (int32) q_w[o][c] * (int32) q_a[c]
// (exact in int32; (float)isum is exact too, |isum| <= 32*8*128).  Scale
// application in FP32: acc = 0; acc = fma(s_w[o][g], isum, acc) for g
// ascending; out = acc * s_a.  isum_out [N][K/32] optional.
static void linear_w4a8_row(int N, int K, const int8_t* aq, float sa, const int8_t* wq,
                            const float* ws, float* out, int32_t* isum_out) {
  const int G = K / kGroup;
  for (int o = 0; o < N; ++o) {
    float acc = 0.0f;
    for (int g = 0; g < G; ++g) {
      int32_t is = 0;
      for (int c = g * kGroup; c < (g + 1) * kGroup; ++c)
        is += (int32_t)wq[(int64_t)o * K + c] * (int32_t)aq[c];
      if (isum_out) isum_out[(int64_t)o * G + g] = is;
      acc = std::fma(ws[(int64_t)o * G + g], (float)is, acc);
    }
    out[o] = acc * sa;
  }
}

int ora_linear_w4a8(int64_t rows, int N, int K, const int8_t* aq, const float* sa,
                    const int8_t* wq, const float* ws, float* out, int32_t* isum) {
  if (K % kGroup) return -1;
  const int G = K / kGroup;
  for (int64_t r = 0; r < rows; ++r)
    linear_w4a8_row(N, K, aq + r * K, sa[r], wq, ws, out + r * N,
                    isum ? isum + r * (int64_t)N * G : nullptr);
  return 0;
}

// One SwiGLU expert FFN on one INT8 row: gate rows 0..h-1 and up rows h..2h-1
// of the stacked gate/up weight, a = SiLU(g) * u in FP32 with
// SiLU(z) = z / (1 + exp_ref(-z)), INT8 re-quantisation of that hidden row,
// then the down product.
//   wgu_q [2h][d] / wgu_s [2h][d/32], wd_q [d][h] / wd_s [d][h/32].
static void ffn_w4a8_row(int d, int h, const int8_t* xq, float sx, const int8_t* wgu_q,
                         const float* wgu_s, const int8_t* wd_q, const float* wd_s,
                         int8_t* hq, float* hs, float* f, int32_t* isum_gu,
                         int32_t* isum_d, float* a_out) {
  std::vector<float> gu(2 * h);
  linear_w4a8_row(2 * h, d, xq, sx, wgu_q, wgu_s, gu.data(), isum_gu);
  std::vector<float> a(h);
  for (int o = 0; o < h; ++o) a[o] = silu32(gu[o]) * gu[h + o];
  if (a_out)
    for (int o = 0; o < h; ++o) a_out[o] = a[o];
  ora_quant_act_i8(1, h, a.data(), hq, hs);
  linear_w4a8_row(d, h, hq, *hs, wd_q, wd_s, f, isum_d);
}

int ora_ffn_w4a8(int64_t rows, int d, int h, const int8_t* xq, const float* sx,
                 const int8_t* wgu_q, const float* wgu_s, const int8_t* wd_q,
                 const float* wd_s, int8_t* hq, float* hs, float* f, int32_t* isum_gu,
                 int32_t* isum_d, float* a_out) {
  if (d % kGroup || h % kGroup) return -1;
  for (int64_t r = 0; r < rows; ++r)
    ffn_w4a8_row(d, h, xq + r * d, sx[r], wgu_q, wgu_s, wd_q, wd_s, hq + r * h, hs + r,
                 f + r * d, isum_gu ? isum_gu + r * (int64_t)2 * h * (d / kGroup) : nullptr,
                 isum_d ? isum_d + r * (int64_t)d * (h / kGroup) : nullptr,
                 a_out ? a_out + r * (int64_t)h : nullptr);
  return 0;
}

// Plain floating-point SwiGLU FFN on one row.  mode 0: FP32 operands,
// evaluated in double.  mode 1: operands rounded to BF16 first (x, both
// weights), the hidden row rounded to BF16 before the down product.
static void ffn_float_row(int d, int h, const float* x, const float* wgu, const float* wd,
                          int mode, double* f) {
  std::vector<double> xv(d);
  for (int c = 0; c < d; ++c) xv[c] = mode ? round_bf16(x[c]) : x[c];
  std::vector<double> gu(2 * h);
  for (int o = 0; o < 2 * h; ++o) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) {
      float wv = wgu[(int64_t)o * d + c];
      acc += xv[c] * (double)(mode ? round_bf16(wv) : wv);
    }
    gu[o] = acc;
  }
  std::vector<double> a(h);
  for (int o = 0; o < h; ++o) {
    a[o] = silu(gu[o]) * gu[h + o];
    if (mode) a[o] = round_bf16((float)a[o]);
  }
  for (int o = 0; o < d; ++o) {
    double acc = 0.0;
    for (int c = 0; c < h; ++c) {
      float wv = wd[(int64_t)o * h + c];
      acc += a[c] * (double)(mode ? round_bf16(wv) : wv);
    }
    f[o] = acc;
  }
}

int ora_ffn_float(int64_t rows, int d, int h, const float* x, const float* wgu,
                  const float* wd, int mode, double* f) {
  for (int64_t r = 0; r < rows; ++r) ffn_float_row(d, h, x + r * d, wgu, wd, mode, f + r * d);
  return 0;
}

// Combine (eq. (*) with the "weighted scatter through the inverse
// permutation" of the custom-kernel section): y[t] = sum_j w[t][j] f[t][j] +
// ys[t], slots summed in j order, in double.  f is in token-slot order
// [T][k][d].  ys may be null (no shared expert).
int ora_combine(int64_t T, int k, int d, const double* f, const double* w, const double* ys,
                double* y) {
  for (int64_t t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w[t * k + j] * f[(t * k + j) * d + c];
      y[t * d + c] = acc + (ys ? ys[t * d + c] : 0.0);
    }
  return 0;
}

// FP32 combine of the INT4/INT8 path: acc = 0; acc = fma(w[t][j], f[t][j][c],
// acc) for j ascending; y = acc + ys (ys may be null).
int ora_combine_f32(int64_t T, int k, int d, const float* f, const float* w, const float* ys,
                    float* y) {
  for (int64_t t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc = std::fma(w[t * k + j], f[(t * k + j) * d + c], acc);
      y[t * d + c] = ys ? acc + ys[t * d + c] : acc;
    }
  return 0;
}

// RMSNorm used between stacked layers in the decode workload (not part of
// eq. (*)): y = x / sqrt(mean(x^2) + eps), unit gain, in double.
int ora_rmsnorm(int64_t rows, int cols, double eps, const float* x, double* y) {
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int c = 0; c < cols; ++c) ss += (double)x[r * cols + c] * (double)x[r * cols + c];
    double inv = 1.0 / std::sqrt(ss / cols + eps);
    for (int c = 0; c < cols; ++c) y[r * cols + c] = (double)x[r * cols + c] * inv;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Whole layer, eq. (*).
//   wfmt 0: FP32 weights and activations, no quantisation.
//   wfmt 1: INT4 group-32 weights (eq. (6)), per-token INT8 activations.
//   wfmt 2: BF16 weights and activations, output rounded to BF16.
//   gating 0: softmax over all E, no renormalisation; 1: sigmoid + top-k norm;
//   plus 2: the bias takes part in the selection only (see ora_router).
// Inputs (FP32, row-major): x [T][d]; wr [E][d]; bias [E] (nullable);
//   w_gu [E][2h][d] (gate rows first, then up rows); w_d [E][d][h];
//   ws_gu [2hs][d]; ws_d [d][hs] (both ignored when hs == 0).
// Outputs: y [T][d] double; every other pointer in ora_out is optional.
struct ora_out {
  double* y;         // [T][d]
  int32_t* idx;      // [T][k]
  double* w;         // [T][k]
  float* logits;     // [T][E]
  int8_t* xq;        // [T][d]        (wfmt 1)
  float* sx;         // [T]           (wfmt 1)
  int8_t* hq;        // [T][k][h]     (wfmt 1)
  float* hs;         // [T][k]        (wfmt 1)
  double* f;         // [T][k][d]     routed expert outputs, before gating
  double* ys;        // [T][d]        shared expert output
  int8_t* hq_s;      // [T][hs]       (wfmt 1)
  float* hs_s;       // [T]           (wfmt 1)
};

int ora_forward(int d, int E, int h, int hs, int k, int wfmt, int gating, int64_t T,
                const float* x, const float* wr, const float* bias, const float* w_gu,
                const float* w_d, const float* ws_gu, const float* ws_d, int nthreads,
                ora_out* out) {
  if (d % 64 || h % kGroup || hs % kGroup || k < 1 || k > E || !out || !out->y) return -1;
  if (wfmt < 0 || wfmt > 2 || gating < 0 || gating > 3) return -1;
  const int sel_only = gating >> 1;  // gating | 2: the bias steers the selection only
  std::vector<int32_t> idx(T * k);
  std::vector<double> w(T * k);
  int rc = (gating & 1) == 0
               ? ora_router(T, d, E, k, x, wr, bias, out->logits, idx.data(), w.data(), sel_only)
               : ora_router_sigmoid(T, d, E, k, x, wr, bias, idx.data(), w.data(), sel_only);
  if (rc) return rc;
  if (out->idx) std::copy(idx.begin(), idx.end(), out->idx);
  if (out->w) std::copy(w.begin(), w.end(), out->w);

  // Weights quantised once per call (eq. (6)); only for the INT4 format.
  std::vector<int8_t> gu_q, d_q, sgu_q, sd_q, xq;
  std::vector<float> gu_s, d_s, sgu_s, sd_s, sx;
  if (wfmt == 1) {
    gu_q.resize((int64_t)E * 2 * h * d);  gu_s.resize((int64_t)E * 2 * h * d / kGroup);
    d_q.resize((int64_t)E * d * h);       d_s.resize((int64_t)E * d * h / kGroup);
    ora_quant_w4g32((int64_t)E * 2 * h, d, w_gu, gu_q.data(), gu_s.data());
    ora_quant_w4g32((int64_t)E * d, h, w_d, d_q.data(), d_s.data());
    if (hs) {
      sgu_q.resize((int64_t)2 * hs * d);  sgu_s.resize((int64_t)2 * hs * d / kGroup);
      sd_q.resize((int64_t)d * hs);       sd_s.resize((int64_t)d * hs / kGroup);
      ora_quant_w4g32(2 * hs, d, ws_gu, sgu_q.data(), sgu_s.data());
      ora_quant_w4g32(d, hs, ws_d, sd_q.data(), sd_s.data());
    }
    xq.resize(T * d);
    sx.resize(T);
    ora_quant_act_i8(T, d, x, xq.data(), sx.data());
    if (out->xq) std::copy(xq.begin(), xq.end(), out->xq);
    if (out->sx) std::copy(sx.begin(), sx.end(), out->sx);
  }

  // INT4 path: FP32 throughout (see the precision policy at the top);
  // FP32/BF16 weight paths: double.
  std::vector<double> f((int64_t)T * k * d);
  std::vector<double> ys(hs ? (int64_t)T * d : 0);
  std::vector<float> f32(wfmt == 1 ? (int64_t)T * k * d : 0);
  std::vector<float> ys32(wfmt == 1 && hs ? (int64_t)T * d : 0);
  const int64_t gu_q_stride = (int64_t)2 * h * d, gu_s_stride = gu_q_stride / kGroup;
  const int64_t d_q_stride = (int64_t)d * h, d_s_stride = d_q_stride / kGroup;

#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : 1;
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (wfmt == 1) {
        std::vector<int8_t> hq(h);
        float hsc = 0.0f;
        ffn_w4a8_row(d, h, xq.data() + t * d, sx[t], gu_q.data() + e * gu_q_stride,
                     gu_s.data() + e * gu_s_stride, d_q.data() + e * d_q_stride,
                     d_s.data() + e * d_s_stride, hq.data(), &hsc,
                     f32.data() + (t * k + j) * d, nullptr, nullptr, nullptr);
        if (out->hq) std::copy(hq.begin(), hq.end(), out->hq + (t * k + j) * h);
        if (out->hs) out->hs[t * k + j] = hsc;
      } else {
        ffn_float_row(d, h, x + t * d, w_gu + e * gu_q_stride, w_d + e * d_q_stride,
                      wfmt == 2 ? 1 : 0, f.data() + (t * k + j) * d);
      }
    }
    if (hs) {
      if (wfmt == 1) {
        std::vector<int8_t> hq(hs);
        float hsc = 0.0f;
        ffn_w4a8_row(d, hs, xq.data() + t * d, sx[t], sgu_q.data(), sgu_s.data(),
                     sd_q.data(), sd_s.data(), hq.data(), &hsc, ys32.data() + t * d, nullptr,
                     nullptr, nullptr);
        if (out->hq_s) std::copy(hq.begin(), hq.end(), out->hq_s + t * hs);
        if (out->hs_s) out->hs_s[t] = hsc;
      } else {
        ffn_float_row(d, hs, x + t * d, ws_gu, ws_d, wfmt == 2 ? 1 : 0, ys.data() + t * d);
      }
    }
  }
  if (wfmt == 1) {
    std::copy(f32.begin(), f32.end(), f.begin());
    if (hs) std::copy(ys32.begin(), ys32.end(), ys.begin());
    std::vector<float> w32(w.begin(), w.end()), y32((int64_t)T * d);
    ora_combine_f32(T, k, d, f32.data(), w32.data(), hs ? ys32.data() : nullptr, y32.data());
    std::copy(y32.begin(), y32.end(), out->y);
  } else {
    ora_combine(T, k, d, f.data(), w.data(), hs ? ys.data() : nullptr, out->y);
  }
  if (out->f) std::copy(f.begin(), f.end(), out->f);
  if (out->ys && hs) std::copy(ys.begin(), ys.end(), out->ys);
  if (wfmt == 2)
    for (int64_t i = 0; i < T * d; ++i) out->y[i] = round_bf16((float)out->y[i]);
  return 0;
}

// FP32 exponential of the INT4 path, exposed for its pin.
void ora_exp_ref(int64_t n, const float* x, float* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = exp_ref(x[i]);
}

// BF16 rounding exposed for the pins.
void ora_round_bf16(int64_t n, const float* x, float* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = round_bf16(x[i]);
}

// ---------------------------------------------------------------------------
// Grouped-query attention of one new token per sequence over an INT8 KV cache
// (the decoder block around the MoE-FFN: GQA with n_kv key/value heads of
// width d_h, KV cache held in 8 bits; sections "MoE preliminaries and three
// design factors" and eq. (5)).  Plain definition in double:
//   query head h reads key/value head g = h / (n_h / n_kv);
//   k_t = s_k[t] * k_q[t], v_t = s_v[t] * v_q[t] (the cached codes and the
//   per-(position, head) scales);
//   score_t = (q_h . k_t) / sqrt(d_h), p = softmax over t = 0..T-1,
//   out_h = sum_t p_t v_t.
// Layouts: q [B][n_h][d_h] FP32; caches [B][n_kv][max_T][d_h] int8, scales
// [B][n_kv][max_T] FP32 (positions 0..T-1 used); out [B][n_h][d_h] double.
int ora_attn_decode(int64_t B, int nh, int nkv, int dh, int64_t T, int64_t maxT, const float* q,
                    const int8_t* kq, const int8_t* vq, const float* ks, const float* vs,
                    double* out) {
  if (B < 0 || nkv < 1 || nh < nkv || nh % nkv || dh < 1 || T < 1 || T > maxT) return -1;
  const int grp = nh / nkv;
  std::vector<double> sc(T);
  for (int64_t b = 0; b < B; ++b)
    for (int h = 0; h < nh; ++h) {
      const int g = h / grp;
      const float* qh = q + (b * nh + h) * dh;
      const int64_t base = (b * nkv + g) * maxT;
      double m = -INFINITY;
      for (int64_t t = 0; t < T; ++t) {
        double dot = 0.0;
        for (int c = 0; c < dh; ++c)
          dot += (double)qh[c] * ((double)ks[base + t] * (double)kq[(base + t) * dh + c]);
        sc[t] = dot / std::sqrt((double)dh);
        m = std::max(m, sc[t]);
      }
      double den = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        sc[t] = std::exp(sc[t] - m);
        den += sc[t];
      }
      double* o = out + (b * nh + h) * dh;
      for (int c = 0; c < dh; ++c) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
          acc += sc[t] * ((double)vs[base + t] * (double)vq[(base + t) * dh + c]);
        o[c] = acc / den;
      }
    }
  return 0;
}

// ---------------------------------------------------------------------------
// Training-side pieces of the layer: [P1] section "Pre-training" (the MoE
// stability list: balancing through an expert bias updated from the batch's
// load, no auxiliary loss; the efficiency list: drop-and-pad dispatch with
// capacity factor 1.5) and section "Quantisation-aware training" (eq. (6)
// applied as fake quantisation during training).

// Aux-loss-free balancing.  load_e = number of (token, slot) assignments of
// the batch routed to e; the mean load is T*k/E.  Every bias moves by lambda
// towards balance:
//   b_e <- b_e + lambda   if load_e is below the mean,
//   b_e <- b_e - lambda   if above, unchanged if equal   (one FP32 add),
// the comparison taken exactly in integers (T*k against E*load_e).
// load (optional) receives load_e.  Returns -1 if an id is out of range.
int ora_bias_update(int64_t T, int E, int k, const int32_t* idx, float lambda, float* bias,
                    int32_t* load) {
  std::vector<int64_t> c(E, 0);
  for (int64_t i = 0; i < T * k; ++i) {
    if (idx[i] < 0 || idx[i] >= E) return -1;
    c[idx[i]]++;
  }
  for (int e = 0; e < E; ++e) {
    const int64_t below = T * k - (int64_t)E * c[e];  // > 0: load under the mean
    if (below > 0) bias[e] = bias[e] + lambda;
    else if (below < 0) bias[e] = bias[e] - lambda;
    if (load) load[e] = (int32_t)c[e];
  }
  return 0;
}

// Drop-and-pad dispatch: every expert gets a buffer of C rows.  Reading:
// assignments are admitted in token order (t ascending, then slot j); the
// first C of an expert are kept, the rest dropped (their term leaves the
// sum of eq. (*)).
//   buf[e][p]   = id t*k+j of expert e's p-th kept assignment, -1 for the
//                 padding rows p >= kept_e                      [E][C]
// and the kept assignments as a dropless routing:
//   offsets_c   = exclusive prefix sum of kept_e = min(load_e, C)   [E+1]
//   perm_c[offsets_c[e] + p] = buf[e][p] for p < kept_e               [T*k]
//                 (entries past offsets_c[E] set to -1)
//   inv_c[t*k+j] = its row in perm_c, -1 if dropped                 [T*k]
int ora_drop_pad(int64_t T, int E, int k, int64_t C, const int32_t* idx, int32_t* buf,
                 int32_t* offsets_c, int32_t* perm_c, int32_t* inv_c) {
  if (C < 0) return -1;
  for (int64_t i = 0; i < T * k; ++i)
    if (idx[i] < 0 || idx[i] >= E) return -1;
  std::vector<int64_t> fill(E, 0);
  for (int64_t i = 0; i < (int64_t)E * C; ++i) buf[i] = -1;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      const int e = idx[a];
      if (fill[e] < C) buf[(int64_t)e * C + fill[e]] = (int32_t)a;
      fill[e]++;
    }
  int64_t run = 0;
  for (int e = 0; e < E; ++e) {
    offsets_c[e] = (int32_t)run;
    run += std::min(fill[e], C);
  }
  offsets_c[E] = (int32_t)run;
  for (int64_t a = 0; a < T * k; ++a) {
    perm_c[a] = -1;
    inv_c[a] = -1;
  }
  for (int e = 0; e < E; ++e)
    for (int64_t p = 0; p < std::min(fill[e], C); ++p) {
      const int32_t a = buf[(int64_t)e * C + p];
      perm_c[offsets_c[e] + p] = a;
      inv_c[a] = (int32_t)(offsets_c[e] + p);
    }
  return 0;
}

// Fake quantisation (QAT), eq. (6) with b bits over groups of `group`
// consecutive elements of a row (weights: b = 4, group 32; activations:
// b = 8, group = the row):
//   s = (2 * max|x_g|) / (2^b - 1)                    (FP32, IEEE division)
//   u = round_half_even(x / s)                        (FP32 division)
//   xbar = s * clamp(u, -2^(b-1), 2^(b-1) - 1)        (FP32 product)
// Backward with straight-through rounding: the derivative of the rounding is
// taken as 1 and the clamp's as its own at u, so
//   gin = gout where -2^(b-1) <= u <= 2^(b-1) - 1, else 0;
// an all-zero group (s = 0) gives xbar = 0 and passes the gradient.  Since
// |x / s| <= (2^b - 1) / 2, only a positive group maximum whose quotient
// rounds up to 2^(b-1) is clipped.  xbar and the gradient pair are optional.
int ora_fake_quant(int64_t rows, int64_t cols, int bits, int64_t group, const float* x,
                   float* xbar, const float* gout, float* gin) {
  if ((bits != 4 && bits != 8) || group < 1 || cols % group) return -1;
  const float levels = bits == 4 ? 15.0f : 255.0f;
  const float qmin = bits == 4 ? -8.0f : -128.0f, qmax = bits == 4 ? 7.0f : 127.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g0 = 0; g0 < cols; g0 += group) {
      const int64_t base = r * cols + g0;
      float amax = 0.0f;
      for (int64_t c = 0; c < group; ++c) amax = std::max(amax, std::fabs(x[base + c]));
      const float s = (2.0f * amax) / levels;
      for (int64_t c = 0; c < group; ++c) {
        const int64_t i = base + c;
        bool pass = true;
        float v = 0.0f;
        if (s != 0.0f) {
          const float u = std::nearbyint(x[i] / s);
          pass = u >= qmin && u <= qmax;
          v = s * std::min(std::max(u, qmin), qmax);
        }
        if (xbar) xbar[i] = v;
        if (gin) gin[i] = pass ? gout[i] : 0.0f;
      }
    }
  return 0;
}

// ---------------------------------------------------------------------------
// QAT forward and backward of the routed experts ([P1] "Pre-training":
// every expert's FFN batched into grouped matrix products; "Quantisation-
// aware training": weights and activations fake-quantised, eq. (6)).  Rows
// are the kept assignments in expert order: expert e owns rows
// [offsets[e], offsets[e+1]) of xs (the fake-quantised input rows).
// Weights are fake-quantised FP32: wgu [E][2h][d] (gate rows first), wd
// [E][d][h].  Per row r of expert e:
//   gu = wgu_e xs_r                           (gate g = gu[0:h], up u = gu[h:2h])
//   a  = silu32(g) * u                         (FP32, the SwiGLU of R6)
//   abar = fake quant of a, b = 8, one group per row (eq. (6))
//   f  = wd_e abar
// Products and sums in double; the a / abar step in FP32 as stated, since
// it decides INT8 codes.
static void train_act_row(int h, const float* gu_row, float* a, float* abar, float* pass) {
  float amax = 0.0f;
  for (int j = 0; j < h; ++j) {
    a[j] = silu32(gu_row[j]) * gu_row[h + j];
    amax = std::max(amax, std::fabs(a[j]));
  }
  const float s = (2.0f * amax) / 255.0f;
  for (int j = 0; j < h; ++j) {
    if (s == 0.0f) {
      abar[j] = 0.0f;
      pass[j] = 1.0f;
      continue;
    }
    const float u = std::nearbyint(a[j] / s);
    pass[j] = (u >= -128.0f && u <= 127.0f) ? 1.0f : 0.0f;
    abar[j] = s * std::min(std::max(u, -128.0f), 127.0f);
  }
}

int ora_expert_train_forward(int E, int d, int h, const int32_t* offsets, const float* xs,
                             const float* wgu, const float* wd, float* gu, float* abar, float* f) {
  std::vector<float> a(h), pass(h);
  for (int e = 0; e < E; ++e) {
    const float* Wg = wgu + (int64_t)e * 2 * h * d;
    const float* Wd = wd + (int64_t)e * d * h;
    for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
      const float* x = xs + r * d;
      float* g = gu + r * 2 * h;
      for (int j = 0; j < 2 * h; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)Wg[(int64_t)j * d + c] * (double)x[c];
        g[j] = (float)acc;
      }
      train_act_row(h, g, a.data(), abar + r * h, pass.data());
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < h; ++j) acc += (double)Wd[(int64_t)c * h + j] * (double)abar[r * h + j];
        f[r * d + c] = (float)acc;
      }
    }
  }
  return 0;
}

// Backward of the above given the forward's gu and the gradient df of the
// expert output rows (straight-through rounding in the activation quantiser,
// its clamp differentiated at the rounded quotient; the row scale held
// constant):
//   dabar = wd_e^T df_r;  da = dabar * pass(a)
//   dg = da * u * silu'(g),  du = da * silu(g),   silu'(g) = sig(g) (1 + g (1 - sig(g)))
//   dxs_r = wgu_e^T [dg, du]
//   dwd_e  = sum over the expert's rows of df_r abar_r^T      [d][h]
//   dwgu_e = sum over the expert's rows of [dg, du]_r xs_r^T [2h][d]
// abar and pass are recomputed from gu by the FP32 rule above; everything
// else in double.  An expert without rows gets zero weight gradients.
int ora_expert_backward(int E, int d, int h, const int32_t* offsets, const float* xs,
                        const float* wgu, const float* wd, const float* gu, const float* df,
                        double* dxs, double* dwgu, double* dwd) {
  std::vector<float> a(h), abar(h), pass(h);
  std::vector<double> dgu(2 * h);
  for (int e = 0; e < E; ++e) {
    const float* Wg = wgu + (int64_t)e * 2 * h * d;
    const float* Wd = wd + (int64_t)e * d * h;
    double* dWg = dwgu + (int64_t)e * 2 * h * d;
    double* dWd = dwd + (int64_t)e * d * h;
    for (int64_t i = 0; i < (int64_t)2 * h * d; ++i) dWg[i] = 0.0;
    for (int64_t i = 0; i < (int64_t)d * h; ++i) dWd[i] = 0.0;
    for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
      const float* g = gu + r * 2 * h;
      const float* x = xs + r * d;
      const float* dfr = df + r * d;
      train_act_row(h, g, a.data(), abar.data(), pass.data());
      for (int j = 0; j < h; ++j) {
        double dab = 0.0;
        for (int c = 0; c < d; ++c) dab += (double)Wd[(int64_t)c * h + j] * (double)dfr[c];
        const double da = dab * pass[j];
        const double gj = g[j], uj = g[h + j];
        const double sig = 1.0 / (1.0 + std::exp(-gj));
        dgu[j] = da * uj * sig * (1.0 + gj * (1.0 - sig));
        dgu[h + j] = da * gj * sig;
      }
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = 0; j < 2 * h; ++j) acc += (double)Wg[(int64_t)j * d + c] * dgu[j];
        dxs[r * d + c] = acc;
      }
      for (int c = 0; c < d; ++c)
        for (int j = 0; j < h; ++j) dWd[(int64_t)c * h + j] += (double)dfr[c] * (double)abar[j];
      for (int j = 0; j < 2 * h; ++j)
        for (int c = 0; c < d; ++c) dWg[(int64_t)j * d + c] += dgu[j] * (double)x[c];
    }
  }
  return 0;
}

// Router backward of the training step ([P1] "Pre-training", stability list:
// FP32 router, router z-loss with weight lambda_z, sigmoid gating with
// per-token top-k renormalisation as the training gate).  Given the
// gradient dy of the layer output and the kept expert outputs f (rows of the
// kept routing, inv[t*k+j] its row or -1 when dropped):
//   g_j   = dy_t . f_inv(t,j)  (0 when dropped)        gradient of gate weight j
//   z     = the logits the gate reads: x_t Wr^T + bias (or without the bias
//           when gating & 2: selection-only bias)
//   softmax gate (gating & 1 == 0): w_j = p_idx(j), p = softmax(z) over all E:
//           dz_e = p_e (G_e - sum_j p_idx(j) g_j), G_e = g_j if e = idx(j), else 0
//   sigmoid gate: w_j = sig(z_idx(j)) / S, S = sum over the k of sig:
//           dz_idx(j) = sig'(z_idx(j)) / S (g_j - sum_i w_i g_i), other e: 0
//   z-loss  (lambda_z / T) sum_t lse(z_t)^2 adds (2 lambda_z / T) lse(z_t) softmax(z_t)_e
//   dWr = dz^T x  [E][d];  dx_t += dz_t Wr  [T][d] (accumulated into dx)
// The bias gets no gradient (it follows the load).  Double precision.
int ora_router_backward(int64_t T, int d, int E, int k, int gating, const float* x, const float* wr,
                        const float* bias, const int32_t* idx, const float* f, const int32_t* inv,
                        const float* dy, double lambda_z, double* dz, double* dwr, double* dx) {
  std::vector<double> z(E), p(E), g(k);
  for (int64_t i = 0; i < (int64_t)E * d; ++i) dwr[i] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const float* xt = x + t * d;
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += (double)xt[c] * (double)wr[(int64_t)e * d + c];
      z[e] = acc + ((bias && !(gating & 2)) ? (double)bias[e] : 0.0);
    }
    for (int j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      double acc = 0.0;
      if (r >= 0)
        for (int c = 0; c < d; ++c) acc += (double)dy[t * d + c] * (double)f[(int64_t)r * d + c];
      g[j] = acc;
    }
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) m = std::max(m, z[e]);
    double S = 0.0;
    for (int e = 0; e < E; ++e) S += std::exp(z[e] - m);
    for (int e = 0; e < E; ++e) p[e] = std::exp(z[e] - m) / S;
    const double lse = m + std::log(S);
    double* dzt = dz + t * E;
    for (int e = 0; e < E; ++e) dzt[e] = 2.0 * lambda_z / (double)T * lse * p[e];
    if (!(gating & 1)) {
      double pg = 0.0;
      for (int j = 0; j < k; ++j) pg += p[idx[t * k + j]] * g[j];
      for (int e = 0; e < E; ++e) dzt[e] -= p[e] * pg;
      for (int j = 0; j < k; ++j) dzt[idx[t * k + j]] += p[idx[t * k + j]] * g[j];
    } else {
      double Ssig = 0.0;
      std::vector<double> sg(k);
      for (int j = 0; j < k; ++j) {
        sg[j] = 1.0 / (1.0 + std::exp(-z[idx[t * k + j]]));
        Ssig += sg[j];
      }
      double wg = 0.0;
      for (int j = 0; j < k; ++j) wg += sg[j] / Ssig * g[j];
      for (int j = 0; j < k; ++j) dzt[idx[t * k + j]] += sg[j] * (1.0 - sg[j]) / Ssig * (g[j] - wg);
    }
    for (int e = 0; e < E; ++e)
      for (int c = 0; c < d; ++c) {
        dwr[(int64_t)e * d + c] += dzt[e] * (double)xt[c];
        dx[t * d + c] += dzt[e] * (double)wr[(int64_t)e * d + c];
      }
  }
  return 0;
}

}  // extern "C"
