// Grouped-query attention of one new token per sequence over an INT8 KV cache,
// the decoder-block neighbour of the MoE-FFN (MobileMoE close reading: each
// layer is GQA attention with n_kv key/value heads plus the FFN, section "MoE
// preliminaries and three design factors"; the KV cache is held in 8 bits,
// eq. (5) in section "On-device objective and memory function"; n_kv = 4 and
// d_h = 64 in section "Pre-training").
//
// Cache layout: codes [B][n_kv][max_T][64] int8 and scales [B][n_kv][max_T]
// FP32: one symmetric INT8 scale per (position, head) vector, the row rule of
// the activations (s = 2 max|v| / 255, codes clamp(rint(v / s))).
//
// Decode is split over the context (flash-decoding): workgroups take runs of
// 64-position blocks of one (sequence, key/value head) and write one partial
// softmax record per query head of the group; a second kernel merges them.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace mm {
namespace {

constexpr int kDh = 64;        // head width (one lane per channel)
constexpr int kMaxGrp = 8;     // query heads per key/value head
constexpr int kRec = 68;       // partial record: m, l, two pad words, o[64] (16-byte rows)

// One wave per (sequence, head) vector of the new token: K and V quantised
// into the cache at position pos[b] (positions outside [0, max_T) are not
// written).
__global__ __launch_bounds__(256) void k_kv_append(int64_t B, int nkv, int64_t maxT,
                                                   const int32_t* __restrict__ pos,
                                                   const float* __restrict__ k_new,
                                                   const float* __restrict__ v_new,
                                                   int8_t* __restrict__ kc, int8_t* __restrict__ vc,
                                                   float* __restrict__ ks, float* __restrict__ vs) {
  const int lane = threadIdx.x & 63;
  const int64_t vec = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * nkv + g
  if (vec >= B * nkv) return;
  const int64_t b = vec / nkv;
  const int p = pos[b];
  if (p < 0 || p >= maxT) return;
  const int64_t slot = vec * maxT + p;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float v = (which ? v_new : k_new)[vec * kDh + lane];
    const float amax = max64(fabsf(v));
    const float s = (2.0f * amax) / 255.0f, y = quant_recip(s);
    (which ? vc : kc)[slot * kDh + lane] = s != 0.0f ? quant_i8(v, s, y) : (int8_t)0;
    if (lane == 0) (which ? vs : ks)[slot] = s;
  }
}

__device__ __forceinline__ void unpack_i8x4(uint32_t w, float (&f)[4]) {
  f[0] = (float)(int8_t)(w & 0xFFu);
  f[1] = (float)(int8_t)((w >> 8) & 0xFFu);
  f[2] = (float)(int8_t)((w >> 16) & 0xFFu);
  f[3] = (float)(int8_t)(w >> 24);
}

// Split of the context: a workgroup takes one (sequence b, key/value head g)
// pair, vec = b * nkv + g, and 4 * nblk consecutive blocks of 64 positions;
// wave w takes nblk of them and keeps its own running softmax over them (per
// query head of the group: maximum m, per-lane sums of exp(score - m), and
// exp(score - m)-weighted values, rescaled when m grows).  The four waves are
// merged at the end into one partial record per query head: [m, l, -, -,
// o[64]], l = sum of exp(score - m), o = sum of exp(score - m) s_v v_q.
// Positions at or past the sequence's length give m = -inf, l = 0, o = 0.
// Within a block, lane i owns position i for the scores and channels
// 4 (i & 15) .. + 3 of positions 4 j + (i >> 4), j < 16, for the values; all
// of a block's loads are issued before the first is used.
template <int kG>
__global__ __launch_bounds__(256) void k_attn_split(int nh, int nkv, int64_t maxT, int64_t max_len,
                                                    int nsplit, int nblk,
                                                    const int32_t* __restrict__ lens,
                                                    const float* __restrict__ q,
                                                    const int8_t* __restrict__ kc,
                                                    const int8_t* __restrict__ vc,
                                                    const float* __restrict__ ks,
                                                    const float* __restrict__ vs,
                                                    float* __restrict__ part) {
  __shared__ float s_q[kG][kDh];
  __shared__ float s_m[4][kG], s_l[4][kG];
  __shared__ float s_o[4][kG][kDh];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t vec = (int64_t)blockIdx.x / nsplit;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t b = vec / nkv;
  const int g = (int)(vec % nkv);
  const int64_t len = min((int64_t)max(lens[b], 0), max_len);
  for (int i = threadIdx.x; i < kG * kDh; i += 256)
    s_q[i / kDh][i % kDh] = q[(b * nh + (int64_t)g * kG) * kDh + i];
  __syncthreads();

  const int8_t* kv_base = kc + vec * maxT * kDh;
  const int8_t* vv_base = vc + vec * maxT * kDh;
  const float* ks_base = ks + vec * maxT;
  const float* vs_base = vs + vec * maxT;
  float m_run[kG], l_run[kG], acc[kG][4];
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.0f;
  }
  const int64_t blk0 = ((int64_t)split * 4 + wave) * nblk;
  for (int bi = 0; bi < nblk; ++bi) {
    const int64_t tb = (blk0 + bi) * 64;
    if (tb >= len) break;  // wave-uniform
    // re-read q from workgroup memory each block rather than holding 64 kG
    // registers of it across the loop
    asm volatile("" ::: "memory");
    const int64_t t = tb + lane;
    const bool valid = t < len;
    uint4 kw[4];
    float kscale = 0.0f, vscale = 0.0f;
    if (valid) {
      const uint4* kr = reinterpret_cast<const uint4*>(kv_base + t * kDh);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) kw[c4] = kr[c4];
      kscale = ks_base[t] * 0.125f;  // 1 / sqrt(64)
      vscale = vs_base[t];
    } else {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) kw[c4] = make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t vw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t tt = tb + 4 * j + (lane >> 4);
      vw[j] = tt < len ? *reinterpret_cast<const uint32_t*>(vv_base + tt * kDh + 4 * (lane & 15))
                       : 0u;
    }
    float sc[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) sc[h] = 0.0f;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const uint32_t ww[4] = {kw[c4].x, kw[c4].y, kw[c4].z, kw[c4].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[4];
        unpack_i8x4(ww[j], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c4 * 16 + j * 4 + e;
#pragma unroll
          for (int h = 0; h < kG; ++h) sc[h] = fmaf(s_q[h][c], f[e], sc[h]);
        }
      }
    }
    float pw[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      const float s = sc[h] * kscale;
      const float m_new = fmaxf(m_run[h], max64(valid ? s : -INFINITY));
      const float alpha = expf(m_run[h] - m_new);  // 0 on the first block
      m_run[h] = m_new;
      const float pv = valid ? expf(s - m_new) : 0.0f;
      l_run[h] = fmaf(l_run[h], alpha, pv);
      pw[h] = pv * vscale;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float f[4];
      unpack_i8x4(vw[j], f);
      const int src = 4 * j + (lane >> 4);
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const float p = __shfl(pw[h], src);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] = fmaf(p, f[e], acc[h][e]);
      }
    }
  }
  // this wave's record into workgroup memory
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const float l = wave_sum(l_run[h]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) s_o[wave][h][4 * lane + e] = v;
    }
    if (lane == 0) {
      s_m[wave][h] = m_run[h];
      s_l[wave][h] = l;
    }
  }
  __syncthreads();
  // merge the four waves: record [m, l, -, -, o[64]] per query head
  float* rec = part + ((vec * nsplit + split) * kMaxGrp) * kRec;
  for (int i = threadIdx.x; i < kG * kDh; i += 256) {
    const int h = i / kDh, c = i % kDh;
    const float m = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float o = 0.0f, l = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = s_m[w][h] == -INFINITY ? 0.0f : expf(s_m[w][h] - m);
        o = fmaf(a, s_o[w][h][c], o);
        l = fmaf(a, s_l[w][h], l);
      }
    }
    rec[h * kRec + 4 + c] = o;
    if (c == 0) {
      rec[h * kRec] = m;
      rec[h * kRec + 1] = l;
    }
  }
}

// One wave per (sequence, query head): merges the chunks.  Lanes take the
// chunks' maxima and sums 64 at a time; for the numerator lane takes channels
// 4 (lane & 15) .. + 3 of chunk 4 j + (lane >> 4), four loads in flight.
__global__ __launch_bounds__(256) void k_attn_merge(int64_t B, int nh, int nkv, int nsplit,
                                                    const float* __restrict__ part,
                                                    float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= B * nh) return;
  const int64_t b = bh / nh;
  const int h = (int)(bh % nh), grp = nh / nkv, g = h / grp, hl = h % grp;
  const float* rec0 = part + (((b * nkv + g) * nsplit) * kMaxGrp + hl) * kRec;
  const int64_t stride = (int64_t)kMaxGrp * kRec;
  // first loads: maxima and sums of chunks lane, lane + 64, ... and the
  // numerator rows of chunks 0..15, all before the first is needed
  float m_l = lane < nsplit ? rec0[lane * stride] : -INFINITY;
  float l_l = lane < nsplit ? rec0[lane * stride + 1] : 0.0f;
  float mi[4];
  float4 o[4];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = i0 + 4 * jj + (lane >> 4);
      if (i < nsplit) {
        mi[jj] = rec0[i * stride];
        o[jj] = reinterpret_cast<const float4*>(rec0 + i * stride + 4)[lane & 15];
      } else {
        mi[jj] = -INFINITY;
        o[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  load_batch(0);
  float m = m_l;
  for (int i = lane + 64; i < nsplit; i += 64) m = fmaxf(m, rec0[i * stride]);
  m = max64(m);
  float4* o4 = reinterpret_cast<float4*>(out + bh * kDh);
  if (m == -INFINITY) {  // no position: zero output
    if (lane < 16) o4[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  float den = m_l == -INFINITY ? 0.0f : expf(m_l - m) * l_l;
  for (int i = lane + 64; i < nsplit; i += 64) {
    const float mj = rec0[i * stride];
    if (mj != -INFINITY) den = fmaf(expf(mj - m), rec0[i * stride + 1], den);
  }
  den = wave_sum(den);
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < nsplit; i0 += 16) {
    if (i0 > 0) load_batch(i0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float a = mi[jj] == -INFINITY ? 0.0f : expf(mi[jj] - m);
      num.x = fmaf(a, o[jj].x, num.x);
      num.y = fmaf(a, o[jj].y, num.y);
      num.z = fmaf(a, o[jj].z, num.z);
      num.w = fmaf(a, o[jj].w, num.w);
    }
  }
  float r[4] = {num.x, num.y, num.z, num.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] += __shfl_xor(r[e], 16);
    r[e] += __shfl_xor(r[e], 32);
  }
  if (lane < 16) {
    const float inv = 1.0f / den;
    o4[lane] = make_float4(r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv);
  }
}

}  // namespace

// Blocks of 64 positions per wave: one, unless the whole launch would hold
// more than 8192 waves (eight per SIMD of the chip), then as many as keep it
// there.
static int attn_nblk(int64_t B, int nkv, int64_t max_len) {
  const int64_t nb = (max_len + 63) / 64;
  return (int)std::max<int64_t>(1, (B * nkv * nb + 8191) / 8192);
}

static int attn_nsplit(int64_t max_len, int nblk) {
  const int64_t nb = (max_len + 63) / 64;
  return (int)((nb + 4 * (int64_t)nblk - 1) / (4 * (int64_t)nblk));
}

size_t attn_partial_bytes(int64_t B, int nkv, int64_t max_len) {
  const int nsplit = attn_nsplit(max_len, attn_nblk(B, nkv, max_len));
  return (size_t)(B * nkv * nsplit) * kMaxGrp * kRec * sizeof(float);
}

hipError_t launch_kv_append(int64_t B, int nkv, int64_t maxT, const int32_t* pos,
                            const float* k_new, const float* v_new, int8_t* kc, int8_t* vc,
                            float* ks, float* vs, hipStream_t st) {
  const int64_t vecs = B * nkv;
  hipLaunchKernelGGL(k_kv_append, dim3((unsigned)((vecs + 3) / 4)), dim3(256), 0, st, B, nkv, maxT,
                     pos, k_new, v_new, kc, vc, ks, vs);
  return hipGetLastError();
}

hipError_t launch_attn_decode(int64_t B, int nh, int nkv, int64_t maxT, int64_t max_len,
                              const int32_t* lens, const float* q, const int8_t* kc,
                              const int8_t* vc, const float* ks, const float* vs, float* part,
                              float* out, hipStream_t st) {
  const int nblk = attn_nblk(B, nkv, max_len);
  const int nsplit = attn_nsplit(max_len, nblk);
  const dim3 grid((unsigned)(B * nkv * nsplit));
  switch (nh / nkv) {
#define MM_ATTN_G(G)                                                                          \
  case G:                                                                                     \
    hipLaunchKernelGGL(k_attn_split<G>, grid, dim3(256), 0, st, nh, nkv, maxT, max_len, nsplit, \
                       nblk, lens, q, kc, vc, ks, vs, part);                                  \
    break;
    MM_ATTN_G(1) MM_ATTN_G(2) MM_ATTN_G(3) MM_ATTN_G(4)
    MM_ATTN_G(5) MM_ATTN_G(6) MM_ATTN_G(7) MM_ATTN_G(8)
#undef MM_ATTN_G
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3((unsigned)((B * nh + 3) / 4)), dim3(256), 0, st, B, nh, nkv,
                     nsplit, part, out);
  return hipGetLastError();
}

}  // namespace mm
