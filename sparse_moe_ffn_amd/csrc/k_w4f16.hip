// W4A8 grouped products on the f16 matrix cores with exact group sums.
//
// MobileMoE close reading, section "Custom MoE kernel": after the count sort
// each expert runs one batched product over its contiguous rows (fused gate/up
// with SwiGLU, then down); section "Quantisation-aware training", eq. (6):
// INT4 weights with one FP32 scale per 32 weights along the reduction, INT8
// activations.  Every group sum isum_g = sum_k a_k w_k is an integer with
// |isum_g| <= 32 * 128 * 8 = 2^15, and every partial sum of it is an integer
// of at most that size, so v_mfma_f32_32x32x16_f16 -- f16 operands holding
// the codes exactly, FP32 accumulation -- returns isum_g exactly, already as
// an FP32 value.  Each output then takes one fused multiply-add per group,
//     acc = fma(s_w[col][g], isum_g, acc)   for g ascending,
// the order the other product kernels and the CPU oracle use, so results are
// bit-identical to them.  (The int8 matrix cores return int32 sums that need
// a convert before that FMA: twice the vector-ALU work per group, which is
// what bounds these products.)
//
// Operands.  Activations are f16 paired codes (common.h), written so by the
// quantisers.  Weights are the prepacked INT4 chunks (common.h), unpacked to
// f16 two at a time: with the top bit of each nibble flipped (offset binary,
// nibble = q + 8) and the exponent bits of 1024 set, two low nibbles of a
// 32-bit word become the f16 pair 1024 + (q + 8), two high nibbles the pair
// 1024 + 16 (q + 8); one packed f16 subtraction of 1032 or 1152 leaves q or
// 16 q exactly.  The slot order this gives is the paired order of the
// activations, whose high-nibble partners are stored divided by 16, so every
// product is a * q exactly.
//
// Tiling.  A workgroup of 2 x kWN waves owns kTM rows of one expert (128;
// routed tiles found on the device from the offsets; a dense problem with
// few tiles takes 64-row tiles, since its reduction cannot be split) and
// 64 kWN weight rows (gate/up: 32 kWN gate rows and the matching up rows, so
// SwiGLU is applied in registers; down: 64 kWN output columns).  The
// reduction runs in K blocks of two quantisation groups: the block's
// activation tile (f16, 128 bytes per row), its raw prepacked weight chunks
// and their scales are staged through LDS (two stages), loaded into
// registers two blocks ahead of the math, so each global byte feeds every
// wave that needs it.  Wave (wm, wn) computes rows kTM/2 wm .. of the tile
// against its two 32-column tiles, unpacking its own weight fragments to f16
// in registers.  Workgroup ids are remapped so that the tiles of one expert
// stay on one XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kXcd = 8;
constexpr int kBM = 128;   // most rows per workgroup tile
constexpr int kLds = 80;   // LDS bytes per tile row (64 bytes of codes + 16 of padding)

struct F16Prob {
  ExpertArgs a;
  int nsplit, K, N;
  const uint16_t* act;  // f16 paired codes [.][K]
  const float* act_scale;
  const uint8_t* wq;
  const float* wsc;
  float* out;
  int32_t* isum;  // exact group sums [rows][wrows][G] (test twins), or null
};

// 8 prepacked nibbles (one 32-bit word) -> 8 f16 values in paired slot order
// (4 words): slots 0,1 and 4,5 hold q, slots 2,3 and 6,7 hold 16 q.  (w & m)
// ^ c keeps two nibbles, flips their top bit (two's complement to offset
// binary) and sets the exponent bits of 1024.
__device__ __forceinline__ v4i nib_to_f16(uint32_t w) {
  const uint32_t t = w >> 8;
  const v2h k1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const v2h k16 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  v4i r;
  r[0] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, (w & 0x000F000Fu) ^ 0x64086408u) + k1);
  r[1] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, (w & 0x00F000F0u) ^ 0x64806480u) + k16);
  r[2] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, (t & 0x000F000Fu) ^ 0x64086408u) + k1);
  r[3] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, (t & 0x00F000F0u) ^ 0x64806480u) + k16);
  return r;
}

__device__ __forceinline__ v16f mfma2(v4i a0, v4i a1, v4i b0, v4i b1) {
  v16f d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a0),
                                                   __builtin_bit_cast(v8h, b0), v16f{}, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a1),
                                                __builtin_bit_cast(v8h, b1), d, 0, 0, 0);
}

// Capture of the exact group sums (test twins only): isum[(p0 + row) *
// wrows + col][g], col = the weight row of the lane's column.
struct Capture {
  int32_t* isum;
  int64_t wrows;
  int G, g, p0, rows_left;  // rows_left: rows of the wave's first row tile onward
  int col[2];               // weight row of this lane's column in each column tile
};

// One group of one wave: kMT row tiles x 2 column tiles.  a/b: this lane's
// fragments (two K steps each), sc: the true FP32 scales of the lane's column
// in each column tile.  The MFMAs of the next tile are issued before the
// previous tile's epilogue, so matrix cores and vector ALU overlap.
// Row tiles at or past mt_active (wave-uniform) are skipped.
template <int kMT, bool kCapture>
__device__ __forceinline__ void group_math(v16f (&acc)[2][2], const v4i (&a)[2][2],
                                           const v4i (&b)[2][2], const float (&sc)[2],
                                           const Capture& cap, int lane, int mt_active) {
  constexpr int kT = 2 * kMT;  // tile t: row tile t / 2, column tile t % 2
  v16f d[2];
#pragma unroll
  for (int t = 0; t <= kT; ++t) {
    if (t < kT && (t >> 1) < mt_active) {
      d[t & 1] = mfma2(a[t >> 1][0], a[t >> 1][1], b[t & 1][0], b[t & 1][1]);
      if constexpr (kCapture) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = (t >> 1) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < cap.rows_left)
            cap.isum[((int64_t)(cap.p0 + row) * cap.wrows + cap.col[t & 1]) * cap.G + cap.g] =
                (int32_t)d[t & 1][r];
        }
      }
    }
    if (t > 0 && ((t - 1) >> 1) < mt_active) {
      const int p = t - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[p >> 1][p & 1][r] = fmaf(sc[p & 1], d[p & 1][r], acc[p >> 1][p & 1][r]);
    }
  }
}

// Workgroup memory of one tile: two stages, each holding two quantisation
// groups (a K block of 64) -- the activation tile (128 rows x 128 bytes), the
// raw prepacked weight chunks (2 kWN chunks x 2 groups x 512 bytes) and their
// scales (2 kWN x 2 x 32 floats) -- and the rows' activation scales.  A tile
// row holds eight 16-byte parts (part 4 gg + q: group gg of the block, codes
// 8 q .. 8 q + 7 of the group); part p of row r sits at slot p ^ (r & 7), so
// the fragment reads of 8 consecutive rows hit 8 different bank groups.
template <int kWN>
struct F16Smem {
  __attribute__((aligned(16))) uint8_t A[2][kBM * 128];
  __attribute__((aligned(16))) uint8_t Braw[2][2 * kWN * 2 * kChunkBytes];
  __attribute__((aligned(16))) float S[2][2 * kWN * 2 * 32];
  float R[kBM];
};

__device__ __forceinline__ uint32_t swz(int row, int part) {
  return (uint32_t)(row * 128 + ((part ^ (row & 7)) << 4));
}

// One workgroup tile of problem P: logical tile id = mt * nsplit + split,
// slot i of XCD x (kDense: the rows are the tokens in order, per_dense slots
// per XCD; otherwise routed, expert-sorted rows with tiles found from the
// offsets).  Called by the whole workgroup; every exit before the main loop
// is taken by all of its waves together.
// kTM: rows of the tile (128, or 64 to spread a dense problem over more
// workgroups), kTM / 2 per wave row.
template <int kWN, int kTM, bool kGateUp, bool kDense, bool kCapture>
__device__ __forceinline__ void f16_tile(F16Smem<kWN>& sm, const F16Prob& P, int x, int i,
                                         int per_dense) {
  static_assert(kTM == 64 || kTM == kBM, "tile rows");
  constexpr int kBN = 64 * kWN;                          // weight rows per workgroup
  constexpr int kThreads = 128 * kWN;
  constexpr int kWR = kTM / 2;                           // rows per wave
  constexpr int kMT = kWR / 32;                          // row tiles per wave
  constexpr int kAPieces = kTM * 128 / (16 * kThreads);  // 16-byte activation pieces per thread
  constexpr int kBPieces = 2 * kWN * 2 * kChunkBytes / (16 * kThreads);  // 16-byte weight pieces
  static_assert(kBPieces * 16 * kThreads == 2 * kWN * 2 * kChunkBytes, "weight pieces");
  static_assert(2 * kWN * 2 * 32 == kThreads, "one scale per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const ExpertArgs& a = P.a;
  const int nsplit = P.nsplit, K = P.K;
  const int rows = (int)a.rows;
  int mt, split, p0, n, e;
  if constexpr (kDense) {
    const int logical = x * per_dense + i;
    mt = logical / nsplit;
    split = logical % nsplit;
    p0 = mt * kTM;
    n = min(kTM, rows - p0);
    e = 0;
  } else {
    const RoutedTiles rt = routed_tiles(a.offsets, a.E, rows, kTM);
    const int per = (rt.total * nsplit + kXcd - 1) / kXcd;
    if (i >= per) return;
    const int logical = x * per + i;
    mt = logical / nsplit;
    split = logical % nsplit;
    routed_pick(rt, kTM, mt, p0, n, e);
  }
  if (n <= 0) return;
  const int G = K / kGroup, KB = G / 2, h = a.h;
  const int64_t wrows = kGateUp ? 2 * (int64_t)h : P.N;

  auto src_row = [&](int r) {
    const int rr = r < n ? r : 0;  // padding rows read the tile's first row (never stored)
    int src = p0 + rr;
    if constexpr (kGateUp && !kDense) {
      src = a.perm[p0 + rr] / a.k;
      if ((unsigned)src >= (unsigned)a.T) src = 0;  // stays in bounds for a corrupt perm
    }
    return src;
  };
  auto rb_of = [&](int cb) {  // prepacked 32-row block of chunk cb of the tile
    if constexpr (kGateUp)
      return cb < kWN ? split * kWN + cb : h / 32 + split * kWN + (cb - kWN);
    else
      return split * 2 * kWN + cb;
  };
  // Staging of one K block, flat over the workgroup: activation piece q (q =
  // tid + kThreads c) is row q / 8, slot q % 8 (it carries part (q % 8) ^
  // (row & 7)); weight piece q is bytes 16 q .. of the chunks (chunk q / 64,
  // whose prepacked groups 2 kb and 2 kb + 1 are contiguous); scale tid is
  // chunk tid / 64, group (tid / 32) % 2, row tid % 32.
  const uint16_t* ga[kAPieces];
#pragma unroll
  for (int c = 0; c < kAPieces; ++c) {
    const int q = tid + kThreads * c, r = q >> 3;
    const int part = (q & 7) ^ (r & 7);  // group (part >> 2), codes 8 (part & 3) ..
    ga[c] = P.act + (int64_t)src_row(r) * K + (part >> 2) * 32 + (part & 3) * 8;
  }
  if (tid < kTM) sm.R[tid] = P.act_scale[src_row(tid)];
  const int64_t ebase = (int64_t)e * (wrows / 32);
  const uint8_t* gb[kBPieces];
#pragma unroll
  for (int c = 0; c < kBPieces; ++c) {
    const int q = tid + kThreads * c, cb = q >> 6;
    gb[c] = P.wq + (ebase + rb_of(cb)) * G * kChunkBytes + (q & 63) * 16;
  }
  const float* gs = P.wsc + (ebase + rb_of(tid >> 6)) * G * 32 + (tid & 63);

  // Global loads run two K blocks ahead of the math, in two register slots
  // (block kb in slot kb % 2; the loop is unrolled by two so the slots are
  // fixed registers).  Past the last block the last one is re-read (valid,
  // unused).
  struct Regs {
    v4i a[kAPieces], b[kBPieces];
    float s;
  } r0, r1;
  auto gload = [&](int kb, Regs& r) __attribute__((always_inline)) {
    kb = min(kb, KB - 1);
#pragma unroll
    for (int c = 0; c < kAPieces; ++c) r.a[c] = *reinterpret_cast<const v4i*>(ga[c] + kb * 64);
#pragma unroll
    for (int c = 0; c < kBPieces; ++c)
      r.b[c] = *reinterpret_cast<const v4i*>(gb[c] + (int64_t)kb * 2 * kChunkBytes);
    r.s = gs[(int64_t)kb * 64];
  };
  auto lstore = [&](int st, const Regs& r) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kAPieces; ++c)
      *reinterpret_cast<v4i*>(&sm.A[st][16 * (tid + kThreads * c)]) = r.a[c];
#pragma unroll
    for (int c = 0; c < kBPieces; ++c)
      *reinterpret_cast<v4i*>(&sm.Braw[st][16 * (tid + kThreads * c)]) = r.b[c];
    sm.S[st][tid] = r.s;
  };

  // this wave's fragment rows and weight chunks
  const int fr = lane & 31, fq = 2 * (lane >> 5);
  int arow[2], bcb[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) arow[m] = wm * kWR + (m % kMT) * 32 + fr;
  if constexpr (kGateUp) {
    bcb[0] = wn;
    bcb[1] = kWN + wn;
  } else {
    bcb[0] = 2 * wn;
    bcb[1] = 2 * wn + 1;
  }
  const int rows_w = min(max(n - wm * kWR, 0), kWR);  // rows of this wave
  Capture cap{P.isum, wrows, G, 0, p0 + wm * kWR, rows_w, {0, 0}};
  if constexpr (kCapture) {
#pragma unroll
    for (int j = 0; j < 2; ++j) cap.col[j] = rb_of(bcb[j]) * 32 + fr;
  }

  v16f acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = v16f{};

  // Pipeline: block kb + 1's global loads are in flight while block kb is
  // computed from LDS; then they go to the other LDS stage, and one barrier
  // per block makes them visible (and frees the stage just computed).
  gload(0, r0);
  gload(1, r1);
  lstore(0, r0);
  gload(2, r0);
  __syncthreads();
  // iteration kb: compute block kb from LDS stage kb % 2, store block kb + 1
  // (register slot (kb + 1) % 2) to the other stage, load block kb + 3 into
  // that slot
  auto step = [&](int kb, Regs& next) __attribute__((always_inline)) {
    const int st = kb & 1;
    if (rows_w > 0) {
      // every LDS read of the block first, then the math of its two groups
      uint2 wr[2][2];
      v4i av[2][2][2];
      float sc[2][2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // prepack lane L = lane of chunk bcb[j], group gg of the block
          wr[gg][j] = *reinterpret_cast<const uint2*>(
              &sm.Braw[st][(bcb[j] * 2 + gg) * kChunkBytes + 8 * lane]);
          sc[gg][j] = sm.S[st][(bcb[j] * 2 + gg) * 32 + fr];
        }
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
          av[gg][m][0] = *reinterpret_cast<const v4i*>(&sm.A[st][swz(arow[m], 4 * gg + fq)]);
          av[gg][m][1] = *reinterpret_cast<const v4i*>(&sm.A[st][swz(arow[m], 4 * gg + fq + 1)]);
        }
      }
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        v4i bv[2][2];
        float scale[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // this lane's 16 nibbles, unpacked to f16 in registers
          bv[j][0] = nib_to_f16(wr[gg][j].x);
          bv[j][1] = nib_to_f16(wr[gg][j].y);
          scale[j] = sc[gg][j] * 16.0f;  // prepacked scales are divided by 16
        }
        cap.g = 2 * kb + gg;
        group_math<kMT, kCapture>(acc, av[gg], bv, scale, cap, lane, (rows_w + 31) >> 5);
      }
    }
    if (kb + 1 < KB) {
      lstore(st ^ 1, next);
      gload(kb + 3, next);
    }
    __syncthreads();
  };
  for (int kb = 0; kb < KB; kb += 2) {  // KB is even
    step(kb, r1);
    step(kb + 1, r0);
  }

  // epilogue: times the row's activation scale; gate/up applies SwiGLU
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * kWR + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= n) continue;
      const float s = sm.R[row];
      if constexpr (kGateUp) {
        P.out[(int64_t)(p0 + row) * h + split * 32 * kWN + wn * 32 + fr] =
            silu(acc[m][0][r] * s) * (acc[m][1][r] * s);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          P.out[(int64_t)(p0 + row) * P.N + split * kBN + wn * 64 + j * 32 + fr] = acc[m][j][r] * s;
      }
    }
}

// Routed (P0) and shared (P1) products of one kind in one launch: every XCD's
// first per1 slots take shared tiles (the longer ones start first), the rest
// routed tiles.
template <int kWN, int kTM1, bool kGateUp, bool kCapture>
__global__ __launch_bounds__(128 * kWN) void k_w4f16_pair(F16Prob P0, F16Prob P1, int per1) {
  __shared__ F16Smem<kWN> sm;
  const int b = (int)blockIdx.x, x = b % kXcd, i = b / kXcd;
  if (i < per1)
    f16_tile<kWN, kTM1, kGateUp, true, kCapture>(sm, P1, x, i, per1);
  else
    f16_tile<kWN, kBM, kGateUp, false, kCapture>(sm, P0, x, i - per1, 0);
}

// One problem alone (routed or dense).
constexpr int kWNDefault = 2;

unsigned slots_per_xcd(int64_t tiles) { return (unsigned)((tiles + kXcd - 1) / kXcd); }

F16Prob gateup_prob(const ExpertArgs& a, const uint16_t* x16, const float* sx, const uint8_t* wq,
                    const float* ws, float* out, int32_t* isum) {
  return F16Prob{a, a.h / (32 * kWNDefault), a.d, 2 * a.h, x16, sx, wq, ws, out, isum};
}

F16Prob down_prob(const ExpertArgs& a, const uint16_t* h16, const float* hs, const uint8_t* wq,
                  const float* ws, float* f, int32_t* isum) {
  ExpertArgs b = a;
  b.perm = nullptr;
  return F16Prob{b, a.d / (64 * kWNDefault), a.h, a.d, h16, hs, wq, ws, f, isum};
}

// The dense problem takes 64-row tiles when 128-row ones would leave it fewer
// workgroups than two per CU (its reduction cannot be split: the group sums
// are added in one fixed order).
template <bool kGateUp>
hipError_t launch_pair(const F16Prob& R, const F16Prob& D, hipStream_t st) {
  const bool d64 = tile_bound(D.a, kBM) * D.nsplit < 512;
  const unsigned per1 = slots_per_xcd(tile_bound(D.a, d64 ? 64 : kBM) * D.nsplit);
  const unsigned per0 = slots_per_xcd(tile_bound(R.a, kBM) * R.nsplit);
  const dim3 grid(kXcd * (per0 + per1)), block(128 * kWNDefault);
  const bool cap = R.isum != nullptr || D.isum != nullptr;
#define MM_F16_PAIR(TM, CAP) \
  hipLaunchKernelGGL((k_w4f16_pair<kWNDefault, TM, kGateUp, CAP>), grid, block, 0, st, R, D, (int)per1)
  if (d64) {
    if (cap) MM_F16_PAIR(64, true); else MM_F16_PAIR(64, false);
  } else {
    if (cap) MM_F16_PAIR(kBM, true); else MM_F16_PAIR(kBM, false);
  }
#undef MM_F16_PAIR
  return hipGetLastError();
}

}  // namespace

bool f16_products_fit(int d, int h, int hs) {
  auto ok = [](int K, int N, int step) { return K > 0 && K % 64 == 0 && N > 0 && N % step == 0; };
  return ok(d, h, 32 * kWNDefault) && ok(d, hs, 32 * kWNDefault) && ok(h, d, 64 * kWNDefault) &&
         ok(hs, d, 64 * kWNDefault);
}

hipError_t launch_gateup_f16_pair(const ExpertArgs& ar, const ExpertArgs& as, const uint16_t* x16,
                                  const float* sx, const uint8_t* wq_r, const float* ws_r,
                                  const uint8_t* wq_s, const float* ws_s, float* abuf_r,
                                  float* abuf_s, int32_t* isum_r, int32_t* isum_s,
                                  hipStream_t st) {
  return launch_pair<true>(gateup_prob(ar, x16, sx, wq_r, ws_r, abuf_r, isum_r),
                           gateup_prob(as, x16, sx, wq_s, ws_s, abuf_s, isum_s), st);
}

hipError_t launch_down_f16_pair(const ExpertArgs& ar, const ExpertArgs& as, const uint16_t* h16_r,
                                const float* hs_r, const uint16_t* h16_s, const float* hs_s,
                                const uint8_t* wq_r, const float* ws_r, const uint8_t* wq_s,
                                const float* ws_s, float* f, float* ys, int32_t* isum_r,
                                int32_t* isum_s, hipStream_t st) {
  return launch_pair<false>(down_prob(ar, h16_r, hs_r, wq_r, ws_r, f, isum_r),
                            down_prob(as, h16_s, hs_s, wq_s, ws_s, ys, isum_s), st);
}

}  // namespace mm
