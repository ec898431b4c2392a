// Device-side helpers shared by the libmobmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

constexpr int kWave = 64;
constexpr int kGroup = 32;  // INT4 quantisation group along the reduction dim

// Prepacked INT4 layout (written by k_prepack_int4, read by the expert kernels).
// A [rows][cols] matrix is cut into chunks of 32 rows x 32 columns (one
// quantisation group of 32 output rows).  Chunk (rb, g) is 512 bytes at byte
// offset ((rb * G) + g) * 512, G = cols / 32.  Inside a chunk, "lane" L in
// 0..63 owns 8 bytes at offset L * 8: row rb*32 + (L % 32), columns
// g*32 + 16*(L / 32) + i for i = 0..15.  Those 16 nibbles are stored so that a
// shift/mask unpack yields them in ascending order: in 32-bit word w (0 or 1)
// byte b (0..3) holds column 8w+b in its low nibble and 8w+b+4 in its high
// nibble.  This is the operand order of one wave's B fragment for
// v_mfma_i32_32x32x32_i8 (column = lane % 32, k = 16*(lane/32) + i).
// Scales: FP32 at index (rb * G + g) * 32 + (row % 32), pre-divided by 16
// (the unpack below yields 16 * q).
constexpr int kChunkBytes = 512;

// Unpacks one 32-bit word of 8 prepacked nibbles into two words of four int8
// lanes each, every value multiplied by 16 (exact: 16*q is in [-128, 112]).
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = (w << 4) & 0xF0F0F0F0u;
  hi = w & 0xF0F0F0F0u;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) v = v + __shfl_xor(v, s);
  return v;
}

// DPP lane moves within rows of 16 lanes (gfx9 encodings).
enum : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,   // lane i of each 8 <- lane 7-i
  kDppMirror = 0x140        // lane i of each 16 <- lane 15-i
};

// Every control above reads a lane of the same row, so no source lane is out
// of range; bound_ctrl set lets the compiler fold the move into the VALU
// instruction that uses it (v_add_f32_dpp, v_max_f32_dpp).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Sum of the 64 lanes as a balanced pairwise tree over lane indices: pairs at
// distance 1, 2, 4, 8 (inside each 16-lane row, with DPP moves; after each
// step all lanes of a group hold the same value, so a mirror partner is as
// good as the xor partner), then rows (0+1) and (2+3), then their sum.  Every
// lane returns the same value.  IEEE addition is commutative, so the result
// equals the tree evaluated in any lane order.
__device__ __forceinline__ float tree_sum64(float v) {
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  v = v + dpp<kDppHalfMirror>(v);
  v = v + dpp<kDppMirror>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Maximum over the 64 lanes (exact; order does not matter).
__device__ __forceinline__ float max64(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// e^x, FP32: Cody-Waite reduction x = n*ln2 + r (ln 2 split into a 15-bit head,
// whose product with any |n| <= 128 is exact, and the remainder), then the
// degree-7 Taylor polynomial of e^r in Horner form with fused multiply-adds,
// then scaling by 2^n.  Every step is an IEEE-defined FP32 operation, so any
// implementation of the same steps returns the same bits.  Accurate to about
// 1.3 ulp on [-87.33, 88.72]; +inf above, 0 below.
namespace expc {
constexpr double kLn2 = 0.69314718055994530942;
constexpr float kHi = 0.693145751953125f;  // 11357 / 2^14
constexpr float kLo = (float)(kLn2 - 0.693145751953125);
constexpr float kLog2e = (float)(1.0 / kLn2);
}  // namespace expc

__device__ __forceinline__ float exp_fp32(float x) {
  if (x >= 88.72f) return __builtin_huge_valf();
  if (x <= -87.33f) return 0.0f;
  const float n = rintf(x * expc::kLog2e);
  float r = fmaf(n, -expc::kHi, x);
  r = fmaf(n, -expc::kLo, r);
  float p = 1.0f / 5040.0f;
  p = fmaf(p, r, 1.0f / 720.0f);
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

// SiLU(z) = z * sigmoid(z), written z / (1 + e^-z) with IEEE division.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + exp_fp32(-z)); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Tile lookup for the routed (expert-sorted) layout: expert e owns rows
// [offsets[e], offsets[e+1]) cut into ceil(n_e / rows_per_tile) tiles,
// numbered expert by expert.  Called by all 64 lanes of one wave: lane e
// computes its expert's tile count, an inclusive scan over the lanes gives
// each expert's first tile, and the lane whose range holds tile `mt` writes
// (first row, rows, expert) to *p0, *n, *e; if none does, lane 0 writes n = 0.
// Offsets are clamped to [0, rows] so a corrupt table cannot move a tile out
// of bounds.  E <= 64.
__device__ __forceinline__ void routed_tile(const int32_t* __restrict__ offsets, int E, int rows,
                                            int rows_per_tile, int mt, int* p0, int* n, int* e) {
  const int lane = threadIdx.x & 63;
  int beg = 0, end = 0;
  if (lane < E) {
    beg = min(max(offsets[lane], 0), rows);
    end = min(max(offsets[lane + 1], beg), rows);
  }
  const int nt = (end - beg + rows_per_tile - 1) / rows_per_tile;
  int inc = nt;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int v = __shfl_up(inc, s);
    if (lane >= s) inc += v;
  }
  const int first = inc - nt;
  const bool mine = lane < E && mt >= first && mt < inc;
  const uint64_t owners = __ballot(mine);  // all 64 lanes take part
  if (mine) {
    *p0 = beg + (mt - first) * rows_per_tile;
    *n = min(rows_per_tile, end - *p0);
    *e = lane;
  }
  if (lane == 0 && owners == 0ull) {
    *p0 = 0;
    *n = 0;
    *e = 0;
  }
}

// The routed tile table of a one-wave workgroup, in registers: lane e holds
// expert e's row segment [beg, end) and its tiles [first, inc); total is the
// tile count over all experts (wave-uniform).  All 64 lanes call.
struct RoutedTiles {
  int beg, end, first, inc, total;
};

__device__ __forceinline__ RoutedTiles routed_tiles(const int32_t* __restrict__ offsets, int E,
                                                    int rows, int rows_per_tile) {
  const int lane = threadIdx.x & 63;
  RoutedTiles t{0, 0, 0, 0, 0};
  if (lane < E) {
    t.beg = min(max(offsets[lane], 0), rows);
    t.end = min(max(offsets[lane + 1], t.beg), rows);
  }
  const int nt = (t.end - t.beg + rows_per_tile - 1) / rows_per_tile;
  int inc = nt;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int v = __shfl_up(inc, s);
    if (lane >= s) inc += v;
  }
  t.first = inc - nt;
  t.inc = inc;
  t.total = __builtin_amdgcn_readlane(inc, 63);
  return t;
}

// First row, row count and expert of tile mt from the table (n = 0: no such
// tile), wave-uniform.  All 64 lanes call.
__device__ __forceinline__ void routed_pick(const RoutedTiles& t, int rows_per_tile, int mt,
                                            int& p0, int& n, int& e) {
  const bool mine = mt >= t.first && mt < t.inc;  // lanes >= E: first == inc
  const uint64_t owners = __ballot(mine);
  if (owners == 0ull) {
    p0 = 0;
    n = 0;
    e = 0;
    return;
  }
  const int own = __ffsll((unsigned long long)owners) - 1;
  const int my_p0 = t.beg + (mt - t.first) * rows_per_tile;
  p0 = __builtin_amdgcn_readlane(my_p0, own);
  n = min(rows_per_tile, __builtin_amdgcn_readlane(t.end, own) - p0);
  e = own;
}

// routed_tile for a one-wave workgroup: the same lookup, with the result
// returned wave-uniform in registers (n = 0: no such tile).  All 64 lanes call.
__device__ __forceinline__ void routed_tile_wave(const int32_t* __restrict__ offsets, int E,
                                                 int rows, int rows_per_tile, int mt, int& p0,
                                                 int& n, int& e) {
  routed_pick(routed_tiles(offsets, E, rows, rows_per_tile), rows_per_tile, mt, p0, n, e);
}

// INT8 activation matrices [R][C] are row-major, or, inside the one-call
// layer where the matrix-core kernels read them, group-major: the 32 codes of
// (row r, group g = c / 32) at byte (g * R + r) * 32 + c % 32, so that the 32
// rows of one MFMA tile and one group are 1 KB of contiguous memory.  Byte
// offset of (r, c); gm_rows = R for group-major, 0 for row-major.
__device__ __forceinline__ int64_t act_offset(int64_t r, int64_t c, int64_t cols, int64_t gm_rows) {
  return gm_rows ? ((c >> 5) * gm_rows + r) * 32 + (c & 31) : r * cols + c;
}

// F16 paired activation codes, the operand form of the f16 matrix-core
// products (k_w4f16.hip): a row-major [R][C] matrix of 16-bit values in which
// each aligned block of 8 columns is reordered -- column c of the block
// (0..7) sits at slot (c odd ? 4 + c/2 : c/2) -- and column c holds its INT8
// code as an f16 value, divided by 16 for c >= 4 (exact: at most 8
// significant bits).  This matches the order in which those kernels unpack the
// prepacked INT4 weights (two nibbles per 32-bit operand, the high nibbles of
// a byte scaled by 16), so the product of each pair is exactly code * weight.
// Passed as gm_rows = kF16Paired where a quantiser takes a layout.
constexpr int64_t kF16Paired = -1;

__device__ __forceinline__ int64_t f16p_index(int64_t r, int64_t c, int64_t cols) {
  const int cc = (int)(c & 7);
  return r * cols + (c & ~(int64_t)7) + ((cc & 1) ? 4 + (cc >> 1) : (cc >> 1));
}

__device__ __forceinline__ uint16_t f16p_value(int code, int64_t c) {
  const float v = (c & 4) ? (float)code * 0.0625f : (float)code;
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Stores one INT8 code in the layout gm_rows names: 0 row-major int8, > 0
// group-major int8 (that many rows), kF16Paired f16 paired (q is then a
// buffer of 2 * R * C bytes).
__device__ __forceinline__ void store_code(void* q, int64_t r, int64_t c, int64_t cols,
                                           int64_t gm_rows, int code) {
  if (gm_rows == kF16Paired)
    static_cast<uint16_t*>(q)[f16p_index(r, c, cols)] = f16p_value(code, c);
  else
    static_cast<int8_t*>(q)[act_offset(r, c, cols, gm_rows)] = (int8_t)code;
}

// Per-row INT8 code of v given the row scale s (s > 0): clamp(rint(v / s)).
__device__ __forceinline__ int8_t quant_i8(float v, float s) {
  float r = rintf(v / s);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int8_t)(int)r;
}

// The same code without a division per element.  y = quant_recip(s), once
// per row: the hardware reciprocal (within 1 ulp of 1/s), or NaN for tiny s.
// With |v| <= amax, |v / s| <= 127.5, so t = v * y differs from the rounded
// quotient fl(v / s) by less than 4e-5 (1 ulp of 1/s and two roundings, each
// relative 2^-23 or less, at most 128 in size).  Unless t lies within 2^-12
// of a half-integer, both are then strictly inside the same interval
// (k - 1/2, k + 1/2) and round to the same k; in that window (and for NaN
// y) the IEEE quotient is taken instead.  Codes are thus identical to
// quant_i8(v, s).
__device__ __forceinline__ float quant_recip(float s) {
  return s >= 0x1p-100f ? __builtin_amdgcn_rcpf(s) : __builtin_nanf("");
}
__device__ __forceinline__ int8_t quant_i8(float v, float s, float y) {
  const float t = v * y;
  float r = rintf(t);
  if (!(fabsf(t - r) < 0.5f - 0x1p-12f)) r = rintf(v / s);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int8_t)(int)r;
}

// Branch-free INT8 code of v with y = quant_recip(s): quant_i8's fast case;
// slow becomes true where quant_i8 would take its exact division instead.
__device__ __forceinline__ int quant_code_fast(float v, float y, bool& slow) {
  const float t = v * y;
  const float r = rintf(t);
  slow |= !(fabsf(t - r) < 0.5f - 0x1p-12f);
  return (int)fminf(fmaxf(r, -128.0f), 127.0f);
}

}  // namespace mm
