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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Per-row INT8 code of v given the row scale s (s > 0): clamp(rint(v / s)).
__device__ __forceinline__ int8_t quant_i8(float v, float s) {
  float r = rintf(v / s);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int8_t)(int)r;
}

}  // namespace mm
