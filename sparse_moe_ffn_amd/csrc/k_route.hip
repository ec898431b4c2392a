// Stable count sort of the T*k (token, slot) assignments by expert id.
//
// MobileMoE close reading, section "Custom MoE kernel": tokens are reordered
// by their assigned expert with a counting sort so that each expert's tokens
// are contiguous and each expert runs one batched product on its slice.
// Inference routing is dropless (section "Supervised fine-tuning").
//
// Up to kOneMax slots: one workgroup does it all (k_route_one, below); past
// that, one workgroup's scattered writes take longer than a second launch.
// Beyond that, two kernels, no host synchronisation and no order-dependent
// atomics:
//   k_route_count    one workgroup per block of 256 slots: per-expert counts
//                    of the block (integer LDS atomics; the result does not
//                    depend on their order) -> ws[block][E].
//   k_route_scatter  one workgroup per block: sums the counts of all earlier
//                    blocks per expert and of all blocks (for the offsets),
//                    then ranks each slot among the equal ids of its block in
//                    slot order and writes perm / inv_perm.  Block 0 also
//                    writes expert_offsets.
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

constexpr int kBlockSlots = 256;

__global__ __launch_bounds__(kBlockSlots) void k_route_count(int64_t Tk, int E,
                                                             const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ counts) {
  __shared__ int cnt[64];
  const int tid = threadIdx.x;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  const int64_t slot = (int64_t)blockIdx.x * kBlockSlots + tid;
  if (slot < Tk) {
    const int e = idx[slot];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < E) counts[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

// Sources of the per-expert counts of the earlier blocks and of all blocks:
// kCounts the table of k_route_count; kSingle none (the whole table fits one
// block, T*k <= 256, decode batches: the block counts its own slots); kHist
// the router's per-workgroup counts (4 tokens, 4k slots each; bytes
// hist[e * hstride + b], b < nrb; rpb router workgroups per block), so no
// counting kernel runs.
enum { kCounts = 0, kSingle = 1, kHist = 2 };

// Sum of the first `lim` of the 16 byte counts in wd (all 16 when lim >= 16,
// none when lim <= 0).  lim is the same on every lane of the wave.
__device__ __forceinline__ int hist_piece_sum(const uint32_t (&wd)[4], int64_t lim) {
  if (lim <= 0) return 0;
  int sum = 0;
  if (lim >= 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sum = (int)__builtin_amdgcn_udot4(wd[i], 0x01010101u, (uint32_t)sum, false);
    return sum;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t l = lim - 4 * i;  // bytes of word i below the limit
    const uint32_t m = l >= 4 ? 0xFFFFFFFFu : l <= 0 ? 0u : (1u << (8 * (int)l)) - 1u;
    sum = (int)__builtin_amdgcn_udot4(wd[i] & m, 0x01010101u, (uint32_t)sum, false);
  }
  return sum;
}

template <int kMode>
__global__ __launch_bounds__(kBlockSlots) void k_route_scatter(
    int64_t Tk, int E, int64_t nblk, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    const uint8_t* __restrict__ hist = nullptr, int64_t nrb = 0, int64_t hstride = 0,
    int rpb = 0) {
  __shared__ int part_before[4][64];
  __shared__ int part_total[4][64];
  __shared__ int base[64];    // offsets[e] + count of e in earlier blocks
  __shared__ int wcnt[4][64];  // count of e in each wave of this block
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t blk = blockIdx.x;
  // this thread's slot id, read first so that its latency overlaps the counts
  const int64_t slot = blk * kBlockSlots + tid;
  const int eraw = slot < Tk ? idx[slot] : -1;

  if constexpr (kMode == kSingle) {
    part_before[wv][lane] = 0;
    part_total[wv][lane] = 0;
    wcnt[wv][lane] = 0;
    __syncthreads();
    if (tid < Tk) {
      const int e = idx[tid];
      if ((unsigned)e < (unsigned)E) atomicAdd(&part_total[0][e], 1);
    }
  } else if constexpr (kMode == kHist) {
    // expert `lane`, quarter `wv` of the router workgroups, 16 bytes a load
    // (hstride % 64 == 0; bytes past nrb are not counted)
    // The loads of a batch of kHistBatch 16-byte pieces are all issued
    // before any is summed, so a lane pays one memory round trip per batch
    // instead of one per piece.  A piece's block indices are the same for
    // every lane (only the expert row differs), so whether a piece lies
    // wholly below a limit is a wave-uniform test; only a piece that
    // straddles one is masked byte by byte.
    constexpr int kHistBatch = 8;
    int before = 0, total = 0;
    if (lane < E) {
      const int64_t q = hstride / 4, b0 = wv * q, bend = blk * rpb;  // router blocks before this block
      const int64_t npiece = q / 16;
      const uint4* row = reinterpret_cast<const uint4*>(hist + (int64_t)lane * hstride + b0);
      for (int64_t c0 = 0; c0 < npiece; c0 += kHistBatch) {
        uint4 v[kHistBatch];
#pragma unroll
        for (int j = 0; j < kHistBatch; ++j)
          v[j] = c0 + j < npiece ? row[c0 + j] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < kHistBatch; ++j) {
          const int64_t pb = b0 + 16 * (c0 + j);  // block index of the piece's first byte
          const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
          total += hist_piece_sum(wd, nrb - pb);
          before += hist_piece_sum(wd, bend - pb);
        }
      }
    }
    part_before[wv][lane] = before;
    part_total[wv][lane] = total;
    wcnt[wv][lane] = 0;
  } else {
    // Per-expert sums over blocks: 4 threads per expert, interleaved blocks.
    int before = 0, total = 0;
    if (lane < E) {
      for (int64_t b = wv; b < nblk; b += 4) {
        const int c = counts[b * E + lane];
        total += c;
        if (b < blk) before += c;
      }
    }
    part_before[wv][lane] = before;
    part_total[wv][lane] = total;
    wcnt[wv][lane] = 0;
  }
  __syncthreads();
  // Expert offsets: exclusive scan of the totals over the experts (one lane
  // per expert, E <= 64), then each expert's base for this block.
  if (tid < 64) {
    const int e = tid;
    int tot = 0, bef = 0;
    if (e < E) {
      tot = part_total[0][e] + part_total[1][e] + part_total[2][e] + part_total[3][e];
      bef = part_before[0][e] + part_before[1][e] + part_before[2][e] + part_before[3][e];
    }
    int inc = tot;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int v = __shfl_up(inc, s);
      if (lane >= s) inc += v;
    }
    const int excl = inc - tot;
    if (e < E) {
      if (blk == 0) offsets[e] = excl;
      base[e] = excl + bef;
      if (blk == 0 && e == E - 1) offsets[E] = inc;
    }
  }

  // Rank inside the wave: the lanes holding the same id are found with one
  // ballot per id bit (ids < 64).
  const bool valid = (unsigned)eraw < (unsigned)E;  // out-of-range ids are skipped
  const int e = valid ? eraw : 0;
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t ones = __ballot(valid && ((e >> b) & 1));
    same &= ((e >> b) & 1) ? ones : ~ones;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & below);
  if (valid && rank == 0) wcnt[wv][e] = __popcll(same);
  __syncthreads();
  if (valid) {
    int pos = base[e] + rank;
    for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
    perm[pos] = (int32_t)slot;
    inv_perm[slot] = pos;
  }
}

// Whole table in one workgroup of 16 waves.  Wave w owns the contiguous
// chunk [w * C, (w + 1) * C) of slots and walks it in rounds of 64: the lanes
// of a round holding the same id are found with one ballot per id bit, so a
// slot's rank among equal ids of earlier lanes is a popcount and the round's
// count per id is added by the lowest such lane (no atomics).  Pass 1 gives
// each wave's count per id; from those, one wave forms the expert offsets and
// each wave's base per id (offset + counts of the earlier waves); pass 2 walks
// the chunk again and writes perm / inv_perm.  The ids stay in registers
// between the passes.
constexpr int kOneWaves = 16;
constexpr int kOneRounds = 2;  // rounds per wave: up to 16 * 64 * 2 slots
constexpr int64_t kOneMax = (int64_t)kOneWaves * 64 * kOneRounds;

__global__ __launch_bounds__(64 * kOneWaves) void k_route_one(int64_t Tk, int E,
                                                              const int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm) {
  __shared__ int wc[kOneWaves][64];  // pass 1: count per (wave, id); then base per (wave, id)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int C = (int)((Tk + kOneWaves * 64 - 1) / (kOneWaves * 64)) * 64;  // chunk, multiple of 64
  const int rounds = C / 64;
  const int64_t c0 = (int64_t)wv * C;
  wc[wv][lane] = 0;
  int ev[kOneRounds];
#pragma unroll
  for (int r = 0; r < kOneRounds; ++r) {
    ev[r] = -1;
    const int64_t slot = c0 + r * 64 + lane;
    if (r < rounds && slot < Tk) ev[r] = idx[slot];
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto same_of = [&](int eraw, bool& valid, int& e) {
    valid = (unsigned)eraw < (unsigned)E;  // out-of-range ids are skipped
    e = valid ? eraw : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? ones : ~ones;
    }
    return same;
  };
  // wc[wv][.] is written by this wave only, in program order: no barrier
  // is needed between its rounds.
#pragma unroll
  for (int r = 0; r < kOneRounds; ++r) {
    if (r >= rounds) break;
    bool valid;
    int e;
    const uint64_t same = same_of(ev[r], valid, e);
    if (valid && __popcll(same & below) == 0) wc[wv][e] += __popcll(same);
  }
  __syncthreads();
  if (wv == 0) {  // lane e: offsets and per-wave bases of id e
    int tot = 0;
    if (lane < E)
      for (int w = 0; w < kOneWaves; ++w) tot += wc[w][lane];
    int inc = tot;
#pragma unroll
    for (int s2 = 1; s2 < 64; s2 <<= 1) {
      const int v = __shfl_up(inc, s2);
      if (lane >= s2) inc += v;
    }
    int base = inc - tot;
    if (lane < E) {
      offsets[lane] = base;
      if (lane == E - 1) offsets[E] = inc;
      for (int w = 0; w < kOneWaves; ++w) {
        const int c = wc[w][lane];
        wc[w][lane] = base;
        base += c;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kOneRounds; ++r) {
    if (r >= rounds) break;
    bool valid;
    int e;
    const uint64_t same = same_of(ev[r], valid, e);
    const int rank = __popcll(same & below);
    int pos = 0;
    if (valid) pos = wc[wv][e] + rank;
    if (valid && rank == 0) wc[wv][e] += __popcll(same);  // after every lane read its base
    if (valid) {
      const int64_t slot = c0 + r * 64 + lane;
      perm[pos] = (int32_t)slot;
      inv_perm[slot] = pos;
    }
  }
}

}  // namespace

int64_t route_blocks(int64_t Tk) { return (Tk + kBlockSlots - 1) / kBlockSlots; }

hipError_t launch_route(int64_t Tk, int E, const int32_t* idx, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, int32_t* ws, hipStream_t st) {
  const int64_t nblk = route_blocks(Tk);
  if (nblk > 1 && Tk <= kOneMax) {
    hipLaunchKernelGGL(k_route_one, dim3(1), dim3(64 * kOneWaves), 0, st, Tk, E, idx, offsets, perm,
                       inv_perm);
    return hipGetLastError();
  }
  if (nblk == 1) {
    hipLaunchKernelGGL(k_route_scatter<kSingle>, dim3(1), dim3(kBlockSlots), 0, st, Tk, E, nblk, idx,
                       ws, offsets, perm, inv_perm, nullptr, 0, 0, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_route_count, dim3((unsigned)nblk), dim3(kBlockSlots), 0, st, Tk, E, idx, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_route_scatter<kCounts>, dim3((unsigned)nblk), dim3(kBlockSlots), 0, st, Tk, E,
                     nblk, idx, ws, offsets, perm, inv_perm, nullptr, 0, 0, 0);
  return hipGetLastError();
}

int64_t route_hist_stride(int64_t T) { return ((T + 3) / 4 + 63) / 64 * 64; }

// Where launch_route would run the two-kernel sort and the router writes
// the histogram (more than 64 tokens: the 4-token router form).
bool route_hist_applies(int64_t T, int k) {
  return T > 64 && T * k > kOneMax && kBlockSlots % (4 * k) == 0;
}

hipError_t launch_route_hist(int64_t T, int k, int E, const int32_t* idx, const uint8_t* hist,
                             int32_t* offsets, int32_t* perm, int32_t* inv_perm, hipStream_t st) {
  const int64_t Tk = T * k, nblk = route_blocks(Tk);
  if (kBlockSlots % (4 * k) != 0) return hipErrorInvalidValue;
  const int rpb = kBlockSlots / (4 * k);  // 4-token router workgroups per block of slots
  hipLaunchKernelGGL(k_route_scatter<kHist>, dim3((unsigned)nblk), dim3(kBlockSlots), 0, st, Tk, E,
                     nblk, idx, nullptr, offsets, perm, inv_perm, hist, (T + 3) / 4,
                     route_hist_stride(T), rpb);
  return hipGetLastError();
}

}  // namespace mm
