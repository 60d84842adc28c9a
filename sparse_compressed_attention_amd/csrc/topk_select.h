// Workgroup-local top-k selection used by the top-k kernels and by the fused
// indexer + top-k kernel: an MSB-first radix select over order-preserving
// uint32 keys held in registers (each thread a contiguous segment), then an
// ordered compaction that emits the selection in ascending position order.
// No locks, no floating-point atomics, deterministic; the order is (key
// desc, position asc), a strict total order.
#pragma once

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {
namespace topk_sel {

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

// BLOCK threads per workgroup (512 or 1024): rows that are few get the
// larger workgroup, so each thread holds and scans half as many keys.
template <int BLOCK>
struct TopkShared {
  static constexpr int kWaves = BLOCK / 64;
  // two histograms: a pass clears the next pass's while it finds its digit
  int hist[2][kBins];
  int wsum[kWaves];
  int sel[4];
  uint32_t red[2][kWaves];
};

// Wave-wide inclusive scans on DPP lane moves (VALU, no LDS round trip):
// shifts by 1, 2, 4 and 8 within each row of 16 lanes (a lane with no
// source adds 0), then the last lane of row 0 added into row 1 and of row 2
// into row 3 (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31).
// Lane 63 ends with the whole wave's result.
__device__ __forceinline__ int wave_inclusive_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}
// Largest value over the wave (unsigned; a lane with no source takes 0,
// which never exceeds its own value)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
// Smallest value over the wave (through the largest complement)
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum of all.  Contains a barrier: every thread must call it, and two
// calls must be separated by another barrier (the per-wave sums are reused).
template <int BLOCK>
__device__ int block_exclusive_scan(int v, TopkShared<BLOCK>& sh, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int x = wave_inclusive_add(v);
  if (lane == 63) sh.wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TopkShared<BLOCK>::kWaves; ++w) {
    const int s = sh.wsum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  *total = tot;
  return before + x - v;
}

// Selection state after the radix passes: keys with (key & pmask) > prefix
// are in, keys with (key & pmask) == prefix are in for the first need_eq of
// them in index order.
struct Sel {
  uint32_t prefix, pmask;
  int need_eq;
};

// K-th largest among the valid keys of the workgroup (1 <= K <= count); bit j
// of `valid` marks key j of this thread's segment.
template <int BLOCK, int SEG>
__device__ Sel radix_select(const uint32_t (&key)[SEG], uint32_t valid, int K, TopkShared<BLOCK>& sh) {
  constexpr int kBpt = kBins / BLOCK;   // histogram bins per thread in the scan
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kBins; i += BLOCK) sh.hist[0][i] = 0;
  // smallest / largest valid key of the workgroup
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    if ((valid >> j) & 1u) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = sh.red[0][0];
  kmax = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < TopkShared<BLOCK>::kWaves; ++w) {
    kmin = min(kmin, sh.red[0][w]);
    kmax = max(kmax, sh.red[1][w]);
  }
  Sel s;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0) {                       // every valid key is the same value
    s.prefix = kmax;
    s.pmask = 0xffffffffu;
    s.need_eq = K;
    return s;
  }
  int top = 31 - __builtin_clz(diff);    // highest differing bit
  s.pmask = top == 31 ? 0u : ~((2u << top) - 1u);
  s.prefix = kmax & s.pmask;
  int rem = K;
  int hb = 0;                            // this pass's histogram (cleared)
  while (true) {
    const int nb = top + 1 < kDigitBits ? top + 1 : kDigitBits;
    const int lo = top - nb + 1;
    const uint32_t dmask = (1u << nb) - 1u;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      if (((valid >> j) & 1u) && (key[j] & s.pmask) == s.prefix) atomicAdd(&sh.hist[hb][(key[j] >> lo) & dmask], 1);
    }
    __syncthreads();
    // thread t owns bins 2047 - kBpt t - i, i < kBpt (descending digit order)
    int c[kBpt];
    int tsum = 0;
#pragma unroll
    for (int i = 0; i < kBpt; ++i) {
      c[i] = sh.hist[hb][kBins - 1 - (kBpt * threadIdx.x + i)];
      tsum += c[i];
    }
    int tot;
    const int before = block_exclusive_scan(tsum, sh, &tot);
    if (before < rem && rem <= before + tsum) {
      int acc = before;
#pragma unroll
      for (int i = 0; i < kBpt; ++i) {
        if (acc < rem && rem <= acc + c[i]) {
          sh.sel[0] = kBins - 1 - (kBpt * threadIdx.x + i);
          sh.sel[1] = acc;
          sh.sel[2] = c[i];
        }
        acc += c[i];
      }
    }
    // the next pass's histogram: its last reads were before this pass's
    // scan barrier
    for (int i = threadIdx.x; i < kBins; i += BLOCK) sh.hist[hb ^ 1][i] = 0;
    __syncthreads();
    // sel is written again only after the next pass's histogram barrier,
    // which every thread reaches after reading it here
    const uint32_t d = (uint32_t)sh.sel[0];
    const int above = sh.sel[1];
    const int in_bin = sh.sel[2];
    hb ^= 1;
    s.prefix |= d << lo;
    s.pmask |= dmask << lo;
    rem -= above;
    if (rem == in_bin || lo == 0) break;   // the whole bin is in, or every bit is fixed
    top = lo - 1;
  }
  s.need_eq = rem;
  return s;
}

// Ordered compaction: out_fn(rank, j) for every selected key j of this
// thread's segment; ranks run 0..K-1 in ascending position.
template <int BLOCK, int SEG, typename OutFn>
__device__ void emit_selected(const uint32_t (&key)[SEG], uint32_t valid, const Sel& s, TopkShared<BLOCK>& sh,
                              OutFn out_fn) {
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    if ((valid >> j) & 1u) {
      const uint32_t m = key[j] & s.pmask;
      gt += m > s.prefix;
      eq += m == s.prefix;
    }
  }
  static_assert(kTopkMaxChunk < 65536 && kTopkMaxCand < 65536, "packed 16-bit counts");
  // one scan of both counts, packed as (gt << 16) | eq: over a workgroup each
  // sum is at most 16384, so the low half never carries into the high half;
  // the keys equal to the prefix are taken in position order, so the ones
  // taken before this thread are min(eq_before, need_eq)
  int tot;
  const int packed = block_exclusive_scan((gt << 16) | eq, sh, &tot);
  const int gt_before = packed >> 16, eq_before = packed & 0xffff;
  const int take_eq = max(0, min(eq, s.need_eq - eq_before));
  int off = gt_before + min(eq_before, s.need_eq);
  int eq_seen = 0;
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    if ((valid >> j) & 1u) {
      const uint32_t m = key[j] & s.pmask;
      bool take = m > s.prefix;
      if (m == s.prefix) {
        take = eq_seen < take_eq;
        ++eq_seen;
      }
      if (take) out_fn(off++, j);
    }
  }
}

}  // namespace topk_sel
}  // namespace csa
