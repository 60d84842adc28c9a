// Step 2 of the CSA path: per-query causal top-k over the indexer scores.
//
// "DSV4 Audit -- Decode Repetition + Precision / Tensor-Core Plan", B2 and
// "ROADMAP -- Stage E ...", E7: the top-k over indexer scores must be a
// warp/wave-local reduction with no global lock (a serial single-thread heap
// merge at top_k = 1024 was a latency source).
//
// Design (no locks, no floating-point atomics, deterministic):
//  * scores become order-preserving uint32 keys; ties are broken by the lower
//    index, which gives a strict total order (key desc, index asc);
//  * stage 1: one workgroup (512 threads) per (row, chunk of <= 16384
//    entries).  Every thread keeps a contiguous segment of SEG keys in
//    registers.  An MSB-first radix select finds the chunk's k-th key: it
//    starts at the highest bit where the chunk's smallest and largest keys
//    differ (the bits above are shared by every key, and starting there
//    spreads the first histogram instead of piling the whole chunk into one
//    or two bins), uses 11-bit digits with 2048-bin LDS histograms filled by
//    integer atomics, finds the digit with a workgroup prefix sum over the
//    bins, and stops as soon as the selected bin holds exactly the keys still
//    needed;
//  * an ordered compaction (two workgroup prefix sums over the contiguous
//    per-thread segments) emits the chunk's selection in ascending index
//    order -- the final answer when the row fits one chunk, else the chunk's
//    candidates (key, index);
//  * stage 2 (long rows only): one workgroup per row repeats the selection
//    over the concatenated candidates.  The global top-k is contained in the
//    union of the chunks' top-k under the same total order, so the merge is
//    exact.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

constexpr int kTopkBlock = 512;
constexpr int kTopkWaves = kTopkBlock / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

struct TopkShared {
  int hist[kBins];
  int wsum[kTopkWaves];
  int sel[4];
  uint32_t red[2][kTopkWaves];
};

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum of all.  Contains barriers: every thread must call it.
__device__ int block_exclusive_scan(int v, TopkShared& sh, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh.wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int s = sh.wsum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
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
template <int SEG>
__device__ Sel radix_select(const uint32_t (&key)[SEG], uint32_t valid, int K, TopkShared& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // smallest / largest valid key of the workgroup
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    if ((valid >> j) & 1u) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
  }
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = sh.red[0][0];
  kmax = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) {
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
  while (true) {
    const int nb = top + 1 < kDigitBits ? top + 1 : kDigitBits;
    const int lo = top - nb + 1;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kTopkBlock) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      if (((valid >> j) & 1u) && (key[j] & s.pmask) == s.prefix) atomicAdd(&sh.hist[(key[j] >> lo) & dmask], 1);
    }
    __syncthreads();
    // thread t owns bins 2047-4t .. 2044-4t (descending digit order)
    int c[4];
    int tsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = sh.hist[kBins - 1 - (4 * threadIdx.x + i)];
      tsum += c[i];
    }
    int tot;
    const int before = block_exclusive_scan(tsum, sh, &tot);
    if (before < rem && rem <= before + tsum) {
      int acc = before;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc < rem && rem <= acc + c[i]) {
          sh.sel[0] = kBins - 1 - (4 * threadIdx.x + i);
          sh.sel[1] = acc;
          sh.sel[2] = c[i];
        }
        acc += c[i];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh.sel[0];
    const int above = sh.sel[1];
    const int in_bin = sh.sel[2];
    __syncthreads();
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
template <int SEG, typename OutFn>
__device__ void emit_selected(const uint32_t (&key)[SEG], uint32_t valid, const Sel& s, TopkShared& sh,
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
  int tot;
  const int eq_before = block_exclusive_scan(eq, sh, &tot);
  const int take_eq = max(0, min(eq, s.need_eq - eq_before));
  int off = block_exclusive_scan(gt + take_eq, sh, &tot);
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

template <int SEG>
__global__ __launch_bounds__(kTopkBlock) void topk_chunk_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const int t = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x - t * p.n_chunks;
  const int nv = (int)max<int64_t>(0, min<int64_t>(p.n_visible[t], p.ld));
  const int c0 = ch * p.chunk;
  const int n = max(0, min(nv - c0, p.chunk));
  const int i0 = threadIdx.x * SEG;
  const int cnt = max(0, min(SEG, n - i0));
  const float* src = p.scores + (size_t)t * p.ld + c0 + i0;
  uint32_t key[SEG];
  if (cnt == SEG && ((((uintptr_t)src) & 15) == 0)) {
    // whole segment: 16-byte loads
#pragma unroll
    for (int j = 0; j < SEG; j += 4) {
      const v4f v = *reinterpret_cast<const v4f*>(src + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j + e] = float_order_key(v[e]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < SEG; ++j) key[j] = j < cnt ? float_order_key(src[j]) : 0u;
  }
  const uint32_t valid = cnt >= 32 ? 0xffffffffu : ((1u << cnt) - 1u);
  const int K = min(p.k, n);
  if (p.n_chunks == 1) {
    int32_t* o = p.out + (size_t)t * p.k;
    if (K > 0) {
      const Sel s = radix_select<SEG>(key, valid, K, sh);
      emit_selected<SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) o[rank] = c0 + i0 + j;
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) o[i] = -1;
  } else {
    const size_t base = ((size_t)t * p.n_chunks + ch) * p.k;
    uint32_t* ck = p.cand_key + base;
    int32_t* ci = p.cand_idx + base;
    if (K > 0) {
      const Sel s = radix_select<SEG>(key, valid, K, sh);
      emit_selected<SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) {
          ck[rank] = key[j];
          ci[rank] = c0 + i0 + j;
        }
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) {
      ck[i] = 0u;
      ci[i] = -1;
    }
  }
}

// Candidates of a row arrive in chunk order and ascending index within each
// chunk, so position order is index order; empty slots (index -1) are masked.
template <int SEG>
__global__ __launch_bounds__(kTopkBlock) void topk_merge_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const int t = blockIdx.x;
  const int ncand = p.n_chunks * p.k;
  const int i0 = threadIdx.x * SEG;
  const size_t base = (size_t)t * ncand;
  uint32_t key[SEG];
  int32_t idx[SEG];
  uint32_t valid = 0u;
  const uint32_t* ksrc = p.cand_key + base + i0;
  const int32_t* isrc = p.cand_idx + base + i0;
  if (i0 + SEG <= ncand && ((((uintptr_t)ksrc) | ((uintptr_t)isrc)) & 15) == 0) {
    // whole segment: 16-byte loads
#pragma unroll
    for (int j = 0; j < SEG; j += 4) {
      const v4i kv = *reinterpret_cast<const v4i*>(ksrc + j);
      const v4i iv = *reinterpret_cast<const v4i*>(isrc + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[j + e] = (uint32_t)kv[e];
        idx[j + e] = iv[e];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      key[j] = 0u;
      idx[j] = -1;
      if (i0 + j < ncand) {
        key[j] = ksrc[j];
        idx[j] = isrc[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < SEG; ++j) valid |= (idx[j] >= 0 ? 1u : 0u) << j;
  int total;
  block_exclusive_scan(__builtin_popcount(valid), sh, &total);
  const int K = min(p.k, total);
  int32_t* o = p.out + (size_t)t * p.k;
  if (K > 0) {
    const Sel s = radix_select<SEG>(key, valid, K, sh);
    emit_selected<SEG>(key, valid, s, sh, [&](int rank, int j) {
      if (rank < K) o[rank] = idx[j];
    });
  }
  for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) o[i] = -1;
}

template <int SEG>
hipError_t launch_chunk(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(topk_chunk_kernel<SEG>, dim3(p.T * p.n_chunks), dim3(kTopkBlock), 0, stream, p);
  return hipPeekAtLastError();
}
template <int SEG>
hipError_t launch_merge(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(topk_merge_kernel<SEG>, dim3(p.T), dim3(kTopkBlock), 0, stream, p);
  return hipPeekAtLastError();
}

int seg_for(int n) {
  const int per = (n + kTopkBlock - 1) / kTopkBlock;
  return per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : 32;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  hipError_t e;
  switch (seg_for(p.chunk)) {
    case 4: e = launch_chunk<4>(p, stream); break;
    case 8: e = launch_chunk<8>(p, stream); break;
    case 16: e = launch_chunk<16>(p, stream); break;
    default: e = launch_chunk<32>(p, stream); break;
  }
  if (e != hipSuccess || p.n_chunks == 1) return e;
  switch (seg_for(p.n_chunks * p.k)) {
    case 4: return launch_merge<4>(p, stream);
    case 8: return launch_merge<8>(p, stream);
    case 16: return launch_merge<16>(p, stream);
    default: return launch_merge<32>(p, stream);
  }
}

}  // namespace csa
