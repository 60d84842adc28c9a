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
//  * stage 1: one workgroup per (row, chunk of <= 16384 entries) copies its
//    chunk into LDS and finds the chunk's k-th key by an MSB-first radix
//    select (8-bit digits, LDS histograms with integer atomics, one wave
//    scanning the 256 bins);
//  * an ordered compaction (two workgroup prefix sums over contiguous
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

__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int s = sh[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Finds the K-th largest key (1 <= K <= number of valid keys) among keys[0,n)
// whose valid flag holds (valid == nullptr: all).  Returns the key and how
// many keys equal to it belong to the top K.
__device__ void radix_select(const uint32_t* keys, const int32_t* valid, int n, int K, int* hist,
                             int* misc, uint32_t* kth, int* need_eq) {
  uint32_t prefix = 0, pmask = 0;
  int rem = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kTopkBlock) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kTopkBlock) {
      if (valid && valid[i] < 0) continue;
      const uint32_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int c[4];
      int s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        s += c[j];
      }
      int x = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const int before = x - s;   // keys whose digit is above this lane's digits
      if (before < rem && rem <= x) {
        int acc = before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < rem && rem <= acc + c[j]) {
            misc[0] = 255 - 4 * lane - j;
            misc[1] = acc;
          }
          acc += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    pmask |= 0xffu << shift;
    rem -= misc[1];
    __syncthreads();
  }
  *kth = prefix;
  *need_eq = rem;
}

// Ordered compaction of the selection: out_fn(rank, i) for every selected i,
// ranks 0..K-1 in ascending i.
template <typename OutFn>
__device__ void emit_selected(const uint32_t* keys, const int32_t* valid, int n, uint32_t kth, int need_eq,
                              int* shscan, OutFn out_fn) {
  const int seg = (n + kTopkBlock - 1) / kTopkBlock;
  const int i0 = min(n, (int)threadIdx.x * seg);
  const int i1 = min(n, i0 + seg);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    if (valid && valid[i] < 0) continue;
    const uint32_t key = keys[i];
    gt += key > kth;
    eq += key == kth;
  }
  int tot;
  const int eq_before = block_exclusive_scan(eq, shscan, &tot);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  int off = block_exclusive_scan(gt + take_eq, shscan, &tot);
  int eq_seen = 0;
  for (int i = i0; i < i1; ++i) {
    if (valid && valid[i] < 0) continue;
    const uint32_t key = keys[i];
    bool take = key > kth;
    if (key == kth) {
      take = eq_seen < take_eq;
      ++eq_seen;
    }
    if (take) out_fn(off++, i);
  }
}

__global__ __launch_bounds__(kTopkBlock) void topk_chunk_kernel(TopkParams p) {
  extern __shared__ uint32_t skeys[];
  __shared__ int hist[256];
  __shared__ int misc[2];
  __shared__ int shscan[kTopkWaves];
  const int t = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x - t * p.n_chunks;
  const int nv = (int)max<int64_t>(0, min<int64_t>(p.n_visible[t], p.ld));
  const int c0 = ch * p.chunk;
  const int n = max(0, min(nv - c0, p.chunk));
  const float* src = p.scores + (size_t)t * p.ld + c0;
  for (int i = threadIdx.x; i < n; i += kTopkBlock) skeys[i] = float_order_key(src[i]);
  __syncthreads();
  const int K = min(p.k, n);
  if (p.n_chunks == 1) {
    int32_t* o = p.out + (size_t)t * p.k;
    if (K > 0) {
      uint32_t kth;
      int need_eq;
      radix_select(skeys, nullptr, n, K, hist, misc, &kth, &need_eq);
      emit_selected(skeys, nullptr, n, kth, need_eq, shscan, [&](int rank, int i) {
        if (rank < K) o[rank] = c0 + i;
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) o[i] = -1;
  } else {
    const size_t base = ((size_t)t * p.n_chunks + ch) * p.k;
    uint32_t* ck = p.cand_key + base;
    int32_t* ci = p.cand_idx + base;
    if (K > 0) {
      uint32_t kth;
      int need_eq;
      radix_select(skeys, nullptr, n, K, hist, misc, &kth, &need_eq);
      emit_selected(skeys, nullptr, n, kth, need_eq, shscan, [&](int rank, int i) {
        if (rank < K) {
          ck[rank] = skeys[i];
          ci[rank] = c0 + i;
        }
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) {
      ck[i] = 0u;
      ci[i] = -1;
    }
  }
}

__global__ __launch_bounds__(kTopkBlock) void topk_merge_kernel(TopkParams p) {
  extern __shared__ uint32_t smem[];
  __shared__ int hist[256];
  __shared__ int misc[2];
  __shared__ int shscan[kTopkWaves];
  const int t = blockIdx.x;
  const int ncand = p.n_chunks * p.k;
  uint32_t* keys = smem;
  int32_t* idx = reinterpret_cast<int32_t*>(smem + ncand);
  const size_t base = (size_t)t * ncand;
  for (int i = threadIdx.x; i < ncand; i += kTopkBlock) {
    keys[i] = p.cand_key[base + i];
    idx[i] = p.cand_idx[base + i];
  }
  const int nv = (int)max<int64_t>(0, min<int64_t>(p.n_visible[t], p.ld));
  int nvalid = 0;
  for (int ch = 0; ch < p.n_chunks; ++ch) nvalid += min(p.k, max(0, min(nv - ch * p.chunk, p.chunk)));
  __syncthreads();
  const int K = min(p.k, nvalid);
  int32_t* o = p.out + (size_t)t * p.k;
  if (K > 0) {
    uint32_t kth;
    int need_eq;
    radix_select(keys, idx, ncand, K, hist, misc, &kth, &need_eq);
    emit_selected(keys, idx, ncand, kth, need_eq, shscan, [&](int rank, int i) {
      if (rank < K) o[rank] = idx[i];
    });
  }
  for (int i = K + threadIdx.x; i < p.k; i += kTopkBlock) o[i] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_merge_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 8 * kTopkMaxCand);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds1 = (size_t)p.chunk * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(p.T * p.n_chunks), dim3(kTopkBlock), lds1, stream, p);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess || p.n_chunks == 1) return e;
  const size_t lds2 = (size_t)p.n_chunks * p.k * 8;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(p.T), dim3(kTopkBlock), lds2, stream, p);
  return hipPeekAtLastError();
}

}  // namespace csa
