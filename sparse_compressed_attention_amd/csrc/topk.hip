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
//  * stage 1: one workgroup (512 threads, or 1024 when rows x chunks are
//    fewer than the CUs) per (row, chunk of <= 16384 entries).  Every thread keeps a contiguous segment of SEG keys in
//    registers.  An MSB-first radix select finds the chunk's k-th key: it
//    starts at the highest bit where the chunk's smallest and largest keys
//    differ (the bits above are shared by every key, and starting there
//    spreads the first histogram instead of piling the whole chunk into one
//    or two bins), uses 11-bit digits with 2048-bin LDS histograms filled by
//    integer atomics, finds the digit with a workgroup prefix sum over the
//    bins, and stops as soon as the selected bin holds exactly the keys still
//    needed;
//  * an ordered compaction (one workgroup prefix sum over the contiguous
//    per-thread segments, of the counts above and equal to the threshold
//    packed in one word) emits the chunk's selection in ascending index
//    order -- the final answer when the row fits one chunk, else the chunk's
//    candidates (key, index);
//  * stage 2 (long rows only): one workgroup per row repeats the selection
//    over the concatenated candidates.  The global top-k is contained in the
//    union of the chunks' top-k under the same total order, so the merge is
//    exact.
#include "csa_device.h"
#include "csa_internal.h"
#include "topk_select.h"

namespace csa {

namespace {

using namespace topk_sel;

// (launch bounds: at least six waves per SIMD, three 512-thread workgroups
// per CU; at 32 keys per thread that caps a wave at 80 registers, and the
// few it spills cost less than the lost occupancy would)
template <int BLOCK, int SEG>
__global__ __launch_bounds__(BLOCK, 6) void topk_chunk_kernel(TopkParams p) {
  __shared__ TopkShared<BLOCK> sh;
  const int t = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x - t * p.n_chunks;
  const int nv_raw = p.n_visible[t];   // in flight together with the scores
  const int c0 = ch * p.chunk;
  const int i0 = threadIdx.x * SEG;
  // The scores are read without waiting for the visible count: a thread
  // loads the part of its segment that lies inside the row's allocated
  // columns [0, ld); columns past the visible count are masked below and
  // never used.
  const int avail = (int)max<int64_t>(0, min<int64_t>(SEG, min<int64_t>(p.ld - c0, p.chunk) - i0));
  const float* src = p.scores + (size_t)t * p.ld + c0 + i0;
  uint32_t key[SEG];
  if (avail == SEG && ((((uintptr_t)src) & 15) == 0)) {
    // whole segment: 16-byte loads
#pragma unroll
    for (int j = 0; j < SEG; j += 4) {
      const v4f v = *reinterpret_cast<const v4f*>(src + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j + e] = float_order_key(v[e]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < SEG; ++j) key[j] = j < avail ? float_order_key(src[j]) : 0u;
  }
  const int nv = (int)max<int64_t>(0, min<int64_t>(nv_raw, p.ld));
  const int n = max(0, min(nv - c0, p.chunk));
  const int cnt = max(0, min(SEG, n - i0));
  const uint32_t valid = cnt >= 32 ? 0xffffffffu : ((1u << cnt) - 1u);
  const int K = min(p.k, n);
  if (p.n_chunks == 1) {
    int32_t* o = p.out + (size_t)t * p.k;
    if (K > 0) {
      const Sel s = radix_select<BLOCK, SEG>(key, valid, K, sh);
      emit_selected<BLOCK, SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) o[rank] = c0 + i0 + j;
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += BLOCK) o[i] = -1;
  } else {
    const size_t base = ((size_t)t * p.n_chunks + ch) * p.k;
    uint32_t* ck = p.cand_key + base;
    int32_t* ci = p.cand_idx + base;
    if (K > 0) {
      const Sel s = radix_select<BLOCK, SEG>(key, valid, K, sh);
      emit_selected<BLOCK, SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) {
          ck[rank] = key[j];
          ci[rank] = c0 + i0 + j;
        }
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += BLOCK) {
      ck[i] = 0u;
      ci[i] = -1;
    }
  }
}

// Candidates of a row arrive in chunk order and ascending index within each
// chunk, so position order is index order; empty slots (index -1) are masked.
template <int BLOCK, int SEG>
__global__ __launch_bounds__(BLOCK) void topk_merge_kernel(TopkParams p) {
  __shared__ TopkShared<BLOCK> sh;
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
    const Sel s = radix_select<BLOCK, SEG>(key, valid, K, sh);
    emit_selected<BLOCK, SEG>(key, valid, s, sh, [&](int rank, int j) {
      if (rank < K) o[rank] = idx[j];
    });
  }
  for (int i = K + threadIdx.x; i < p.k; i += BLOCK) o[i] = -1;
}

template <int BLOCK, int SEG>
hipError_t launch_chunk(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((topk_chunk_kernel<BLOCK, SEG>), dim3(p.T * p.n_chunks), dim3(BLOCK), 0, stream, p);
  return hipPeekAtLastError();
}
template <int BLOCK, int SEG>
hipError_t launch_merge(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((topk_merge_kernel<BLOCK, SEG>), dim3(p.T), dim3(BLOCK), 0, stream, p);
  return hipPeekAtLastError();
}

// keys per thread for n keys over a workgroup of `block` threads
int seg_for(int n, int block) {
  const int per = (n + block - 1) / block;
  return per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : 32;
}

template <int BLOCK>
hipError_t launch_chunk_b(const TopkParams& p, hipStream_t stream) {
  switch (seg_for(p.chunk, BLOCK)) {
    case 4: return launch_chunk<BLOCK, 4>(p, stream);
    case 8: return launch_chunk<BLOCK, 8>(p, stream);
    case 16: return launch_chunk<BLOCK, 16>(p, stream);
    default: return launch_chunk<BLOCK, 32>(p, stream);
  }
}
template <int BLOCK>
hipError_t launch_merge_b(const TopkParams& p, hipStream_t stream) {
  switch (seg_for(p.n_chunks * p.k, BLOCK)) {
    case 4: return launch_merge<BLOCK, 4>(p, stream);
    case 8: return launch_merge<BLOCK, 8>(p, stream);
    case 16: return launch_merge<BLOCK, 16>(p, stream);
    default: return launch_merge<BLOCK, 32>(p, stream);
  }
}

}  // namespace

hipError_t launch_topk_merge(const TopkParams& p, hipStream_t stream) {
  return p.T < 256 ? launch_merge_b<1024>(p, stream) : launch_merge_b<512>(p, stream);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  // fewer workgroups than CUs, and more than four keys per thread at 512
  // threads: 1024 threads each
  const bool wide = (int64_t)p.T * p.n_chunks < 256 && p.chunk > 4 * 512;
  const hipError_t e = wide ? launch_chunk_b<1024>(p, stream) : launch_chunk_b<512>(p, stream);
  if (e != hipSuccess || p.n_chunks == 1) return e;
  return p.T < 256 ? launch_merge_b<1024>(p, stream) : launch_merge_b<512>(p, stream);
}

}  // namespace csa
