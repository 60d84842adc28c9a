// Step 1 of the CSA path: lightning-indexer scores on FP8 MFMA (and, as a
// variant, on MXFP4 operands with the scaled FP4 MFMA).
//
// "DSV4 Audit -- Decode Repetition + Precision / Tensor-Core Plan", B2: the
// indexer logits are the einsum 'tnd,cd->tnc' of per-token index queries
// (n heads x d dims) with one key per compressed entry, reduced by a
// weighted ReLU over the heads ("weighted-ReLU MQA logits"), run on the
// tensor units in FP8 over every visible compressed entry.
//
// Mapping on gfx950: one workgroup (8 waves) scores one query row over a
// chunk of 512 entries; each wave owns 64 consecutive entries = 4 groups of
// 16.  Per group a wave runs one v_mfma 16x16x128 FP8 per 16 index heads:
// A = the query's index heads (rows) x 128 dims; B = 16 entry keys x 128
// dims, loaded straight from memory into the operand registers (each key
// byte is used once, so no LDS staging).  The workgroup reads the query
// operand once (one tile of 16 heads per wave, waves 0-3) and shares it
// through LDS.
// The pages of the wave's groups come from one vector load (lane u fetches
// group u's page id; a group of 16 never straddles a page because the page
// size is a multiple of 16), then all of the wave's key loads are issued
// before the first MFMA.  Short workgroups at four waves per SIMD keep 8 KB
// in flight per wave and let the hardware rebalance ragged rows as
// workgroups finish.  Prefill chunks (many queries of one sequence) take the
// many-query kernel below, and the fused indexer + top-k kernels follow it.  The ReLU, the head weights and the reduction over
// heads stay in registers; the head reduction crosses the four 16-lane
// groups with two permlane swaps.  The scan is HBM-bound (128 FLOP/byte).
#include "csa_device.h"
#include "csa_internal.h"
#include "topk_select.h"

#include <algorithm>

namespace csa {

namespace {

// max(x, 0) as one v_med3_f32 (fmaxf on an MFMA result costs a canonicalising
// v_max first)
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.0e38f); }

// Weighted ReLU of one 16-entry group's MFMA outputs over this lane's 16
// heads (heads 16 ht + 4 g + i of entry r), as two FMA chains.
__device__ __forceinline__ float wrelu16(const v4f (&a)[4], const v4f (&w)[4]) {
  float s0 = w[0][0] * relu(a[0][0]);
  float s1 = w[2][0] * relu(a[2][0]);
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    s0 = __builtin_fmaf(w[0][i], relu(a[0][i]), s0);
    s1 = __builtin_fmaf(w[2][i], relu(a[2][i]), s1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s0 = __builtin_fmaf(w[1][i], relu(a[1][i]), s0);
    s1 = __builtin_fmaf(w[3][i], relu(a[3][i]), s1);
  }
  return s0 + s1;
}

// Sum over the four 16-lane groups of four values at once (a reduce-
// scatter): x_u is this lane's partial of group u; lane group g gets group
// g's total.  Three permlane swaps for four groups instead of two per group:
// the 32-lane swaps leave groups 0, 1 in the lower half and 2, 3 in the
// upper half (summed over the halves), the 16-lane swap the even and odd
// groups in the even and odd rows.
__device__ __forceinline__ float reduce4_scatter(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x0), __float_as_int(x2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x1), __float_as_int(x3), false, false);
  const float ya = __int_as_float(a[0]) + __int_as_float(a[1]);
  const float yb = __int_as_float(b[0]) + __int_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_int(ya), __float_as_int(yb), false, false);
  return __int_as_float(c[0]) + __int_as_float(c[1]);
}

// kWaves waves of kGroups groups of 16 entries: a workgroup scores
// kWaves * kGroups * 16 consecutive entries of one query row.  kQLds: the
// workgroup reads the query operand from memory once and hands it to its
// waves through LDS (else every wave loads its own copy).
//
// kFp4: MXFP4 operands (the pages' FP4 indexer variant, "DSV4 Audit", B2):
// q and k rows are E2M1 codes, two per byte (even element in the low
// nibble), with one E8M0 scale per 32 dims; a lane's 32 dims are exactly one
// scale block, so each lane hands its block's scale byte to the scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, FP4 x FP4).  A key row is D_I / 2
// bytes plus D_I / 32 scale bytes: about half the bytes of the FP8 scan.
template <int kWaves, int kGroups, int kOcc, bool kQLds, bool kFp4>
__global__ __launch_bounds__(64 * kWaves, kOcc) void index_scores_kernel(IndexParams p) {
  static_assert(!kQLds || kWaves >= 4, "four waves fill the shared query operand");
  static_assert(kGroups <= 64, "one page-id lane per group");
  static_assert(kGroups % 4 == 0, "groups are reduced four at a time");
  constexpr int kWaveEntries = 16 * kGroups;
  constexpr int kChunk = kWaves * kWaveEntries;
  __shared__ v8i qs[kQLds ? 4 * 64 : 1];
  __shared__ int qss[kQLds && kFp4 ? 4 * 64 : 1];
  // chunk-major grid: every row's first chunks are dispatched before any
  // row's later ones, so the workgroups past a short row's visible range
  // (which exit after one round trip) come last instead of between busy ones
  const int chunk = blockIdx.x / p.T;
  const int t = blockIdx.x - chunk * p.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const bool dim_ok = 32 * g < p.D_I;

  // ---- first round trip: the query operand and head weights (they depend
  // only on t), the position and the page ids, all issued before anything
  // is waited for.  Query operand: 4 tiles of 16 index heads; lane holds
  // head 16 ht + r, dims [32 g, 32 g + 32).  Weights of output rows
  // (heads 16 ht + 4 g + i), read as one 16-byte load per tile.
  auto load_q = [&](int ht, int& sc) -> v8i {
    const int h = 16 * ht + r;
    v8i a = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    sc = 0;
    if (h < p.H_I && dim_ok) {
      const size_t row = (size_t)t * p.H_I + h;
      if constexpr (kFp4) {
        const v4i v = ld16(p.q_idx + row * (p.D_I / 2) + 16 * g);
        a = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        sc = p.q_sc[row * (p.D_I / 32) + g];
      } else {
        const uint8_t* src = p.q_idx + row * p.D_I + 32 * g;
        const v4i lo = ld16(src), hi = ld16(src + 16);
        a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    return a;
  };
  v8i qa[4];
  int qsc[4] = {0, 0, 0, 0};
  if (kQLds) {
    if (wave < 4) qa[0] = load_q(wave, qsc[0]);   // wave w < 4 fetches tile w
  } else {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) qa[ht] = load_q(ht, qsc[ht]);
  }
  v4f wv[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h0 = 16 * ht + 4 * g;
    if (h0 + 3 < p.H_I && (p.H_I & 3) == 0 && ((uintptr_t)p.w & 15) == 0) {
      wv[ht] = *reinterpret_cast<const v4f*>(p.w + (size_t)t * p.H_I + h0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[ht][i] = h0 + i < p.H_I ? p.w[(size_t)t * p.H_I + h0 + i] : 0.0f;
    }
  }
  // without q_seq, query t belongs to sequence t (a decode batch), and the
  // page ids need no load before them
  const int seq = p.q_seq ? p.q_seq[t] : t;
  const int pos = p.q_pos[t];
  const int e_begin = chunk * kChunk + wave * kWaveEntries;
  const bool seq_ok = seq >= 0 && seq < p.B;
  // Page of every group (lane u < kGroups fetches group u's page id); a
  // group of 16 never straddles a page because the page size is a multiple
  // of 16.
  int my_page = -1;
  if (seq_ok && lane < kGroups) {
    const int pi = (e_begin + 16 * lane) / p.page_size;
    if (pi < p.max_pages) my_page = p.page_table[(size_t)seq * p.max_pages + pi];
  }
  int nv = 0;
  if (seq_ok && pos >= 0) nv = min(pos / p.ratio_m, p.n_comp[seq]);
  nv = max(0, min(nv, (int)min<int64_t>(p.ld, 0x7fffffff)));
  if (chunk == 0 && threadIdx.x == 0) p.n_visible[t] = nv;
  // a workgroup whose first entry is past the visible range has nothing to
  // do (uniform, so the LDS hand-over below is never split)
  if (chunk * kChunk >= nv) return;
  const int e_end = min(nv, e_begin + kWaveEntries);

  // ---- all key loads back to back.  Group u covers entries
  // e_begin + 16 u + (0..15); lane (g, r) loads entry r's dims [32 g, 32 g + 32).
  int poff = e_begin % p.page_size;        // uniform: offset of group u in its page
  v8i kb[kGroups];
  int ksc[kGroups];
  uint32_t ok_mask = 0;                    // uniform: group has a valid page
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int e0 = e_begin + 16 * u;
    const int page = __builtin_amdgcn_readlane(my_page, u);
    const bool ok = e0 < e_end && page >= 0 && page < p.num_pages;
    ok_mask |= (ok ? 1u : 0u) << u;
    v8i x = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    int xs = 0;
    if (ok && dim_ok && e0 + r < e_end) {
      const size_t row = (size_t)page * p.page_size + poff + r;
      if constexpr (kFp4) {
        const v4i v = ld16(p.k_idx + row * (p.D_I / 2) + 16 * g);
        x = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        xs = p.k_sc[row * (p.D_I / 32) + g];
      } else {
        const uint8_t* src = p.k_idx + row * p.D_I + 32 * g;
        const v4i lo = ld16(src), hi = ld16(src + 16);
        x = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    kb[u] = x;
    ksc[u] = xs;
    poff += 16;
    if (poff >= p.page_size) poff -= p.page_size;
  }
  if (kQLds) {
    // the query tile arrived with the page ids, ahead of the keys
    if (wave < 4) {
      qs[wave * 64 + lane] = qa[0];
      if constexpr (kFp4) qss[wave * 64 + lane] = qsc[0];
    }
    lds_barrier();
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      qa[ht] = qs[ht * 64 + lane];
      if constexpr (kFp4) qsc[ht] = qss[ht * 64 + lane];
    }
  }
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) wv[ht] *= p.qk_scale;
  if (e_begin >= nv) return;

  // ---- software pipeline: the MFMAs of group u + 1 go out before the
  // weighted ReLU of group u; every four groups one reduce-scatter over the
  // lane groups, after which lane (g, r) holds entry r of group 4 j + g
  float* out = p.scores + (size_t)t * p.ld;
  auto mfmas = [&](const v8i& k, int ks, v4f (&acc)[4]) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      // rows of absent heads are zero
      if constexpr (kFp4)
        acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], k, (v4f){0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                   qsc[ht], 0, ks);
      else
        acc[ht] = mfma_f8_128(qa[ht], k, (v4f){0.f, 0.f, 0.f, 0.f});
    }
  };
  v4f acc[2][4];
  float xg[4];
  mfmas(kb[0], ksc[0], acc[0]);
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    if (u + 1 < kGroups) mfmas(kb[u + 1], ksc[u + 1], acc[(u + 1) & 1]);
    xg[u & 3] = wrelu16(acc[u & 1], wv);
    if ((u & 3) == 3) {
      const float tot = reduce4_scatter(xg[0], xg[1], xg[2], xg[3]);
      const int ug = u - 3 + g;
      const int e = e_begin + 16 * ug + r;
      if (e < e_end) out[e] = ((ok_mask >> ug) & 1u) ? tot : -__builtin_inff();
    }
  }
}

// ---- many queries of one sequence (prefill) -----------------------------
// All queries scan the same compressed keys, so a workgroup of kMqQ waves
// takes kMqQ queries (one per wave) and walks the whole key range in chunks
// of 256 entries, each staged once in LDS and scored against all kMqQ
// queries: the indexer becomes a GEMM [queries x heads] x [entries] whose
// key tile is read from memory once per kMqQ queries.  The next chunk's keys
// are loaded into registers while the current chunk is scored (LDS double
// buffer); page ids run two chunks ahead.  LDS layout: the MFMA B operand of
// group u (16 entries) for lane l at (u * 64 + l) * 32 bytes, so every lane
// reads its 32 bytes contiguously.
constexpr int kMqQ = 16;
constexpr int kMqGroups = 16;
constexpr int kMqChunk = 16 * kMqGroups;
static_assert(kMqGroups % kMqQ == 0, "groups split evenly over the waves");
static_assert(kMqGroups % 4 == 0, "groups are reduced four at a time");

//
// kFp4 (MXFP4 operands, as in the one-query kernel): a lane's LDS slot of a
// group holds its 16 code bytes in dwords 0-3 and its block's scale byte in
// dword 4; the scaled MFMA reads only dwords 0-3 of an FP4 operand.
//
// kQ queries (waves) per workgroup.  The scores kernel runs one 16-wave
// workgroup per CU (64 KB of LDS, registers for four waves per SIMD), so a
// staged chunk serves 16 queries.  kFused: one 8-wave workgroup per CU; the
// scores never leave the chip.  Every wave keeps a candidate buffer of (key, entry) pairs in LDS, in
// entry order, and a threshold: an entry goes in only if its
// order-preserving key is above the threshold (later entries are higher in
// index, so one tied with the threshold ranks below every kept one).  When a
// buffer could overflow in the next chunk, the waves cut their buffers to a
// little more than k entries by a threshold found by bisection over key
// values (exactly k where ties decide), which becomes the new insertion
// threshold.  After the last chunk each buffer is cut to the exact top k of
// the workgroup's key range, written as the row's answer (one range) or as
// candidates for the top-k merge.  The scores come from the same code as in
// the scores kernel, so the selection is bit-identical to csa_index_scores +
// csa_topk.
constexpr int kFtMqCap = 1792;   // candidate slots per wave (8 waves: 84 KB of LDS)
constexpr int kFtMqMaxK = 1024;   // largest k: a cut leaves room for at least one chunk
static_assert(kFtMqCap - kMqChunk >= kFtMqMaxK, "a buffer cut to k has room for a chunk");
template <bool kFp4, int kQ, bool kFused>
__global__ __launch_bounds__(64 * kQ, kFused ? 1 : 4) void index_scores_mq_kernel(IndexParams p, TopkParams tp,
                                                                                int n_split) {
  static_assert(!kFused || !kFp4, "fused indexer + top-k: E4M3 operands");
  constexpr int kMqGpw = kMqGroups / kQ;    // groups loaded per wave per chunk
  static_assert(kMqGroups % kQ == 0 && kMqGpw >= 1, "groups split evenly over the waves");
  __shared__ __attribute__((aligned(16))) v8i ks[2][kMqGroups * 64];
  __shared__ uint32_t okw[2][kQ];
  // fused: each wave's candidate keys and entries, and whether its buffer
  // needs a cut before the next chunk
  __shared__ uint32_t fck[kFused ? kQ : 1][kFused ? kFtMqCap : 1];
  __shared__ uint16_t fci[kFused ? kQ : 1][kFused ? kFtMqCap : 1];
  __shared__ int fneed[2][kQ];
  // workgroup = (query block, part of the key range): n_split parts when
  // the query blocks alone would leave CUs idle
  const int qb = blockIdx.x / n_split;
  const int split = blockIdx.x - qb * n_split;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const bool dim_ok = 32 * g < p.D_I;
  const int t = qb * kQ + wave;
  const bool q_ok = t < p.T;

  // ---- this wave's query operand and weights (layout as in the
  // one-query kernel)
  v8i qa[4];
  int qsc[4];
  v4f wv[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = 16 * ht + r;
    qa[ht] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    qsc[ht] = 0;
    if (q_ok && h < p.H_I && dim_ok) {
      const size_t row = (size_t)t * p.H_I + h;
      if constexpr (kFp4) {
        const v4i v = ld16(p.q_idx + row * (p.D_I / 2) + 16 * g);
        qa[ht] = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        qsc[ht] = p.q_sc[row * (p.D_I / 32) + g];
      } else {
        const uint8_t* src = p.q_idx + row * p.D_I + 32 * g;
        const v4i lo = ld16(src), hi = ld16(src + 16);
        qa[ht] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    const int h0 = 16 * ht + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = (q_ok && h0 + i < p.H_I) ? p.w[(size_t)t * p.H_I + h0 + i] : 0.0f;
  }

  // ---- visible counts of the workgroup's queries (all in sequence 0)
  const int nc = p.n_comp[0];
  int nv_max = 0, nv_own = 0;
#pragma unroll
  for (int w = 0; w < kQ; ++w) {
    const int tw = qb * kQ + w;
    int nv = 0;
    if (tw < p.T) {
      const int pos = p.q_pos[tw];
      if ((p.q_seq ? p.q_seq[tw] : tw) == 0 && pos >= 0) nv = min(pos / p.ratio_m, nc);
      nv = max(0, min(nv, (int)min<int64_t>(p.ld, 0x7fffffff)));
      if (split == 0 && w == wave && lane == 0) p.n_visible[tw] = nv;
    }
    nv_max = max(nv_max, nv);
    if (w == wave) nv_own = nv;
  }
  const int n_all = (nv_max + kMqChunk - 1) / kMqChunk;
  const int per = (n_all + n_split - 1) / n_split;
  const int c_begin = split * per;
  const int n_ch = min(n_all, c_begin + per);   // chunks [c_begin, n_ch) of this workgroup

  // ---- fused: this wave's candidate buffer (wave-local; the wave's LDS
  // operations complete in order, so a wait for them is its only fence)
  uint32_t* bk = fck[kFused ? wave : 0];
  uint16_t* bi = fci[kFused ? wave : 0];
  int fcnt = 0;           // candidates in the buffer (ascending entry order)
  bool full = false;      // a cut has happened: only keys above ftau go in
  uint32_t ftau = 0;
  auto wave_sync = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
  };
  auto lanes_below = [&](uint64_t m) -> int {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  };
  // Cuts the buffer (fcnt > U >= K >= 1) to the entries above a threshold
  // thr that keeps between K and U of them, or, when ties leave no such
  // threshold (and always when U == K), to exactly its top K: the keys above
  // thr plus the first need_eq keys equal to it.  Either way every dropped
  // entry, and every later entry whose key is not above thr, has at least K
  // kept entries ranked above it, so thr becomes the insertion threshold.
  // thr comes from a bisection over key values; each probe counts the keys
  // above it with one compare and one ballot popcount per 64 slots (keys
  // and entries are read into registers once, lane l holding slots 64 q + l).
  auto shrink = [&](int K, int U) __attribute__((always_inline)) {
    constexpr int kR = kFtMqCap / 64;
    uint32_t kr[kR], ir[kR];
    uint32_t vmin = 0xffffffffu, vmax = 0u;
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const bool v = 64 * q + lane < fcnt;
      kr[q] = v ? bk[64 * q + lane] : 0u;   // empty slots: key 0, above no probe
      ir[q] = v ? bi[64 * q + lane] : 0u;
      vmin = v ? min(vmin, kr[q]) : vmin;
      vmax = v ? max(vmax, kr[q]) : vmax;
    }
    vmin = topk_sel::wave_min_u32(vmin);
    vmax = topk_sel::wave_max_u32(vmax);
    auto count_above = [&](uint32_t x) {
      int n = 0;
#pragma unroll
      for (int q = 0; q < kR; ++q) n += __builtin_popcountll(__ballot(kr[q] > x));
      return n;
    };
    // count_above(lo) >= K > count_above(hi)
    int64_t lo = (int64_t)vmin - 1, hi = vmax;
    int c_lo = fcnt, c_hi = 0;
    while (c_lo > U && hi - lo > 1) {
      const uint32_t mid = (uint32_t)(lo + ((hi - lo) >> 1));
      const int c = count_above(mid);
      if (c >= K) {
        lo = mid;
        c_lo = c;
      } else {
        hi = mid;
        c_hi = c;
      }
    }
    uint32_t thr;
    int need_eq = 0;
    if (c_lo <= U) {
      thr = (uint32_t)lo;         // lo >= 0 here: it moved at least once
    } else {
      thr = (uint32_t)hi;         // hi == lo + 1: the keys equal to hi decide
      need_eq = K - c_hi;
    }
    // ordered compaction in place (outputs never pass inputs, all of which
    // are in registers)
    int n_out = 0, eq_seen = 0;
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const bool valid = 64 * q + lane < fcnt;
      const bool eq = valid && kr[q] == thr;
      const uint64_t eqb = __ballot(eq);
      const bool take = (valid && kr[q] > thr) || (eq && eq_seen + lanes_below(eqb) < need_eq);
      const uint64_t tb = __ballot(take);
      if (take) {
        const int pos = n_out + lanes_below(tb);
        bk[pos] = kr[q];
        bi[pos] = (uint16_t)ir[q];
      }
      n_out += __builtin_popcountll(tb);
      eq_seen += __builtin_popcountll(eqb);
    }
    fcnt = n_out;
    ftau = thr;
    full = true;
    wave_sync();
  };
  // the row's answer (one key range) or its candidates for the merge:
  // min(k, fcnt) entries in ascending order, then padding
  auto emit = [&]() {
    if (fcnt > tp.k) shrink(tp.k, tp.k);
    wave_sync();
    if (n_split == 1) {
      int32_t* o = tp.out + (size_t)t * tp.k;
      for (int j = lane; j < tp.k; j += 64) o[j] = j < fcnt ? (int32_t)bi[j] : -1;
    } else {
      const size_t base = ((size_t)t * n_split + split) * tp.k;
      for (int j = lane; j < tp.k; j += 64) {
        tp.cand_key[base + j] = j < fcnt ? bk[j] : 0u;
        tp.cand_idx[base + j] = j < fcnt ? (int32_t)bi[j] : -1;
      }
    }
  };
  if (c_begin >= n_ch) {                        // uniform over the workgroup
    if constexpr (kFused) {
      if (q_ok) emit();
    }
    return;
  }

  // page id of group (4 w + j) of chunk c, fetched by lane j (< kMqGpw)
  auto load_page = [&](int c) -> int {
    int pg = -1;
    if (lane < kMqGpw && c < n_ch) {
      const int pi = (c * kMqChunk + 16 * (kMqGpw * wave + lane)) / p.page_size;
      if (pi < p.max_pages) pg = p.page_table[pi];
    }
    return pg;
  };
  // this wave's groups of chunk c: lane (g, r) entry r's dims [32 g, 32 g + 32)
  auto load_keys = [&](int c, int pg, v8i (&kl)[kMqGpw], uint32_t& okbits) {
    okbits = 0;
#pragma unroll
    for (int j = 0; j < kMqGpw; ++j) {
      const int u = kMqGpw * wave + j;
      const int eg = c * kMqChunk + 16 * u;
      const int page = __builtin_amdgcn_readlane(pg, j);
      const bool ok = eg < nv_max && page >= 0 && page < p.num_pages;
      okbits |= (ok ? 1u : 0u) << u;
      kl[j] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
      if (ok && dim_ok && eg + r < nv_max) {
        const size_t row = (size_t)page * p.page_size + eg % p.page_size + r;
        if constexpr (kFp4) {
          const v4i v = ld16(p.k_idx + row * (p.D_I / 2) + 16 * g);
          kl[j] = (v8i){v[0], v[1], v[2], v[3], (int)p.k_sc[row * (p.D_I / 32) + g], 0, 0, 0};
        } else {
          const uint8_t* src = p.k_idx + row * p.D_I + 32 * g;
          const v4i lo = ld16(src), hi = ld16(src + 16);
          kl[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
    }
  };
  auto store_keys = [&](int b, const v8i (&kl)[kMqGpw], uint32_t okbits) {
#pragma unroll
    for (int j = 0; j < kMqGpw; ++j) ks[b][(kMqGpw * wave + j) * 64 + lane] = kl[j];
    if (lane == 0) okw[b][wave] = okbits;
  };

  v8i kl[kMqGpw];
  uint32_t okbits;
  int pg_next = load_page(c_begin + 1);
  {
    const int pg0 = load_page(c_begin);
    load_keys(c_begin, pg0, kl, okbits);
  }
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) wv[ht] *= p.qk_scale;
  store_keys(0, kl, okbits);
  __syncthreads();

  float* out = kFused ? nullptr : p.scores + (size_t)t * p.ld;
  auto mfmas = [&](const v8i& k, v4f (&acc)[4]) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      // rows of absent heads are zero
      if constexpr (kFp4)
        acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], k, (v4f){0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                   qsc[ht], 0, k[4]);
      else
        acc[ht] = mfma_f8_128(qa[ht], k, (v4f){0.f, 0.f, 0.f, 0.f});
    }
  };

  for (int c = c_begin; c < n_ch; ++c) {
    const int b = (c - c_begin) & 1;
    // next chunk's keys into registers (page ids one chunk further ahead)
    const bool more = c + 1 < n_ch;
    if (more) {
      load_keys(c + 1, pg_next, kl, okbits);
      pg_next = load_page(c + 2);
    }
    const int e0 = c * kMqChunk;
    if (q_ok && e0 < nv_own) {
      uint32_t ok_mask = 0;
#pragma unroll
      for (int w = 0; w < kQ; ++w) ok_mask |= okw[b][w];
      const int e_end = min(nv_own, e0 + kMqChunk);
      // Scores kernel: one accumulator set; the other waves of its SIMD (four
      // per SIMD) hide the MFMA latency, and the registers a second set would
      // take are what allow that occupancy.  Fused kernel (two waves per
      // SIMD): the MFMAs of group u + 1 go before the weighted ReLU of group
      // u, into a second set.  One reduce-scatter per four groups.
      constexpr int kAcc = kFused ? 2 : 1;
      v4f acc[kAcc][4];
      float xg[4];
      float sq[kMqGroups / 4];   // fused: entry e0 + 64 i + lane of the chunk
      if constexpr (kFused) {
        const v8i kb = ks[b][lane];
        mfmas(kb, acc[0]);
      }
#pragma unroll
      for (int u = 0; u < kMqGroups; ++u) {
        if constexpr (kFused) {
          if (u + 1 < kMqGroups) {
            const v8i kb = ks[b][(u + 1) * 64 + lane];
            mfmas(kb, acc[(u + 1) & 1]);
          }
        } else {
          const v8i kb = ks[b][u * 64 + lane];
          mfmas(kb, acc[0]);
        }
        xg[u & 3] = wrelu16(acc[u % kAcc], wv);
        if ((u & 3) == 3) {
          const float tot = reduce4_scatter(xg[0], xg[1], xg[2], xg[3]);
          const int ug = u - 3 + g;
          const float v = ((ok_mask >> ug) & 1u) ? tot : -__builtin_inff();
          if constexpr (kFused) {
            sq[u >> 2] = v;
          } else {
            const int e = e0 + 16 * ug + r;
            if (e < e_end) out[e] = v;
          }
        }
      }
      if constexpr (kFused) {
        // lane l holds entry e0 + 64 i + l of block i: ballots in lane order
        // keep the buffer in entry order
        // (room for the whole chunk: fcnt <= kFtMqCap - kMqChunk here)
        uint32_t key[kMqGroups / 4];
        uint64_t bal[kMqGroups / 4];
#pragma unroll
        for (int i = 0; i < kMqGroups / 4; ++i) {
          key[i] = float_order_key(sq[i]);
          bal[i] = __ballot(e0 + 64 * i + lane < e_end && (!full || key[i] > ftau));
        }
#pragma unroll
        for (int i = 0; i < kMqGroups / 4; ++i) {
          if ((bal[i] >> lane) & 1u) {
            const int pos = fcnt + lanes_below(bal[i]);
            bk[pos] = key[i];
            bi[pos] = (uint16_t)(e0 + 64 * i + lane);
          }
          fcnt += __builtin_popcountll(bal[i]);
        }
      }
    }
    if (more) store_keys(b ^ 1, kl, okbits);
    if constexpr (kFused) {
      if (lane == 0) fneed[b][wave] = fcnt > kFtMqCap - kMqChunk;
    }
    __syncthreads();
    if constexpr (kFused) {
      // when any wave's buffer could overflow in the next chunk, every wave
      // above U cuts now: the cuts of the workgroup run side by side instead
      // of one after another between the chunk barriers.  U a little above
      // k lets the bisection stop early (measured on 2048 queries x 16384
      // entries, k 512: 310 us with U = k + 128 and 1792 slots, 320 us with
      // U halfway to the trigger and 1280 slots)
      int any = 0;
#pragma unroll
      for (int w = 0; w < kQ; ++w) any |= fneed[b][w];
      const int U = min(tp.k + 128, kFtMqCap - kMqChunk);
      if (any && more && fcnt > U) shrink(tp.k, U);
    }
  }
  if constexpr (kFused) {
    if (q_ok) emit();
  }
}

// ---- fused indexer + top-k ------------------------------------------------
// "DSV4 Audit", B2: score and select with a wave-local reduction and no
// global lock.  One workgroup (8 waves) per (row, chunk of kRounds x 512
// entries): the chunk's scores are computed as in the one-query kernel
// (a wave scores 64 entries per round, the next round's keys in flight
// while the current one is scored) but kept in LDS, then the workgroup
// selects the chunk's top-k with the same radix selection as the top-k
// kernels.  A row of one chunk gets its final answer here; longer rows
// leave per-chunk candidates for the top-k merge.  The scores never go to
// HBM.
constexpr int kFtWaves = 8;
constexpr int kFtRound = kFtWaves * 4 * 16;   // entries per round: 4 groups of 16 per wave

template <int kRounds>
__global__ __launch_bounds__(64 * kFtWaves, 1) void index_topk_kernel(IndexParams p, TopkParams tp) {
  constexpr int kChunk = kRounds * kFtRound;
  constexpr int kThreads = 64 * kFtWaves;
  constexpr int SEG = kChunk / kThreads;       // keys per thread in the selection
  static_assert(SEG == 4 || SEG == 8 || SEG == 16, "selection segment");
  static_assert(4 * kRounds <= 64, "one page-id lane per group");
  __shared__ __attribute__((aligned(16))) float sc[kChunk];
  __shared__ v8i qs[4 * 64];
  __shared__ topk_sel::TopkShared<kThreads> sh;
  const int chunk = blockIdx.x / p.T;           // chunk-major, as the one-query kernel
  const int t = blockIdx.x - chunk * p.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const bool dim_ok = 32 * g < p.D_I;
  const int c0 = chunk * kChunk;

  // ---- first round trip: query tile (waves 0-3, shared through LDS),
  // weights, position, and the page ids of all of this wave's groups
  // (lane 4 rd + u holds group u of round rd)
  v8i qa[4];
  if (wave < 4) {
    const int h = 16 * wave + r;
    qa[0] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    if (h < p.H_I && dim_ok) {
      const uint8_t* src = p.q_idx + ((size_t)t * p.H_I + h) * p.D_I + 32 * g;
      const v4i lo = ld16(src), hi = ld16(src + 16);
      qa[0] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  v4f wv[4];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h0 = 16 * ht + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[ht][i] = h0 + i < p.H_I ? p.w[(size_t)t * p.H_I + h0 + i] : 0.0f;
  }
  const int seq = p.q_seq ? p.q_seq[t] : t;
  const int pos = p.q_pos[t];
  const bool seq_ok = seq >= 0 && seq < p.B;
  int my_page = -1;
  if (seq_ok && lane < 4 * kRounds) {
    const int rd = lane >> 2, u = lane & 3;
    const int pi = (c0 + rd * kFtRound + wave * 64 + 16 * u) / p.page_size;
    if (pi < p.max_pages) my_page = p.page_table[(size_t)seq * p.max_pages + pi];
  }
  int nv = 0;
  if (seq_ok && pos >= 0) nv = min(pos / p.ratio_m, p.n_comp[seq]);
  nv = max(0, (int)min<int64_t>(nv, p.ld));     // the page table's entries at most
  if (chunk == 0 && threadIdx.x == 0) p.n_visible[t] = nv;
  const int n = max(0, min(kChunk, nv - c0));   // visible entries of this chunk (uniform)

  // keys of round rd for this wave: group u covers entries
  // c0 + rd * kFtRound + 64 wave + 16 u + (0..15)
  auto load_round = [&](int rd, v8i (&kb)[4], uint32_t& okm) {
    okm = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int le = rd * kFtRound + wave * 64 + 16 * u;   // chunk-local first entry
      const int page = __builtin_amdgcn_readlane(my_page, 4 * rd + u);
      const bool ok = le < n && page >= 0 && page < p.num_pages;
      okm |= (ok ? 1u : 0u) << u;
      v8i x = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
      if (ok && dim_ok && le + r < n) {
        const int poff = (c0 + le) % p.page_size;
        const uint8_t* src = p.k_idx + ((size_t)page * p.page_size + poff + r) * p.D_I + 32 * g;
        const v4i lo = ld16(src), hi = ld16(src + 16);
        x = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      kb[u] = x;
    }
  };
  v8i kb[2][4];
  uint32_t okm[2];
  load_round(0, kb[0], okm[0]);
  if (wave < 4) qs[wave * 64 + lane] = qa[0];
  lds_barrier();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) qa[ht] = qs[ht * 64 + lane];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) wv[ht] *= p.qk_scale;

  auto mfmas = [&](const v8i& k, v4f (&acc)[4]) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = mfma_f8_128(qa[ht], k, (v4f){0.f, 0.f, 0.f, 0.f});
  };
#pragma unroll
  for (int rd = 0; rd < kRounds; ++rd) {
    const int cur = rd & 1;
    if (rd + 1 < kRounds) load_round(rd + 1, kb[cur ^ 1], okm[cur ^ 1]);
    const int le0 = rd * kFtRound + wave * 64;
    if (le0 < n) {
      v4f acc[2][4];
      float xg[4];
      mfmas(kb[cur][0], acc[0]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u + 1 < 4) mfmas(kb[cur][u + 1], acc[(u + 1) & 1]);
        xg[u] = wrelu16(acc[u & 1], wv);
      }
      // lane (g, r) now holds entry r of group g
      const float tot = reduce4_scatter(xg[0], xg[1], xg[2], xg[3]);
      const int le = le0 + 16 * g + r;
      if (le < n) sc[le] = ((okm[cur] >> g) & 1u) ? tot : -__builtin_inff();
    }
  }
  __syncthreads();   // the chunk's scores are in LDS

  // ---- selection over the chunk (thread i: scores [SEG i, SEG i + SEG))
  const int i0 = threadIdx.x * SEG;
  uint32_t key[SEG];
#pragma unroll
  for (int j = 0; j < SEG; j += 4) {
    const v4f v = *reinterpret_cast<const v4f*>(sc + i0 + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[j + e] = float_order_key(v[e]);
  }
  const int cnt = max(0, min(SEG, n - i0));
  const uint32_t valid = cnt >= 32 ? 0xffffffffu : ((1u << cnt) - 1u);
  const int K = min(tp.k, n);
  if (tp.n_chunks == 1) {
    int32_t* o = tp.out + (size_t)t * tp.k;
    if (K > 0) {
      const topk_sel::Sel s = topk_sel::radix_select<kThreads, SEG>(key, valid, K, sh);
      topk_sel::emit_selected<kThreads, SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) o[rank] = c0 + i0 + j;
      });
    }
    for (int i = K + threadIdx.x; i < tp.k; i += kThreads) o[i] = -1;
  } else {
    const size_t base = ((size_t)t * tp.n_chunks + chunk) * tp.k;
    uint32_t* ck = tp.cand_key + base;
    int32_t* ci = tp.cand_idx + base;
    if (K > 0) {
      const topk_sel::Sel s = topk_sel::radix_select<kThreads, SEG>(key, valid, K, sh);
      topk_sel::emit_selected<kThreads, SEG>(key, valid, s, sh, [&](int rank, int j) {
        if (rank < K) {
          ck[rank] = key[j];
          ci[rank] = c0 + i0 + j;
        }
      });
    }
    for (int i = K + threadIdx.x; i < tp.k; i += kThreads) {
      ck[i] = 0u;
      ci[i] = -1;
    }
  }
}

template <int kWaves, int kGroups, int kOcc, bool kQLds, bool kFp4>
hipError_t launch_decode(IndexParams p, int64_t span, hipStream_t stream) {
  constexpr int kChunk = kWaves * kGroups * 16;
  p.chunk = kChunk;
  p.n_chunks = (int)std::max<int64_t>(1, (span + kChunk - 1) / kChunk);
  const int64_t blocks = (int64_t)p.T * p.n_chunks;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((index_scores_kernel<kWaves, kGroups, kOcc, kQLds, kFp4>), dim3((unsigned)blocks),
                     dim3(64 * kWaves), 0, stream, p);
  return hipPeekAtLastError();
}

}  // namespace

hipError_t launch_index_scores(const IndexParams& p_in, hipStream_t stream) {
  IndexParams p = p_in;
  const int64_t span = std::min<int64_t>(p.ld, (int64_t)p.max_pages * p.page_size);
  if (p.B == 1 && p.T >= 2 * kMqQ) {
    // one sequence, many queries: key tiles shared through LDS
    p.chunk = kMqChunk;
    p.n_chunks = (int)std::max<int64_t>(1, (span + kMqChunk - 1) / kMqChunk);
    const int64_t n_qb = (p.T + kMqQ - 1) / kMqQ;
    const int64_t span_ch = std::max<int64_t>(1, (span + kMqChunk - 1) / kMqChunk);
    // about 256 workgroups, one per CU (a 16-wave workgroup fills the four
    // waves per SIMD its registers allow), parts of at least 4 chunks
    const int n_split = (int)std::max<int64_t>(1, std::min<int64_t>((256 + n_qb - 1) / n_qb, span_ch / 4));
    const TopkParams none{};
    if (p.fp4)
      hipLaunchKernelGGL((index_scores_mq_kernel<true, kMqQ, false>), dim3((unsigned)(n_qb * n_split)),
                         dim3(64 * kMqQ), 0, stream, p, none, n_split);
    else
      hipLaunchKernelGGL((index_scores_mq_kernel<false, kMqQ, false>), dim3((unsigned)(n_qb * n_split)),
                         dim3(64 * kMqQ), 0, stream, p, none, n_split);
    return hipPeekAtLastError();
  }
  // MXFP4 operands: twice the groups per wave (a key row is half as long, so
  // the same bytes in flight)
  if (p.fp4) return launch_decode<4, 8, 4, true, true>(p, span, stream);
  // 8 waves of 4 groups (512 entries per workgroup): 0.4 us faster at c2
  // and 1.2 us at c3 than 4 waves (fewer workgroups to dispatch and fewer
  // of them past a short row's end)
  return launch_decode<8, 4, 4, true, false>(p, span, stream);
}

hipError_t launch_index_topk_prefill(const IndexParams& p, const TopkParams& tp, hipStream_t stream) {
  static_assert(kFtMqMaxK == kIndexTopkPrefillMaxK, "candidate buffer sized for the largest k");
  if (p.B != 1 || p.T < 1 || tp.k < 1 || tp.k > kFtMqMaxK || tp.n_chunks < 1 || p.ld > kIndexTopkPrefillMaxSpan)
    return hipErrorInvalidValue;
  const int64_t n_qb = (p.T + kIndexTopkPrefillQ - 1) / kIndexTopkPrefillQ;
  const int n_split = tp.n_chunks;
  if (n_qb * n_split >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((index_scores_mq_kernel<false, kIndexTopkPrefillQ, true>), dim3((unsigned)(n_qb * n_split)),
                     dim3(64 * kIndexTopkPrefillQ), 0, stream, p, tp, n_split);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess || n_split == 1) return e;
  return launch_topk_merge(tp, stream);
}

hipError_t launch_index_topk(const IndexParams& p_in, const TopkParams& tp_in, hipStream_t stream) {
  IndexParams p = p_in;
  TopkParams tp = tp_in;
  const int64_t blocks = (int64_t)p.T * tp.n_chunks;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  switch (tp.chunk) {
    case 4 * kFtRound:
      hipLaunchKernelGGL(index_topk_kernel<4>, dim3((unsigned)blocks), dim3(64 * kFtWaves), 0, stream, p, tp);
      break;
    case 8 * kFtRound:
      hipLaunchKernelGGL(index_topk_kernel<8>, dim3((unsigned)blocks), dim3(64 * kFtWaves), 0, stream, p, tp);
      break;
    case 16 * kFtRound:
      hipLaunchKernelGGL(index_topk_kernel<16>, dim3((unsigned)blocks), dim3(64 * kFtWaves), 0, stream, p, tp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess || tp.n_chunks == 1) return e;
  return launch_topk_merge(tp, stream);
}

}  // namespace csa
