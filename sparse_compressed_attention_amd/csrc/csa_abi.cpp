// C ABI of libcsa.so: argument validation on the host, launch-shape choices
// (chunking, workgroup split of long key ranges), launches and status codes.
// The contract of every entry point is documented in include/csa.h.
//
// "ROADMAP -- Stage E ...", E4: the launch path returns a code and checks
// hipPeekAtLastError() after each launch; it never synchronises the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>

#include "csa.h"
#include "csa_internal.h"

using namespace csa;

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- top-k chunking -------------------------------------------------------
struct TopkPlan {
  int chunk = 0, n_chunks = 0;
  size_t ws_bytes = 0;
  bool ok = false;
};
TopkPlan plan_topk(int32_t T, int64_t ld, int32_t k) {
  TopkPlan pl;
  if (ld <= kTopkMaxChunk) {
    pl.chunk = (int)ld;
    pl.n_chunks = 1;
    pl.ok = true;
    return pl;
  }
  for (int chunk : {8192, 4096, kTopkMaxChunk}) {
    const int64_t n = ceil_div(ld, chunk);
    if (n * k <= kTopkMaxCand) {
      pl.chunk = chunk;
      pl.n_chunks = (int)n;
      pl.ws_bytes = (size_t)T * (size_t)n * (size_t)k * 8u;
      pl.ok = true;
      return pl;
    }
  }
  return pl;
}

// ---- fused indexer + top-k: chunk of entries per workgroup ----------------
// The smallest of 2048, 4096, 8192 entries whose candidates (chunks x k) the
// merge can take, or one chunk for the whole row.
TopkPlan plan_index_topk(int32_t T, int64_t span, int32_t k) {
  TopkPlan pl;
  for (int chunk : {2048, 4096, 8192}) {
    const int64_t n = std::max<int64_t>(1, ceil_div(span, chunk));
    if (n == 1 || n * k <= kTopkMaxCand) {
      pl.chunk = chunk;
      pl.n_chunks = (int)n;
      pl.ws_bytes = n > 1 ? (size_t)T * (size_t)n * (size_t)k * 8u : 0;
      pl.ok = true;
      return pl;
    }
  }
  return pl;
}

// Many queries of one sequence (B == 1, T >= 16, k <= 1024, at most 65536
// entries): workgroups of 8 queries sharing each key tile, the key range cut
// into n parts of at least 1024 entries when there are fewer query blocks
// than CUs; candidates of n parts x k per row go to the merge.
TopkPlan plan_index_topk_prefill(int32_t T, int64_t span, int32_t k) {
  TopkPlan pl;
  if (T < 16 || k < 1 || k > kIndexTopkPrefillMaxK || span < 1 || span > kIndexTopkPrefillMaxSpan) return pl;
  const int64_t n_qb = ceil_div(T, kIndexTopkPrefillQ);
  const int64_t n = std::max<int64_t>(
      1, std::min<int64_t>({ceil_div(256, n_qb), ceil_div(span, 256) / 4, (int64_t)(kTopkMaxCand / k)}));
  pl.chunk = (int)ceil_div(span, n);
  pl.n_chunks = (int)n;
  pl.ws_bytes = n > 1 ? (size_t)T * (size_t)n * (size_t)k * 8u : 0;
  pl.ok = true;
  return pl;
}

// ---- attention split of the key range over workgroups ---------------------
constexpr int kTargetBlocks = 256;   // one workgroup per CU on MI355X
struct AttnPlan {
  int ht = 2, n_hg = 0, n_splits = 1, per_split = 0;
  size_t ws_bytes = 0;
};
size_t partial_bytes(int64_t T, int64_t H, int D, int splits) {
  return (size_t)splits * (size_t)T * (size_t)H * part_row_bytes(D);
}
// Preferred plan, then shrunk to what `ws_avail` holds.  Returns false when
// even the minimum number of splits does not fit.
bool plan_attn(int64_t T, int32_t H, int D, int64_t max_slots, size_t ws_avail, bool limit_ws, AttnPlan* out) {
  AttnPlan pl;
  // 64 heads per workgroup (two waves per SIMD) when that alone gives a
  // workgroup per CU, else 32 heads per workgroup and, if still too few,
  // split key ranges
  pl.ht = (T * ceil_div(H, 64) >= kTargetBlocks) ? 4 : 2;
  pl.n_hg = (int)ceil_div(H, 16 * pl.ht);
  // the kernel pads the selected slots to whole tiles (at most kAttnTile - 1 more)
  const int64_t slots = std::max<int64_t>(1, max_slots + kAttnTile - 1);
  const int64_t min_splits = ceil_div(slots, kAttnMaxSlots);
  if (min_splits > kAttnMaxSplits) return false;   // key range beyond what one merge combines
  const int64_t base = std::max<int64_t>(1, T * pl.n_hg);
  int64_t splits = std::max<int64_t>(min_splits, ceil_div(kTargetBlocks, base));
  splits = std::min<int64_t>(splits, ceil_div(slots, kAttnTile));
  splits = std::min<int64_t>(splits, kAttnMaxSplits);
  splits = std::max<int64_t>(splits, min_splits);
  if (limit_ws && splits > 1) {
    const size_t one = partial_bytes(T, H, D, 1);
    const int64_t fit = one ? (int64_t)(ws_avail / one) : 0;
    if (fit < splits) splits = std::max<int64_t>(min_splits, fit);
    if (splits > 1 && fit < splits) return false;
    splits = std::max<int64_t>(1, splits);
  }
  int64_t per = ceil_div(ceil_div(slots, splits), kAttnTile) * kAttnTile;
  per = std::min<int64_t>(per, kAttnMaxSlots);
  splits = ceil_div(slots, per);
  pl.n_splits = (int)splits;
  pl.per_split = (int)per;
  pl.ws_bytes = splits > 1 ? partial_bytes(T, H, D, (int)splits) : 0;
  if (limit_ws && pl.ws_bytes > ws_avail) return false;
  *out = pl;
  return true;
}

bool dims_supported(int dn, int dr) { return (dn == 448 && dr == 64) || (dn == 48 && dr == 16); }

int check_cache(const csa_latent_cache* c) {
  if (!c || !c->nope || !c->rope || !c->page_table || !c->n_comp) return CSA_ERR_INVALID_ARG;
  if (!aligned16(c->nope) || !aligned16(c->rope)) return CSA_ERR_INVALID_ARG;
  if (c->num_seqs < 1 || c->num_pages < 1 || c->page_size < 16 || c->page_size % 16 || c->max_pages < 1 || c->ratio_m < 1)
    return CSA_ERR_INVALID_ARG;
  if ((int64_t)c->num_pages * c->page_size >= (int64_t)1 << 30) return CSA_ERR_UNSUPPORTED;
  if (!(c->nope_scale > 0.0f) || !std::isfinite(c->nope_scale)) return CSA_ERR_INVALID_ARG;
  if (!dims_supported(c->D_nope, c->D_rope)) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int csa_version(void) { return 130; }

const char* csa_status_string(int code) {
  switch (code) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported shape";
    case CSA_ERR_LAUNCH: return "kernel launch failed";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_TOO_LARGE: return "partial results exceed the library's fixed scratch buffer";
    default: return "unknown status";
  }
}

// Checks and launch shared by the FP8 and MXFP4 indexer entry points.
static int index_scores_common(IndexParams& p, const int32_t* page_table, const int32_t* n_comp, int32_t num_pages,
                               int32_t page_size, int32_t max_pages, int32_t B, const int32_t* q_pos,
                               const int32_t* q_seq, int32_t T, int32_t H_I, int32_t D_I, int32_t ratio_m,
                               float* scores, int64_t ld_scores, int32_t* n_visible, void* stream) {
  if (!p.q_idx || !p.w || !p.k_idx || !page_table || !n_comp || !q_pos || !scores || !n_visible)
    return CSA_ERR_INVALID_ARG;
  if (!aligned16(p.q_idx) || !aligned16(p.k_idx)) return CSA_ERR_INVALID_ARG;
  if (B < 1 || num_pages < 1 || page_size < 16 || page_size % 16 || max_pages < 1 || ratio_m < 1 || ld_scores < 1)
    return CSA_ERR_INVALID_ARG;
  if (H_I < 1 || H_I > 64 || !(D_I == 32 || D_I == 64 || D_I == 96 || D_I == 128)) return CSA_ERR_UNSUPPORTED;
  p.page_table = page_table;
  p.n_comp = n_comp;
  p.q_pos = q_pos;
  p.q_seq = q_seq;
  p.scores = scores;
  p.n_visible = n_visible;
  p.ld = ld_scores;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.max_pages = max_pages;
  p.B = B;
  p.T = T;
  p.H_I = H_I;
  p.D_I = D_I;
  p.ratio_m = ratio_m;
  // entries per workgroup (and the grid) are chosen by the launcher
  if ((int64_t)T * ceil_div(std::min<int64_t>(ld_scores, (int64_t)max_pages * page_size), 256) >= ((int64_t)1 << 31))
    return CSA_ERR_UNSUPPORTED;
  return launch_status(launch_index_scores(p, (hipStream_t)stream));
}

int csa_index_scores(const uint8_t* q_idx, float q_idx_scale, const float* w, const uint8_t* k_idx,
                     float k_idx_scale, const int32_t* page_table, const int32_t* n_comp, int32_t num_pages,
                     int32_t page_size, int32_t max_pages, int32_t B, const int32_t* q_pos, const int32_t* q_seq,
                     int32_t T, int32_t H_I, int32_t D_I, int32_t ratio_m, float* scores, int64_t ld_scores,
                     int32_t* n_visible, void* stream) {
  if (T < 0) return CSA_ERR_INVALID_ARG;
  if (T == 0) return CSA_OK;
  if (!(q_idx_scale > 0.0f) || !(k_idx_scale > 0.0f) || !std::isfinite(q_idx_scale) || !std::isfinite(k_idx_scale))
    return CSA_ERR_INVALID_ARG;
  IndexParams p{};
  p.q_idx = q_idx;
  p.w = w;
  p.k_idx = k_idx;
  p.qk_scale = q_idx_scale * k_idx_scale;
  return index_scores_common(p, page_table, n_comp, num_pages, page_size, max_pages, B, q_pos, q_seq, T, H_I, D_I,
                             ratio_m, scores, ld_scores, n_visible, stream);
}

int csa_index_scores_mxfp4(const uint8_t* q_idx, const uint8_t* q_idx_sc, const float* w, const uint8_t* k_idx,
                           const uint8_t* k_idx_sc, const int32_t* page_table, const int32_t* n_comp,
                           int32_t num_pages, int32_t page_size, int32_t max_pages, int32_t B, const int32_t* q_pos,
                           const int32_t* q_seq, int32_t T, int32_t H_I, int32_t D_I, int32_t ratio_m,
                           float* scores, int64_t ld_scores, int32_t* n_visible, void* stream) {
  if (T < 0) return CSA_ERR_INVALID_ARG;
  if (T == 0) return CSA_OK;
  if (!q_idx_sc || !k_idx_sc) return CSA_ERR_INVALID_ARG;
  IndexParams p{};
  p.q_idx = q_idx;
  p.w = w;
  p.k_idx = k_idx;
  p.q_sc = q_idx_sc;
  p.k_sc = k_idx_sc;
  p.fp4 = 1;
  p.qk_scale = 1.0f;
  return index_scores_common(p, page_table, n_comp, num_pages, page_size, max_pages, B, q_pos, q_seq, T, H_I, D_I,
                             ratio_m, scores, ld_scores, n_visible, stream);
}

size_t csa_index_topk_workspace_size(int32_t T, int64_t max_entries, int32_t k) {
  if (T < 1 || max_entries < 1 || k < 1 || k > kTopkMaxK) return CSA_WORKSPACE_UNSUPPORTED;
  const TopkPlan pl = plan_index_topk(T, max_entries, k);
  if (!pl.ok) return CSA_WORKSPACE_UNSUPPORTED;
  // one sequence may take the many-query plan (B is not an argument here)
  const TopkPlan pm = plan_index_topk_prefill(T, max_entries, k);
  return pm.ok ? std::max(pl.ws_bytes, pm.ws_bytes) : pl.ws_bytes;
}

int csa_index_topk(const uint8_t* q_idx, float q_idx_scale, const float* w, const uint8_t* k_idx, float k_idx_scale,
                   const int32_t* page_table, const int32_t* n_comp, int32_t num_pages, int32_t page_size,
                   int32_t max_pages, int32_t B, const int32_t* q_pos, const int32_t* q_seq, int32_t T, int32_t H_I,
                   int32_t D_I, int32_t ratio_m, int32_t k, int32_t* topk_idx, int32_t* n_visible, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (T < 0) return CSA_ERR_INVALID_ARG;
  if (T == 0) return CSA_OK;
  if (!q_idx || !w || !k_idx || !page_table || !n_comp || !q_pos || !topk_idx || !n_visible)
    return CSA_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(k_idx)) return CSA_ERR_INVALID_ARG;
  if (B < 1 || num_pages < 1 || page_size < 16 || page_size % 16 || max_pages < 1 || ratio_m < 1)
    return CSA_ERR_INVALID_ARG;
  if (!(q_idx_scale > 0.0f) || !(k_idx_scale > 0.0f) || !std::isfinite(q_idx_scale) || !std::isfinite(k_idx_scale))
    return CSA_ERR_INVALID_ARG;
  if (H_I < 1 || H_I > 64 || !(D_I == 32 || D_I == 64 || D_I == 96 || D_I == 128)) return CSA_ERR_UNSUPPORTED;
  if (k < 1 || k > kTopkMaxK) return CSA_ERR_UNSUPPORTED;
  const int64_t span = (int64_t)max_pages * page_size;
  const TopkPlan pl0 = plan_index_topk(T, span, k);
  if (!pl0.ok) return CSA_ERR_UNSUPPORTED;
  const TopkPlan pm = B == 1 ? plan_index_topk_prefill(T, span, k) : TopkPlan();
  const TopkPlan& pl = pm.ok ? pm : pl0;
  if (pl.n_chunks > 1 && (!workspace || !aligned16(workspace) || workspace_bytes < pl.ws_bytes))
    return CSA_ERR_WORKSPACE;
  if ((int64_t)T * pl.n_chunks >= ((int64_t)1 << 31)) return CSA_ERR_UNSUPPORTED;
  IndexParams p{};
  p.q_idx = q_idx;
  p.w = w;
  p.k_idx = k_idx;
  p.qk_scale = q_idx_scale * k_idx_scale;
  p.page_table = page_table;
  p.n_comp = n_comp;
  p.q_pos = q_pos;
  p.q_seq = q_seq;
  p.n_visible = n_visible;
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.max_pages = max_pages;
  p.B = B;
  p.T = T;
  p.H_I = H_I;
  p.D_I = D_I;
  p.ratio_m = ratio_m;
  TopkParams tp{};
  tp.out = topk_idx;
  tp.T = T;
  tp.k = k;
  tp.chunk = pl.chunk;
  tp.n_chunks = pl.n_chunks;
  if (pl.n_chunks > 1) {
    tp.cand_key = static_cast<uint32_t*>(workspace);
    tp.cand_idx = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + pl.ws_bytes / 2);
  }
  // rows see at most the page table's entries (as csa_index_scores with
  // ld_scores = max_pages * page_size)
  p.ld = span;
  if (pm.ok) return launch_status(launch_index_topk_prefill(p, tp, (hipStream_t)stream));
  return launch_status(launch_index_topk(p, tp, (hipStream_t)stream));
}

size_t csa_topk_workspace_size(int32_t T, int64_t ld_scores, int32_t k) {
  if (T < 1 || ld_scores < 1 || k < 1 || k > kTopkMaxK) return CSA_WORKSPACE_UNSUPPORTED;
  const TopkPlan pl = plan_topk(T, ld_scores, k);
  return pl.ok ? pl.ws_bytes : CSA_WORKSPACE_UNSUPPORTED;
}

int csa_topk(const float* scores, int64_t ld_scores, const int32_t* n_visible, int32_t T, int32_t k,
             int32_t* topk_idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0) return CSA_ERR_INVALID_ARG;
  if (T == 0) return CSA_OK;
  if (!scores || !n_visible || !topk_idx || ld_scores < 1) return CSA_ERR_INVALID_ARG;
  if (k < 1 || k > kTopkMaxK) return CSA_ERR_UNSUPPORTED;
  const TopkPlan pl = plan_topk(T, ld_scores, k);
  if (!pl.ok) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)T * pl.n_chunks >= ((int64_t)1 << 31)) return CSA_ERR_UNSUPPORTED;
  if (pl.n_chunks > 1 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)))
    return CSA_ERR_WORKSPACE;
  TopkParams p{};
  p.scores = scores;
  p.n_visible = n_visible;
  p.out = topk_idx;
  p.ld = ld_scores;
  p.T = T;
  p.k = k;
  p.chunk = pl.chunk;
  p.n_chunks = pl.n_chunks;
  if (pl.n_chunks > 1) {
    p.cand_key = static_cast<uint32_t*>(workspace);
    p.cand_idx = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + pl.ws_bytes / 2);
  }
  return launch_status(launch_topk(p, (hipStream_t)stream));
}

size_t csa_attn_workspace_size(int32_t n_queries, int32_t H, int32_t D_nope, int32_t D_rope,
                               int32_t max_keys_per_query) {
  if (n_queries < 1 || H < 1 || !dims_supported(D_nope, D_rope) || max_keys_per_query < 0)
    return CSA_WORKSPACE_UNSUPPORTED;
  AttnPlan pl;
  if (!plan_attn(n_queries, H, D_nope + D_rope, max_keys_per_query, 0, false, &pl)) return CSA_WORKSPACE_UNSUPPORTED;
  return pl.ws_bytes;
}

// inverse RoPE base: 0 (no rotation) or a finite value > 0
static bool rope_theta_ok(float theta) { return theta == 0.0f || (std::isfinite(theta) && theta > 0.0f); }
static void set_inv_rope(AttnParams& p, float theta) {
  p.inv_rope = theta > 0.0f ? 1 : 0;
  p.rope_log2_theta = theta > 0.0f ? std::log2((double)theta) : 0.0;
}

static int run_attn(AttnParams& p, int64_t max_slots, void* workspace, size_t workspace_bytes, void* stream) {
  p.sm_log2 = p.sm_scale * 1.4426950408889634f;
  p.pscale = std::ldexp(1.0f, 8 - kAttnTau);
  p.inv_pscale = std::ldexp(1.0f, kAttnTau - 8);
  p.lat_over_swa = p.lat_scale / p.swa_scale;
  // division by the page size as a multiply-shift: with l = ceil(log2 d),
  // M = ceil(2^(32 + l) / d) has M d - 2^(32 + l) < d <= 2^l, so
  // floor(n M / 2^(32 + l)) == floor(n / d) for every n < 2^31
  {
    int l = 0;
    while ((1LL << l) < p.page_size) ++l;
    const unsigned __int128 num = (unsigned __int128)1 << (32 + l);
    p.ps_magic = (uint64_t)((num + (unsigned)p.page_size - 1) / (unsigned)p.page_size);
    p.ps_shift = 32 + l;
  }
  if (max_slots + kAttnTile - 1 > (int64_t)kAttnMaxSplits * kAttnMaxSlots) return CSA_ERR_UNSUPPORTED;
  AttnPlan pl;
  const size_t avail = (workspace && aligned16(workspace)) ? workspace_bytes : 0;
  if (!plan_attn(p.T, p.H, p.D_nope + p.D_rope, max_slots, avail, true, &pl)) return CSA_ERR_WORKSPACE;
  p.ht = pl.ht;
  p.n_hg = pl.n_hg;
  p.n_splits = pl.n_splits;
  p.per_split = pl.per_split;
  p.part = pl.n_splits > 1 ? static_cast<uint8_t*>(workspace) : nullptr;
  const int64_t blocks = (p.T >= 8 ? ceil_div(p.T, 8) * 8 : (int64_t)p.T) * p.n_hg * p.n_splits;
  if (blocks >= ((int64_t)1 << 31)) return CSA_ERR_UNSUPPORTED;
  return launch_status(launch_attn(p, (hipStream_t)stream));
}

// Checks and launch of csa_decode_attn and csa_decode_attn_noalloc; the
// scratch of the latter is resolved only once the arguments are known good.
// The top-k scores of csa_topk_decode_attn (the selection runs inside the
// attention kernel); nullptr scores for the other decode calls.
struct FusedTopk {
  const float* scores = nullptr;
  int64_t ld = 0;
  const int32_t* n_visible = nullptr;
  int32_t* topk_out = nullptr;
};

static int decode_attn(const uint16_t* q, int64_t q_stride, const csa_latent_cache* cache, const int32_t* topk_idx,
                       int32_t k, const csa_swa_ring* swa, const int32_t* q_pos, const float* sink,
                       float softmax_scale, float inv_rope_theta, int32_t B, int32_t H, uint16_t* out, float* lse,
                       void* workspace, size_t workspace_bytes, bool use_scratch, void* stream,
                       const FusedTopk& ft = FusedTopk()) {
  if (B < 0 || H < 1) return CSA_ERR_INVALID_ARG;
  if (B == 0) return CSA_OK;
  int rc = check_cache(cache);
  if (rc != CSA_OK) return rc;
  if (B > cache->num_seqs) return CSA_ERR_INVALID_ARG;
  if (!q || !q_pos || !sink || !out || !swa || !swa->nope || !swa->rope || !swa->pos) return CSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(swa->nope) || !aligned16(swa->rope)) return CSA_ERR_INVALID_ARG;
  const int D = cache->D_nope + cache->D_rope;
  if (q_stride < (int64_t)H * D || q_stride % 8) return CSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(swa->nope_scale > 0.0f) || !std::isfinite(swa->nope_scale))
    return CSA_ERR_INVALID_ARG;
  if (!rope_theta_ok(inv_rope_theta)) return CSA_ERR_INVALID_ARG;
  if (swa->W < 1 || swa->W > 1024) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)B * swa->W >= (int64_t)1 << 30) return CSA_ERR_UNSUPPORTED;
  if (topk_idx && (k < 0 || k > kTopkMaxK)) return CSA_ERR_UNSUPPORTED;
  AttnParams p{};
  p.q = q;
  p.q_stride = q_stride;
  p.lat_nope = cache->nope;
  p.lat_rope = cache->rope;
  p.page_table = cache->page_table;
  p.n_comp = cache->n_comp;
  p.topk = topk_idx;
  p.scores = ft.scores;
  p.ld_scores = ft.ld;
  p.n_visible = ft.n_visible;
  p.topk_out = ft.topk_out;
  p.swa_nope = swa->nope;
  p.swa_rope = swa->rope;
  p.swa_pos = swa->pos;
  p.q_pos = q_pos;
  p.sink = sink;
  p.out = out;
  p.lse = lse;
  p.lat_scale = cache->nope_scale;
  p.swa_scale = swa->nope_scale;
  p.sm_scale = softmax_scale;
  set_inv_rope(p, inv_rope_theta);
  p.num_pages = cache->num_pages;
  p.page_size = cache->page_size;
  p.max_pages = cache->max_pages;
  p.ratio_m = cache->ratio_m;
  p.k = (topk_idx || ft.scores) ? k : 0;
  p.W = swa->W;
  p.prefill_seq = -1;
  p.T = B;
  p.H = H;
  p.D_nope = cache->D_nope;
  p.D_rope = cache->D_rope;
  const int64_t max_slots =
      ((topk_idx || ft.scores) ? (int64_t)k : (int64_t)cache->max_pages * cache->page_size) + swa->W;
  if (use_scratch) {
    if (attn_scratch_address(&workspace) != hipSuccess) return CSA_ERR_LAUNCH;
    workspace_bytes = kAttnScratchBytes;
    const int rc = run_attn(p, max_slots, workspace, workspace_bytes, stream);
    return rc == CSA_ERR_WORKSPACE ? CSA_ERR_TOO_LARGE : rc;
  }
  return run_attn(p, max_slots, workspace, workspace_bytes, stream);
}

int csa_decode_attn(const uint16_t* q, int64_t q_stride, const csa_latent_cache* cache, const int32_t* topk_idx,
                    int32_t k, const csa_swa_ring* swa, const int32_t* q_pos, const float* sink,
                    float softmax_scale, float inv_rope_theta, int32_t B, int32_t H, uint16_t* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_attn(q, q_stride, cache, topk_idx, k, swa, q_pos, sink, softmax_scale, inv_rope_theta, B, H, out, lse,
                     workspace, workspace_bytes, false, stream);
}

int csa_topk_decode_attn(const float* scores, int64_t ld_scores, const int32_t* n_visible, int32_t k,
                         int32_t* topk_idx, const uint16_t* q, int64_t q_stride, const csa_latent_cache* cache,
                         const csa_swa_ring* swa, const int32_t* q_pos, const float* sink, float softmax_scale,
                         float inv_rope_theta, int32_t B, int32_t H, uint16_t* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (B < 0) return CSA_ERR_INVALID_ARG;
  if (B == 0) return CSA_OK;
  if (!scores || !n_visible || ld_scores < 1) return CSA_ERR_INVALID_ARG;
  if (k < 1 || k > kTopkMaxK || ld_scores > kAttnSelMax) return CSA_ERR_UNSUPPORTED;
  FusedTopk ft;
  ft.scores = scores;
  ft.ld = ld_scores;
  ft.n_visible = n_visible;
  ft.topk_out = topk_idx;
  return decode_attn(q, q_stride, cache, nullptr, k, swa, q_pos, sink, softmax_scale, inv_rope_theta, B, H, out, lse,
                     workspace, workspace_bytes, false, stream, ft);
}

int csa_decode_attn_noalloc(const uint16_t* q, int64_t q_stride, const csa_latent_cache* cache,
                            const int32_t* topk_idx, int32_t k, const csa_swa_ring* swa, const int32_t* q_pos,
                            const float* sink, float softmax_scale, float inv_rope_theta, int32_t B, int32_t H,
                            uint16_t* out, float* lse, void* stream) {
  return decode_attn(q, q_stride, cache, topk_idx, k, swa, q_pos, sink, softmax_scale, inv_rope_theta, B, H, out, lse,
                     nullptr, 0, true, stream);
}

int csa_prefill_attn(const uint16_t* q, int64_t q_stride, const csa_latent_cache* cache, int32_t seq,
                     const int32_t* topk_idx, int32_t k, const uint8_t* swa_nope, const uint16_t* swa_rope,
                     float swa_scale, int32_t swa_first_pos, int32_t swa_len, int32_t W, const int32_t* q_pos,
                     int32_t T, const float* sink, float softmax_scale, float inv_rope_theta, int32_t H,
                     uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || H < 1 || seq < 0 || swa_len < 0) return CSA_ERR_INVALID_ARG;
  if (T == 0) return CSA_OK;
  int rc = check_cache(cache);
  if (rc != CSA_OK) return rc;
  if (seq >= cache->num_seqs) return CSA_ERR_INVALID_ARG;
  if (!q || !q_pos || !sink || !out) return CSA_ERR_INVALID_ARG;
  if (swa_len > 0 && (!swa_nope || !swa_rope || !aligned16(swa_nope) || !aligned16(swa_rope)))
    return CSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return CSA_ERR_INVALID_ARG;
  const int D = cache->D_nope + cache->D_rope;
  if (q_stride < (int64_t)H * D || q_stride % 8) return CSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !rope_theta_ok(inv_rope_theta)) return CSA_ERR_INVALID_ARG;
  if (swa_len > 0 && (!(swa_scale > 0.0f) || !std::isfinite(swa_scale))) return CSA_ERR_INVALID_ARG;
  if (W < 1 || W > 1024) return CSA_ERR_UNSUPPORTED;
  if (swa_len >= (1 << 30)) return CSA_ERR_UNSUPPORTED;
  if (topk_idx && (k < 0 || k > kTopkMaxK)) return CSA_ERR_UNSUPPORTED;
  AttnParams p{};
  p.q = q;
  p.q_stride = q_stride;
  p.lat_nope = cache->nope;
  p.lat_rope = cache->rope;
  p.page_table = cache->page_table;
  p.n_comp = cache->n_comp;
  p.topk = topk_idx;
  p.swa_nope = swa_nope;
  p.swa_rope = swa_rope;
  p.swa_pos = nullptr;
  p.q_pos = q_pos;
  p.sink = sink;
  p.out = out;
  p.lse = lse;
  p.lat_scale = cache->nope_scale;
  p.swa_scale = swa_len > 0 ? swa_scale : cache->nope_scale;
  p.sm_scale = softmax_scale;
  set_inv_rope(p, inv_rope_theta);
  p.num_pages = cache->num_pages;
  p.page_size = cache->page_size;
  p.max_pages = cache->max_pages;
  p.ratio_m = cache->ratio_m;
  p.k = topk_idx ? k : 0;
  p.W = W;
  p.prefill_seq = seq;
  p.swa_first_pos = swa_first_pos;
  p.swa_len = swa_len;
  p.T = T;
  p.H = H;
  p.D_nope = cache->D_nope;
  p.D_rope = cache->D_rope;
  const int64_t max_slots = (topk_idx ? (int64_t)k : (int64_t)cache->max_pages * cache->page_size) + W;
  return run_attn(p, max_slots, workspace, workspace_bytes, stream);
}

// ---- graph capture of a whole step ("ROADMAP -- Stage E ...", E9: a
// decode step free of synchronisation is captured once and replayed; the
// calls above never allocate or synchronise, so a sequence of them can be
// recorded as it is) --------------------------------------------------------
struct csa_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

int csa_graph_capture_begin(void* stream) {
  if (!stream) return CSA_ERR_INVALID_ARG;   // the legacy default stream cannot be captured
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &st) != hipSuccess) return CSA_ERR_INVALID_ARG;
  if (st != hipStreamCaptureStatusNone) return CSA_ERR_INVALID_ARG;
  return hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal) == hipSuccess
             ? CSA_OK
             : CSA_ERR_LAUNCH;
}

int csa_graph_capture_end(void* stream, csa_graph** graph) {
  if (!stream || !graph) return CSA_ERR_INVALID_ARG;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture((hipStream_t)stream, &g) != hipSuccess || !g) {
    (void)hipGetLastError();   // a failed capture leaves its error behind; it is reported here
    if (g) (void)hipGraphDestroy(g);
    return CSA_ERR_LAUNCH;
  }
  hipGraphExec_t ex = nullptr;
  if (hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess || !ex) {
    (void)hipGetLastError();
    (void)hipGraphDestroy(g);
    return CSA_ERR_LAUNCH;
  }
  csa_graph* h = new (std::nothrow) csa_graph{g, ex};
  if (!h) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return CSA_ERR_LAUNCH;
  }
  *graph = h;
  return CSA_OK;
}

int csa_graph_launch(const csa_graph* graph, void* stream) {
  if (!graph) return CSA_ERR_INVALID_ARG;
  return hipGraphLaunch(graph->exec, (hipStream_t)stream) == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

void csa_graph_destroy(csa_graph* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

}  // extern "C"
