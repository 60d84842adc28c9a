// Host-side checks of libcsa's C ABI: argument validation and launch
// planning (chunking of the top-k, key-range splits of the attention,
// workspace sizing), built with csa_abi.cpp and the launcher stand-ins of
// launch_stubs.cpp under AddressSanitizer and UndefinedBehaviorSanitizer.
// No GPU is touched: every device pointer is an aligned stand-in address
// that the host code only checks, never dereferences.  Exit status 0 when
// every check holds.
#include <cstdint>
#include <cstdio>

#include "csa.h"
#include "launch_stubs.h"

using namespace csa;

static int g_fail = 0;
#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      if (++g_fail <= 20) {                                           \
        fprintf(stderr, "FAIL line %d: %s: ", __LINE__, #cond);       \
        fprintf(stderr, __VA_ARGS__);                                 \
        fprintf(stderr, "\n");                                        \
      }                                                               \
    }                                                                 \
  } while (0)

static void* dev(uint64_t i) { return reinterpret_cast<void*>((uint64_t(1) << 36) + (i << 12)); }

struct Rng {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return uint32_t(s >> 33);
  }
  int64_t range(int64_t lo, int64_t hi) { return lo + int64_t(next() % uint64_t(hi - lo + 1)); }
};

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

static void invalid_arguments() {
  // null pointers, negative sizes, bad scales: rejected before any launch
  const int before = g_stub.n_index + g_stub.n_topk + g_stub.n_attn + g_stub.n_index_topk;
  auto* u8 = static_cast<const uint8_t*>(dev(1));
  auto* f = static_cast<const float*>(dev(2));
  auto* i32 = static_cast<const int32_t*>(dev(3));
  CHECK(csa_index_scores(nullptr, 1.f, f, u8, 1.f, i32, i32, 4, 64, 2, 1, i32, nullptr, 4, 64, 128, 4,
                         (float*)dev(4), 256, (int32_t*)dev(5), nullptr) == CSA_ERR_INVALID_ARG, "null q_idx");
  CHECK(csa_index_scores(u8, 0.f, f, u8, 1.f, i32, i32, 4, 64, 2, 1, i32, nullptr, 4, 64, 128, 4, (float*)dev(4),
                         256, (int32_t*)dev(5), nullptr) == CSA_ERR_INVALID_ARG, "zero scale");
  CHECK(csa_index_scores(u8, 1.f, f, u8, 1.f, i32, i32, 4, 64, 2, 1, i32, nullptr, -1, 64, 128, 4, (float*)dev(4),
                         256, (int32_t*)dev(5), nullptr) == CSA_ERR_INVALID_ARG, "negative T");
  CHECK(csa_index_scores(u8 + 4, 1.f, f, u8, 1.f, i32, i32, 4, 64, 2, 1, i32, nullptr, 4, 64, 128, 4,
                         (float*)dev(4), 256, (int32_t*)dev(5), nullptr) == CSA_ERR_INVALID_ARG, "misaligned q_idx");
  CHECK(csa_topk(nullptr, 64, i32, 4, 16, (int32_t*)dev(6), nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG, "null scores");
  CHECK(csa_topk(f, 0, i32, 4, 16, (int32_t*)dev(6), nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG, "ld 0");
  csa_latent_cache cache{u8, (const uint16_t*)dev(7), 1.f, i32, i32, 2, 8, 64, 4, 448, 64, 4};
  csa_swa_ring ring{u8, (const uint16_t*)dev(8), 1.f, i32, 128};
  const float nan = __builtin_nanf("");
  CHECK(csa_decode_attn((const uint16_t*)dev(9), 512 * 128, &cache, i32, 16, &ring, i32, f, nan, 0.f, 2, 128,
                        (uint16_t*)dev(10), nullptr, nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG, "NaN softmax scale");
  cache.nope_scale = -1.f;
  CHECK(csa_decode_attn((const uint16_t*)dev(9), 512 * 128, &cache, i32, 16, &ring, i32, f, 0.04f, 0.f, 2, 128,
                        (uint16_t*)dev(10), nullptr, nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG, "negative cache scale");
  cache.nope_scale = 1.f;
  CHECK(csa_decode_attn((const uint16_t*)dev(9), 512 * 128, &cache, i32, 16, nullptr, i32, f, 0.04f, 0.f, 2, 128,
                        (uint16_t*)dev(10), nullptr, nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG, "null ring");
  CHECK(csa_decode_attn_noalloc((const uint16_t*)dev(9), 512 * 128, nullptr, i32, 16, &ring, i32, f, 0.04f, 0.f, 2,
                                128, (uint16_t*)dev(10), nullptr, nullptr) == CSA_ERR_INVALID_ARG, "null cache");
  CHECK(csa_prefill_attn((const uint16_t*)dev(9), 512 * 128, &cache, 5, i32, 16, u8, (const uint16_t*)dev(8), 1.f,
                         0, 100, 128, i32, 4, f, 0.04f, 0.f, 128, (uint16_t*)dev(10), nullptr, nullptr, 0,
                         nullptr) == CSA_ERR_INVALID_ARG, "prefill sequence beyond the cache");
  const int after = g_stub.n_index + g_stub.n_topk + g_stub.n_attn + g_stub.n_index_topk;
  CHECK(before == after, "an invalid call reached a launcher");
}

// Attention planning over random shapes: the reported workspace suffices,
// the split covers every key slot, and a smaller workspace either fits a
// coarser split or is refused.
static void attention_plans(Rng& rng, bool prefill) {
  for (int iter = 0; iter < 4000; ++iter) {
    const bool tiny = rng.next() & 1;
    const int dn = tiny ? 48 : 448, dr = tiny ? 16 : 64, D = dn + dr;
    const int hs[] = {1, 8, 40, 128, 200};
    const int H = hs[rng.range(0, 4)];
    const int T = (int)rng.range(1, prefill ? 4096 : 1200);
    const bool hca = rng.next() % 3 == 0;
    const int ps = 16 * (int)rng.range(1, 8);
    const int maxp = (int)rng.range(1, hca ? 3000 : 64);
    const int k = hca ? 0 : (int)rng.range(0, 2048);
    const int W = (int)rng.range(1, 1024);
    const int num_seqs = prefill ? (int)rng.range(1, 4) : T + (int)rng.range(0, 3);
    csa_latent_cache cache{(const uint8_t*)dev(11), (const uint16_t*)dev(12), 0.7f, (const int32_t*)dev(13),
                           (const int32_t*)dev(14), num_seqs, (int32_t)rng.range(1, 1 << 16), ps, maxp, dn, dr,
                           hca ? 128 : 4};
    const int64_t max_sel = hca ? (int64_t)maxp * ps : k;
    const int64_t max_keys = max_sel + W;
    const size_t ws = csa_attn_workspace_size(T, H, dn, dr, (int32_t)max_keys);
    const int32_t* topk = hca ? nullptr : (const int32_t*)dev(15);
    csa_swa_ring ring{(const uint8_t*)dev(16), (const uint16_t*)dev(17), 0.3f, (const int32_t*)dev(18), W};
    auto call = [&](void* wsp, size_t wsb) {
      if (prefill)
        return csa_prefill_attn((const uint16_t*)dev(19), (int64_t)H * D, &cache, 0, topk, k, (const uint8_t*)dev(16),
                                (const uint16_t*)dev(17), 0.3f, 1000, 2000, W, (const int32_t*)dev(20), T,
                                (const float*)dev(21), 0.04f, 0.f, H, (uint16_t*)dev(22), (float*)dev(23), wsp, wsb,
                                nullptr);
      return csa_decode_attn((const uint16_t*)dev(19), (int64_t)H * D, &cache, topk, k, &ring, (const int32_t*)dev(20),
                             (const float*)dev(21), 0.04f, 0.f, T, H, (uint16_t*)dev(22), (float*)dev(23), wsp, wsb,
                             nullptr);
    };
    const int64_t need_slots = round_up(max_sel, kAttnTile) + W;
    const int n0 = g_stub.n_attn;
    if (ws == CSA_WORKSPACE_UNSUPPORTED) {
      CHECK(call(dev(24), size_t(1) << 40) == CSA_ERR_UNSUPPORTED, "T %d H %d slots %lld", T, H, (long long)need_slots);
      CHECK(g_stub.n_attn == n0, "unsupported shape launched");
      continue;
    }
    const int rc = call(ws ? dev(24) : nullptr, ws);
    CHECK(rc == CSA_OK, "rc %d T %d H %d k %d W %d maxp %d ps %d", rc, T, H, k, W, maxp, ps);
    if (rc != CSA_OK) continue;
    const AttnParams& a = g_stub.attn;
    CHECK(a.n_splits >= 1 && a.n_splits <= kAttnMaxSplits, "splits %d", a.n_splits);
    CHECK(a.per_split > 0 && a.per_split % kAttnTile == 0 && a.per_split <= kAttnMaxSlots, "per_split %d", a.per_split);
    CHECK((int64_t)a.n_splits * a.per_split >= need_slots, "splits %d x %d < %lld slots", a.n_splits, a.per_split,
          (long long)need_slots);
    CHECK((a.n_splits == 1) == (a.part == nullptr), "partials pointer");
    CHECK((a.ht == 2 || a.ht == 4) && a.n_hg * 16 * a.ht >= H, "head groups");
    const uint64_t part_bytes = (uint64_t)a.n_splits * T * H * part_row_bytes(D);
    CHECK(a.n_splits == 1 || part_bytes <= ws, "partials %llu > workspace %zu", (unsigned long long)part_bytes, ws);
    // half the workspace: a coarser split that fits, or refused
    if (ws > 0) {
      const size_t half = ws / 2 / 16 * 16;
      const int rc2 = call(half ? dev(24) : nullptr, half);
      CHECK(rc2 == CSA_OK || rc2 == CSA_ERR_WORKSPACE, "rc2 %d", rc2);
      if (rc2 == CSA_OK) {
        const AttnParams& b = g_stub.attn;
        const uint64_t pb = (uint64_t)b.n_splits * T * H * part_row_bytes(D);
        CHECK(b.n_splits == 1 ? half == 0 || true : pb <= half, "coarser partials %llu > %zu", (unsigned long long)pb,
              half);
        CHECK((int64_t)b.n_splits * b.per_split >= need_slots && b.per_split <= kAttnMaxSlots, "coarser split");
      }
    }
    if (!prefill) {
      // the allocation-free variant: the library's 16 MiB array instead of a workspace
      const int rc3 = csa_decode_attn_noalloc((const uint16_t*)dev(19), (int64_t)H * D, &cache, topk, k, &ring,
                                              (const int32_t*)dev(20), (const float*)dev(21), 0.04f, 0.f, T, H,
                                              (uint16_t*)dev(22), (float*)dev(23), nullptr);
      // the fewest splits the planner can use: the selected slots may be
      // padded by up to a tile
      const int64_t plan_slots = max_keys + kAttnTile - 1;
      const uint64_t min_part = (uint64_t)((plan_slots + kAttnMaxSlots - 1) / kAttnMaxSlots) * T * H * part_row_bytes(D);
      if (rc3 == CSA_OK) {
        const AttnParams& c = g_stub.attn;
        CHECK(c.n_splits == 1 || (uint64_t)c.n_splits * T * H * part_row_bytes(D) <= CSA_NOALLOC_SCRATCH_BYTES,
              "no-alloc partials beyond the scratch");
      } else {
        CHECK(rc3 == CSA_ERR_TOO_LARGE && min_part > CSA_NOALLOC_SCRATCH_BYTES,
              "no-alloc rc %d: T %d H %d D %d keys %lld, minimum partials %llu", rc3, T, H, D, (long long)max_keys,
              (unsigned long long)min_part);
      }
    }
  }
}

static void topk_plans(Rng& rng) {
  for (int iter = 0; iter < 4000; ++iter) {
    const int T = (int)rng.range(1, 5000);
    const int64_t ld = rng.range(1, 1 << 21);
    const int k = (int)rng.range(1, 2100);
    const size_t ws = csa_topk_workspace_size(T, ld, k);
    const int rc = csa_topk((const float*)dev(30), ld, (const int32_t*)dev(31), T, k, (int32_t*)dev(32),
                            ws && ws != CSA_WORKSPACE_UNSUPPORTED ? dev(33) : nullptr,
                            ws == CSA_WORKSPACE_UNSUPPORTED ? 0 : ws, nullptr);
    if (k > kTopkMaxK) {
      CHECK(ws == CSA_WORKSPACE_UNSUPPORTED && rc == CSA_ERR_UNSUPPORTED, "k %d", k);
      continue;
    }
    if (ws == CSA_WORKSPACE_UNSUPPORTED) {
      CHECK(rc == CSA_ERR_UNSUPPORTED, "rc %d for unsupported T %d ld %lld k %d", rc, T, (long long)ld, k);
      continue;
    }
    CHECK(rc == CSA_OK || rc == CSA_ERR_UNSUPPORTED, "rc %d", rc);
    if (rc != CSA_OK) continue;
    const TopkParams& t = g_stub.topk;
    CHECK((int64_t)t.chunk * t.n_chunks >= ld && t.chunk <= kTopkMaxChunk, "chunks %d x %d < ld %lld", t.chunk,
          t.n_chunks, (long long)ld);
    if (t.n_chunks > 1) {
      CHECK((int64_t)t.n_chunks * k <= kTopkMaxCand, "candidates");
      CHECK((uint64_t)T * t.n_chunks * k * 8 <= ws, "candidate bytes beyond the workspace");
      CHECK((uint8_t*)t.cand_idx - (uint8_t*)t.cand_key == (ptrdiff_t)(ws / 2), "candidate halves");
    } else {
      CHECK(ws == 0, "workspace asked for a single chunk");
    }
  }
}

static void index_plans(Rng& rng) {
  for (int iter = 0; iter < 3000; ++iter) {
    const int T = (int)rng.range(1, 3000);
    const int HI = (int)rng.range(1, 70);
    const int dis[] = {16, 32, 64, 96, 128, 160};
    const int DI = dis[rng.range(0, 5)];
    const int ps = 16 * (int)rng.range(1, 8);
    const int maxp = (int)rng.range(1, 4000);
    const int64_t ld = rng.range(1, (int64_t)maxp * ps + 64);
    const bool supported = HI <= 64 && (DI == 32 || DI == 64 || DI == 96 || DI == 128);
    const int rc = csa_index_scores((const uint8_t*)dev(40), 0.5f, (const float*)dev(41), (const uint8_t*)dev(42), 0.25f,
                                    (const int32_t*)dev(43), (const int32_t*)dev(44), 1000, ps, maxp, 3,
                                    (const int32_t*)dev(45), nullptr, T, HI, DI, 4, (float*)dev(46), ld,
                                    (int32_t*)dev(47), nullptr);
    CHECK(supported ? rc == CSA_OK : rc == CSA_ERR_UNSUPPORTED, "rc %d HI %d DI %d", rc, HI, DI);
    if (rc == CSA_OK) {
      const IndexParams& p = g_stub.index;
      CHECK(p.T == T && p.ld == ld && p.H_I == HI && p.D_I == DI && p.qk_scale == 0.125f, "index params");
    }
    // fused indexer + top-k (one sequence: possibly the many-query plan)
    const int k = (int)(rng.range(0, 1) ? rng.range(1, 2100) : rng.range(1, 1100));
    const int B = rng.range(0, 1) ? 1 : 3;
    const int64_t span = (int64_t)maxp * ps;
    const size_t ws = csa_index_topk_workspace_size(T, span, k);
    const int np0 = g_stub.n_index_topk_prefill;
    const int rc2 = csa_index_topk((const uint8_t*)dev(40), 0.5f, (const float*)dev(41), (const uint8_t*)dev(42), 0.25f,
                                   (const int32_t*)dev(43), (const int32_t*)dev(44), 1000, ps, maxp, B,
                                   (const int32_t*)dev(45), nullptr, T, HI, DI, 4, k, (int32_t*)dev(48),
                                   (int32_t*)dev(47), ws && ws != CSA_WORKSPACE_UNSUPPORTED ? dev(49) : nullptr,
                                   ws == CSA_WORKSPACE_UNSUPPORTED ? 0 : ws, nullptr);
    if (!supported || ws == CSA_WORKSPACE_UNSUPPORTED) {
      CHECK(rc2 == CSA_ERR_UNSUPPORTED, "fused rc %d", rc2);
    } else {
      CHECK(rc2 == CSA_OK || rc2 == CSA_ERR_UNSUPPORTED, "fused rc %d", rc2);
      if (rc2 == CSA_OK) {
        const TopkParams& t = g_stub.topk;
        const bool many = g_stub.n_index_topk_prefill != np0;
        CHECK(many == (B == 1 && T >= 16 && k <= kIndexTopkPrefillMaxK && span <= kIndexTopkPrefillMaxSpan),
              "plan choice B %d T %d k %d span %lld", B, T, k, (long long)span);
        CHECK(g_stub.index.ld == span, "fused key range");
        CHECK((int64_t)t.chunk * t.n_chunks >= span, "fused chunks");
        CHECK(t.n_chunks == 1 || (uint64_t)T * t.n_chunks * k * 8 <= ws, "fused candidates beyond the workspace");
        CHECK((int64_t)t.n_chunks * k <= kTopkMaxCand || t.n_chunks == 1, "merge input beyond its capacity");
      }
    }
  }
}

// Steps 2-4 in one call: rows up to 8192 scores, k up to 2048; the
// attention plan is csa_decode_attn's with k selected slots.
static void topk_attention_plans(Rng& rng) {
  for (int iter = 0; iter < 2000; ++iter) {
    const int B = (int)rng.range(1, 600);
    const int H = 128, dn = 448, dr = 64, D = dn + dr;
    const int64_t ld = rng.range(1, 9000);
    const int k = (int)rng.range(1, 2100);
    const int W = (int)rng.range(1, 1024);
    csa_latent_cache cache{(const uint8_t*)dev(60), (const uint16_t*)dev(61), 0.7f, (const int32_t*)dev(62),
                           (const int32_t*)dev(63), B, 4096, 64, 128, dn, dr, 4};
    csa_swa_ring ring{(const uint8_t*)dev(64), (const uint16_t*)dev(65), 0.3f, (const int32_t*)dev(66), W};
    const bool ok_shape = ld <= kAttnSelMax && k <= kTopkMaxK;
    const size_t ws = ok_shape ? csa_attn_workspace_size(B, H, dn, dr, k + W) : 0;
    const int n0 = g_stub.n_attn;
    const int rc = csa_topk_decode_attn((const float*)dev(67), ld, (const int32_t*)dev(68), k, (int32_t*)dev(69),
                                        (const uint16_t*)dev(70), (int64_t)H * D, &cache, &ring,
                                        (const int32_t*)dev(71), (const float*)dev(72), 0.04f, 0.f, B, H,
                                        (uint16_t*)dev(73), nullptr, ws ? dev(74) : nullptr, ws, nullptr);
    if (!ok_shape) {
      CHECK(rc == CSA_ERR_UNSUPPORTED && g_stub.n_attn == n0, "ld %lld k %d rc %d", (long long)ld, k, rc);
      continue;
    }
    CHECK(rc == CSA_OK, "rc %d", rc);
    if (rc != CSA_OK) continue;
    const AttnParams& a = g_stub.attn;
    CHECK(a.scores == dev(67) && a.ld_scores == ld && a.topk == nullptr && a.k == k && a.topk_out == dev(69),
          "fused top-k parameters");
    CHECK((int64_t)a.n_splits * a.per_split >= round_up(k, kAttnTile) + W, "fused split covers the slots");
  }
}

int main() {
  Rng rng{20260};
  invalid_arguments();
  attention_plans(rng, false);
  attention_plans(rng, true);
  topk_plans(rng);
  index_plans(rng);
  topk_attention_plans(rng);
  CHECK(g_stub.n_index_topk_prefill > 0, "the many-query fused plan was never taken");
  printf("host ABI checks: %d failures (attention launches %d, top-k %d, indexer %d, fused %d)\n", g_fail,
         g_stub.n_attn, g_stub.n_topk, g_stub.n_index, g_stub.n_index_topk);
  return g_fail ? 1 : 0;
}
