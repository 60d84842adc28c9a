// Steps 3+4 of the CSA path: gather of the selected compressed latents plus
// the sliding window, and shared-latent attention with a per-head sink.
//
// Sources:
//  "DSV4 Inference Kernel", Architecture: the latent (T, 512) is shared by all
//    128 query heads (key = value), sink weights merge the sparse and SWA
//    attention.
//  "DSV4 Audit -- Decode Repetition + Precision / Tensor-Core Plan", A3: the
//    query attends [top-k compressed entries] ++ [SWA window]; B1: FP8 nope
//    dims go to the matrix units without a BF16 dequantised copy, q is
//    quantised to FP8, the 64 rope dims stay BF16.
//  "ROADMAP -- Stage E ...", E1: one fused gather straight from the paged FP8
//    cache (no Python loop, no BF16 materialisation); E4: (o, lse); E5: batch
//    in the grid.
//
// Mapping on gfx950 (eight computing waves per workgroup, two per SIMD; in
// the decode shape a ninth wave only issues the tile copies):
//  * a workgroup owns one query, HT x 16 heads and a range of key slots (the
//    range is split over workgroups only when there are few queries);
//  * wave (ht, dp): heads [16 ht, 16 ht + 16) of the group and dim part dp of
//    ND parts of the latent.  Few queries: HT = 2, ND = 4 (part dp < 3 owns
//    nope block dp, part 3 the last 64 nope dims and the rope dims).  Many
//    queries: HT = 4, ND = 2 (dim halves).  Every 64-key tile is handled
//    whole by all parts of a head tile: each computes the scores over its own
//    dims, the partial score tiles are added through LDS in one fixed order,
//    all parts run the same online softmax (bit-identical state), and each
//    accumulates O for its own dims only.  O and q of a wave are a part of a
//    head tile's, which keeps a wave's registers small enough for two waves
//    per SIMD, and no merge of softmax states is needed at the end;
//  * gather: key descriptors (top-k index -> page table -> row, or window slot
//    -> row) are resolved once into LDS; each 64-key tile is copied from HBM
//    straight into LDS with global_load_lds_dwordx4 (no register staging),
//    three tiles in flight (ring of 3 buffers, prefetch distance 2).  The
//    tile is a grid of 256-byte blocks, each holding one 16-byte chunk of 16
//    keys; one DMA instruction fills four blocks (16 keys x 64 contiguous
//    bytes of their rows), so it touches 16 cache lines instead of 64, and
//    every lane keeps one key for all of its DMAs.  Inside a block the key
//    rows are XOR-ed with 8 on alternate blocks, which keeps the QK reads and
//    both transpose reads free of LDS bank conflicts.  Masked keys (padding,
//    invalid entries, the ragged tail) copy a static row of zeros, so no
//    operand needs a per-key mask.  The cache's FP8/BF16 bytes go to the MFMA
//    unchanged;
//  * QK: S^T (keys x heads) = X . Q^T on v_mfma 16x16x128 FP8, with q split
//    into two E4M3 terms hi + lo sharing a power-of-two per-head scale (the K
//    dimension is [hi | lo], X read once and used for both), plus the rope
//    dims on v_mfma 16x16x32 BF16; four 16-key subtiles in flight;
//  * online softmax in FP32, exp2 domain; each lane owns one head.  The
//    running max is raised lazily: only when a tile's max exceeds it by more
//    than 2^tau (tau = 4), so probabilities stay <= 2^tau and the O rescale
//    runs on few tiles.  The sink joins the max and the denominator in FP32
//    after the last tile, so P is always quantised relative to the largest
//    key logit, however large the sink;
//  * PV: O^T (dims x heads) += X^T . P^T on v_mfma 16x16x128 FP8 with
//    K = [64 keys, P hi | 64 keys, P lo] (P x 2^(8 - tau) as two E4M3 terms,
//    the keys' E4M3 codes unscaled; the key source's FP8 scale is applied in
//    FP32, with one rescale of the accumulators where the key range passes
//    from compressed entries to window rows); X^T comes from the same LDS tile through
//    ds_read_b64_tr_b8 (two reads per 16 dims, used for both terms).  Rope
//    dims use ds_read_b64_tr_b16 and v_mfma 16x16x32 BF16 with P in BF16.
//    Each dim part exponentiates and packs P for its own 16-key subtiles
//    only, and the parts swap those through LDS.
#include <mutex>

#include "csa_device.h"
#include "csa_internal.h"
#include "topk_select.h"

namespace csa {

namespace {

constexpr int kSwaFlag = 1 << 30;
constexpr int kNBuf = 3;

template <int DN, int DR>
struct Cfg {
  static constexpr int NFB = DN / 128;                       // full 128-dim nope blocks
  static constexpr int REM = DN % 128;                       // combined hi|lo block (<= 64 dims)
  static constexpr int NBLK = NFB + (REM > 0 ? 1 : 0);
  static constexpr int B0 = (NBLK + 1) / 2;                  // nope blocks of dim half 0 (ND = 2)
  static constexpr int CHN = DN / 16;                        // 16-byte nope chunks of a row
  static constexpr int CHR = DR / 8;                         // 16-byte rope chunks of a row
  static constexpr int CHNP = (CHN + 3) & ~3;                // padded to whole quads
  static constexpr int CHRP = (CHR + 3) & ~3;
  static constexpr int NQ = (CHNP + CHRP) / 4;               // quads = DMAs per wave per tile
  static constexpr int TILE_BYTES = NQ * 4 * 1024;
  static_assert(DN % 16 == 0 && DR % 16 == 0, "dims must be multiples of 16");
  static_assert(REM <= 64, "remainder block must fit one combined hi|lo MFMA");
};

// What dim part DP of ND (2 or 4) of a head tile owns: nope blocks
// [BB, BE) (128 dims each; block NFB is the combined hi|lo block of the last
// REM <= 64 nope dims) and, in the last part, the rope dims.  Two parts split
// the nope blocks in half; four parts take one nope block each.
template <int DN, int DR, int ND, int DP>
struct Part {
  using C = Cfg<DN, DR>;
  static_assert(ND == 2 || ND == 4, "two or four dim parts");
  static_assert(ND == 2 || C::NBLK == ND, "four parts take one nope block each");
  static constexpr bool LAST = DP == ND - 1;
  static constexpr int BB = ND == 2 ? (DP == 0 ? 0 : C::B0) : DP;
  static constexpr int BE = ND == 2 ? (DP == 0 ? C::B0 : C::NBLK) : DP + 1;
  static constexpr int FB = (BE < C::NFB ? BE : C::NFB) - (BB < C::NFB ? BB : C::NFB);   // full blocks
  static constexpr int FB0 = BB;                                         // first full block
  static constexpr bool COMB = C::REM > 0 && BB <= C::NFB && C::NFB < BE;
  static constexpr int NR = LAST ? (DR + 31) / 32 : 0;                   // rope k-steps of QK
  static constexpr int D0 = 128 * BB < DN ? 128 * BB : DN;               // nope dims [D0, D1)
  static constexpr int D1 = 128 * BE < DN ? 128 * BE : DN;
  static constexpr int PT0 = D0 / 16;                                    // first nope dim tile of PV
  static constexpr int NPT = (D1 - D0) / 16;
  static constexpr int NRT = LAST ? DR / 16 : 0;                         // rope dim tiles of PV
  static constexpr int NO = NPT + NRT;                                   // O accumulators
  static constexpr int NQB = FB + (COMB ? 1 : 0);
  static_assert(NO >= 1, "every dim part owns output dims");
};

// key (0..31) held by byte e (0..7) of a lane in 16-lane group g: the keys
// of the two 16-key subtiles that the QK output layout puts in that lane.
__device__ __forceinline__ int kappa(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }
// Byte offset of 16-byte chunk c of tile key k.  Block (q, rg, cc) =
// ((c / 4) * 4 + k / 16) * 4 + c % 4 holds chunk c of keys [16 rg, 16 rg + 16);
// inside it key row k % 16 is XOR-ed with 8 when (k / 16 + c) is odd.  With
// q = c / 4, the four blocks (q, rg, 0..3) are one contiguous KB: the target
// of one DMA instruction.
__device__ __forceinline__ int chunk_off(int k, int c) {
  const int rg = k >> 4;
  return ((((c >> 2) << 2) + rg) * 4 + (c & 3)) * 256 + 16 * ((k & 15) ^ (((rg ^ c) & 1) << 3));
}
// chunk_off(k, c) - chunk_base(c) for keys k = 16 st + row: the part that
// depends on the key (c enters only through its parity)
__device__ __forceinline__ int chunk_base(int c) { return (((c >> 2) << 4) + (c & 3)) * 256; }
__device__ __forceinline__ int key_part(int k, int parity) {
  const int rg = k >> 4;
  return rg * 1024 + 16 * ((k & 15) ^ (((rg ^ parity) & 1) << 3));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// One global_load_lds_dwordx4: every lane copies 16 bytes from `src` to LDS
// byte address lds_base + 16 * lane.  Issued through asm so that the
// compiler's wait-count pass does not see an LDS write in flight: left to
// itself it drains vmcnt before every later LDS access, which would wait for
// the prefetched tiles too.  The kernel orders these copies itself (wait_vmcnt
// + barrier before a tile is read; a buffer is refilled only after the
// barrier that follows its last read).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ int page_div(int n, const AttnParams& p) {
  return (int)(((uint64_t)(uint32_t)n * p.ps_magic) >> p.ps_shift);
}

// Source of the tile rows of masked keys.
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[512] = {};

struct Block {
  int t, hg, split, seq;
  int pos, nc;
  int n_sel, sel_end, kv0, nkeys;   // slots: [0, n_sel) selected, [sel_end, sel_end + W) window
};

template <int DN, int DR, int DP, int HT, int ND, bool kProd>
__device__ __forceinline__ void attn_wave(const AttnParams& p, const Block& bk, uint8_t* xs0, int32_t* desc,
                                          v4f* sx, v2i* pxh, v2i* pxb, int wave, const int32_t* sel) {
  using C = Cfg<DN, DR>;
  using HF = Part<DN, DR, ND, DP>;
  constexpr int D = DN + DR;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int r = lane & 15;
  constexpr int kWaves = ND * HT;             // waves (head tile, dim part): wave = DP * HT + ht
  constexpr int kThreads = 64 * kWaves;
  const int ht = wave % HT;
  const int h = bk.hg * (16 * HT) + ht * 16 + r;
  const bool tile_ok = bk.hg * (16 * HT) + ht * 16 < p.H;
  const bool head_ok = h < p.H;
  const bool prefill = p.prefill_seq >= 0;
  const int t = bk.t, seq = bk.seq, kv0 = bk.kv0, nkeys = bk.nkeys, n_sel = bk.n_sel, sel_end = bk.sel_end;

  // ---- query rows of this dim part (packed BF16), issued first so that
  // their latency overlaps the descriptor round trips
  v4i qraw[HF::NQB > 0 ? HF::NQB : 1][4];
  v4i qrope[HF::NR > 0 ? HF::NR : 1];
  {
    const uint16_t* qrow = p.q + (size_t)t * p.q_stride + (size_t)h * D;
#pragma unroll
    for (int b = 0; b < HF::NQB; ++b) {
      const bool comb = b == HF::FB;
      const int d0 = comb ? 128 * C::NFB + 32 * (g & 1) : 128 * (HF::FB0 + b) + 32 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int dd = d0 + 8 * c;
        v4i raw = (v4i){0, 0, 0, 0};
        if (head_ok && dd < DN) raw = ld16(qrow + dd);
        qraw[b][c] = raw;
      }
    }
#pragma unroll
    for (int rr = 0; rr < HF::NR; ++rr) {
      const int dd = 32 * rr + 8 * g;
      v4i raw = (v4i){0, 0, 0, 0};
      if (head_ok && dd < DR) raw = ld16(qrow + DN + dd);
      qrope[rr] = raw;
    }
  }
  const float sink_raw = head_ok ? p.sink[h] : 0.0f;

  // ---- key descriptors of this workgroup's slots: row | source flag, -1 =
  // skip.  First-level loads (top-k index or ring position) need nothing
  // loaded before them; then all page-table loads: two round trips.
  const int32_t* pt = p.page_table + (size_t)seq * p.max_pages;
  constexpr int kSPT = kAttnMaxSlots / kThreads;   // slots per thread
  int v1[kSPT];
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + kThreads * j;
    const int slot = kv0 + s;
    int v = -1;
    if (s < nkeys) {
      if (slot < n_sel) {
        v = sel ? sel[slot] : p.topk ? p.topk[(size_t)t * p.k + slot] : slot;
      } else if (slot >= sel_end && !prefill) {
        v = p.swa_pos[(size_t)seq * p.W + (slot - sel_end)];
      }
    }
    v1[j] = v;
  }
  int v2[kSPT];
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + kThreads * j;
    const int idx = v1[j];
    int page = -1;
    if (s < nkeys && kv0 + s < n_sel && idx >= 0) {
      const int pi = page_div(idx, p);
      if (pi < p.max_pages) page = pt[pi];
    }
    v2[j] = page;
  }
  const int pos = bk.pos;
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + kThreads * j;
    if (s >= nkeys) continue;
    const int slot = kv0 + s;
    int d = -1;
    if (slot < n_sel) {
      const int idx = v1[j], page = v2[j];
      if (idx < bk.nc && page >= 0 && page < p.num_pages)
        d = page * p.page_size + (idx - page_div(idx, p) * p.page_size);
    } else if (slot >= sel_end) {
      const int jw = slot - sel_end;
      if (!prefill) {
        const int pp = v1[j];
        if (pp >= 0 && pp <= pos && pp > pos - p.W) d = (seq * p.W + jw) | kSwaFlag;
      } else {
        const int pp = pos - p.W + 1 + jw;
        if (pp >= 0 && pp >= p.swa_first_pos && pp - p.swa_first_pos < p.swa_len)
          d = (pp - p.swa_first_pos) | kSwaFlag;
      }
    }
    desc[s] = d;
  }

  __syncthreads();   // descriptors visible

  // ---- tile DMA: wave w fills the quads of keys [16 w, 16 w + 16); lane l
  // copies 16 bytes of chunk 4 q + l / 16 of key dkey into LDS byte
  // (q * 4 + w) * 1024 + 16 l.  Masked keys copy a row of zeros, so that
  // every wave issues the same number of DMAs per tile and those keys add
  // nothing to S or O.
  const int dcc = lane >> 4;
  const int drg = wave & 3;                   // row group (16 keys) this wave copies
  const int dq0 = wave >> 2;                  // first quad; then every kQStep-th
  const int dkey = 16 * drg + ((lane & 15) ^ (((drg ^ dcc) & 1) << 3));
  const uint8_t* tsrc_n = p.lat_nope;   // this lane's row of the tile being issued
  const uint8_t* tsrc_r = reinterpret_cast<const uint8_t*>(p.lat_rope);
  auto prep_tile = [&](int tile) {
    const int s = tile * kAttnTile + dkey;
    const int d = s < nkeys ? desc[s] : -1;
    const uint8_t* nsrc = kZeroRow;
    const uint8_t* rsrc = kZeroRow;
    if (d >= 0) {
      const size_t row = (size_t)(d & ~kSwaFlag);
      if (d & kSwaFlag) {
        nsrc = p.swa_nope + row * DN;
        rsrc = reinterpret_cast<const uint8_t*>(p.swa_rope + row * DR);
      } else {
        nsrc = p.lat_nope + row * DN;
        rsrc = reinterpret_cast<const uint8_t*>(p.lat_rope + row * DR);
      }
    }
    tsrc_n = nsrc;
    tsrc_r = rsrc;
  };
  constexpr int kQStep = kWaves / 4;                 // waves sharing a row group
  constexpr int kQMax = (C::NQ + kQStep - 1) / kQStep;  // quads per wave (at most)
  constexpr int kParts = 3;                          // a tile's DMAs go out in three parts
  constexpr int kPerPart = (kQMax + kParts - 1) / kParts;
  auto issue_quads = [&](int buf, int part) {
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(CSA_LDS uint8_t*)(xs0 + buf * C::TILE_BYTES) + (uint32_t)drg * 1024u;
#pragma unroll
    for (int q = 0; q < C::NQ; ++q) {
      if (q % kQStep != dq0) continue;
      if (part >= 0 && (q / kQStep) / kPerPart != part) continue;
      const int c = 4 * q + dcc;
      const uint8_t* src;
      if (4 * q < C::CHNP) {
        src = (C::CHN == C::CHNP || c < C::CHN) ? tsrc_n + 16 * c : tsrc_n;
      } else {
        const int cr = c - C::CHNP;
        src = (C::CHR == C::CHRP || cr < C::CHR) ? tsrc_r + 16 * cr : tsrc_r;
      }
      dma16(src, lds_base + q * 4096);
    }
  };

  const int n_tiles = (nkeys + kAttnTile - 1) / kAttnTile;
  if constexpr (!kProd) {   // with a producer wave, it issues every tile copy
    if (n_tiles > 0) {
      prep_tile(0);
      issue_quads(0, -1);
    }
    if (n_tiles > 1) {
      prep_tile(1);
      issue_quads(1, -1);
    }
  }

  // ---- query operands: q split into two E4M3 terms hi + lo with a shared
  // power-of-two per-head scale over this part's nope dims
  v8i qhi[HF::FB > 0 ? HF::FB : 1], qlo[HF::FB > 0 ? HF::FB : 1], qcomb;
  v8bf qr[HF::NR > 0 ? HF::NR : 1];
  float cq = 0.0f;
  const float cr = p.sm_log2;
  {
    auto qval = [&](int b, int c, int e) -> float {
      const uint32_t w = (uint32_t)qraw[b][c][e >> 1];
      return bf16_bits_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
    };
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b < HF::NQB; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(qval(b, c, e)));
    amax = max_over_groups(amax);
    const float s = e4m3_pow2_scale(amax);
    const float inv = 1.0f / s;
    cq = head_ok ? cr * s : 0.0f;
#pragma unroll
    for (int b = 0; b < HF::NQB; ++b) {
      v8i hi, lo;
#pragma unroll
      for (int w4 = 0; w4 < 8; ++w4) {
        float x[4], res[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = qval(b, w4 >> 1, 4 * (w4 & 1) + e) * inv;
        const int hw = pack4_fp8(x[0], x[1], x[2], x[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = x[e] - fp8_to_f32(hw, e);
        hi[w4] = hw;
        lo[w4] = pack4_fp8(res[0], res[1], res[2], res[3]);
      }
      if (b < HF::FB) {
        qhi[b] = hi;
        qlo[b] = lo;
      } else {
        qcomb = (g < 2) ? hi : lo;
      }
    }
#pragma unroll
    for (int rr = 0; rr < HF::NR; ++rr) qr[rr] = __builtin_bit_cast(v8bf, qrope[rr]);
  }
  const float cql = cq * p.lat_scale, cqs = cq * p.swa_scale;

  // ---- softmax state (exp2 domain), identical in every dim part.  The sink
  // stays out of the running max: the probabilities are quantised relative to
  // the largest key logit, and the sink joins the max and the denominator in
  // FP32 at the end (split 0 only).
  const bool sink_here = bk.split == 0 && head_ok;
  const float sink2 = head_ok ? sink_raw * kLog2e : -__builtin_inff();
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  // The FP8 accumulator holds p x (E4M3 code) in the unit of one key source's
  // scale: the compressed entries' until the first window tile, whose arrival
  // rescales the nope accumulators by lat_scale / swa_scale (tiles never mix
  // the two sources, and the window tiles come last).
  bool o_swa = kv0 >= sel_end;
  v4f O[HF::NO];
#pragma unroll
  for (int i = 0; i < HF::NO; ++i) O[i] = (v4f){0.f, 0.f, 0.f, 0.f};

  // loop-invariant per-lane parts of the LDS offsets
  int qk_off[4][2];                                          // key 16 st + r, chunk parity
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qk_off[st][0] = key_part(16 * st + r, 0);
    qk_off[st][1] = key_part(16 * st + r, 1);
  }
  const int qk_g = ((g >> 1) * 16 + 2 * (g & 1)) * 256;      // chunk_base(2 g) for the full blocks
  int pv_off[2][2];                                          // tr8 rows: keys 32 u + kappa(g, r / 2), parity
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    pv_off[u][0] = key_part(32 * u + kappa(g, r >> 1), 0) + 8 * (r & 1);
    pv_off[u][1] = key_part(32 * u + kappa(g, r >> 1), 1) + 8 * (r & 1);
  }
  const int rb_ = (r >> 1) & 1;                              // rope tr16: chunk parity of this lane
  int rp_off[2][2];                                          // [u][lo/hi key group]
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    rp_off[u][0] = rb_ * 256 + key_part(32 * u + kappa(g, r >> 2), rb_) + 8 * (r & 1);
    rp_off[u][1] = rb_ * 256 + key_part(32 * u + kappa(g, 4 + (r >> 2)), rb_) + 8 * (r & 1);
  }
  v4f* sx_own = sx + (size_t)wave * 4 * 64 + lane;
  const v4f* sx_tile = sx + (size_t)ht * 4 * 64 + lane;   // part dp of this head tile at + dp HT 4 64

  // ---- one tile's steps
  v4f acc[4], racc[4];
  // QK: partial scores over this part's dims of the tile in buffer xq
  auto qk = [&](const uint8_t* xq) {
    // -- partial scores over this part's dims: four 16-key subtiles; the
    //    operands of the next step are read before the MFMAs of this one
    // (no branch on the head tile: a tile beyond H has zero q rows, and the
    // branch would make the compiler clear the accumulators with moves)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      acc[st] = (v4f){0.f, 0.f, 0.f, 0.f};
      racc[st] = acc[st];
    }
    {
      constexpr int NSTEP = HF::FB + (HF::COMB ? 1 : 0);
      auto read_step = [&](int step, v8i (&x)[4]) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (step < HF::FB) {
            // chunks 8 (FB0 + step) + 2 g and + 1 (even, odd)
            const uint8_t* base = xq + (HF::FB0 + step) * 8192 + qk_g;
            const v4i lo = *reinterpret_cast<const v4i*>(base + qk_off[st][0]);
            const v4i hi = *reinterpret_cast<const v4i*>(base + 256 + qk_off[st][1]);
            x[st] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            // chunks 8 NFB + 2 (g & 1) and + 1
            const uint8_t* base = xq + C::NFB * 8192 + 512 * (g & 1);
            v4i lo = (v4i){0, 0, 0, 0}, hi = lo;
            if (32 * (g & 1) < C::REM) lo = *reinterpret_cast<const v4i*>(base + qk_off[st][0]);
            if (32 * (g & 1) + 16 < C::REM) hi = *reinterpret_cast<const v4i*>(base + 256 + qk_off[st][1]);
            x[st] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
      };
      v8i x[2][4];
      v4i y[HF::NR > 0 ? HF::NR : 1][4];
      if (NSTEP > 0) read_step(0, x[0]);
#pragma unroll
      for (int rr = 0; rr < HF::NR; ++rr) {
        // rope chunk CHNP + 4 rr + g (parity g & 1)
        const uint8_t* base = xq + ((C::CHNP / 4 + rr) * 16 + g) * 256;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          y[rr][st] = (v4i){0, 0, 0, 0};
          if (32 * rr + 8 * g < DR) y[rr][st] = *reinterpret_cast<const v4i*>(base + qk_off[st][g & 1]);
        }
      }
#pragma unroll
      for (int step = 0; step < NSTEP; ++step) {
        if (step + 1 < NSTEP) read_step(step + 1, x[(step + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (step < HF::FB) {
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[st] = mfma_f8_128(x[step & 1][st], qhi[step], acc[st]);
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[st] = mfma_f8_128(x[step & 1][st], qlo[step], acc[st]);
        } else {
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[st] = mfma_f8_128(x[step & 1][st], qcomb, acc[st]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int rr = 0; rr < HF::NR; ++rr)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          racc[st] = mfma_bf16_32(__builtin_bit_cast(v8bf, y[rr][st]), qr[rr], racc[st]);
    }
  };
  // valid keys of tile `it` (the same in every wave): bit k = key k.  Masked
  // keys were copied from a zero row, so they add nothing to S or O; dim
  // part 0 gives them -inf in the exchanged score.
  auto tile_mask = [&](int it) -> uint64_t {
    const int sk = it * kAttnTile + lane;
    const int dk = sk < nkeys ? desc[sk] : -1;
    return __ballot(dk >= 0);
  };
  // own partial (scaled) of the exchanged score
  auto own_part = [&](uint64_t vmask, bool tile_swa, v4f (&part)[4]) {
    const bool full = vmask == ~0ull;
    // -- own partial (scaled), exchanged with the other dim parts of the
    //    head tile.  Part 0 also subtracts the running max (so the sum S' is
    //    the exp2 argument) and carries -inf for masked keys (lane keys
    //    16 st + 4 g + i).
    const float msub = (m_run == -__builtin_inff()) ? 0.0f : m_run;
    const float ks = tile_swa ? cqs : cql;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (DP == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[st][i] = __builtin_fmaf(acc[st][i], ks, -msub);
      } else {
        part[st] = acc[st] * ks + racc[st] * cr;
      }
    }
    if (DP == 0 && !full) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t vw = st < 2 ? (uint32_t)vmask : (uint32_t)(vmask >> 32);
        const uint32_t bits = vw >> (16 * (st & 1) + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((bits >> i) & 1u)) part[st][i] = -__builtin_inff();
      }
    }
  };
  // online softmax and PV of tile `it` (tot: the exchanged score, summed over
  // the dim parts in the same order in every part)
  // Each dim part exponentiates and packs the probabilities of its own
  // 16-key subtiles only (st % ND == dp; the max still comes from the whole
  // tile, so every part takes the same rescale decisions), and the parts swap
  // their P through LDS; the denominator is kept per part and summed at the
  // end.
  constexpr bool kSplitP = ND > 1;
  constexpr int kOwnSt = 4 / ND;   // subtiles per part
  // online softmax of tile `it` (tot: the exchanged score, summed over the
  // dim parts in the same order in every part); P of subtile st, when this
  // part computes it, is pq[st] = (hi, lo E4M3 of p x kq; p as two BF16 pairs)
  auto soft = [&](int it, const v4f (&tot)[4], float tmax, bool tile_swa, v4i (&pq)[4]) {
    const float msub = (m_run == -__builtin_inff()) ? 0.0f : m_run;   // as subtracted in own_part
    // -- lane: head h, keys 16 st + 4 g + i; tot = S - msub
    const bool m_inf = m_run == -__builtin_inff();
    const bool grow = m_inf ? (tmax > -__builtin_inff()) : (tmax > (float)kAttnTau);
    float delta = 0.0f;
    if (__ballot(grow)) {
      // raise the running max to the tile max on the lanes that grew
      delta = grow ? tmax : 0.0f;
      const float alpha = grow ? (m_inf ? 0.0f : __builtin_amdgcn_exp2f(-tmax)) : 1.0f;
      if (grow) m_run = msub + tmax;
      l_run *= alpha;
      if (it > 0) {
#pragma unroll
        for (int i = 0; i < HF::NO; ++i) O[i] *= alpha;
      }
    }
    const float kq = p.pscale;
    float psum = 0.0f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (kSplitP && st % ND != DP) continue;
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(tot[st][i] - delta);   // exp2(-inf) = 0 for masked keys
        psum += pr[i];
      }
      // nope operand bytes: hi of p x 2^(8 - tau), lo = the rounding
      // residual; rope operand: p in BF16
      const float x0 = pr[0] * kq, x1 = pr[1] * kq, x2 = pr[2] * kq, x3 = pr[3] * kq;
      const int w = pack4_fp8(x0, x1, x2, x3);
      const v2f b01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const v2f b23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      pq[st] = (v4i){w, pack4_fp8(x0 - b01[0], x1 - b01[1], x2 - b23[0], x3 - b23[1]),
                     (int)pack2_bf16(pr[0], pr[1]), (int)pack2_bf16(pr[2], pr[3])};
    }
    l_run += psum;
  };
  // PV of the tile in buffer xb with the probabilities pq of all 16-key subtiles
  auto pv = [&](const uint8_t* xb, const v4i (&pq)[4]) {
    // -- B operand for nope: bytes [hi of the lane's 16 keys | lo of them]
    v8i pb;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      pb[st] = pq[st][0];
      pb[4 + st] = pq[st][1];
    }
    // -- PV: O^T[dims x heads] += X^T[dims x K] P^T[K x heads]; A = the
    //    two 8-key transpose reads, used for the hi and the lo half of K.
    //    Reads of the next batch go out before the MFMAs of this one.
    {
      constexpr int PB = 4;   // dim tiles per batch
      constexpr int NB = (HF::NPT + PB - 1) / PB;
      v2i ra[2][PB], rb[2][PB];
      auto read_batch = [&](int bt, v2i (&a)[PB], v2i (&b)[PB]) {
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int dt = bt * PB + j;
          if (dt < HF::NPT) {
            const int c = HF::PT0 + dt;
            const uint8_t* cb = xb + chunk_base(c);
            a[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CSA_LDS v2i*)(cb + pv_off[0][c & 1]));
            b[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CSA_LDS v2i*)(cb + pv_off[1][c & 1]));
          }
        }
      };
      if (NB > 0) read_batch(0, ra[0], rb[0]);
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        if (bt + 1 < NB) read_batch(bt + 1, ra[(bt + 1) & 1], rb[(bt + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const int dt = bt * PB + j;
          if (dt < HF::NPT) {
            const v2i a0 = ra[bt & 1][j], a1 = rb[bt & 1][j];
            const v8i a = (v8i){a0[0], a0[1], a1[0], a1[1], a0[0], a0[1], a1[0], a1[1]};
            O[dt] = mfma_f8_128(a, pb, O[dt]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (HF::NRT > 0) {
      // rope, BF16: MFMA u covers keys 32 u + kappa(g, 0..7); rope dim tile
      // j = chunks CHNP + 2 j (+1)
      v4i pbf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) pbf[u] = (v4i){pq[2 * u][2], pq[2 * u][3], pq[2 * u + 1][2], pq[2 * u + 1][3]};
      v4i ya[HF::NRT > 0 ? HF::NRT : 1][2];
#pragma unroll
      for (int j = 0; j < HF::NRT; ++j) {
        const uint8_t* cb = xb + ((C::CHNP / 4 + (j >> 1)) * 16 + 2 * (j & 1)) * 256;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const v2i lo = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(cb + rp_off[u][0])));
          const v2i hi = __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(cb + rp_off[u][1])));
          ya[j][u] = (v4i){lo[0], lo[1], hi[0], hi[1]};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < HF::NRT; ++j)
          O[HF::NPT + j] = mfma_bf16_32(__builtin_bit_cast(v8bf, ya[j][u]), __builtin_bit_cast(v8bf, pbf[u]),
                                        O[HF::NPT + j]);
    }
  };

  // ---- the tiles: a barrier for each tile's arrival and one for the score
  // exchange; the other waves on the SIMD hide each other's latencies
  int buf = 0;
  for (int it = 0; it < n_tiles; ++it, buf = (buf + 1 == kNBuf) ? 0 : buf + 1) {
    // tile `it` landed in LDS (this wave's DMAs), then everyone's (barrier);
    // the barrier also retires every wave's reads of the buffer reused next
    asm volatile("" ::: "memory");
    if constexpr (!kProd) {
      if (it + 1 < n_tiles) wait_vmcnt<C::NQ / kQStep>(); else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool refill = !kProd && it + 2 < n_tiles;
    const int nbuf = buf == 0 ? 2 : buf - 1;
    if (refill) {
      prep_tile(it + 2);
      issue_quads(nbuf, 0);
    }
    const uint8_t* xb = xs0 + buf * C::TILE_BYTES;
    const uint64_t vmask = tile_mask(it);
    const bool tile_swa = kv0 + it * kAttnTile >= sel_end;
    qk(xb);
    v4f part[4];
    own_part(vmask, tile_swa, part);
#pragma unroll
    for (int st = 0; st < 4; ++st) sx_own[st * 64] = part[st];
    if (refill) issue_quads(nbuf, 1);
    lds_barrier();
    // the scores of this part's own subtiles (four parts) or of all of them
    // (two): the parts' partials (own from registers, the others from LDS)
    // summed in one fixed order
    constexpr bool kSplitMax = ND == 4;
    v4f tot[4];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (kSplitMax && st % ND != DP) continue;
      v4f pp[ND];
#pragma unroll
      for (int dp = 0; dp < ND; ++dp) pp[dp] = dp == DP ? part[st] : sx_tile[(dp * HT * 4 + st) * 64];
      tot[st] = ND == 2 ? pp[0] + pp[1] : (pp[0] + pp[1]) + (pp[ND - 2] + pp[ND - 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, tot[st][i]);
    }
    float tmax = max_over_groups(mloc);
    if constexpr (kSplitMax) {
      // the tile max over the parts, swapped through this part's slot of its
      // own subtile DP, which no other part reads (one more barrier, for 36
      // fewer adds)
      *reinterpret_cast<float*>(sx_own + DP * 64) = tmax;
      lds_barrier();
#pragma unroll
      for (int dp = 0; dp < ND; ++dp)
        if (dp != DP) tmax = fmaxf(tmax, *reinterpret_cast<const float*>(sx_tile + (dp * HT * 4 + dp) * 64));
    }
    v4i pq[4];
    soft(it, tot, tmax, tile_swa, pq);
    if constexpr (kSplitP) {
      // this part's subtiles of P to LDS (E4M3 hi/lo for every part; BF16,
      // used by the rope dims, for the last part only), the other parts' back
#pragma unroll
      for (int j = 0; j < kOwnSt; ++j) {
        const int st = DP + ND * j;
        pxh[(wave * kOwnSt + j) * 64 + lane] = (v2i){pq[st][0], pq[st][1]};
        if (!HF::LAST) pxb[((ht * (ND - 1) + DP) * kOwnSt + j) * 64 + lane] = (v2i){pq[st][2], pq[st][3]};
      }
      lds_barrier();
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int dq = st % ND, j = st / ND;
        if (dq == DP) continue;
        const v2i hl = pxh[((dq * HT + ht) * kOwnSt + j) * 64 + lane];
        pq[st][0] = hl[0];
        pq[st][1] = hl[1];
        if (HF::LAST) {
          const v2i bf = pxb[((ht * (ND - 1) + dq) * kOwnSt + j) * 64 + lane];
          pq[st][2] = bf[0];
          pq[st][3] = bf[1];
        }
      }
    }
    if (tile_swa && !o_swa) {
      // first window tile: the nope accumulators change unit (uniform branch,
      // taken at most once)
#pragma unroll
      for (int i = 0; i < HF::NPT; ++i) O[i] *= p.lat_over_swa;
      o_swa = true;
    }
    __builtin_amdgcn_sched_barrier(0);
    pv(xb, pq);
    if (refill) issue_quads(nbuf, 2);
  }
  // the denominator: per part with split P (summed here over the parts in
  // one order; the exchange buffer is free once the last tile's P is)
  float L = sum_over_groups(l_run);
  if constexpr (kSplitP) {
    float* lx = reinterpret_cast<float*>(sx);
    lx[wave * 64 + lane] = L;
    lds_barrier();
    float lp[ND];
#pragma unroll
    for (int dp = 0; dp < ND; ++dp) lp[dp] = lx[(dp * HT + ht) * 64 + lane];
    L = ND == 2 ? lp[0] + lp[1] : (lp[0] + lp[1]) + (lp[ND - 2] + lp[ND - 1]);
  }
  if (!tile_ok) return;

  // ---- the sink joins the max and the denominator (split 0): M = max(m, sink),
  // O and L rescaled by 2^(m - M), plus 2^(sink - M) in L
  float M = m_run, oscale = 1.0f;
  if (sink_here) {
    const float Ms = fmaxf(m_run, sink2);
    if (Ms > -__builtin_inff()) {
      oscale = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - Ms);
      L = L * oscale + __builtin_amdgcn_exp2f(sink2 - Ms);
      M = Ms;
    }
  }
  const float nope_unit = (o_swa ? p.swa_scale : p.lat_scale) * p.inv_pscale * oscale;

  // ---- output of this part's dims (the softmax state is the same in every part)
  const bool final_out = p.n_splits == 1;
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
  // inverse RoPE of the rope dims at the query position, when this
  // workgroup writes the final output (split outputs are rotated by the
  // merge).  Lane i < DR / 2 forms the rotation of pair i; every lane then
  // fetches the two pairs of each of its rope tiles (dims 4g .. 4g + 3 of
  // tile j are pairs 8j + 2g and 8j + 2g + 1), outside the head branch so
  // that every lane takes part in the swaps.
  float2 rcs[HF::NRT > 0 ? HF::NRT : 1][2];
  const bool rot = HF::LAST && final_out && p.inv_rope;
  if constexpr (HF::NRT > 0) {
    if (rot) {
      const float2 own = lane < DR / 2 ? inv_rope_cs(bk.pos, lane, DR, p.rope_log2_theta) : make_float2(1.0f, 0.0f);
#pragma unroll
      for (int j = 0; j < HF::NRT; ++j)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int pr = 8 * j + 2 * g + e;
          rcs[j][e] = make_float2(__shfl(own.x, pr, 64), __shfl(own.y, pr, 64));
        }
    }
  }
  if (head_ok) {
#pragma unroll
    for (int j = 0; j < HF::NO; ++j) {
      const bool nope = j < HF::NPT;
      const float unit = nope ? nope_unit : oscale;
      const int dim = nope ? 16 * (HF::PT0 + j) + 4 * g : DN + 16 * (j - HF::NPT) + 4 * g;
      v4f v = O[j] * unit;
      if constexpr (HF::NRT > 0) {
        if (!nope && rot) {
          const int jr = j >= HF::NPT ? j - HF::NPT : 0;
          const float2 a = rotate2(v[0], v[1], rcs[jr][0]);
          const float2 b = rotate2(v[2], v[3], rcs[jr][1]);
          v = (v4f){a.x, a.y, b.x, b.y};
        }
      }
      // the final output, or this split's output normalised by its own
      // denominator (BF16, like the output; the merge weighs it by L)
      const v2i pk = (v2i){(int)pack2_bf16(v[0] * invL, v[1] * invL), (int)pack2_bf16(v[2] * invL, v[3] * invL)};
      if (final_out) {
        *reinterpret_cast<v2i*>(p.out + ((size_t)t * p.H + h) * D + dim) = pk;
      } else {
        *reinterpret_cast<v2i*>(p.part + (((size_t)bk.split * p.T + t) * p.H + h) * part_row_bytes(D) + 2 * dim) = pk;
      }
    }
    if (DP == 0 && g == 0) {
      if (final_out) {
        if (p.lse) p.lse[(size_t)t * p.H + h] = (L > 0.0f) ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
      } else {
        float* dst = reinterpret_cast<float*>(p.part + (((size_t)bk.split * p.T + t) * p.H + h) * part_row_bytes(D) + 2 * D);
        dst[0] = M;
        dst[1] = L;
      }
    }
  }
}

// The DMA producer of a workgroup (one extra wave, decode shape): it issues
// every tile copy, so that the stalls of the per-CU limit on vector-memory
// instructions in flight fall on it and not on the waves that compute.  It
// copies the same 1 KB blocks the computing waves would (block (q, rg): 16
// keys of row group rg, 64 bytes of each, lane l one key and one 16-byte
// chunk), waits for a tile's copies before the tile's arrival barrier, and
// meets every barrier the computing waves execute: one after the
// descriptors, per tile the arrival, the score exchange, the tile max (four
// dim parts) and the P exchange, and the denominator exchange after the
// last tile.  A tile's 4 NQ copies go out in three parts, one after each
// of the arrival, score-exchange and P-exchange barriers (spread over the
// tile: c2 27.8 us, against 28.2 with two parts after the arrival and 29.4
// with all of them).
template <int DN, int DR, int ND>
__device__ __forceinline__ void attn_producer(const AttnParams& p, const Block& bk, uint8_t* xs0, const int32_t* desc) {
  using C = Cfg<DN, DR>;
  constexpr int kN = 4 * C::NQ;            // copies per tile
  static_assert(kN < 64, "a tile's copies fit the vmcnt range");
  constexpr int kPer = (kN + 2) / 3;
  const int lane = threadIdx.x & 63;
  const int dcc = lane >> 4;
  __syncthreads();   // the descriptors are visible
  const int nkeys = bk.nkeys;
  const int n_tiles = (nkeys + kAttnTile - 1) / kAttnTile;
  const uint8_t* sn[4];
  const uint8_t* sr[4];
  auto prep = [&](int tile) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int key = 16 * rg + ((lane & 15) ^ (((rg ^ dcc) & 1) << 3));
      const int s = tile * kAttnTile + key;
      const int d = s < nkeys ? desc[s] : -1;
      const uint8_t* nsrc = kZeroRow;
      const uint8_t* rsrc = kZeroRow;
      if (d >= 0) {
        const size_t row = (size_t)(d & ~kSwaFlag);
        if (d & kSwaFlag) {
          nsrc = p.swa_nope + row * DN;
          rsrc = reinterpret_cast<const uint8_t*>(p.swa_rope + row * DR);
        } else {
          nsrc = p.lat_nope + row * DN;
          rsrc = reinterpret_cast<const uint8_t*>(p.lat_rope + row * DR);
        }
      }
      sn[rg] = nsrc;
      sr[rg] = rsrc;
    }
  };
  auto issue = [&](int buf, int part) {
    const uint32_t base = (uint32_t)(uintptr_t)(CSA_LDS uint8_t*)(xs0 + buf * C::TILE_BYTES);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (part >= 0 && i / kPer != part) continue;
      const int q = i >> 2, rg = i & 3;
      const int c = 4 * q + dcc;
      const uint8_t* src;
      if (4 * q < C::CHNP) {
        src = (C::CHN == C::CHNP || c < C::CHN) ? sn[rg] + 16 * c : sn[rg];
      } else {
        const int cr = c - C::CHNP;
        src = (C::CHR == C::CHRP || cr < C::CHR) ? sr[rg] + 16 * cr : sr[rg];
      }
      dma16(src, base + (uint32_t)(q * 4096 + rg * 1024));
    }
  };
  if (n_tiles > 0) {
    prep(0);
    issue(0, -1);
  }
  if (n_tiles > 1) {
    prep(1);
    issue(1, -1);
  }
  int buf = 0;
  for (int it = 0; it < n_tiles; ++it, buf = (buf + 1 == kNBuf) ? 0 : buf + 1) {
    asm volatile("" ::: "memory");
    if (it + 1 < n_tiles) wait_vmcnt<kN>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();   // arrival; the buffer refilled next is retired
    asm volatile("" ::: "memory");
    const bool refill = it + 2 < n_tiles;
    const int nbuf = buf == 0 ? 2 : buf - 1;
    if (refill) {
      prep(it + 2);
      issue(nbuf, 0);
    }
    __builtin_amdgcn_s_barrier();                 // score exchange
    if (refill) issue(nbuf, 1);
    if constexpr (ND == 4) __builtin_amdgcn_s_barrier();   // tile max
    __builtin_amdgcn_s_barrier();                 // P exchange
    if (refill) issue(nbuf, 2);
  }
  __builtin_amdgcn_s_barrier();   // denominator exchange
}

// HT = 16-head tiles per workgroup, ND = dim parts per head tile; one wave
// per (tile, part), so ND * HT waves.  Few queries: HT = 2 with ND = 4 (eight
// waves on 32 heads, two per SIMD, so that one wave's softmax runs while the
// other's MFMAs do).  Enough (query, head group) pairs to fill the GPU
// without splitting key ranges: HT = 4 with ND = 2 (each tile shared by 64
// heads, again two waves per SIMD).
//
// kProd: one more wave, the DMA producer (the decode shape, when the
// workgroup does not select its own top-k).
template <int DN, int DR, int HT, int ND, bool kProd>
__global__ __launch_bounds__(64 * (ND * HT + (kProd ? 1 : 0)), 1) void attn_kernel(AttnParams p) {
  using C = Cfg<DN, DR>;
  // the tile ring (also the selection histograms of csa_topk_decode_attn
  // before the first tile, which need more than the small tiles' ring)
  constexpr size_t kRing = (size_t)kNBuf * C::TILE_BYTES;
  constexpr size_t kSelHist = sizeof(topk_sel::TopkShared<64 * ND * HT>);
  __shared__ __attribute__((aligned(16))) uint8_t xs[kRing > kSelHist ? kRing : (kSelHist + 15) / 16 * 16];
  __shared__ int32_t desc[kAttnMaxSlots];
  __shared__ v4f sx[ND * HT * 4 * 64];   // partial score tiles, [wave][subtile][lane]
  // each part's subtiles of P: E4M3 hi/lo [wave][subtile][lane]; BF16 of the
  // parts other than the last [ht][part][subtile][lane]
  __shared__ v2i pxh[ND * HT * (4 / ND) * 64];
  __shared__ v2i pxb[(ND > 1 ? HT * (ND - 1) * (4 / ND) : 1) * 64];

  // ---- which (query, head group, split).  Workgroups go to the 8 XCDs
  // round-robin by id.  With 8 or more queries, queries are spread over the
  // XCDs and all workgroups of one query share an XCD (and its L2, which then
  // serves the head groups' repeated reads of the same rows).  With 1, 2 or 4
  // queries each query takes 8 / T XCDs of its own, so its rows are fetched
  // into as few L2s as the CUs allow (c3 HCA 23.8 -> 22.9 us against
  // spreading every query over all eight); other counts spread them.
  const int nb = p.n_hg * p.n_splits;
  const int bid = blockIdx.x;
  Block bk;
  int jb;
  if (p.T >= 8) {
    const int local = bid >> 3;
    bk.t = (local / nb) * 8 + (bid & 7);
    jb = local % nb;
  } else if (8 % p.T == 0) {
    const int G = 8 / p.T;              // XCDs per query
    const int xcd = bid & 7;
    bk.t = xcd / G;
    jb = (bid >> 3) * G + (xcd - bk.t * G);
    if (jb >= nb) return;
  } else {
    bk.t = bid / nb;
    jb = bid - bk.t * nb;
  }
  if (bk.t >= p.T) return;
  bk.hg = jb / p.n_splits;
  bk.split = jb - bk.hg * p.n_splits;
  const bool prefill = p.prefill_seq >= 0;
  bk.seq = prefill ? p.prefill_seq : bk.t;
  bk.pos = p.q_pos[bk.t];
  bk.nc = p.n_comp[bk.seq];
  // with a top-k list the slot count needs nothing loaded, so the
  // descriptor loads need not wait for the position
  if (p.topk || p.scores) {
    bk.n_sel = p.k;
  } else {
    bk.n_sel = bk.pos >= 0 ? max(0, min(bk.pos / p.ratio_m, bk.nc)) : 0;
  }
  // the selected slots are padded to whole tiles, so that no tile mixes
  // compressed entries and window rows
  bk.sel_end = (bk.n_sel + kAttnTile - 1) & ~(kAttnTile - 1);
  const int n_slots = bk.sel_end + p.W;
  bk.kv0 = bk.split * p.per_split;
  if (bk.split > 0 && bk.kv0 >= n_slots) {
    // empty split: an empty state (M = -inf, L = 0), which the merge weighs
    // by zero without reading the split's output
    const int h = bk.hg * 16 * HT + (int)threadIdx.x;
    if ((int)threadIdx.x < 16 * HT && h < p.H) {
      constexpr int D = DN + DR;
      float* dst = reinterpret_cast<float*>(p.part + (((size_t)bk.split * p.T + bk.t) * p.H + h) * part_row_bytes(D) + 2 * D);
      dst[0] = -__builtin_inff();
      dst[1] = 0.0f;
    }
    return;
  }
  bk.nkeys = max(0, min(n_slots, bk.kv0 + p.per_split) - bk.kv0);

  // ---- top-k from the indexer scores (csa_topk_decode_attn): the
  // workgroup selects its query's top-k itself, with the top-k kernels'
  // radix selection (the same rule, so the same indices).  The histograms
  // live in the tile ring and the indices in the score-exchange buffer,
  // which hold nothing yet.
  const int32_t* sel = nullptr;
  if (!kProd && p.scores) {
    using namespace topk_sel;
    constexpr int kThreads = 64 * ND * HT;
    constexpr int kSelSeg = kAttnSelMax / kThreads;
    static_assert(sizeof(TopkShared<kThreads>) <= sizeof(xs), "selection histograms fit the tile ring");
    static_assert(kTopkMaxK * sizeof(int32_t) <= sizeof(sx), "selected indices fit the exchange buffer");
    auto& shs = *reinterpret_cast<TopkShared<kThreads>*>(xs);
    int32_t* selw = reinterpret_cast<int32_t*>(sx);
    const int t = bk.t;
    const int i0 = threadIdx.x * kSelSeg;
    const float* src = p.scores + (size_t)t * p.ld_scores + i0;
    const int nv_raw = p.n_visible[t];
    // loaded without waiting for the visible count; columns past it are
    // masked below
    const int avail = (int)max<int64_t>(0, min<int64_t>(kSelSeg, p.ld_scores - i0));
    uint32_t key[kSelSeg];
    if (avail == kSelSeg && ((((uintptr_t)src) & 15) == 0)) {
#pragma unroll
      for (int j = 0; j < kSelSeg; j += 4) {
        const v4f v = *reinterpret_cast<const v4f*>(src + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[j + e] = float_order_key(v[e]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelSeg; ++j) key[j] = j < avail ? float_order_key(src[j]) : 0u;
    }
    const int n = (int)max<int64_t>(0, min<int64_t>(nv_raw, p.ld_scores));
    const int cnt = max(0, min(kSelSeg, n - i0));
    const uint32_t valid = cnt >= 32 ? 0xffffffffu : ((1u << cnt) - 1u);
    const int K = min(p.k, n);
    if (K > 0) {
      const Sel sl = radix_select<kThreads, kSelSeg>(key, valid, K, shs);
      emit_selected<kThreads, kSelSeg>(key, valid, sl, shs, [&](int rank, int j) {
        if (rank < K) selw[rank] = i0 + j;
      });
    }
    for (int i = K + threadIdx.x; i < p.k; i += kThreads) selw[i] = -1;
    __syncthreads();
    // one workgroup of the query also hands the indices to the caller
    if (p.topk_out && bk.hg == 0 && bk.split == 0)
      for (int i = threadIdx.x; i < p.k; i += kThreads) p.topk_out[(size_t)t * p.k + i] = selw[i];
    sel = selw;
  }

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < ND * HT + (kProd ? 1 : 0));
  if constexpr (kProd) {
    if (wave == ND * HT) {
      attn_producer<DN, DR, ND>(p, bk, xs, desc);
      return;
    }
  }
  if constexpr (ND == 4) {
    if (wave >= 3 * HT)
      attn_wave<DN, DR, 3, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
    else if (wave >= 2 * HT)
      attn_wave<DN, DR, 2, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
    else if (wave >= HT)
      attn_wave<DN, DR, 1, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
    else
      attn_wave<DN, DR, 0, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
  } else {
    if (wave >= HT)
      attn_wave<DN, DR, 1, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
    else
      attn_wave<DN, DR, 0, HT, ND, kProd>(p, bk, xs, desc, sx, pxh, pxb, wave, sel);
  }
}

// Combines the per-split partial states (the split's output normalised by
// its denominator, in BF16; running max in log2 units; denominator) of every
// (query, head) into the output and lse.  Every split leaves a state (an
// empty split an empty one: M = -inf, L = 0), so the merge needs nothing
// but the partials.  128 threads per (query, head): thread i loads every
// split's (M, L) and dims [4 i, 4 i + 4) of every split's output at once
// (one round trip for up to kMergeRegs splits, two passes beyond), then
// weighs them in registers, the splits summed in order.
constexpr int kMergeRegs = 16;
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int D = p.D_nope + p.D_rope;
  const size_t RB = part_row_bytes(D);
  const int pair = blockIdx.x * 2 + (threadIdx.x >> 7);   // (query, head) of this thread's team
  const int sub = threadIdx.x & 127;
  if (pair >= p.T * p.H) return;
  const int t = pair / p.H;
  const int h = pair - t * p.H;
  const int n = p.n_splits;
  const int pos = p.inv_rope ? p.q_pos[t] : 0;
  const size_t pstride = (size_t)p.T * p.H * RB;   // one split (bytes)
  const uint8_t* row = p.part + ((size_t)t * p.H + h) * RB;
  const int d0 = 4 * sub;
  const bool dim_ok = d0 < D;
  auto unpack = [](v2i w) -> v4f {
    return (v4f){__uint_as_float((uint32_t)w[0] << 16), __uint_as_float((uint32_t)w[0] & 0xffff0000u),
                 __uint_as_float((uint32_t)w[1] << 16), __uint_as_float((uint32_t)w[1] & 0xffff0000u)};
  };
  // weight of a split against the merged max Ms: L_s 2^(M_s - Ms), zero for
  // an empty split (whose output row is never read into the sum)
  auto weight = [](float2 ml, float Ms) -> float {
    return ml.x == -__builtin_inff() ? 0.0f : ml.y * __builtin_amdgcn_exp2f(ml.x - Ms);
  };
  float M = -__builtin_inff(), L = 0.0f;
  v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
  if (n <= kMergeRegs) {
    float2 ml[kMergeRegs];
    v2i v[kMergeRegs];
#pragma unroll
    for (int s = 0; s < kMergeRegs; ++s) {
      if (s < n) {
        ml[s] = *reinterpret_cast<const float2*>(row + s * pstride + 2 * D);
        v[s] = dim_ok ? *reinterpret_cast<const v2i*>(row + s * pstride + 2 * d0) : (v2i){0, 0};
      }
    }
#pragma unroll
    for (int s = 0; s < kMergeRegs; ++s)
      if (s < n) M = fmaxf(M, ml[s].x);
    const float Ms = (M == -__builtin_inff()) ? 0.0f : M;
#pragma unroll
    for (int s = 0; s < kMergeRegs; ++s) {
      if (s < n) {
        const float w = weight(ml[s], Ms);
        L += w;
        if (w > 0.0f) acc += unpack(v[s]) * w;
      }
    }
  } else {
    for (int s = 0; s < n; ++s) M = fmaxf(M, reinterpret_cast<const float*>(row + s * pstride + 2 * D)[0]);
    const float Ms = (M == -__builtin_inff()) ? 0.0f : M;
    for (int s = 0; s < n; ++s) {
      const float w = weight(*reinterpret_cast<const float2*>(row + s * pstride + 2 * D), Ms);
      L += w;
      if (w > 0.0f && dim_ok) acc += unpack(*reinterpret_cast<const v2i*>(row + s * pstride + 2 * d0)) * w;
    }
  }
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
  if (dim_ok) {
    if (d0 >= p.D_nope && p.inv_rope) {
      // inverse RoPE of rope pairs (d0 - D_nope) / 2 and the next one
      const int pr = (d0 - p.D_nope) >> 1;
      const float2 a = rotate2(acc[0], acc[1], inv_rope_cs(pos, pr, p.D_rope, p.rope_log2_theta));
      const float2 b = rotate2(acc[2], acc[3], inv_rope_cs(pos, pr + 1, p.D_rope, p.rope_log2_theta));
      acc = (v4f){a.x, a.y, b.x, b.y};
    }
    *reinterpret_cast<v2i*>(p.out + ((size_t)t * p.H + h) * D + d0) =
        (v2i){(int)pack2_bf16(acc[0] * invL, acc[1] * invL), (int)pack2_bf16(acc[2] * invL, acc[3] * invL)};
  }
  if (sub == 0 && p.lse) p.lse[(size_t)t * p.H + h] = (L > 0.0f) ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
}

template <int DN, int DR>
hipError_t launch_attn_t(const AttnParams& p, hipStream_t stream) {
  const int nb = p.n_hg * p.n_splits;
  const int blocks = p.T >= 8 ? ((p.T + 7) / 8) * 8 * nb : (8 % p.T == 0) ? 8 * ((nb + 8 / p.T - 1) / (8 / p.T)) : p.T * nb;
  constexpr int kNd = Cfg<DN, DR>::NBLK == 4 ? 4 : 2;   // dim parts of the 32-head shape
  if (p.ht == 4)
    hipLaunchKernelGGL((attn_kernel<DN, DR, 4, 2, false>), dim3(blocks), dim3(512), 0, stream, p);
  else if (p.scores)   // the selection in the prologue runs on the computing waves alone
    hipLaunchKernelGGL((attn_kernel<DN, DR, 2, kNd, false>), dim3(blocks), dim3(64 * 2 * kNd), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_kernel<DN, DR, 2, kNd, true>), dim3(blocks), dim3(64 * (2 * kNd + 1)), 0, stream, p);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  static_assert((DN + DR) / 4 <= 128, "one 128-thread team per (query, head)");
  const int mblocks = (p.T * p.H + 1) / 2;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(mblocks), dim3(256), 0, stream, p);
  return hipPeekAtLastError();
}

}  // namespace

// Partial-result scratch of the allocation-free decode entry point: one
// array per GPU, held until the process ends.  In host code `scratch` is a
// host-side stand-in, never a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

hipError_t attn_scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn(const AttnParams& p, hipStream_t stream) {
  if (p.D_nope == 448 && p.D_rope == 64) return launch_attn_t<448, 64>(p, stream);
  if (p.D_nope == 48 && p.D_rope == 16) return launch_attn_t<48, 16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace csa
