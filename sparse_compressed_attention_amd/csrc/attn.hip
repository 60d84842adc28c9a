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
// Mapping on gfx950 (256 threads = 4 waves per workgroup):
//  * a workgroup owns one query, 32 heads and a range of key slots (the range
//    is split over workgroups only when there are few queries);
//  * wave (ht, kh): heads [16 ht, 16 ht + 16) of the group; within every
//    64-key tile it takes keys [32 kh, 32 kh + 32).  The two kh waves of a head
//    tile merge their softmax states through LDS at the end;
//  * gather: key descriptors (top-k index -> page table -> row, or window slot
//    -> row) are resolved once into LDS; each 64-key tile is copied from HBM
//    straight into LDS with global_load_lds_dwordx4 (no register staging),
//    three tiles in flight (ring of 3 buffers, prefetch distance 2).  The
//    tile is stored as "planes": plane c holds the c-th 16-byte chunk of all
//    64 rows, so one DMA instruction writes one whole plane and every lane
//    keeps one row (key) for all of its DMAs.  Rows 16..31 and 48..63 are
//    XOR-swizzled by 4 slots so that the transpose reads below never hit the
//    same LDS banks.  The cache's FP8/BF16 bytes go to the MFMA unchanged;
//  * QK: S^T (keys x heads) = X . Q^T on v_mfma 16x16x128 FP8, with q split
//    into two E4M3 terms hi + lo sharing a power-of-two per-head scale (the K
//    dimension is [hi | lo], X read once and used for both), plus the rope
//    dims on v_mfma 16x16x32 BF16; the two 16-key subtiles are interleaved
//    and the next X operands are read from LDS before the current MFMAs;
//  * online softmax in FP32, exp2 domain; each lane owns one head, so the
//    rescale of O needs no cross-lane traffic.  The running max is raised
//    lazily: only when a tile's max exceeds it by more than 2^tau (tau = 4),
//    so probabilities stay <= 2^tau and the O rescale runs on few tiles.  The
//    sink starts the running max and denominator (zero value);
//  * PV: O^T (dims x heads) += X^T . P^T: X^T is read from the same LDS tile
//    with ds_read_b64_tr_b8 (nope, FP8; P as two E4M3 terms hi + lo after a
//    2^(8 - tau) scale) and ds_read_b64_tr_b16 (rope, BF16, P in BF16); bytes
//    of masked keys are cleared in registers; P never leaves registers.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

constexpr int kSwaFlag = 1 << 30;
constexpr int kNBuf = 3;
constexpr int kPlane = kAttnTile * 16;   // bytes per plane (64 rows x 16 B)

template <int DN, int DR>
struct Cfg {
  static constexpr int NFB = DN / 128;                                       // full 128-dim blocks
  static constexpr int REM = DN % 128;                                       // combined hi|lo block
  static constexpr int NR = (DR + 31) / 32;                                  // rope k-steps
  static constexpr int ND = DN / 16;                                         // PV nope dim tiles
  static constexpr int NDR = DR / 16;                                        // PV rope dim tiles
  static constexpr int NDT = ND + NDR;
  static constexpr int HALF = NDT / 2;
  static constexpr int CHN = DN / 16;                                        // nope planes
  static constexpr int CHR = 2 * DR / 16;                                    // rope planes
  static constexpr int CH = CHN + CHR;
  static constexpr int PPW = (CH + 3) / 4;                                   // planes per wave (max)
  static constexpr int PMIN = CH / 4;                                        // planes per wave (min)
  static constexpr int TILE_BYTES = CH * kPlane;
  static_assert(DN % 16 == 0 && DR % 16 == 0, "dims must be multiples of 16");
  static_assert(REM <= 64, "remainder block must fit one combined hi|lo MFMA");
  static_assert(NDT % 2 == 0, "dim tiles split evenly between the two key halves");
  static_assert(PMIN >= 1, "every wave issues at least one plane per tile");
};

// key (0..31) of this wave's half-tile held by byte e (0..7) of a lane in
// 16-lane group g, as produced by the QK output layout of two 16-key subtiles.
__device__ __forceinline__ int kappa(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }
// LDS slot of key k inside a plane (an involution).
__device__ __forceinline__ int slot_of(int k) { return k ^ (((k >> 4) & 1) << 2); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <int DN, int DR>
__global__ __launch_bounds__(256, 1) void attn_kernel(AttnParams p) {
  using C = Cfg<DN, DR>;
  constexpr int D = DN + DR;

  __shared__ __attribute__((aligned(16))) uint8_t xs[kNBuf][C::TILE_BYTES];
  __shared__ int32_t desc[kAttnMaxSlots];

  // ---- which (query, head group, split).  Workgroups go to the 8 XCDs
  // round-robin by id.  With 8 or more queries, queries are spread over the
  // XCDs and all workgroups of one query share an XCD (and its L2, which then
  // serves the head groups' repeated reads of the same rows); with fewer,
  // a query's workgroups are spread over all XCDs instead.
  const int nb = p.n_hg * p.n_splits;
  const int bid = blockIdx.x;
  int t, jb;
  if (p.T >= 8) {
    const int local = bid >> 3;
    t = (local / nb) * 8 + (bid & 7);
    jb = local % nb;
  } else {
    t = bid / nb;
    jb = bid - t * nb;
  }
  if (t >= p.T) return;
  const int hg = jb / p.n_splits;
  const int split = jb - hg * p.n_splits;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const int ht = wave & 1;
  const int kh = wave >> 1;
  const int h = hg * 32 + ht * 16 + r;
  const bool tile_ok = hg * 32 + ht * 16 < p.H;
  const bool head_ok = h < p.H;
  const bool prefill = p.prefill_seq >= 0;
  const int seq = prefill ? p.prefill_seq : t;
  const int pos = p.q_pos[t];
  const int nc = p.n_comp[seq];
  const int nv = pos >= 0 ? max(0, min(pos / p.ratio_m, nc)) : 0;
  const int n_sel = p.topk ? p.k : nv;
  const int n_slots = n_sel + p.W;
  const int kv0 = split * p.per_split;
  if (split > 0 && kv0 >= n_slots) return;   // empty split: the merge skips it
  const int kv1 = min(n_slots, kv0 + p.per_split);
  const int nkeys = max(0, kv1 - kv0);

  // ---- query rows: loads issued first (packed BF16, 64 VGPRs) so their
  // latency overlaps the descriptor round trips; converted after the first
  // tile DMAs are issued
  v4i qraw[C::NFB + 1][4];
  v4i qrope[C::NR];
  {
    const uint16_t* qrow = p.q + (size_t)t * p.q_stride + (size_t)h * D;
#pragma unroll
    for (int b = 0; b <= C::NFB; ++b) {
      const bool comb = (b == C::NFB);
      const int d0 = comb ? 128 * C::NFB + 32 * (g & 1) : 128 * b + 32 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int dd = d0 + 8 * c;
        v4i raw = (v4i){0, 0, 0, 0};
        if (head_ok && (!comb || C::REM > 0) && dd < DN) raw = ld16(qrow + dd);
        qraw[b][c] = raw;
      }
    }
#pragma unroll
    for (int rr = 0; rr < C::NR; ++rr) {
      const int dd = 32 * rr + 8 * g;
      v4i raw = (v4i){0, 0, 0, 0};
      if (head_ok && dd < DR) raw = ld16(qrow + DN + dd);
      qrope[rr] = raw;
    }
  }
  const float sink_raw = head_ok ? p.sink[h] : 0.0f;

  // ---- key descriptors of this workgroup's slots: row | source flag, -1 =
  // skip.  All first-level loads (top-k index or ring position) are issued
  // together, then all page-table loads: two round trips in total.
  const int32_t* pt = p.page_table + (size_t)seq * p.max_pages;
  constexpr int kSPT = kAttnMaxSlots / 256;   // slots per thread
  int v1[kSPT];
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + 256 * j;
    const int slot = kv0 + s;
    int v = -1;
    if (s < nkeys) {
      if (slot < n_sel) {
        v = p.topk ? p.topk[(size_t)t * p.k + slot] : slot;
      } else if (!prefill) {
        v = p.swa_pos[(size_t)seq * p.W + (slot - n_sel)];
      }
    }
    v1[j] = v;
  }
  int v2[kSPT];
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + 256 * j;
    const int slot = kv0 + s;
    const int idx = v1[j];
    int page = -1;
    if (s < nkeys && slot < n_sel && idx >= 0 && idx < nc && idx / p.page_size < p.max_pages)
      page = pt[idx / p.page_size];
    v2[j] = page;
  }
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int s = threadIdx.x + 256 * j;
    if (s >= nkeys) continue;
    const int slot = kv0 + s;
    int d = -1;
    if (slot < n_sel) {
      const int idx = v1[j], page = v2[j];
      if (page >= 0 && page < p.num_pages) d = page * p.page_size + idx % p.page_size;
    } else {
      const int jw = slot - n_sel;
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

  // ---- tile DMA: lane -> the key whose plane slot is `lane`, planes
  // c = wave + 4 i.  Masked keys copy a dummy row (row 0) so that every wave
  // issues the same number of DMAs per tile; their bytes are never used.
  const int dkey = slot_of(lane);
  auto issue_tile = [&](int tile, int buf) {
    const int s = tile * kAttnTile + dkey;
    const int d = s < nkeys ? desc[s] : -1;
    const uint8_t* nsrc = p.lat_nope;
    const uint8_t* rsrc = reinterpret_cast<const uint8_t*>(p.lat_rope);
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
    uint8_t* base = xs[buf];
#pragma unroll
    for (int i = 0; i < C::PPW; ++i) {
      const int c = wave + 4 * i;
      if (c < C::CH) {
        const uint8_t* src = (c < C::CHN) ? nsrc + 16 * c : rsrc + 16 * (c - C::CHN);
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                         (void CSA_LDS*)(base + c * kPlane), 16, 0, 0);
      }
    }
  };

  const int n_tiles = (nkeys + kAttnTile - 1) / kAttnTile;
  if (n_tiles > 0) issue_tile(0, 0);
  if (n_tiles > 1) issue_tile(1, 1);

  // ---- query operands: q split into two E4M3 terms hi + lo with a shared
  // power-of-two per-head scale (registers for the whole kernel)
  v8i qhi[C::NFB > 0 ? C::NFB : 1], qlo[C::NFB > 0 ? C::NFB : 1], qcomb;
  v8bf qr[C::NR];
  float cq = 0.0f;
  const float cr = p.sm_log2;
  {
    auto qval = [&](int b, int c, int e) -> float {
      const uint32_t w = (uint32_t)qraw[b][c][e >> 1];
      return bf16_bits_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
    };
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b <= C::NFB; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(qval(b, c, e)));
    amax = max_over_groups(amax);
    const float s = e4m3_pow2_scale(amax);
    const float inv = 1.0f / s;
    cq = head_ok ? cr * s : 0.0f;
#pragma unroll
    for (int b = 0; b <= C::NFB; ++b) {
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
      if (b < C::NFB) {
        qhi[b] = hi;
        qlo[b] = lo;
      } else {
        qcomb = (g < 2) ? hi : lo;
      }
    }
#pragma unroll
    for (int rr = 0; rr < C::NR; ++rr) qr[rr] = __builtin_bit_cast(v8bf, qrope[rr]);
  }
  if (C::NFB == 0) {
    qhi[0] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    qlo[0] = qhi[0];
  }

  // ---- softmax state (exp2 domain); only one wave per head carries the sink
  const bool sink_here = split == 0 && kh == 0 && head_ok;
  const float sink2 = head_ok ? sink_raw * kLog2e : -__builtin_inff();
  float m_run = sink_here ? sink2 : -__builtin_inff();
  float l_run = (sink_here && g == 0 && sink2 > -__builtin_inff()) ? 1.0f : 0.0f;
  v4f O[C::NDT];
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) O[i] = (v4f){0.f, 0.f, 0.f, 0.f};


  const int sl_q0 = slot_of(32 * kh + r);          // QK rows of subtile 0 / 1
  const int sl_q1 = slot_of(32 * kh + 16 + r);
  int buf = 0;
  for (int it = 0; it < n_tiles; ++it, buf = (buf + 1 == kNBuf) ? 0 : buf + 1) {
    // tile `it` landed in LDS (this wave's DMAs), then everyone's (barrier);
    // the barrier also retires every wave's reads of the buffer reused next
    if (it + 1 < n_tiles) wait_vmcnt<C::PMIN>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (it + 2 < n_tiles) issue_tile(it + 2, buf == 0 ? 2 : buf - 1);
    if (!tile_ok) continue;
    const uint8_t* xb = xs[buf];

    // -- QK for the wave's two 16-key subtiles, interleaved
    auto xread = [&](int sl, int c0) -> v8i {
      const v4i lo = *reinterpret_cast<const v4i*>(xb + c0 * kPlane + 16 * sl);
      const v4i hi = *reinterpret_cast<const v4i*>(xb + (c0 + 1) * kPlane + 16 * sl);
      return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto xcomb = [&](int sl) -> v8i {
      const int c0 = 8 * C::NFB + 2 * (g & 1);
      v8i x = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
      if (32 * (g & 1) < C::REM) {
        const v4i lo = *reinterpret_cast<const v4i*>(xb + c0 * kPlane + 16 * sl);
        v4i hi = (v4i){0, 0, 0, 0};
        if (32 * (g & 1) + 16 < C::REM) hi = *reinterpret_cast<const v4i*>(xb + (c0 + 1) * kPlane + 16 * sl);
        x = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      return x;
    };
    v4f a0 = (v4f){0.f, 0.f, 0.f, 0.f}, a1 = a0;
    v8i x0, x1;
    if (C::NFB > 0) {
      x0 = xread(sl_q0, 2 * g);
      x1 = xread(sl_q1, 2 * g);
    } else {
      x0 = xcomb(sl_q0);
      x1 = xcomb(sl_q1);
    }
#pragma unroll
    for (int b = 0; b < C::NFB; ++b) {
      v8i n0, n1;
      if (b + 1 < C::NFB) {
        n0 = xread(sl_q0, 8 * (b + 1) + 2 * g);
        n1 = xread(sl_q1, 8 * (b + 1) + 2 * g);
      } else {
        n0 = xcomb(sl_q0);
        n1 = xcomb(sl_q1);
      }
      a0 = mfma_f8_128(x0, qhi[b], a0);
      a1 = mfma_f8_128(x1, qhi[b], a1);
      a0 = mfma_f8_128(x0, qlo[b], a0);
      a1 = mfma_f8_128(x1, qlo[b], a1);
      x0 = n0;
      x1 = n1;
    }
    if (C::REM > 0) {
      a0 = mfma_f8_128(x0, qcomb, a0);
      a1 = mfma_f8_128(x1, qcomb, a1);
    }
    v4f r0 = (v4f){0.f, 0.f, 0.f, 0.f}, r1 = r0;
#pragma unroll
    for (int rr = 0; rr < C::NR; ++rr) {
      const int c = C::CHN + 4 * rr + g;
      v4i y0 = (v4i){0, 0, 0, 0}, y1 = y0;
      if (32 * rr + 8 * g < DR) {
        y0 = *reinterpret_cast<const v4i*>(xb + c * kPlane + 16 * sl_q0);
        y1 = *reinterpret_cast<const v4i*>(xb + c * kPlane + 16 * sl_q1);
      }
      r0 = mfma_bf16_32(__builtin_bit_cast(v8bf, y0), qr[rr], r0);
      r1 = mfma_bf16_32(__builtin_bit_cast(v8bf, y1), qr[rr], r1);
    }

    // -- online softmax (lane: head h, keys kappa(g, e) of this half-tile)
    float sv[8], kq[8];
    uint32_t m8lo = 0, m8hi = 0;   // byte masks of the valid keys (PV operands)
    float tmax = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int st = e >> 2, i = e & 3;
      const int s = it * kAttnTile + 32 * kh + 16 * st + 4 * g + i;   // = key kappa(g, e)
      const int d = s < nkeys ? desc[s] : -1;
      const bool swa = (d & kSwaFlag) != 0;
      const float an = st ? a1[i] : a0[i];
      const float ar = st ? r1[i] : r0[i];
      const float x = cq * (swa ? p.swa_scale : p.lat_scale) * an + cr * ar;
      kq[e] = swa ? p.pscale_swa : p.pscale_lat;
      sv[e] = (d >= 0 && head_ok) ? x : -__builtin_inff();
      tmax = fmaxf(tmax, sv[e]);
      if (d >= 0) {
        if (e < 4) m8lo |= 0xffu << (8 * e);
        else m8hi |= 0xffu << (8 * (e - 4));
      }
    }
    tmax = max_over_groups(tmax);
    const bool grow = tmax > m_run + (float)kAttnTau;
    if (__ballot(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float alpha = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < C::NDT; ++i) O[i] *= alpha;
      m_run = m_new;
    }
    const float msub = (m_run == -__builtin_inff()) ? 0.0f : m_run;
    float pr[8];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = (sv[e] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(sv[e] - msub);
      psum += pr[e];
    }
    l_run += psum;
    // -- P operands for nope: two E4M3 terms hi + lo of p x key-scale ratio x
    //    2^(8 - tau) (lo = the rounding residual of hi); BF16 for rope
    float px[8], pres[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) px[e] = pr[e] * kq[e];
    const int w0 = pack4_fp8(px[0], px[1], px[2], px[3]);
    const int w1 = pack4_fp8(px[4], px[5], px[6], px[7]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pres[e] = px[e] - fp8_to_f32(w0, e);
      pres[4 + e] = px[4 + e] - fp8_to_f32(w1, e);
    }
    const int w0l = pack4_fp8(pres[0], pres[1], pres[2], pres[3]);
    const int w1l = pack4_fp8(pres[4], pres[5], pres[6], pres[7]);
    const long p8 = (long)(uint32_t)w0 | ((long)(uint32_t)w1 << 32);
    const long p8l = (long)(uint32_t)w0l | ((long)(uint32_t)w1l << 32);
    v4i pbw;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pbw[e] = (int)((uint32_t)f32_to_bf16_bits(pr[2 * e]) | ((uint32_t)f32_to_bf16_bits(pr[2 * e + 1]) << 16));
    const v8bf pbf = __builtin_bit_cast(v8bf, pbw);

    // -- PV: O^T[dims x heads] += X^T[dims x keys] P^T[keys x heads].  The
    //    X^T bytes of masked keys are cleared (their LDS rows are a dummy copy)
    {
      const int krow = 32 * kh + kappa(g, r >> 1);
      const uint8_t* a8 = xb + 16 * slot_of(krow) + 8 * (r & 1);
      // transpose reads in batches of PVB issued ahead of their MFMAs
      constexpr int PVB = 7;
      static_assert(C::ND % PVB == 0 || C::ND < PVB, "PV batch");
      constexpr int NB = C::ND < PVB ? 1 : C::ND / PVB;
      constexpr int BS = C::ND < PVB ? C::ND : PVB;
      v2i abuf[2][BS];
#pragma unroll
      for (int j = 0; j < BS; ++j)
        abuf[0][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CSA_LDS v2i*)(a8 + j * kPlane));
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        if (bt + 1 < NB) {
#pragma unroll
          for (int j = 0; j < BS; ++j)
            abuf[(bt + 1) & 1][j] =
                __builtin_amdgcn_ds_read_tr8_b64_v2i32((CSA_LDS v2i*)(a8 + ((bt + 1) * BS + j) * kPlane));
        }
#pragma unroll
        for (int j = 0; j < BS; ++j) {
          const int dt = bt * BS + j;
          const v2i a = abuf[bt & 1][j];
          const long al = (long)((uint32_t)a[0] & m8lo) | ((long)((uint32_t)a[1] & m8hi) << 32);
          O[dt] = mfma_f8_32(al, p8, O[dt]);
          O[dt] = mfma_f8_32(al, p8l, O[dt]);
        }
      }
      // rope, 16-bit elements: element e of read 0 / read 1 is key kappa(g, e) / kappa(g, 4 + e)
      const uint32_t mr0 = ((m8lo & 0xffu) ? 0xffffu : 0u) | ((m8lo & 0xff00u) ? 0xffff0000u : 0u);
      const uint32_t mr1 = ((m8lo & 0xff0000u) ? 0xffffu : 0u) | ((m8lo & 0xff000000u) ? 0xffff0000u : 0u);
      const uint32_t mr2 = ((m8hi & 0xffu) ? 0xffffu : 0u) | ((m8hi & 0xff00u) ? 0xffff0000u : 0u);
      const uint32_t mr3 = ((m8hi & 0xff0000u) ? 0xffffu : 0u) | ((m8hi & 0xff000000u) ? 0xffff0000u : 0u);
      const int krow0 = 32 * kh + kappa(g, r >> 2);
      const int krow1 = 32 * kh + kappa(g, 4 + (r >> 2));
      const int cpl = C::CHN + ((r >> 1) & 1);
      const uint8_t* b0 = xb + cpl * kPlane + 16 * slot_of(krow0) + 8 * (r & 1);
      const uint8_t* b1 = xb + cpl * kPlane + 16 * slot_of(krow1) + 8 * (r & 1);
#pragma unroll
      for (int dt = 0; dt < C::NDR; ++dt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(b0 + 2 * dt * kPlane));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(b1 + 2 * dt * kPlane));
        v4i packed;
        packed[0] = (int)(((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16)) & mr0);
        packed[1] = (int)(((uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16)) & mr1);
        packed[2] = (int)(((uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16)) & mr2);
        packed[3] = (int)(((uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)) & mr3);
        O[C::ND + dt] = mfma_bf16_32(__builtin_bit_cast(v8bf, packed), pbf, O[C::ND + dt]);
      }
    }
  }
  __syncthreads();   // every wave is done with the tile buffers

  // ---- merge the two key halves (kh) of each head tile through LDS
  const float l_tot = sum_over_groups(l_run);
  float* ex = reinterpret_cast<float*>(&xs[0][0]);                   // [4][HALF][64][4]
  float* stt = ex + 4 * C::HALF * 64 * 4;                              // [4][64][2]
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j)
      *reinterpret_cast<v4f*>(ex + ((wave * C::HALF + j) * 64 + lane) * 4) = O[C::HALF + j];
  } else {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j)
      *reinterpret_cast<v4f*>(ex + ((wave * C::HALF + j) * 64 + lane) * 4) = O[j];
  }
  stt[(wave * 64 + lane) * 2 + 0] = m_run;
  stt[(wave * 64 + lane) * 2 + 1] = l_tot;
  __syncthreads();
  if (!tile_ok) return;
  const int partner = wave ^ 2;
  const float pm = stt[(partner * 64 + lane) * 2 + 0];
  const float pl = stt[(partner * 64 + lane) * 2 + 1];
  const float M = fmaxf(m_run, pm);
  const float Ms = (M == -__builtin_inff()) ? 0.0f : M;
  const float a_self = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - Ms);
  const float a_oth = (pm == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(pm - Ms);
  const float L = l_tot * a_self + pl * a_oth;
  const bool final_out = p.n_splits == 1;
  const float invL = (final_out && L > 0.0f) ? 1.0f / L : 0.0f;

  auto finish = [&](int dt, const v4f& own) {
    const v4f oth = *reinterpret_cast<const v4f*>(ex + ((partner * C::HALF + (dt - kh * C::HALF)) * 64 + lane) * 4);
    const bool nope = dt < C::ND;
    const float unit = nope ? p.nope_unit : 1.0f;
    const int dim = nope ? 16 * dt + 4 * g : DN + 16 * (dt - C::ND) + 4 * g;
    v4f v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (own[i] * a_self + oth[i] * a_oth) * unit;
    if (!head_ok) return;
    if (final_out) {
      const uint32_t b0 = f32_to_bf16_bits(v[0] * invL), b1 = f32_to_bf16_bits(v[1] * invL);
      const uint32_t b2 = f32_to_bf16_bits(v[2] * invL), b3 = f32_to_bf16_bits(v[3] * invL);
      v2i pk = (v2i){(int)(b0 | (b1 << 16)), (int)(b2 | (b3 << 16))};
      *reinterpret_cast<v2i*>(p.out + ((size_t)t * p.H + h) * D + dim) = pk;
    } else {
      float* dst = p.part + (((size_t)split * p.T + t) * p.H + h) * (D + 2) + dim;
      *reinterpret_cast<v4f*>(dst) = v;
    }
  };
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j) finish(j, O[j]);
  } else {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j) finish(C::HALF + j, O[C::HALF + j]);
  }
  if (head_ok && kh == 0 && g == 0) {
    if (final_out) {
      if (p.lse) p.lse[(size_t)t * p.H + h] = (L > 0.0f) ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
    } else {
      float* dst = p.part + (((size_t)split * p.T + t) * p.H + h) * (D + 2) + D;
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// Combines the per-split partial states (unnormalised O, running max in log2
// units, denominator) of every (query, head) into the output and lse.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int D = p.D_nope + p.D_rope;
  const int tpd = D / 4;
  const int hpb = 256 / tpd;
  const int pair = blockIdx.x * hpb + threadIdx.x / tpd;
  if (threadIdx.x >= hpb * tpd || pair >= p.T * p.H) return;
  const int t = pair / p.H;
  const int h = pair - t * p.H;
  const int d0 = (threadIdx.x % tpd) * 4;
  const bool prefill = p.prefill_seq >= 0;
  const int seq = prefill ? p.prefill_seq : t;
  const int pos = p.q_pos[t];
  const int nv = pos >= 0 ? max(0, min(pos / p.ratio_m, p.n_comp[seq])) : 0;
  const int n_slots = (p.topk ? p.k : nv) + p.W;
  const int used = max(1, min(p.n_splits, (n_slots + p.per_split - 1) / p.per_split));
  float M = -__builtin_inff();
  for (int s = 0; s < used; ++s) M = fmaxf(M, p.part[(((size_t)s * p.T + t) * p.H + h) * (D + 2) + D]);
  const float Ms = (M == -__builtin_inff()) ? 0.0f : M;
  float L = 0.0f;
  v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < used; ++s) {
    const float* src = p.part + (((size_t)s * p.T + t) * p.H + h) * (D + 2);
    const float ms = src[D];
    const float a = (ms == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms - Ms);
    L += src[D + 1] * a;
    const v4f v = *reinterpret_cast<const v4f*>(src + d0);
    acc += v * a;
  }
  const float invL = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t b0 = f32_to_bf16_bits(acc[0] * invL), b1 = f32_to_bf16_bits(acc[1] * invL);
  const uint32_t b2 = f32_to_bf16_bits(acc[2] * invL), b3 = f32_to_bf16_bits(acc[3] * invL);
  *reinterpret_cast<v2i*>(p.out + ((size_t)t * p.H + h) * D + d0) =
      (v2i){(int)(b0 | (b1 << 16)), (int)(b2 | (b3 << 16))};
  if (d0 == 0 && p.lse) p.lse[(size_t)t * p.H + h] = (L > 0.0f) ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
}

template <int DN, int DR>
hipError_t launch_attn_t(const AttnParams& p, hipStream_t stream) {
  const int nb = p.n_hg * p.n_splits;
  const int blocks = (p.T >= 8 ? ((p.T + 7) / 8) * 8 : p.T) * nb;
  hipLaunchKernelGGL((attn_kernel<DN, DR>), dim3(blocks), dim3(256), 0, stream, p);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  const int D = DN + DR;
  const int hpb = 256 / (D / 4);
  const int mblocks = (p.T * p.H + hpb - 1) / hpb;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(mblocks), dim3(256), 0, stream, p);
  return hipPeekAtLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t stream) {
  if (p.D_nope == 448 && p.D_rope == 64) return launch_attn_t<448, 64>(p, stream);
  if (p.D_nope == 48 && p.D_rope == 16) return launch_attn_t<48, 16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace csa
