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
//  * the tile is gathered from HBM (top-k index -> page table -> row) into
//    registers and then LDS, double-buffered, in the cache's own FP8/BF16
//    bytes;
//  * QK: S^T (keys x heads) = X . Q^T on v_mfma 16x16x128 FP8, with q split
//    into two E4M3 terms hi + lo sharing a power-of-two per-head scale (the K
//    dimension is [hi | lo], X read once and used for both), plus the rope
//    dims on v_mfma 16x16x32 BF16.  The key scale and the softmax scale are
//    applied per lane in FP32;
//  * online softmax in FP32, exp2 domain; each lane owns one head, so the
//    rescale of O needs no cross-lane traffic; the sink starts the running
//    max and denominator (zero value);
//  * PV: O^T (dims x heads) += X^T . P^T: X^T is read from the same LDS tile
//    with ds_read_b64_tr_b8 (nope, FP8; P as two E4M3 terms hi + lo after a
//    2^8 scale) and ds_read_b64_tr_b16 (rope, BF16, P in BF16); P never leaves
//    registers.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

namespace {

constexpr int kSwaFlag = 1 << 30;

template <int DN, int DR>
struct Cfg {
  static constexpr int NP = ((DN / 16) % 2 == 0) ? DN + 16 : DN;          // LDS pitch, nope
  static constexpr int RB = 2 * DR;                                          // rope bytes
  static constexpr int RP = ((RB / 16) % 2 == 0) ? RB + 16 : RB;          // LDS pitch, rope
  static constexpr int NFB = DN / 128;                                       // full 128-dim blocks
  static constexpr int REM = DN % 128;                                       // combined hi|lo block
  static constexpr int NR = (DR + 31) / 32;                                  // rope k-steps
  static constexpr int ND = DN / 16;                                         // PV nope dim tiles
  static constexpr int NDR = DR / 16;                                        // PV rope dim tiles
  static constexpr int NDT = ND + NDR;
  static constexpr int HALF = NDT / 2;
  static constexpr int CHN = DN / 16;                                        // 16-byte chunks / key
  static constexpr int CHR = RB / 16;
  static constexpr int CH = CHN + CHR;
  static constexpr int CPT = (CH + 3) / 4;                                   // chunks per thread
  static constexpr int TILE_BYTES = kAttnTile * (NP + RP);
  static_assert(DN % 16 == 0 && DR % 16 == 0, "dims must be multiples of 16");
  static_assert(REM <= 64, "remainder block must fit one combined hi|lo MFMA");
  static_assert(NDT % 2 == 0, "dim tiles split evenly between the two key halves");
};

// key (0..31) of this wave's half-tile held by byte e (0..7) of a lane in
// 16-lane group g, as produced by the QK output layout of two 16-key subtiles.
__device__ __forceinline__ int kappa(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

template <int DN, int DR>
__global__ __launch_bounds__(256, 1) void attn_kernel(AttnParams p) {
  using C = Cfg<DN, DR>;
  constexpr int D = DN + DR;

  __shared__ __attribute__((aligned(16))) uint8_t xs[2][C::TILE_BYTES];
  __shared__ int32_t desc[kAttnMaxSlots];

  // ---- which (query, head group, split): queries are spread over the 8
  // XCDs round-robin and all workgroups of one query share an XCD (and its L2).
  const int nb = p.n_hg * p.n_splits;
  const int bid = blockIdx.x;
  const int local = bid >> 3;
  const int t = (local / nb) * 8 + (bid & 7);
  if (t >= p.T) return;
  const int jb = local % nb;
  const int hg = jb / p.n_splits;
  const int split = jb - hg * p.n_splits;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  // ---- key descriptors of this workgroup's slots: row | source flag, -1 = skip
  const int32_t* pt = p.page_table + (size_t)seq * p.max_pages;
  for (int s = threadIdx.x; s < nkeys; s += 256) {
    const int slot = kv0 + s;
    int d = -1;
    if (slot < n_sel) {
      const int idx = p.topk ? p.topk[(size_t)t * p.k + slot] : slot;
      if (idx >= 0 && idx < nc && idx / p.page_size < p.max_pages) {
        const int page = pt[idx / p.page_size];
        if (page >= 0 && page < p.num_pages) d = page * p.page_size + idx % p.page_size;
      }
    } else {
      const int j = slot - n_sel;
      if (!prefill) {
        const int pp = p.swa_pos[(size_t)seq * p.W + j];
        if (pp >= 0 && pp <= pos && pp > pos - p.W) d = (seq * p.W + j) | kSwaFlag;
      } else {
        const int pp = pos - p.W + 1 + j;
        if (pp >= 0 && pp >= p.swa_first_pos && pp - p.swa_first_pos < p.swa_len)
          d = (pp - p.swa_first_pos) | kSwaFlag;
      }
    }
    desc[s] = d;
  }

  // ---- query operands (registers for the whole kernel)
  v8i qhi[C::NFB > 0 ? C::NFB : 1], qlo[C::NFB > 0 ? C::NFB : 1], qcomb;
  v8bf qr[C::NR];
  float cq = 0.0f;
  const float cr = p.sm_scale * kLog2e;
  {
    const uint16_t* qrow = p.q + (size_t)t * p.q_stride + (size_t)h * D;
    float v[C::NFB + 1][32];
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b <= C::NFB; ++b) {
      const bool comb = (b == C::NFB);
      const int d0 = comb ? 128 * C::NFB + 32 * (g & 1) : 128 * b + 32 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int dd = d0 + 8 * c;
        v4i raw = (v4i){0, 0, 0, 0};
        if (head_ok && (!comb || C::REM > 0) && dd < DN) raw = ld16(qrow + dd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = (uint32_t)raw[e >> 1];
          const float f = bf16_bits_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
          v[b][8 * c + e] = f;
          amax = fmaxf(amax, fabsf(f));
        }
      }
    }
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
        for (int e = 0; e < 4; ++e) x[e] = v[b][4 * w4 + e] * inv;
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
    for (int rr = 0; rr < C::NR; ++rr) {
      const int dd = 32 * rr + 8 * g;
      v4i raw = (v4i){0, 0, 0, 0};
      if (head_ok && dd < DR) raw = ld16(qrow + DN + dd);
      qr[rr] = __builtin_bit_cast(v8bf, raw);
    }
  }
  if (C::NFB == 0) {
    qhi[0] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    qlo[0] = qhi[0];
  }

  // ---- softmax state (exp2 domain); only one wave per head carries the sink
  const bool sink_here = split == 0 && kh == 0 && head_ok;
  const float sink2 = head_ok ? p.sink[h] * kLog2e : -__builtin_inff();
  float m_run = sink_here ? sink2 : -__builtin_inff();
  float l_run = (sink_here && g == 0 && sink2 > -__builtin_inff()) ? 1.0f : 0.0f;
  v4f O[C::NDT];
#pragma unroll
  for (int i = 0; i < C::NDT; ++i) O[i] = (v4f){0.f, 0.f, 0.f, 0.f};

  const float smax = fmaxf(p.lat_scale, p.swa_scale);
  const float ratio_lat = p.lat_scale / smax * 256.0f;
  const float ratio_swa = p.swa_scale / smax * 256.0f;

  __syncthreads();   // descriptors visible

  // ---- tile staging: thread -> key (tid / 4), chunks (tid % 4) + 4 j
  const int skey = threadIdx.x >> 2;
  const int spart = threadIdx.x & 3;
  v4i stage[C::CPT];
  auto load_tile = [&](int tile) {
    const int s = tile * kAttnTile + skey;
    const int d = s < nkeys ? desc[s] : -1;
    const uint8_t* nsrc = nullptr;
    const uint8_t* rsrc = nullptr;
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
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int c = spart + 4 * j;
      v4i x = (v4i){0, 0, 0, 0};
      if (d >= 0 && c < C::CH) x = (c < C::CHN) ? ld16(nsrc + 16 * c) : ld16(rsrc + 16 * (c - C::CHN));
      stage[j] = x;
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* base = xs[buf];
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int c = spart + 4 * j;
      if (c < C::CH) {
        uint8_t* dst = (c < C::CHN) ? base + skey * C::NP + 16 * c
                                    : base + kAttnTile * C::NP + skey * C::RP + 16 * (c - C::CHN);
        *reinterpret_cast<v4i*>(dst) = stage[j];
      }
    }
  };

  const int n_tiles = (nkeys + kAttnTile - 1) / kAttnTile;
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1);
    if (tile_ok) {
      const uint8_t* xn = xs[buf];
      const uint8_t* xr = xs[buf] + kAttnTile * C::NP;
      // -- QK for the wave's two 16-key subtiles
      v4f an[2], ar[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kr = 32 * kh + 16 * st + r;
        v4f a = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < C::NFB; ++b) {
          const uint8_t* src = xn + kr * C::NP + 128 * b + 32 * g;
          const v4i x0 = *reinterpret_cast<const v4i*>(src);
          const v4i x1 = *reinterpret_cast<const v4i*>(src + 16);
          const v8i xa = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          a = mfma_f8_128(xa, qhi[b], a);
          a = mfma_f8_128(xa, qlo[b], a);
        }
        if (C::REM > 0) {
          const int off = 32 * (g & 1);
          const uint8_t* src = xn + kr * C::NP + 128 * C::NFB + off;
          v8i xa = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
          if (off < C::REM) {
            const v4i x0 = *reinterpret_cast<const v4i*>(src);
            v4i x1 = (v4i){0, 0, 0, 0};
            if (off + 16 < C::REM) x1 = *reinterpret_cast<const v4i*>(src + 16);
            xa = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          }
          a = mfma_f8_128(xa, qcomb, a);
        }
        an[st] = a;
        v4f b2 = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < C::NR; ++rr) {
          const int dd = 32 * rr + 8 * g;
          v4i x = (v4i){0, 0, 0, 0};
          if (dd < DR) x = *reinterpret_cast<const v4i*>(xr + kr * C::RP + 2 * dd);
          b2 = mfma_bf16_32(__builtin_bit_cast(v8bf, x), qr[rr], b2);
        }
        ar[st] = b2;
      }
      // -- online softmax (lane: head h, keys kappa(g, e))
      float sv[8], kq[8];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int st = e >> 2, i = e & 3;
        const int s = it * kAttnTile + 32 * kh + 16 * st + 4 * g + i;
        const int d = s < nkeys ? desc[s] : -1;
        const bool swa = (d & kSwaFlag) != 0;
        const float ks = swa ? p.swa_scale : p.lat_scale;
        kq[e] = swa ? ratio_swa : ratio_lat;
        const float x = cq * ks * an[st][i] + cr * ar[st][i];
        sv[e] = (d >= 0 && head_ok) ? x : -__builtin_inff();
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = max_over_groups(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float msub = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      const float alpha = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - msub);
      float pr[8];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = (sv[e] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(sv[e] - msub);
        psum += pr[e];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < C::NDT; ++i) O[i] *= alpha;
      }
      // -- P operands for nope: two E4M3 terms hi + lo of p x 2^8 x key-scale
      //    ratio (lo = the rounding residual of hi); BF16 for rope
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
      // -- PV: O^T[dims x heads] += X^T[dims x keys] P^T[keys x heads]
      {
        const int krow = 32 * kh + kappa(g, r >> 1);
        const uint8_t* a8 = xn + krow * C::NP + 8 * (r & 1);
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt) {
          const v2i a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CSA_LDS v2i*)(a8 + 16 * dt));
          const long al = (long)(uint32_t)a[0] | ((long)(uint32_t)a[1] << 32);
          O[dt] = mfma_f8_32(al, p8, O[dt]);
          O[dt] = mfma_f8_32(al, p8l, O[dt]);
        }
        const int krow0 = 32 * kh + kappa(g, r >> 2);
        const int krow1 = 32 * kh + kappa(g, 4 + (r >> 2));
        const uint8_t* b0 = xr + krow0 * C::RP + 8 * (r & 3);
        const uint8_t* b1 = xr + krow1 * C::RP + 8 * (r & 3);
#pragma unroll
        for (int dt = 0; dt < C::NDR; ++dt) {
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(b0 + 32 * dt));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS v4s*)(b1 + 32 * dt));
          v4i packed;
          packed[0] = (int)((uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16));
          packed[1] = (int)((uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16));
          packed[2] = (int)((uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16));
          packed[3] = (int)((uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
          O[C::ND + dt] = mfma_bf16_32(__builtin_bit_cast(v8bf, packed), pbf, O[C::ND + dt]);
        }
      }
    }
    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- merge the two key halves (kh) of each head tile through LDS
  const float l_tot = sum_over_groups(l_run);
  float* ex = reinterpret_cast<float*>(&xs[0][0]);                   // [4][HALF][64][4]
  float* st = ex + 4 * C::HALF * 64 * 4;                               // [4][64][2]
  if (kh == 0) {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j)
      *reinterpret_cast<v4f*>(ex + ((wave * C::HALF + j) * 64 + lane) * 4) = O[C::HALF + j];
  } else {
#pragma unroll
    for (int j = 0; j < C::HALF; ++j)
      *reinterpret_cast<v4f*>(ex + ((wave * C::HALF + j) * 64 + lane) * 4) = O[j];
  }
  st[(wave * 64 + lane) * 2 + 0] = m_run;
  st[(wave * 64 + lane) * 2 + 1] = l_tot;
  __syncthreads();
  if (!tile_ok) return;
  const int partner = wave ^ 2;
  const float pm = st[(partner * 64 + lane) * 2 + 0];
  const float pl = st[(partner * 64 + lane) * 2 + 1];
  const float M = fmaxf(m_run, pm);
  const float Ms = (M == -__builtin_inff()) ? 0.0f : M;
  const float a_self = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - Ms);
  const float a_oth = (pm == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(pm - Ms);
  const float L = l_tot * a_self + pl * a_oth;
  const float nope_unit = smax * (1.0f / 256.0f);
  const bool final_out = p.n_splits == 1;
  const float invL = (final_out && L > 0.0f) ? 1.0f / L : 0.0f;

  auto finish = [&](int dt, const v4f& own) {
    const v4f oth = *reinterpret_cast<const v4f*>(ex + ((partner * C::HALF + (dt - kh * C::HALF)) * 64 + lane) * 4);
    const bool nope = dt < C::ND;
    const float unit = nope ? nope_unit : 1.0f;
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
  const int blocks = ((p.T + 7) / 8) * 8 * nb;
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
