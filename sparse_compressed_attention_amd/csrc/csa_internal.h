// Parameter blocks and launchers shared by the C ABI (csa_abi.cpp) and the
// kernels.  Host-validated before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

struct IndexParams {
  const uint8_t* q_idx;
  const float* w;
  const uint8_t* k_idx;
  const int32_t* page_table;
  const int32_t* n_comp;
  const int32_t* q_pos;
  const int32_t* q_seq;
  float* scores;
  int32_t* n_visible;
  int64_t ld;
  float qk_scale;     // q_idx_scale * k_idx_scale (1 for MXFP4)
  const uint8_t* q_sc; // MXFP4: E8M0 scales [T][H_I][D_I / 32] and
  const uint8_t* k_sc; //        [num_pages][page_size][D_I / 32]
  int fp4;             // q_idx / k_idx are MXFP4 (E2M1 pairs) instead of E4M3
  int num_pages, page_size, max_pages, B;
  int T, H_I, D_I, ratio_m;
  int chunk, n_chunks;   // set by the launcher
};
hipError_t launch_index_scores(const IndexParams& p, hipStream_t stream);

struct TopkParams {
  const float* scores;
  const int32_t* n_visible;
  int32_t* out;
  uint32_t* cand_key;   // [T][n_chunks][k] (multi-chunk rows only)
  int32_t* cand_idx;
  int64_t ld;
  int T, k;
  int chunk, n_chunks;
};
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);
// stage 2 alone: merges per-chunk candidates already in cand_key / cand_idx
hipError_t launch_topk_merge(const TopkParams& p, hipStream_t stream);
// fused indexer + top-k (decode kernel layout, E4M3 operands): scores stay in
// LDS; one workgroup per (row, chunk of `chunk` entries) selects the chunk's
// top-k, then the merge (when a row has several chunks)
hipError_t launch_index_topk(const IndexParams& ip, const TopkParams& tp, hipStream_t stream);
// fused indexer + top-k for many queries of one sequence (ip.B == 1, ip.ld =
// the key range, at most 65536 entries): workgroups of kIndexTopkPrefillQ
// queries share each key tile, each query keeps a candidate buffer in LDS;
// tp.n_chunks parts of the key range per query block, then the merge
hipError_t launch_index_topk_prefill(const IndexParams& ip, const TopkParams& tp, hipStream_t stream);
constexpr int kIndexTopkPrefillQ = 8;
constexpr int kIndexTopkPrefillMaxK = 1024;
constexpr int64_t kIndexTopkPrefillMaxSpan = 65536;
constexpr int kTopkMaxChunk = 16384;
constexpr int kTopkMaxCand = 16384;
constexpr int kTopkMaxK = 2048;

struct AttnParams {
  const uint16_t* q;
  int64_t q_stride;
  const uint8_t* lat_nope;
  const uint16_t* lat_rope;
  const int32_t* page_table;
  const int32_t* n_comp;
  const int32_t* topk;     // [T][k] or nullptr (all visible entries)
  // top-k selected inside the attention kernel (csa_topk_decode_attn):
  // indexer scores [T][ld_scores] and visible counts [T], or nullptr;
  // topk_out [T][k] receives the indices (nullable)
  const float* scores;
  int64_t ld_scores;
  const int32_t* n_visible;
  int32_t* topk_out;
  const uint8_t* swa_nope;
  const uint16_t* swa_rope;
  const int32_t* swa_pos;  // ring positions [B][W] (decode) or nullptr (prefill)
  const int32_t* q_pos;
  const float* sink;
  uint16_t* out;
  float* lse;
  // split partial results or nullptr: rows of part_row_bytes(D) bytes,
  // [n_splits][T][H]: the split's output over its denominator as D BF16,
  // then (M, L) as two floats, then padding to 16 bytes
  uint8_t* part;
  float lat_scale, swa_scale;
  float sm_scale;          // softmax scale (natural-log units)
  // derived on the host (uniform): sm_scale*log2(e); FP8 probability scale
  // 2^(8 - tau) and its inverse; lat_scale / swa_scale (the rescale of the
  // FP8 accumulators where the key range passes to the window rows)
  float sm_log2, pscale, inv_pscale, lat_over_swa;
  // inverse RoPE of the output's rope dims at the query position (inv_rope
  // != 0) with base 2^rope_log2_theta
  double rope_log2_theta;
  int inv_rope;
  // entry / page_size == (entry * ps_magic) >> ps_shift for 0 <= entry < 2^31
  uint64_t ps_magic;
  int ps_shift;
  int num_pages, page_size, max_pages, ratio_m;
  int k, W;
  int prefill_seq;         // -1: decode (query t belongs to sequence t)
  int swa_first_pos, swa_len;
  int T, H;
  int D_nope, D_rope;
  int ht;                  // 16-head tiles per workgroup (2 or 4)
  int n_hg, n_splits, per_split;
};
hipError_t launch_attn(const AttnParams& p, hipStream_t stream);
// Address of the current device's copy of the library's static attention
// scratch array (kAttnScratchBytes), looked up once per device.
hipError_t attn_scratch_address(void** ptr);
constexpr size_t kAttnScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
constexpr int kAttnMaxSlots = 2048;   // key slots one workgroup handles
constexpr int kAttnSelMax = 8192;     // longest score row the attention kernel selects from
constexpr int kAttnTau = 4;           // lazy-rescale threshold (log2 units)
constexpr int kAttnTile = 64;
constexpr int kAttnMaxSplits = 128;   // splits of one query's key slots
// bytes of one split partial row: D BF16 values, (M, L), 16-byte aligned
__host__ __device__ constexpr size_t part_row_bytes(int D) { return (size_t)2 * D + 16; }

}  // namespace csa
