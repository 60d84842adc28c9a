/*
 * csa.h -- C ABI of libcsa.so, the Compressed Sparse Attention (CSA) hot path
 * for one AMD Instinct MI355X (gfx950).
 *
 * The path has four steps, exposed as four calls (plus workspace queries):
 *   csa_index_scores  lightning-indexer scores            (step 1)
 *                     (csa_index_scores_mxfp4: FP4 operands)
 *   csa_index_topk    steps 1+2 fused, scores kept on chip
 *   csa_topk          causal top-k over those scores      (step 2)
 *   csa_decode_attn   gather + sink attention, decode     (steps 3+4)
 *                     (csa_topk_decode_attn: steps 2-4 in one launch)
 *   csa_prefill_attn  gather + sink attention, prefill    (steps 3+4)
 * and graph capture/replay of a whole step (csa_graph_*).
 *
 * Sources (page title and section):
 *   [Audit]   "DSV4 Audit -- Decode Repetition + Precision / Tensor-Core
 *             Plan": A3 (visible compressed blocks; SWA/compressed overlap;
 *             "5. Gather KV"), A4 (inverse RoPE of the attention output),
 *             B1 (FP8_E4M3 nope dims + BF16 rope dims fed to the MMA
 *             without dequantisation), B2 (weighted-ReLU MQA
 *             indexer logits; top-k with no global lock).
 *   [Roadmap] "ROADMAP -- Stage E and the path to a runnable model": E1
 *             (paged FP8 cache + block table + stored scale; gathers of
 *             selected / all compressed entries and of the SWA window), E4
 *             (launch returns a code, errors by peek-at-last-error, no
 *             device sync; attention returns (o, lse)), E5 (batch folded
 *             into the grid), E7 (indexer top-k), E8 (prefill spread over
 *             many workgroups), E9 (graph capture of the decode step).
 *   [README]  "DSV4 Inference Kernel": Architecture (CSA m=4, HCA m'=128,
 *             latent (T, 512) shared by all 128 heads, sink weights merge
 *             the sparse and SWA attention).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    the two struct pointers (csa_latent_cache*, csa_swa_ring*), which point
 *    to HOST structs read during the call.  No step call (csa_index_scores*,
 *    csa_topk, csa_*_attn) keeps a pointer after it returns, allocates
 *    device memory, or synchronises the device; the csa_graph_* calls
 *    create and free graph objects and are meant for set-up, not for the
 *    step itself.  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL = default stream) and runs asynchronously.
 *  - Return value: CSA_OK (0) or a negative error code.  Argument errors are
 *    detected on the host before any launch (nothing is enqueued).  Launch
 *    errors are detected with hipPeekAtLastError() after the launch.
 *  - Data formats: E4M3 = OCP FP8 E4M3FN bytes; BF16 = bfloat16 bit
 *    patterns in uint16_t.  Each FP8 tensor carries one float "scale": the
 *    stored value times the scale is the real value (MXFP4 tensors carry
 *    block scales instead; see csa_index_scores_mxfp4).
 *  - Latent layout: D = D_nope + D_rope dims, nope dims first.  K = V =
 *    the whole latent, shared by all query heads.
 *  - Positions are absolute, 0-based; a query's context includes its own
 *    token.  Compressed entry c covers tokens [c*m, (c+1)*m).  A query at
 *    position pos sees entries c < n_vis = min(floor(pos/m), n_comp[seq])
 *    ([Audit] A3: only blocks strictly before the query's own block).
 *  - Defensive reads: a page-table entry outside [0, num_pages), a top-k
 *    index outside [0, n_comp[seq]) or equal to -1, and an empty ring slot
 *    are never dereferenced: such entries score -inf / are not attended.
 *  - Results are deterministic run to run (no floating-point atomics).
 *  - Calls are safe to issue concurrently on different streams only if
 *    their workspaces are distinct.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_OK 0
#define CSA_ERR_INVALID_ARG (-1)  /* null pointer, bad size/stride/alignment */
#define CSA_ERR_UNSUPPORTED (-2)  /* a shape no kernel is built for         */
#define CSA_ERR_LAUNCH (-3)       /* hipPeekAtLastError() after a launch     */
#define CSA_ERR_WORKSPACE (-4)    /* workspace missing or too small          */
#define CSA_ERR_TOO_LARGE (-5)    /* beyond the fixed scratch of a _noalloc call */

/* Returned by the csa_*_workspace_size queries for arguments that the
 * matching call would reject (a shape with no kernel or an invalid size):
 * 0 means "no workspace needed", this value means "unsupported". */
#define CSA_WORKSPACE_UNSUPPORTED ((size_t)-1)

/* Paged compressed-latent cache of one layer ([Roadmap] E1 "classical paged
 * cache": FP8 entries + BF16 rope + block table + stored scale).
 *   nope       [num_pages][page_size][D_nope] E4M3, 16-byte aligned
 *   rope       [num_pages][page_size][D_rope] BF16, 16-byte aligned
 *   nope_scale dequant multiplier of `nope` (> 0)
 *   page_table [B][max_pages] int32: physical page of logical page j of
 *              sequence b; entry c of sequence b lives at row
 *              page_table[b][c / page_size] * page_size + c % page_size
 *   n_comp     [B] int32: stored entries of each sequence
 *   num_seqs   B, the number of rows of page_table and n_comp
 *   ratio_m    compression ratio m (4 for CSA, 128 for HCA)
 * Supported (D_nope, D_rope): (448, 64) and (48, 16).  page_size % 16 == 0. */
typedef struct csa_latent_cache {
  const uint8_t* nope;
  const uint16_t* rope;
  float nope_scale;
  const int32_t* page_table;
  const int32_t* n_comp;
  int32_t num_seqs;
  int32_t num_pages;
  int32_t page_size;
  int32_t max_pages;
  int32_t D_nope;
  int32_t D_rope;
  int32_t ratio_m;
} csa_latent_cache;

/* Sliding-window ring of the decode batch ([README] KV cache management:
 * "SWA window"; [Roadmap] E1 read_swa_view = FP8 entries + BF16 rope +
 * positions).  One ring of W slots per sequence:
 *   nope [B][W][D_nope] E4M3, rope [B][W][D_rope] BF16, pos [B][W] int32
 * pos holds the absolute token position stored in each slot, -1 if empty.
 * A slot is attended by the query at position q iff q-W+1 <= pos <= q;
 * slot order is irrelevant. */
typedef struct csa_swa_ring {
  const uint8_t* nope;
  const uint16_t* rope;
  float nope_scale;
  const int32_t* pos;
  int32_t W;
} csa_swa_ring;

/* ---- Step 1: indexer scores ([Audit] B2) ------------------------------
 * For each query row t (sequence q_seq[t], or t when q_seq is NULL as in a
 * decode batch; position q_pos[t]) and each
 * visible entry c < n_vis(t):
 *   scores[t*ld_scores + c] =
 *       sum_h w[t][h] * max(0, (q_idx_scale*q_idx[t][h][:]) .
 *                              (k_idx_scale*k_idx[entry c of q_seq[t]][:]))
 * and n_visible[t] = n_vis(t).  Columns c >= n_vis(t) are not written.
 *   q_idx [T][H_I][D_I] E4M3 (16-byte aligned), w [T][H_I] float,
 *   k_idx [num_pages][page_size][D_I] E4M3 (16-byte aligned), paged by
 *   page_table [B][max_pages] / n_comp [B] exactly like the latent cache.
 * Supported: 1 <= H_I <= 64, D_I in {32, 64, 96, 128}, page_size % 16 == 0,
 * ld_scores >= max over rows of n_vis.  Errors: CSA_ERR_INVALID_ARG,
 * CSA_ERR_UNSUPPORTED, CSA_ERR_LAUNCH. */
int csa_index_scores(const uint8_t* q_idx, float q_idx_scale, const float* w,
                     const uint8_t* k_idx, float k_idx_scale,
                     const int32_t* page_table, const int32_t* n_comp,
                     int32_t num_pages, int32_t page_size, int32_t max_pages, int32_t B,
                     const int32_t* q_pos, const int32_t* q_seq, int32_t T,
                     int32_t H_I, int32_t D_I, int32_t ratio_m,
                     float* scores, int64_t ld_scores, int32_t* n_visible,
                     void* stream);

/* ---- Step 1, MXFP4 variant ([Audit] B2: the indexer QK on FP4 tensor
 * units; [Roadmap] E7: FP4 indexer scoring) -------------------------------
 * Same result definition and arguments as csa_index_scores, with q_idx and
 * k_idx in the OCP MX FP4 format instead of E4M3 with a per-tensor scale:
 *   q_idx    [T][H_I][D_I / 2] bytes, k_idx [num_pages][page_size][D_I / 2]
 *            bytes (16-byte aligned): E2M1 codes, two per byte, element 2j
 *            in bits 0-3 and element 2j + 1 in bits 4-7; code = sign bit 3,
 *            exponent bits 2-1, mantissa bit 0 (values 0, 0.5, 1, 1.5, 2,
 *            3, 4, 6 and their negatives);
 *   q_idx_sc [T][H_I][D_I / 32], k_idx_sc [num_pages][page_size][D_I / 32]
 *            bytes: E8M0 block scales, value 2^(byte - 127), one per block of
 *            32 consecutive dims (byte 255 = NaN is not allowed).
 * The real value of element d of a row is e2m1(code_d) * 2^(sc[d/32] - 127).
 * Products are exact in FP32 and accumulate in FP32, so the scores equal
 * the definition on the decoded values up to FP32 summation order.  The key
 * scan reads D_I / 2 + D_I / 32 bytes per entry (68 at D_I = 128), about
 * half of the E4M3 scan.  Errors as csa_index_scores (null scale arrays are
 * CSA_ERR_INVALID_ARG). */
int csa_index_scores_mxfp4(const uint8_t* q_idx, const uint8_t* q_idx_sc, const float* w,
                           const uint8_t* k_idx, const uint8_t* k_idx_sc,
                           const int32_t* page_table, const int32_t* n_comp,
                           int32_t num_pages, int32_t page_size, int32_t max_pages, int32_t B,
                           const int32_t* q_pos, const int32_t* q_seq, int32_t T,
                           int32_t H_I, int32_t D_I, int32_t ratio_m,
                           float* scores, int64_t ld_scores, int32_t* n_visible,
                           void* stream);

/* ---- Step 2: causal top-k ([Audit] B2; [Roadmap] E7) ------------------
 * For each row t, selects the min(k, n_visible[t]) largest of
 * scores[t*ld_scores + 0 .. n_visible[t]-1]; equal scores go to the lower
 * index.  topk_idx[t][0..k) receives the selected indices in ascending
 * order followed by -1 padding.  Lock-free: per-chunk candidate selection
 * then a per-row merge, both with workgroup-local radix selection.
 *   scores [T][ld_scores] float, n_visible [T] int32 (values clamped to
 *   [0, ld_scores]), topk_idx [T][k] int32.
 * The workspace (bytes from csa_topk_workspace_size) may be NULL when
 * ld_scores <= 16384.  csa_topk_workspace_size returns 0 when no workspace
 * is needed and CSA_WORKSPACE_UNSUPPORTED for arguments csa_topk rejects.
 * Supported: 1 <= k <= 2048.
 * Errors: CSA_ERR_INVALID_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE,
 * CSA_ERR_LAUNCH. */
size_t csa_topk_workspace_size(int32_t T, int64_t ld_scores, int32_t k);
int csa_topk(const float* scores, int64_t ld_scores, const int32_t* n_visible,
             int32_t T, int32_t k, int32_t* topk_idx,
             void* workspace, size_t workspace_bytes, void* stream);

/* ---- Steps 1+2 fused ([Audit] B2: weighted-ReLU MQA logits and a top-k
 * with a wave-local reduction and no global lock) --------------------------
 * The result of csa_index_scores followed by csa_topk with ld_scores =
 * max_pages * page_size (same selection rule, bit-identical indices),
 * without writing the scores.  Two plans:
 *   - one sequence (B == 1), T >= 16, k <= 1024, max_pages * page_size <=
 *     65536 (a prefill chunk): workgroups of 8 queries share each key tile
 *     and every query keeps a candidate buffer on chip (entries above a
 *     running threshold, cut back to about k when full); the key range is
 *     split over workgroups when there are fewer query blocks than CUs;
 *   - otherwise one workgroup per (row, chunk of 2048, 4096 or 8192
 *     entries) keeps its chunk's scores in LDS and selects the chunk's
 *     top-k there.
 * Rows whose range was split are finished by the top-k merge over the
 * parts' candidates.  Outputs: topk_idx [T][k] (ascending, -1 padding) and
 * n_visible [T] (clamped to max_pages * page_size).  E4M3 operands only.
 * Workspace: csa_index_topk_workspace_size(T, max_pages * page_size, k)
 * bytes, enough for either plan (0 when no row is split; NULL is then
 * allowed; CSA_WORKSPACE_UNSUPPORTED for arguments csa_index_topk rejects).
 * Supported: 1 <= k <= 2048 and (max_pages * page_size) / 8192 chunks of k
 * candidates within the merge's 16384 (CSA_ERR_UNSUPPORTED otherwise).
 * Errors: CSA_ERR_INVALID_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE,
 * CSA_ERR_LAUNCH. */
size_t csa_index_topk_workspace_size(int32_t T, int64_t max_entries, int32_t k);
int csa_index_topk(const uint8_t* q_idx, float q_idx_scale, const float* w,
                   const uint8_t* k_idx, float k_idx_scale,
                   const int32_t* page_table, const int32_t* n_comp,
                   int32_t num_pages, int32_t page_size, int32_t max_pages, int32_t B,
                   const int32_t* q_pos, const int32_t* q_seq, int32_t T,
                   int32_t H_I, int32_t D_I, int32_t ratio_m, int32_t k,
                   int32_t* topk_idx, int32_t* n_visible,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---- Steps 3+4: gather + shared-latent sink attention ----------------
 * For query t with key set J_t ([Audit] A3 "5. Gather KV"):
 *   compressed entries topk_idx[t][0..k) (entries < 0 or >= n_comp are
 *   skipped; topk_idx == NULL selects HCA mode: every visible entry
 *   c < n_vis(t), [Roadmap] E1 gather_all_compressed_kv), plus the window
 *   tokens with positions in [pos-W+1, pos].  A token both in the window
 *   and in a visible compressed block is attended in both forms ([Audit]
 *   A3, item 2).  Then for every head h ([README] Architecture):
 *     S_j   = softmax_scale * q[t][h][:] . x_j         (x_j dequantised)
 *     M     = max(max_j S_j, sink[h])
 *     den   = sum_j exp(S_j - M) + exp(sink[h] - M)
 *     out[t][h][:] = sum_j exp(S_j - M) x_j / den       (all D dims, BF16)
 *     lse[t][h]    = M + ln(den)                        (natural log)
 * No key and sink = -inf gives out = 0, lse = -inf.
 * Inverse RoPE ([Audit] A4: the attention output is rotated back by
 * RoPE(-pos) at the query's own position, which turns the absolute
 * positions carried by the summed latents into relative ones): when
 * inv_rope_theta > 0, the rope dims of out (dims D_nope + 2i and
 * D_nope + 2i + 1, i < D_rope / 2) are rotated before the BF16 store:
 *     a_i = -q_pos[t] * inv_rope_theta^(-2i / D_rope)
 *     (x, y) -> (x cos a_i - y sin a_i, x sin a_i + y cos a_i)
 * inv_rope_theta == 0 leaves out as defined above; lse is not affected.
 * A negative or non-finite inv_rope_theta is CSA_ERR_INVALID_ARG.
 *   q [.][H][D] BF16 with row stride q_stride (elements between tokens,
 *   >= H*D, multiple of 8), 16-byte aligned; sink [H] float; out [.][H][D]
 *   BF16 contiguous; lse [.][H] float or NULL.
 * Precision: nope products run on FP8 MFMA (q split into two E4M3 terms
 * with a shared per-head power-of-two scale; probabilities, at most 16
 * relative to the running maximum of the key logits, scaled by 16 and split
 * into two E4M3 terms), rope products on BF16 MFMA, accumulation and the
 * softmax in FP32.  Each key source's FP8 scale (cache->nope_scale,
 * swa->nope_scale) is applied in FP32, to the logits and to the FP32
 * accumulators, so the two scales may differ by any ratio.  The sink joins
 * the maximum and the denominator in FP32 after the last key, so it does
 * not coarsen the probabilities however far it lies above the logits.
 * Workspace: needed only when the key range is split across workgroups
 * (few queries, or HCA with long context); csa_attn_workspace_size gives
 * the bytes for the preferred split (0: no split, no workspace needed;
 * CSA_WORKSPACE_UNSUPPORTED: dims with no kernel, or more key slots than
 * 128 splits of 2048 hold), and a smaller workspace makes the call use
 * fewer splits.  CSA_ERR_WORKSPACE if even the minimum split (per
 * workgroup at most 2048 key slots) does not fit.
 * Supported: H >= 1, (D_nope, D_rope) in {(448,64), (48,16)},
 * 1 <= W <= 1024, 0 <= k <= 2048. */
size_t csa_attn_workspace_size(int32_t n_queries, int32_t H, int32_t D_nope,
                               int32_t D_rope, int32_t max_keys_per_query);

/* Decode: B queries (B <= cache->num_seqs), query b belongs to sequence b
 * and sits at q_pos[b]; window rows come from `swa` (one ring per sequence).
 * topk_idx [B][k]. */
int csa_decode_attn(const uint16_t* q, int64_t q_stride,
                    const csa_latent_cache* cache,
                    const int32_t* topk_idx, int32_t k,
                    const csa_swa_ring* swa, const int32_t* q_pos,
                    const float* sink, float softmax_scale,
                    float inv_rope_theta, int32_t B, int32_t H,
                    uint16_t* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Decode with the top-k inside the attention kernel ([Audit] B2: top-k
 * with a wave-local reduction and no global lock; [Roadmap] E7): the result
 * of csa_topk(scores, ld_scores, n_visible, B, k, topk_idx) followed by
 * csa_decode_attn(..., topk_idx, k, ...), in one launch.  Every attention
 * workgroup of query b selects its row's top-k from scores[b][0 ..
 * n_visible[b]) itself, with csa_topk's selection rule (larger score first,
 * equal scores to the lower index), so the indices are identical to
 * csa_topk's; they stay on chip, and are also written to topk_idx [B][k]
 * (ascending, -1 padding) when topk_idx is not NULL.  The other arguments,
 * the result and the workspace (csa_attn_workspace_size with
 * max_keys_per_query = k + W) are those of csa_decode_attn.
 *   scores [B][ld_scores] float, n_visible [B] int32 (clamped to
 *   [0, ld_scores]), as csa_index_scores writes them.
 * Supported: 1 <= ld_scores <= 8192 (one workgroup holds a row) and
 * 1 <= k <= 2048; longer rows are CSA_ERR_UNSUPPORTED (use csa_topk and
 * csa_decode_attn).  Errors as csa_decode_attn. */
int csa_topk_decode_attn(const float* scores, int64_t ld_scores,
                         const int32_t* n_visible, int32_t k, int32_t* topk_idx,
                         const uint16_t* q, int64_t q_stride,
                         const csa_latent_cache* cache, const csa_swa_ring* swa,
                         const int32_t* q_pos, const float* sink, float softmax_scale,
                         float inv_rope_theta, int32_t B, int32_t H,
                         uint16_t* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Decode without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, result and errors as csa_decode_attn,
 * minus the workspace: the partial results of split key ranges go to a
 * static device array inside the library, one per GPU, of
 * CSA_NOALLOC_SCRATCH_BYTES (16 MiB), held until the process ends.  The call itself allocates nothing (no hipMalloc, no
 * allocating library routine); its first call on a device looks up that
 * device's array address once.  When the preferred split does not fit, the
 * call uses fewer splits; CSA_ERR_TOO_LARGE when even the minimum split's
 * partial results exceed the array.  Nothing in the array needs clearing:
 * every split's (max, denominator) state is written by the same call (an
 * empty split's as empty), and the merge uses a split's row only when its
 * state is not empty.  All calls
 * on one GPU share its array, which keeps the last call's contents, so
 * calls that overlap on one GPU (different streams, or graph replays in
 * flight together) race: serialise them. */
int csa_decode_attn_noalloc(const uint16_t* q, int64_t q_stride,
                            const csa_latent_cache* cache,
                            const int32_t* topk_idx, int32_t k,
                            const csa_swa_ring* swa, const int32_t* q_pos,
                            const float* sink, float softmax_scale,
                            float inv_rope_theta, int32_t B, int32_t H,
                            uint16_t* out, float* lse, void* stream);
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* Prefill chunk: T queries of sequence `seq` (< cache->num_seqs) at
 * positions q_pos[T];
 * window rows come from a linear token buffer that holds positions
 * [swa_first_pos, swa_first_pos + swa_len): swa_nope [swa_len][D_nope]
 * E4M3, swa_rope [swa_len][D_rope] BF16 ([Roadmap] E8: prefill spread over
 * many workgroups).  Window positions outside the buffer are skipped. */
int csa_prefill_attn(const uint16_t* q, int64_t q_stride,
                     const csa_latent_cache* cache, int32_t seq,
                     const int32_t* topk_idx, int32_t k,
                     const uint8_t* swa_nope, const uint16_t* swa_rope,
                     float swa_scale, int32_t swa_first_pos, int32_t swa_len,
                     int32_t W, const int32_t* q_pos, int32_t T,
                     const float* sink, float softmax_scale,
                     float inv_rope_theta, int32_t H,
                     uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---- Graph capture of a whole step ([Roadmap] E9: once the decode step is
 * free of synchronisation, capture it once and replay it, removing the host
 * launch overhead; no allocation on the hot path) -------------------------
 * None of the calls above allocates, synchronises or reads a host value
 * back, so a step (e.g. csa_index_scores -> csa_topk -> csa_decode_attn)
 * can be recorded once and replayed with one launch:
 *   csa_graph_capture_begin(s);  ...the step's calls on stream s...;
 *   csa_graph_capture_end(s, &g);  then csa_graph_launch(g, any_stream)
 * per step, and csa_graph_destroy(g) at the end.
 * The graph keeps the device pointers, sizes and scalars of the captured
 * calls: a replay reads the CURRENT contents of the same buffers (new q,
 * new cache rows, new positions), but shapes, pointers, k, W and scales
 * are fixed.  Host structs (csa_latent_cache, csa_swa_ring) are read only
 * during capture.  Buffers must outlive the graph.
 *   begin: `stream` must be a created stream (not NULL) that is not
 *          already capturing (CSA_ERR_INVALID_ARG); capture is thread-local,
 *          so only this thread's work on `stream` is recorded.
 *   end:   ends the capture and instantiates it; *graph = NULL and
 *          CSA_ERR_LAUNCH if the capture was invalidated.
 *   launch: enqueues one replay on `stream` (NULL = default stream); replays
 *          on one stream run in order, and replays of one graph must not
 *          overlap on different streams (they share buffers).
 * The handle is owned by the caller and freed by csa_graph_destroy (NULL
 * is a no-op). */
typedef struct csa_graph csa_graph;
int csa_graph_capture_begin(void* stream);
int csa_graph_capture_end(void* stream, csa_graph** graph);
int csa_graph_launch(const csa_graph* graph, void* stream);
void csa_graph_destroy(csa_graph* graph);

/* Text of a status code (static storage). */
const char* csa_status_string(int code);

/* Library version: major*10000 + minor*100 + patch. */
int csa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
