"""The CSA hot path in plain FP64 NumPy (test infrastructure; see the package
docstring for the source legend and for who may import this).

Notation: a query token t belongs to sequence seq(t), sits at absolute
position pos(t) (0-based; the context includes the query token itself), and
sees a compressed cache of n_comp(seq) entries, entry c covering tokens
[c*m, (c+1)*m).  The latent of an entry is D = D_nope + D_rope wide, nope dims
first, and it serves as both key and value for every query head.
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3_decode, bf16_decode, mxfp4_decode


# --------------------------------------------------------------------------
# Visibility and paged addressing
# --------------------------------------------------------------------------
def n_visible(pos: int, m: int, n_comp: int) -> int:
    """Number of compressed entries a query at `pos` may see.

    [Audit] A3, item 1: a query sees only compressed blocks strictly before
    its own current block, never its own or later blocks.  Its own block is
    floor(pos/m), so the visible entries are c < floor(pos/m).  Reading: this
    holds even when pos is the last token of a block whose entry is already
    stored (that entry is then stored but not visible).  Entries that are not
    stored (c >= n_comp) are never visible.
    """
    return int(min(pos // m, n_comp))


def entry_rows(page_table_row: np.ndarray, page_size: int, idx: np.ndarray) -> np.ndarray:
    """Physical row (page * page_size + slot) of logical entries `idx` of one
    sequence.  [Roadmap] E1: the compressed cache is paged through a block
    table."""
    idx = np.asarray(idx, dtype=np.int64)
    return page_table_row[idx // page_size].astype(np.int64) * page_size + idx % page_size


def dequant_entries(nope: np.ndarray, rope: np.ndarray, scale: float) -> np.ndarray:
    """Latent rows as float64: E4M3 nope dims times the stored scale, then the
    BF16 rope dims ([Audit] B1; [Roadmap] E1 "inverse-scale stored alongside",
    read as a per-tensor multiply-to-dequantise factor)."""
    return np.concatenate([e4m3_decode(nope) * float(scale), bf16_decode(rope)], axis=-1)


# --------------------------------------------------------------------------
# Step 1: lightning-indexer scores
# --------------------------------------------------------------------------
def sequence_index_keys(wl, b: int) -> np.ndarray:
    """All stored indexer keys of sequence b, float64 [n_comp][D_I]."""
    s = wl.spec
    rows = entry_rows(wl.page_table[b], s.page_size, np.arange(int(wl.n_comp[b])))
    flat = wl.k_idx.reshape(-1, s.D_I)
    return e4m3_decode(flat[rows]) * float(wl.k_idx_scale)


def sequence_index_keys_mxfp4(wl, b: int) -> np.ndarray:
    """All stored MXFP4 indexer keys of sequence b, float64 [n_comp][D_I]."""
    s = wl.spec
    rows = entry_rows(wl.page_table[b], s.page_size, np.arange(int(wl.n_comp[b])))
    return mxfp4_decode(wl.k_idx4.reshape(-1, s.D_I // 2)[rows], wl.k_idx4_sc.reshape(-1, s.D_I // 32)[rows])


def index_scores_mxfp4(wl, t: int, keys: np.ndarray | None = None) -> np.ndarray:
    """The indexer scores of index_scores() with q_idx and k_idx taken from
    their MXFP4 copies ([Audit] B2: the QK of the indexer in FP4, as the
    paper does; [Roadmap] E7: FP4 keys and queries with block scales decoded
    by the hardware).  Same formula; only the stored values differ."""
    s = wl.spec
    b = int(wl.q_seq[t])
    nv = n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
    if keys is None:
        keys = sequence_index_keys_mxfp4(wl, b)
    q = mxfp4_decode(wl.q_idx4[t], wl.q_idx4_sc[t])                  # [H_I][D_I]
    logits = q @ keys[:nv].T
    w = wl.w[t].astype(np.float64)
    return w @ np.maximum(logits, 0.0)


def index_scores_unquantised(wl, t: int) -> np.ndarray:
    """The indexer scores of index_scores() on the draws before any
    quantisation (spec.keep_float): the reference against which [Roadmap] E7
    measures an indexer's recall ("recall vs the FP32 oracle").  Same
    formula; only the inputs differ."""
    s = wl.spec
    b = int(wl.q_seq[t])
    nv = n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
    off = int(wl.entry_offset[b])
    keys = wl.k_idx_f32[off:off + nv].astype(np.float64)
    q = wl.q_idx_f32[t].astype(np.float64)
    w = wl.w[t].astype(np.float64)
    return w @ np.maximum(q @ keys.T, 0.0)


def index_scores(wl, t: int, keys: np.ndarray | None = None) -> np.ndarray:
    """Indexer scores of query t over its visible entries, float64 [n_vis].

    [Audit] B2: the indexer logits are the einsum 'tnd,cd->tnc' of the index
    queries (n index heads of d dims per token) with one key per compressed
    entry (MQA-shaped: the key is shared by all index heads), and the kernel
    that replaces it is a weighted-ReLU MQA-logits kernel.  Written out:

        score[t, c] = sum_h w[t, h] * max(0, q_idx[t, h, :] . k_idx[c, :])

    with q_idx and k_idx dequantised by their stored scales.  Reading: no
    extra constant factor (a positive constant cannot change the top-k).
    """
    s = wl.spec
    b = int(wl.q_seq[t])
    nv = n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
    if keys is None:
        keys = sequence_index_keys(wl, b)
    q = e4m3_decode(wl.q_idx[t]) * float(wl.q_idx_scale)           # [H_I][D_I]
    logits = q @ keys[:nv].T                                          # [H_I][nv]
    w = wl.w[t].astype(np.float64)                                    # [H_I]
    return w @ np.maximum(logits, 0.0)


# --------------------------------------------------------------------------
# Step 2: causal top-k
# --------------------------------------------------------------------------
def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best visible entries, int32 [k].

    [Audit] B2 / [Roadmap] E7: the top-k is taken over the indexer scores of
    the visible entries (causality is applied by n_visible: `scores` holds
    exactly the visible entries).  Readings: a larger score wins; equal
    scores go to the lower index; with fewer than k visible entries all of
    them are taken and the rest is -1.  The selection is a set; it is
    returned in ascending index order.
    """
    n = len(scores)
    order = np.lexsort((np.arange(n), -np.asarray(scores, dtype=np.float64)))
    chosen = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: len(chosen)] = chosen
    return out


# --------------------------------------------------------------------------
# Step 3: the key set (gather)
# --------------------------------------------------------------------------
def swa_window(pos: int, W: int) -> tuple[int, int]:
    """Positions [lo, hi] of the sliding window of a query at `pos`.

    [Audit] A3, item 2 and [README] KV cache management: the most recent
    tokens are kept uncompressed in a window of W (=128) tokens.  Reading: the
    window includes the query's own token: positions max(0, pos-W+1) .. pos.
    """
    return max(0, pos - W + 1), pos


def key_rows(wl, t: int, sel: np.ndarray | None) -> tuple[np.ndarray, list]:
    """Dequantised key/value rows of query t, float64 [n][D], and a label per
    row (('c', entry) or ('w', position)).

    [Audit] A3 ("5. Gather KV"): the query attends to [top-k compressed
    entries] ++ [SWA window].  [Audit] A3, item 2: a recent token may be both
    in the window and inside the newest complete compressed block; both
    representations are attended (reading: as distinct keys).  sel=None is
    the HCA mode of [Roadmap] E1 ("gather_all_compressed_kv", no top-k): every
    visible entry is attended.  Window rows come from the decode ring (slot
    membership by the position stored with the slot, [Roadmap] E1
    "read_swa_view ... positions") or, for a prefill chunk, from a linear
    token buffer.
    """
    s = wl.spec
    b = int(wl.q_seq[t])
    pos = int(wl.q_pos[t])
    if sel is None:
        ids = np.arange(n_visible(pos, s.m, int(wl.n_comp[b])))
    else:
        ids = np.asarray([c for c in sel if c >= 0], dtype=np.int64)
    rows = entry_rows(wl.page_table[b], s.page_size, ids)
    comp = dequant_entries(wl.lat_nope.reshape(-1, s.D_nope)[rows],
                           wl.lat_rope.reshape(-1, s.D_rope)[rows], wl.lat_scale)
    labels = [("c", int(c)) for c in ids]
    lo, hi = swa_window(pos, s.W)
    if s.kind == "decode":
        slots = [j for j in range(s.W) if lo <= int(wl.swa_pos[b, j]) <= hi]
        win = dequant_entries(wl.swa_nope[b, slots], wl.swa_rope[b, slots], wl.swa_scale)
        labels += [("w", int(wl.swa_pos[b, j])) for j in slots]
    else:
        ps_ = [p for p in range(lo, hi + 1)
               if wl.swa_first_pos <= p < wl.swa_first_pos + wl.swa_len]
        r = np.asarray(ps_, dtype=np.int64) - wl.swa_first_pos
        win = dequant_entries(wl.swa_nope[r], wl.swa_rope[r], wl.swa_scale)
        labels += [("w", p) for p in ps_]
    return np.concatenate([comp, win], axis=0), labels


# --------------------------------------------------------------------------
# Step 4: shared-latent attention with a per-head sink
# --------------------------------------------------------------------------
def attend(q: np.ndarray, X: np.ndarray, sink: np.ndarray, sigma: float):
    """Attention of all heads over the key rows X, float64.

    [README] Architecture: the latent (D = 512 wide) is shared by all 128
    query heads as both key and value, and per-head sink weights merge the
    sparse and SWA attention.  Written out, per head h over keys j:

        S[h, j] = sigma * q[h, :] . X[j, :]
        M[h]    = max(max_j S[h, j], sink[h])
        den[h]  = sum_j exp(S[h, j] - M[h]) + exp(sink[h] - M[h])
        o[h, :] = sum_j exp(S[h, j] - M[h]) * X[j, :] / den[h]
        lse[h]  = M[h] + ln den[h]

    i.e. the sink is one extra logit with a zero value vector.  Readings: the
    sink logit is not multiplied by sigma; the value is the full latent
    (nope and rope dims), whose rope dims are de-rotated after attention
    ([Audit] A4, not part of this path); lse as returned by [Roadmap] E4.
    An empty key set with a -inf sink gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    S = sigma * (q @ X.T)                                              # [H][n]
    smax = S.max(axis=1) if S.shape[1] else np.full(len(sink), -np.inf)
    M = np.maximum(smax, sink)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    e = np.exp(S - Msafe[:, None])
    den = e.sum(axis=1) + np.exp(sink - Msafe)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(den[:, None] > 0, (e @ X) / np.where(den > 0, den, 1.0)[:, None], 0.0)
        lse = np.where(den > 0, Msafe + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return o, lse


def merge_by_lse(o_a, lse_a, o_b, lse_b):
    """Combine attention over two disjoint key subsets from their (o, lse)
    pairs ([Roadmap] E4 returns lse for this).  The sink must be counted in
    exactly one of the two parts."""
    lse = np.logaddexp(lse_a, lse_b)
    safe = np.where(np.isfinite(lse), lse, 0.0)
    wa = np.where(np.isfinite(lse_a), np.exp(lse_a - safe), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(lse_b - safe), 0.0)
    return o_a * wa[:, None] + o_b * wb[:, None], lse


def query_heads(wl, t: int) -> np.ndarray:
    return bf16_decode(wl.q[t])


def run_attention(wl, sel=None, queries=None):
    """Attention for every query (or the listed ones).  `sel` is [T][k] top-k
    indices (-1 padded) or None for HCA mode.  Returns o [n][H][D], lse [n][H]."""
    s = wl.spec
    ts = range(wl.T) if queries is None else queries
    os_, ls_ = [], []
    for t in ts:
        X, _ = key_rows(wl, t, None if sel is None else sel[t])
        o, lse = attend(query_heads(wl, t), X, wl.sink, s.sigma)
        os_.append(o)
        ls_.append(lse)
    return np.stack(os_), np.stack(ls_)


def run_decode_path(wl, queries=None):
    """The whole path for every query (or the listed ones): scores, top-k,
    attention.  Returns a dict with per-query lists of scores, and arrays
    topk [n][k], o [n][H][D], lse [n][H]."""
    s = wl.spec
    ts = list(range(wl.T)) if queries is None else list(queries)
    keys_cache = {}
    scores, sels = [], []
    for t in ts:
        b = int(wl.q_seq[t])
        if b not in keys_cache:
            keys_cache[b] = sequence_index_keys(wl, b)
        sc = index_scores(wl, t, keys_cache[b])
        scores.append(sc)
        sels.append(topk_select(sc, s.k))
    os_, ls_ = [], []
    for i, t in enumerate(ts):
        X, _ = key_rows(wl, t, sels[i])
        o, lse = attend(query_heads(wl, t), X, wl.sink, s.sigma)
        os_.append(o)
        ls_.append(lse)
    return dict(queries=ts, scores=scores, topk=np.stack(sels), o=np.stack(os_),
                lse=np.stack(ls_))


# --------------------------------------------------------------------------
# After step 4: inverse RoPE of the output's rope dims
# --------------------------------------------------------------------------
def inverse_rope(o: np.ndarray, pos: int, d_nope: int, theta: float) -> np.ndarray:
    """The attention output with its rope dims rotated back by RoPE(-pos).

    [Audit] A4: the attention output is de-rotated at the query's own
    position (not the compressed entries' positions) by the rotation with the
    negated angle, which turns the absolute positions carried by the summed
    latents into relative ones.  Readings (the pages give no formula): the
    rope dims are the last D_rope dims (nope first); they pair up as
    consecutive dims (2i, 2i + 1) of the rope part, taken as the real and
    imaginary part of one complex number; pair i turns at frequency
    theta^(-2i / D_rope), the usual rotary schedule with base theta.  The
    forward rotation at position p multiplies pair i by exp(+1j p f_i), so the
    inverse multiplies it by exp(-1j p f_i).  The nope dims are unchanged.
    `o` is [..., D] (any leading shape).
    """
    o = np.array(o, dtype=np.float64, copy=True)
    d_rope = o.shape[-1] - d_nope
    freq = float(theta) ** (-2.0 * np.arange(d_rope // 2) / d_rope)
    angle = -float(pos) * freq
    c, s = np.cos(angle), np.sin(angle)
    x = o[..., d_nope::2].copy()
    y = o[..., d_nope + 1::2].copy()
    o[..., d_nope::2] = x * c - y * s
    o[..., d_nope + 1::2] = x * s + y * c
    return o
