"""Pins for the FP64 oracle of the CSA path (CPU only).

Each test fixes the oracle to something other than itself: pure-Python brute
force on tiny inputs, hand-derived closed forms (tests/golden), library
routines (scipy's softmax, a full Python sort), and invariants the method
implies (causality, tie rule, ring-order independence, split/merge identity,
top-k=all equals dense attention).  The shapes are deliberately non-square.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import csa_inputs as ci
import oracle
from oracle import csa as oc
from oracle.brute import brute_path

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def tiny_spec(**kw):
    base = dict(name="tiny", kind="decode", ctx_lens=[60, 37, 96], H=5, D_nope=24, D_rope=8,
                H_I=3, D_I=16, k=6, W=7, m=4, page_size=8, shuffle_pages=True)
    base.update(kw)
    return ci.Spec(**base)


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------------ visibility
@pytest.mark.parametrize("pos,m,n_comp,expect", [
    (255, 4, 64, 63), (256, 4, 64, 64), (8191, 4, 2048, 2047), (3, 4, 5, 0),
    (524287, 4, 131072, 131071), (524287, 128, 4096, 4095), (65535, 4, 16384, 16383),
    (63488, 4, 16384, 15872), (1000, 4, 10, 10),
])
def test_n_visible(pos, m, n_comp, expect):
    assert oc.n_visible(pos, m, n_comp) == expect


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("spec_fn", [lambda: ci.spec_for("c0"), tiny_spec,
                                     lambda: tiny_spec(ctx_lens=[33], k=20, shuffle_pages=False)])
def test_oracle_matches_brute_force(spec_fn):
    wl = ci.generate(spec_fn(), seed=7)
    res = oracle.run_decode_path(wl)
    for t in range(wl.T):
        scores, chosen, o, lse = brute_path(wl, t)
        np.testing.assert_allclose(res["scores"][t], scores, rtol=1e-12, atol=1e-12)
        sel = res["topk"][t]
        assert sel[: len(chosen)].tolist() == chosen
        assert np.all(sel[len(chosen):] == -1)
        np.testing.assert_allclose(res["o"][t], np.array(o), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["lse"][t], np.array(lse), rtol=1e-12, atol=1e-12)


def prefill_tiny_spec(**kw):
    base = dict(name="pf_tiny", kind="prefill", ctx_lens=[203], T_prefill=9, H=5, D_nope=24, D_rope=8,
                H_I=3, D_I=16, k=5, W=6, m=4, page_size=8, shuffle_pages=True)
    base.update(kw)
    return ci.Spec(**base)


@pytest.mark.parametrize("spec_fn", [
    prefill_tiny_spec,
    # a chunk at the start of a sequence: early queries' windows reach below
    # position 0, and fewer than k entries are visible
    lambda: prefill_tiny_spec(ctx_lens=[14], T_prefill=11, k=7),
    # a window wider than the chunk's lead-in, pages of 16
    lambda: prefill_tiny_spec(ctx_lens=[150], T_prefill=4, W=9, page_size=16),
])
def test_oracle_matches_brute_force_prefill(spec_fn):
    """The prefill path (window rows from the linear token buffer, every
    query at its own position, all queries on one sequence's paged cache)
    against the brute force, which walks the buffer rows in storage order
    instead of mapping window positions to rows."""
    wl = ci.generate(spec_fn(), seed=23)
    assert wl.spec.kind == "prefill" and wl.T > 1
    res = oracle.run_decode_path(wl)
    for t in range(wl.T):
        scores, chosen, o, lse = brute_path(wl, t)
        np.testing.assert_allclose(res["scores"][t], scores, rtol=1e-12, atol=1e-12)
        sel = res["topk"][t]
        assert sel[: len(chosen)].tolist() == chosen
        assert np.all(sel[len(chosen):] == -1)
        np.testing.assert_allclose(res["o"][t], np.array(o), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["lse"][t], np.array(lse), rtol=1e-12, atol=1e-12)


def test_unquantised_scores_against_loops_without_entry_offsets():
    """index_scores_unquantised on two sequences of different lengths against
    Python loops that find each entry's unquantised key by the E4M3 bytes
    stored at the entry's paged row (not through the per-sequence offsets of
    the kept draws)."""
    spec = ci.Spec(name="uq", kind="decode", ctx_lens=[96, 181], H=4, D_nope=16, D_rope=16, H_I=3, D_I=16,
                   k=4, W=8, page_size=16, shuffle_pages=True, keep_float=True)
    wl = ci.generate(spec, seed=29)
    s = wl.spec
    enc = ci.e4m3_bytes(wl.k_idx_f32, wl.k_idx_scale)
    lookup = {enc[i].tobytes(): i for i in range(enc.shape[0])}
    assert len(lookup) == enc.shape[0]          # every key row has distinct bytes
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        nv = min(int(wl.q_pos[t]) // s.m, int(wl.n_comp[b]))
        got = oracle.index_scores_unquantised(wl, t)
        assert len(got) == nv
        for c in range(nv):
            page = int(wl.page_table[b][c // s.page_size])
            key = wl.k_idx_f32[lookup[wl.k_idx[page, c % s.page_size].tobytes()]]
            tot = 0.0
            for h in range(s.H_I):
                d = 0.0
                for i in range(s.D_I):
                    d += float(wl.q_idx_f32[t][h][i]) * float(key[i])
                if d > 0.0:
                    tot += float(wl.w[t][h]) * d
            assert math.isclose(got[c], tot, rel_tol=1e-12, abs_tol=1e-12), (t, c, got[c], tot)


# ------------------------------------------------------------------ golden closed forms
def _num(v):
    table = {"ln2": math.log(2), "ln4": math.log(4), "ln3": math.log(3),
             "ln2/2": math.log(2) / 2, "2ln2/3": 2 * math.log(2) / 3}
    return table[v] if isinstance(v, str) else float(v)


def test_golden_indexer_closed_form():
    g = json.load(open(GOLDEN))["indexer"]
    # build a one-sequence workload holding exactly these keys/queries
    spec = ci.Spec(name="g", kind="decode", ctx_lens=[20], H=16, D_nope=16, D_rope=16,
                   H_I=2, D_I=2, k=2, W=4, m=4, page_size=4, unit_scale=True)
    wl = ci.generate(spec, seed=1)
    wl.k_idx[:] = 0
    for c, key in enumerate(g["k_idx"]):
        wl.k_idx[c // 4, c % 4] = ci.e4m3_bytes(np.array(key), 1.0)
    wl.q_idx[0] = ci.e4m3_bytes(np.array(g["q_idx"]), 1.0)
    wl.w[0] = np.array(g["w"], dtype=np.float32)
    wl.q_pos[0] = 16          # n_vis = 4
    sc = oracle.index_scores(wl, 0)
    assert sc.tolist() == g["scores"]
    assert oracle.topk_select(sc, 2).tolist() == g["top2"]
    assert oracle.topk_select(sc, 3).tolist() == g["top3"]


def test_golden_attention_closed_form():
    g = json.load(open(GOLDEN))["attention"]
    q = np.array([g["q"]])
    X = np.array([[_num(v) for v in row] for row in g["x"]])
    o, lse = oracle.attend(q, X, np.array([g["sink"]]), 1.0)
    np.testing.assert_allclose(o, [[_num(v) for v in g["o"][0]]], rtol=1e-15)
    np.testing.assert_allclose(lse, [_num(g["lse"])], rtol=1e-15)
    o, lse = oracle.attend(q, X, np.array([-np.inf]), 1.0)
    np.testing.assert_allclose(o, [[_num(v) for v in g["o_sink_neg_inf"][0]]], rtol=1e-15)
    np.testing.assert_allclose(lse, [_num(g["lse_sink_neg_inf"])], rtol=1e-15)


# ------------------------------------------------------------------ indexer invariants
def test_index_scores_nonnegative_and_w_linear():
    wl = ci.generate(tiny_spec(), seed=3)
    for t in range(wl.T):
        sc = oracle.index_scores(wl, t)
        assert np.all(sc >= 0)
    wl2 = dataclasses.replace(wl, w=wl.w * 2)
    for t in range(wl.T):
        np.testing.assert_array_equal(oracle.index_scores(wl2, t), 2 * oracle.index_scores(wl, t))


def test_index_scores_head_permutation_invariant():
    wl = ci.generate(tiny_spec(), seed=4)
    perm = np.array([2, 0, 1])
    wl2 = dataclasses.replace(wl, w=wl.w[:, perm], q_idx=wl.q_idx[:, perm])
    for t in range(wl.T):
        np.testing.assert_allclose(oracle.index_scores(wl2, t), oracle.index_scores(wl, t), rtol=1e-13)


def test_index_score_negated_key_is_zero_and_aligned_key_is_norm():
    """q_idx = -k (E4M3 sign-bit flip, exact) gives score 0 for that entry;
    q_idx = +k gives sum_h w_h * s_q * s_k * |k|^2 (norm via torch's decoder)."""
    wl = ci.generate(tiny_spec(), seed=5)
    s = wl.spec
    b, t, c = 1, 1, 3
    row = int(oc.entry_rows(wl.page_table[b], s.page_size, np.array([c]))[0])
    kbytes = wl.k_idx.reshape(-1, s.D_I)[row]
    wl.q_idx[t][:] = kbytes ^ np.uint8(0x80)
    assert oracle.index_scores(wl, t)[c] == 0.0
    wl.q_idx[t][:] = kbytes
    kv = torch_e4m3(kbytes)
    expect = float(wl.w[t].astype(np.float64).sum()) * wl.q_idx_scale * wl.k_idx_scale * float(kv @ kv)
    np.testing.assert_allclose(oracle.index_scores(wl, t)[c], expect, rtol=1e-12)


def test_single_head_unit_weight_is_relu_dot():
    wl = ci.generate(tiny_spec(H_I=1), seed=6)
    s = wl.spec
    wl.w[:] = 1.0
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        nv = oc.n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
        rows = oc.entry_rows(wl.page_table[b], s.page_size, np.arange(nv))
        K = torch_e4m3(wl.k_idx.reshape(-1, s.D_I)[rows]) * wl.k_idx_scale
        q = torch_e4m3(wl.q_idx[t][0]) * wl.q_idx_scale
        np.testing.assert_allclose(oracle.index_scores(wl, t), np.maximum(K @ q, 0), rtol=1e-13)


# ------------------------------------------------------------------ top-k
def test_topk_matches_python_sort_with_ties():
    rng = np.random.default_rng(11)
    for n, k in [(50, 10), (10, 10), (7, 12), (300, 64), (1, 1), (0, 3)]:
        scores = rng.integers(0, 6, size=n).astype(np.float64)   # many exact ties
        want = sorted(sorted(range(n), key=lambda c: (-scores[c], c))[:k])
        got = oracle.topk_select(scores, k)
        assert got[: len(want)].tolist() == want
        assert np.all(got[len(want):] == -1)


def test_topk_tie_goes_to_lower_index():
    assert oracle.topk_select(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 2).tolist() == [1, 2]
    assert oracle.topk_select(np.array([0.0, 0.0, 0.0]), 2).tolist() == [0, 1]


def test_causality_poisoned_future_blocks_never_selected():
    """Make every not-visible entry (its own block and later) a perfect match
    for the query; the selection must still come from visible entries only."""
    spec = tiny_spec(ctx_lens=[64, 90], q_pos=[41, 70])
    wl = ci.generate(spec, seed=8)
    s = wl.spec
    res0 = oracle.run_decode_path(wl)

    def own_block(pos):   # the block whose token range [c*m, (c+1)*m) holds pos
        return next(c for c in range(10 ** 6) if c * s.m <= pos < (c + 1) * s.m)
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        fut = np.arange(own_block(int(wl.q_pos[t])), int(wl.n_comp[b]))
        rows = oc.entry_rows(wl.page_table[b], s.page_size, fut)
        wl.k_idx.reshape(-1, s.D_I)[rows] = wl.q_idx[t][0]
    res = oracle.run_decode_path(wl)
    for t in range(wl.T):
        sel = res["topk"][t]
        assert np.all(sel[sel >= 0] < own_block(int(wl.q_pos[t])))
        np.testing.assert_array_equal(sel, res0["topk"][t])


def test_topk_all_when_k_exceeds_visible():
    wl = ci.generate(tiny_spec(k=40), seed=9)
    res = oracle.run_decode_path(wl)
    for t in range(wl.T):
        nv = len(res["scores"][t])
        assert res["topk"][t][:nv].tolist() == list(range(nv))
        assert np.all(res["topk"][t][nv:] == -1)


# ------------------------------------------------------------------ attention
def test_sink_neg_inf_is_plain_softmax():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((6, 40))
    X = rng.standard_normal((23, 40))
    o, lse = oracle.attend(q, X, np.full(6, -np.inf), 0.3)
    P = scipy.special.softmax(0.3 * q @ X.T, axis=1)
    np.testing.assert_allclose(o, P @ X, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(0.3 * q @ X.T, axis=1), rtol=1e-13)
    # weights sum to one: equal value rows give back that row
    Xc = np.tile(X[:1], (23, 1))
    o2, _ = oracle.attend(q, Xc, np.full(6, -np.inf), 0.3)
    np.testing.assert_allclose(o2, np.tile(X[:1], (6, 1)), rtol=1e-13)


def test_single_key_plus_sink_closed_form():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 10))
    x = rng.standard_normal((1, 10))
    sink = rng.standard_normal(4)
    o, lse = oracle.attend(q, x, sink, 0.7)
    S = 0.7 * (q @ x[0])
    np.testing.assert_allclose(o, x * (1.0 / (1.0 + np.exp(sink - S)))[:, None], rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.exp(S) + np.exp(sink)), rtol=1e-13)


def test_identical_keys_closed_form():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, 8))
    x = rng.standard_normal((1, 8))
    n = 9
    sink = np.array([0.2, -1.0, 3.0])
    o, _ = oracle.attend(q, np.tile(x, (n, 1)), sink, 1.0)
    S = q @ x[0]
    frac = n * np.exp(S) / (n * np.exp(S) + np.exp(sink))
    np.testing.assert_allclose(o, x * frac[:, None], rtol=1e-12)


def test_split_merge_identity():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((5, 16))
    X = rng.standard_normal((30, 16))
    sink = rng.standard_normal(5)
    o, lse = oracle.attend(q, X, sink, 0.5)
    oa, la = oracle.attend(q, X[:11], sink, 0.5)
    ob, lb = oracle.attend(q, X[11:], np.full(5, -np.inf), 0.5)
    om, lm = oracle.merge_by_lse(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, lse, rtol=1e-13)


def test_empty_key_set_neg_inf_sink():
    o, lse = oracle.attend(np.ones((2, 4)), np.zeros((0, 4)), np.array([-np.inf, -np.inf]), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = oracle.attend(np.ones((1, 4)), np.zeros((0, 4)), np.array([0.5]), 1.0)
    assert np.all(o == 0) and lse[0] == 0.5


def test_topk_all_equals_dense_hca_attention():
    """spec check: selecting every visible entry equals attending all
    visible entries (the HCA mode)."""
    wl = ci.generate(tiny_spec(k=40), seed=16)
    res = oracle.run_decode_path(wl)
    o_dense, l_dense = oracle.run_attention(wl, None)
    np.testing.assert_allclose(res["o"], o_dense, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["lse"], l_dense, rtol=1e-13)


def test_ring_permutation_invariance():
    wl = ci.generate(tiny_spec(), seed=17)
    wlp = ci.with_ring_permuted(wl, seed=99)
    assert not np.array_equal(wlp.swa_pos, wl.swa_pos)
    a = oracle.run_decode_path(wl)
    b = oracle.run_decode_path(wlp)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-12, atol=1e-14)


def test_window_and_newest_block_both_attended():
    """A token inside the newest visible compressed block is also in the
    window: both rows appear in the key set (as distinct keys)."""
    wl = ci.generate(tiny_spec(k=40), seed=18)
    s = wl.spec
    t = 0
    pos = int(wl.q_pos[t])
    nv = oc.n_visible(pos, s.m, int(wl.n_comp[0]))
    X, labels = oracle.key_rows(wl, t, oracle.topk_select(oracle.index_scores(wl, t), s.k))
    comp = [c for kind, c in labels if kind == "c"]
    win = [p for kind, p in labels if kind == "w"]
    assert comp == list(range(nv))
    assert any((nv - 1) * s.m <= p < nv * s.m for p in win)
    assert sorted(win) == list(range(pos - s.W + 1, pos + 1))


def test_prefill_window_from_linear_buffer():
    spec = ci.Spec(name="pf", kind="prefill", ctx_lens=[200], T_prefill=9, H=4, D_nope=16,
                   D_rope=16, H_I=2, D_I=8, k=5, W=6, m=4, page_size=8)
    wl = ci.generate(spec, seed=19)
    assert wl.swa_first_pos == 191 - 5 and wl.swa_len == 9 + 5
    for t in range(wl.T):
        _, labels = oracle.key_rows(wl, t, np.full(5, -1))
        pos = int(wl.q_pos[t])
        assert [p for _, p in labels] == list(range(pos - 5, pos + 1))
