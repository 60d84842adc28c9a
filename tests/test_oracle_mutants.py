"""Each pin must catch a plausible mistake in the oracle.  Mistakes are
planted in the oracle (on the CPU, by monkeypatching) and the matching pin
test is expected to fail."""
import dataclasses

import numpy as np
import pytest

from oracle import csa as oc
import oracle
import tests.test_oracle_path as pins


def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


def test_dropped_sink_is_caught(monkeypatch):
    real = oc.attend

    def no_sink(q, X, sink, sigma):
        return real(q, X, np.full_like(np.asarray(sink, dtype=float), -np.inf), sigma)
    monkeypatch.setattr(oc, "attend", no_sink)
    monkeypatch.setattr(oracle, "attend", no_sink)
    _expect_fail(pins.test_golden_attention_closed_form)
    _expect_fail(pins.test_single_key_plus_sink_closed_form)


def test_sink_scaled_by_sigma_is_caught(monkeypatch):
    real = oc.attend

    def scaled(q, X, sink, sigma):
        return real(q, X, np.asarray(sink) * sigma, sigma)
    monkeypatch.setattr(oracle, "attend", scaled)
    _expect_fail(pins.test_single_key_plus_sink_closed_form)


def test_relu_sign_flip_is_caught(monkeypatch):
    def bad(wl, t, keys=None):
        s = wl.spec
        b = int(wl.q_seq[t])
        nv = oc.n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
        keys = oc.sequence_index_keys(wl, b) if keys is None else keys
        q = oc.e4m3_decode(wl.q_idx[t]) * float(wl.q_idx_scale)
        return wl.w[t].astype(np.float64) @ np.maximum(-(q @ keys[:nv].T), 0.0)
    monkeypatch.setattr(oracle, "index_scores", bad)
    _expect_fail(pins.test_index_score_negated_key_is_zero_and_aligned_key_is_norm)
    _expect_fail(pins.test_golden_indexer_closed_form)


def test_own_block_visible_is_caught(monkeypatch):
    monkeypatch.setattr(oc, "n_visible", lambda pos, m, n: int(min(pos // m + 1, n)))
    _expect_fail(lambda: pins.test_n_visible(255, 4, 64, 63))
    _expect_fail(pins.test_causality_poisoned_future_blocks_never_selected)


def test_tie_to_higher_index_is_caught(monkeypatch):
    def bad(scores, k):
        n = len(scores)
        order = np.lexsort((-np.arange(n), -np.asarray(scores, dtype=np.float64)))
        out = np.full(k, -1, dtype=np.int32)
        ch = np.sort(order[: min(k, n)])
        out[: len(ch)] = ch
        return out
    monkeypatch.setattr(oracle, "topk_select", bad)
    _expect_fail(pins.test_topk_tie_goes_to_lower_index)
    _expect_fail(pins.test_topk_matches_python_sort_with_ties)


def test_value_without_rope_dims_is_caught(monkeypatch):
    real = oc.attend

    def nope_only_values(q, X, sink, sigma):
        o, lse = real(q, X, sink, sigma)
        o = o.copy()
        o[:, -1:] = 0.0
        return o, lse
    monkeypatch.setattr(oracle, "attend", nope_only_values)
    _expect_fail(pins.test_golden_attention_closed_form)


def test_window_excluding_own_token_is_caught(monkeypatch):
    monkeypatch.setattr(oc, "swa_window", lambda pos, W: (max(0, pos - W), pos - 1))
    _expect_fail(pins.test_window_and_newest_block_both_attended)


def test_prefill_buffer_row_off_by_one_is_caught(monkeypatch):
    # the window row of position p read from buffer row p - first + 1
    real = oc.key_rows

    def shifted(wl, t, sel):
        if wl.spec.kind != "prefill":
            return real(wl, t, sel)
        w2 = dataclasses.replace(wl, swa_nope=np.roll(wl.swa_nope, -1, axis=0),
                                 swa_rope=np.roll(wl.swa_rope, -1, axis=0))
        return real(w2, t, sel)
    monkeypatch.setattr(oc, "key_rows", shifted)
    _expect_fail(lambda: pins.test_oracle_matches_brute_force_prefill(pins.prefill_tiny_spec))


def test_entry_offset_of_later_sequences_is_caught(monkeypatch):
    # the kept draws of sequence b > 0 read from the wrong offset
    real = oc.index_scores_unquantised

    def bad(wl, t):
        w2 = dataclasses.replace(wl, entry_offset=wl.entry_offset + (np.arange(wl.B) > 0))
        return real(w2, t)
    monkeypatch.setattr(oracle, "index_scores_unquantised", bad)
    _expect_fail(pins.test_unquantised_scores_against_loops_without_entry_offsets)
