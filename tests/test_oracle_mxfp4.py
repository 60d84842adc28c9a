"""Pins of the oracle's MXFP4 decoders and of its MXFP4 indexer scores (the
FP4 variant of the indexer QK: "DSV4 Audit", B2; "ROADMAP -- Stage E",
E7).  CPU only.

 * E2M1: the value table of the OCP Microscaling specification over all 16
   codes (its eight magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
   negatives).
 * E8M0: torch's float8_e8m0fnu over all 256 codes.
 * Packing: the nibble order of a hand-built byte, and one scale per block
   of 32 dims.
 * Scores: a pure-Python loop over the decoded values on a tiny workload, and
   the FP8 scores themselves when the MXFP4 copy holds the same values.
 * Unquantised reference scores (the recall reference of "ROADMAP", E7): the
   E4M3 scores exactly when the kept draws are replaced by their E4M3 values,
   and the kept draws round to the stored bytes.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import csa_inputs as ci
import oracle
from oracle.codecs import e2m1_decode, e8m0_decode, mxfp4_decode

OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes_match_the_ocp_table():
    vals = e2m1_decode(np.arange(16))
    assert list(vals[:8]) == OCP_E2M1
    assert list(vals[8:]) == [-v for v in OCP_E2M1]
    assert math.copysign(1.0, vals[8]) == -1.0


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0


def test_nibble_order_and_block_scales():
    # byte j holds element 2j in its low nibble: 0x21 -> (0.5, 1.0); 0xF9 ->
    # (-0.5, -6.0)
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21
    packed[0, 1] = 0xF9
    packed[0, 16] = 0x07      # element 32 = 6, in the second block
    sc = np.array([[127, 129]], dtype=np.uint8)   # 1 and 4
    v = mxfp4_decode(packed, sc)
    assert v.shape == (1, 64)
    assert list(v[0, :4]) == [0.5, 1.0, -0.5, -6.0]
    assert v[0, 32] == 24.0
    assert not np.any(v[0, 4:32]) and not np.any(v[0, 33:])


def test_input_encoder_round_trips_grid_values():
    # values on the E2M1 grid times a power of two with the block maximum at
    # 4 or 6 are stored exactly
    rng = np.random.default_rng(7)
    x = rng.choice(np.array(OCP_E2M1 + [-v for v in OCP_E2M1[1:]]), size=(6, 64))
    x[:, 0] = 6.0
    x[:, 32] = -4.0
    x *= np.ldexp(1.0, rng.integers(-5, 6, size=(6, 1)))
    pk, sc = ci.mxfp4_pack(x)
    assert np.array_equal(mxfp4_decode(pk, sc), x)


def tiny_mxfp4_workload(seed):
    spec = ci.Spec(name="tiny_fp4", kind="decode", ctx_lens=[256, 200], H=8, D_nope=48, D_rope=16, H_I=4, D_I=32,
                   k=16, W=32, page_size=16, shuffle_pages=True, mxfp4=True)
    return ci.generate(spec, seed)


def test_mxfp4_scores_against_python_loops():
    wl = tiny_mxfp4_workload(3)
    s = wl.spec
    for t in range(wl.T):
        b = int(wl.q_seq[t])
        nv = oracle.n_visible(int(wl.q_pos[t]), s.m, int(wl.n_comp[b]))
        ours = oracle.index_scores_mxfp4(wl, t)
        assert len(ours) == nv
        q = [[float(v) for v in mxfp4_decode(wl.q_idx4[t][h], wl.q_idx4_sc[t][h])] for h in range(s.H_I)]
        for c in range(nv):
            page = int(wl.page_table[b][c // s.page_size])
            k = [float(v) for v in mxfp4_decode(wl.k_idx4[page, c % s.page_size],
                                               wl.k_idx4_sc[page, c % s.page_size])]
            tot = 0.0
            for h in range(s.H_I):
                d = sum(q[h][i] * k[i] for i in range(s.D_I))
                if d > 0.0:
                    tot += float(wl.w[t][h]) * d
            assert ours[c] == pytest.approx(tot, rel=1e-12, abs=1e-12)


def test_mxfp4_scores_equal_fp8_scores_when_values_agree():
    # store values that both formats hold exactly (E2M1 grid, unit FP8
    # scale): the two score functions must agree
    wl = tiny_mxfp4_workload(4)
    rng = np.random.default_rng(9)
    grid = np.array(OCP_E2M1 + [-v for v in OCP_E2M1[1:]])
    qv = rng.choice(grid, size=wl.q_idx4.shape[:-1] + (wl.spec.D_I,))
    kv = rng.choice(grid, size=wl.k_idx4.shape[:-1] + (wl.spec.D_I,))
    qv[..., 0] = 6.0
    kv[..., 0] = 6.0
    q4, q4s = ci.mxfp4_pack(qv)
    k4, k4s = ci.mxfp4_pack(kv)
    wl2 = dataclasses.replace(wl, q_idx=ci.e4m3_bytes(qv, 1.0), q_idx_scale=1.0, k_idx=ci.e4m3_bytes(kv, 1.0),
                              k_idx_scale=1.0, q_idx4=q4, q_idx4_sc=q4s, k_idx4=k4, k_idx4_sc=k4s)
    for t in range(wl2.T):
        assert np.array_equal(oracle.index_scores_mxfp4(wl2, t), oracle.index_scores(wl2, t))


def test_mxfp4_scores_track_fp8_scores_on_random_data():
    # a plausibility bound, not a pin: the FP4 copy of the same draws gives
    # scores strongly correlated with the FP8 ones
    wl = ci.generate(ci.small_spec(mxfp4=True, ctx_lens=[2048]), seed=11)
    a = oracle.index_scores(wl, 0)
    b = oracle.index_scores_mxfp4(wl, 0)
    assert np.corrcoef(a, b)[0, 1] > 0.95


def test_unquantised_scores_equal_fp8_scores_when_the_draws_are_on_the_grid():
    # replace the kept float draws by their E4M3-decoded values: the
    # unquantised scores must then be the E4M3 scores exactly
    spec = ci.Spec(name="tiny_float", kind="decode", ctx_lens=[256, 200], H=8, D_nope=48, D_rope=16, H_I=4, D_I=32,
                   k=16, W=32, page_size=16, shuffle_pages=True, keep_float=True)
    wl = ci.generate(spec, 12)
    from oracle.codecs import e4m3_decode
    q = e4m3_decode(wl.q_idx) * wl.q_idx_scale
    keys = np.zeros_like(wl.k_idx_f32, dtype=np.float64)
    s = wl.spec
    for b in range(wl.B):
        for c in range(int(wl.n_comp[b])):
            page = int(wl.page_table[b][c // s.page_size])
            keys[int(wl.entry_offset[b]) + c] = e4m3_decode(wl.k_idx[page, c % s.page_size]) * wl.k_idx_scale
    wl2 = dataclasses.replace(wl, q_idx_f32=q, k_idx_f32=keys)
    for t in range(wl.T):
        assert np.allclose(oracle.index_scores_unquantised(wl2, t), oracle.index_scores(wl, t), rtol=1e-13, atol=1e-13)


def test_unquantised_draws_are_the_quantised_ones_before_rounding():
    # the kept draws round to the stored E4M3 bytes (the same draw order)
    spec = ci.Spec(name="tiny_float2", kind="decode", ctx_lens=[256], H=8, D_nope=48, D_rope=16, H_I=4, D_I=32,
                   k=16, W=32, page_size=16, keep_float=True)
    wl = ci.generate(spec, 13)
    assert np.array_equal(ci.e4m3_bytes(wl.q_idx_f32, wl.q_idx_scale), wl.q_idx)


def test_planted_keys_change_only_the_planted_rows():
    # planting draws from a generator of its own: every other array keeps
    # its draws, and exactly plant_topk keys per sequence move, none of them
    # the newest stored entry
    base = dict(name="pl", kind="decode", ctx_lens=[400, 260], H=8, D_nope=48, D_rope=16, H_I=4, D_I=32, k=8,
                W=32, page_size=16, keep_float=True, shuffle_pages=True)
    a = ci.generate(ci.Spec(**base), seed=21)
    b = ci.generate(ci.Spec(**base, plant_topk=8, plant_gain=(0.8, 1.6)), seed=21)
    for name in ("q_idx", "w", "lat_nope", "lat_rope", "q", "sink", "swa_nope", "page_table"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    moved = np.flatnonzero(np.any(a.k_idx_f32 != b.k_idx_f32, axis=1))
    off = a.entry_offset
    for s_ in range(a.B):
        rows = moved[(moved >= off[s_]) & (moved < off[s_] + a.n_comp[s_])] - off[s_]
        assert len(rows) == 8 and rows.max() < a.n_comp[s_] - 1
    # the planted keys stand apart in the unquantised scores (the oracle)
    for t in range(b.T):
        exact = oracle.index_scores_unquantised(b, t)
        srt = np.sort(exact)[::-1]
        assert srt[7] > 1.05 * srt[8]
