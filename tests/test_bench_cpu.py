"""The benchmark's host-side contract, checked without a GPU: one GPU only,
and the algorithmic byte / FLOP accounting its roofline uses."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import csa_inputs as ci

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr


def test_accounting_of_the_tiny_configuration():
    # c0: one query at position 255 sees 63 of 64 entries; top-k 16; window 32
    wl = ci.make_config("c0")
    s = wl.spec
    acc = bench.accounting(wl)
    nv = 63
    assert acc["index_scores"]["flops"] == pytest.approx(2.0 * s.H_I * s.D_I * nv)
    assert acc["index_scores"]["bytes"] == nv * s.D_I + s.H_I * (s.D_I + 4) + nv * 4 + 4
    keys = min(nv, s.k) + s.W
    assert acc["decode_attn"]["flops"] == pytest.approx(4.0 * s.H * keys * s.D)
    # with MXFP4 index keys a row is D_I / 2 code bytes and D_I / 32 scale bytes
    acc4 = bench.accounting(wl, mxfp4=True)
    row4 = s.D_I // 2 + s.D_I // 32
    assert acc4["index_scores"]["bytes"] == nv * row4 + s.H_I * (row4 + 4) + nv * 4 + 4
    assert acc4["decode_attn"] == acc["decode_attn"]


def test_roofline_picks_the_bound_by_intensity():
    hbm = bench.roofline_entry("x", dict(bytes=8e9, flops=1e12), 1.0)       # 125 FLOP/B
    assert hbm["bound"] == "hbm" and hbm["unit"] == "GB/s"
    assert hbm["achieved"] == pytest.approx(8000.0) and hbm["frac"] == pytest.approx(1.0)
    mfma = bench.roofline_entry("x", dict(bytes=1e6, flops=5e12), 1.0)      # 5e6 FLOP/B
    assert mfma["bound"] == "mfma" and mfma["unit"] == "TFLOP/s"
    assert mfma["frac"] == pytest.approx(1.0)
