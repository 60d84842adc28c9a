"""Graph replay of a whole step ("ROADMAP -- Stage E ...", E9: the decode
step, free of synchronisation and allocation, is captured once and
replayed).

Each replay must give exactly the bytes the same step gives when its calls
are issued one by one (the kernels are deterministic), and a replay must see
the current contents of the captured buffers.  The replays are interleaved
with eager work and synchronisations.
"""
import dataclasses
import sys

import numpy as np
import pytest

import csa_inputs as ci
import oracle
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_compressed_attention_amd as csa  # noqa: E402
from csa_inputs.device import to_device, make_path  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def snapshot(path):
    torch.cuda.synchronize()
    res = [path.out.clone(), path.lse.clone()]
    if getattr(path, "topk", None) is not None:
        res.append(path.topk.clone())
    return res


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("case", ["c0", "small_decode", "hca_small", "prefill_small", "mxfp4_inv_rope"])
def test_graph_replay_matches_eager(case):
    say(f"case graph replay {case}")
    opts = {}
    if case == "c0":
        wl = ci.make_config("c0")
    elif case == "mxfp4_inv_rope":
        # the variant entry points are captured as well
        wl = ci.generate(ci.small_spec(shuffle_pages=True, mxfp4=True), seed=136)
        opts = dict(mxfp4=True, inv_rope_theta=10000.0)
    elif case == "small_decode":
        wl = ci.generate(ci.small_spec(shuffle_pages=True), seed=131)
    elif case == "hca_small":
        wl = ci.generate(ci.small_spec(name="hca_small", ctx_lens=[20000, 9000], m=128, with_indexer=False), seed=132)
    else:
        wl = ci.generate(ci.Spec(name="prefill_small", kind="prefill", ctx_lens=[6000], T_prefill=70), seed=133)
    d = to_device(wl, "cuda")
    path = make_path(d, **opts)
    path.run()
    eager = snapshot(path)
    g = csa.StepGraph(path)
    scratch = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        path.out.zero_()
        path.lse.zero_()
        scratch = scratch @ scratch.t() / 512.0        # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = snapshot(path)
        assert same(got, eager), f"replay {rep} differs from the eager step"
    g.close()


def test_graph_replay_reads_current_inputs():
    # new query rows and positions written into the captured buffers are
    # picked up by the next replay; the result is checked against the oracle
    say("case graph replay with refreshed inputs")
    wl = ci.generate(ci.small_spec(ctx_lens=[3000, 2052], shuffle_pages=True), seed=134)
    d = to_device(wl, "cuda")
    path = make_path(d)
    path.run()
    g = csa.StepGraph(path)
    wl2 = ci.generate(ci.small_spec(ctx_lens=[3000, 2052], shuffle_pages=True), seed=135)
    # same shapes and cache, new queries: copy q, q_idx and w of the second draw
    d2 = to_device(wl2, "cuda")
    d.q.copy_(d2.q)
    d.q_idx.copy_(d2.q_idx)
    d.w.copy_(d2.w)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    o = path.out.float().cpu().numpy().astype(np.float64)
    lse = path.lse.cpu().numpy().astype(np.float64)
    topk = path.topk.cpu().numpy()
    # the captured calls keep the first draw's per-tensor scales; the oracle
    # reads the second draw's bytes under those scales, as the GPU does
    wl_mix = dataclasses.replace(wl, q=wl2.q, q_idx=wl2.q_idx, w=wl2.w)
    for t in range(wl.T):
        o_ref, l_ref = P.reference_attention_on(wl_mix, t, topk[t])
        err, cos = P.check_attention(o[t], lse[t], o_ref, l_ref)
        P.check_topk_vs_oracle(topk[t], oracle.index_scores(wl_mix, t), wl.spec.k)
        say(f"  query {t}: max|err| {err:.3e} min cos {cos:.6f}")
    # and the eager calls on the refreshed buffers give the same bytes
    got = snapshot(path)
    path.run()
    assert same(snapshot(path), got)
    g.close()
