"""csa_decode_attn_noalloc (partial results in the library's static scratch
array, no allocation) against csa_decode_attn (caller workspace) through the
C ABI: same kernels, same split plan while the preferred split fits the
scratch, so the outputs must be bit-identical; both are also gated against
the FP64 oracle.  Two calls in a row, the second with a smaller input, then
a problem whose minimum split does not fit the scratch."""
import sys

import numpy as np
import pytest

import csa_inputs as ci
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_compressed_attention_amd as csa  # noqa: E402
from csa_inputs.device import to_device, make_path  # noqa: E402

CSA_ERR_TOO_LARGE = -5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_both(wl, hca):
    s = wl.spec
    d = to_device(wl, "cuda")
    path = make_path(d)
    path.run()                          # indexer + top-k + attention with a workspace
    cache = csa.LatentCache(d.lat_nope, d.lat_rope, d.lat_scale, d.page_table, d.n_comp, s.m)
    swa = csa.SwaRing(d.swa_nope, d.swa_rope, d.swa_scale, d.swa_pos)
    topk = None if hca else path.topk
    k = 0 if hca else s.k
    max_keys = (d.page_table.shape[1] * d.lat_nope.shape[1] if hca else s.k) + s.W
    ws_bytes = csa.csa_attn_workspace_size(wl.T, s.H, s.D_nope, s.D_rope, max_keys)
    assert 0 < ws_bytes <= 16 << 20      # split, and the preferred split fits the scratch
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    out_a = torch.full((wl.T, s.H, s.D), 3.0, dtype=torch.bfloat16, device="cuda")
    lse_a = torch.full((wl.T, s.H), 3.0, dtype=torch.float32, device="cuda")
    out_b = torch.full_like(out_a, -5.0)
    lse_b = torch.full_like(lse_a, -5.0)
    csa.csa_decode_attn(d.q, cache, topk, k, swa, d.q_pos, d.sink, s.sigma, out_a, lse_a, workspace=ws)
    csa.csa_decode_attn_noalloc(d.q, cache, topk, k, swa, d.q_pos, d.sink, s.sigma, out_b, lse_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_a, lse_b)
    o = P.bf16_to_f64(out_b)
    lv = lse_b.cpu().numpy().astype(np.float64)
    sel = None if hca else path.topk.cpu().numpy()
    worst = (0.0, 1.0)
    for t in range(wl.T):
        o_ref, l_ref = P.reference_attention_on(wl, t, None if hca else sel[t])
        err, cos = P.check_attention(o[t], lv[t], o_ref, l_ref)
        worst = (max(worst[0], err), min(worst[1], cos))
    say(f"  {s.name}: {wl.T} queries, {ws_bytes} B of partials; no-alloc == workspace call; "
        f"max|err| {worst[0]:.3e} min cos {worst[1]:.6f}")


def test_noalloc_equals_workspace_call_two_calls_second_smaller():
    say("case no-alloc: c1 (1 query, 2048 entries), then a smaller HCA batch")
    _run_both(ci.make_config("c1"), hca=False)
    spec = ci.small_spec(name="hca_small", ctx_lens=[20000, 9000], m=128, with_indexer=False)
    _run_both(ci.generate(spec, seed=341), hca=True)


def test_noalloc_hca_long_context_then_tiny():
    say("case no-alloc: 4 x 4096-entry HCA rows (many splits), then c0")
    spec = ci.Spec(name="hca_4x4096", kind="decode", ctx_lens=[524288] * 4, m=128, with_indexer=False)
    _run_both(ci.generate(spec, seed=342), hca=True)
    _run_both(ci.make_config("c0"), hca=False)


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 64 HCA queries whose page-table rows span 2048 entries: with the
    # 128-slot window every key range needs at least two splits, and the
    # minimum partial results (2 x 64 x 128 rows of 1040 bytes, 17 MB) exceed the
    # 16 MiB scratch, so the call is refused on the host before any launch.
    # (Every page-table entry is the one zero page and nothing is stored, so
    # even a launch would read in bounds.)
    say("case no-alloc: too large for the scratch")
    T, H, dn, dr, W, ps = 64, 128, 448, 64, 128, 64
    dev = "cuda"
    cache = csa.LatentCache(torch.zeros((1, ps, dn), dtype=torch.uint8, device=dev),
                            torch.zeros((1, ps, dr), dtype=torch.bfloat16, device=dev), 1.0,
                            torch.zeros((T, 2048 // ps), dtype=torch.int32, device=dev),
                            torch.zeros((T,), dtype=torch.int32, device=dev), 128)
    swa = csa.SwaRing(torch.zeros((T, W, dn), dtype=torch.uint8, device=dev),
                      torch.zeros((T, W, dr), dtype=torch.bfloat16, device=dev), 1.0,
                      torch.full((T, W), -1, dtype=torch.int32, device=dev))
    q = torch.zeros((T, H, dn + dr), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    q_pos = torch.zeros((T,), dtype=torch.int32, device=dev)
    sink = torch.zeros((H,), dtype=torch.float32, device=dev)
    need = csa.csa_attn_workspace_size(T, H, dn, dr, 2048 + W)
    assert need > 16 << 20
    with pytest.raises(csa.CsaError) as ei:
        csa.csa_decode_attn_noalloc(q, cache, None, 0, swa, q_pos, sink, 0.0441941738, out)
    assert ei.value.code == CSA_ERR_TOO_LARGE
