"""A decode step driven through the C ABI alone: tests/c_abi/decode_step
(built with the library) links libcsa.so, allocates with hipMalloc, and calls
csa_index_scores -> csa_topk -> csa_decode_attn with no Python or torch in
the process.  Its outputs must be the bytes the Python binding's path gives
on the same inputs (the kernels are deterministic), and must pass the oracle
gates.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import csa_inputs as ci
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from csa_inputs.device import to_device, make_path  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "decode_step")


def write_input(wl, path):
    s = wl.spec
    hdr = np.array([wl.B, s.H, s.D_nope, s.D_rope, s.H_I, s.D_I, s.k, s.W, s.m, s.page_size, wl.num_pages,
                    wl.max_pages, 0, 0, 0, 0], dtype=np.int32)
    fh = np.array([wl.q_idx_scale, wl.k_idx_scale, wl.lat_scale, wl.swa_scale, s.sigma, 0, 0, 0], dtype=np.float32)
    arrays = [wl.q_idx, wl.w.astype(np.float32), wl.k_idx, wl.lat_nope, wl.lat_rope, wl.page_table, wl.n_comp,
              wl.q_pos, wl.q, wl.sink.astype(np.float32), wl.swa_nope, wl.swa_rope, wl.swa_pos]
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(fh.tobytes())
        for a in arrays:
            f.write(np.ascontiguousarray(a).tobytes())


def test_decode_step_through_c_abi_only(tmp_path):
    print("case C-ABI driver (small decode, shuffled pages)", flush=True)
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    wl = ci.generate(ci.small_spec(ctx_lens=[3000, 1508, 2400, 620], shuffle_pages=True), seed=160)
    s = wl.spec
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    write_input(wl, inp)
    res = subprocess.run([DRIVER, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    raw = outp.read_bytes()
    B, H, D, k = wl.B, s.H, s.D, s.k
    n_topk, n_out = B * k * 4, B * H * D * 2
    topk = np.frombuffer(raw[:n_topk], dtype=np.int32).reshape(B, k)
    out_bits = np.frombuffer(raw[n_topk:n_topk + n_out], dtype=np.uint16).reshape(B, H, D)
    lse = np.frombuffer(raw[n_topk + n_out:], dtype=np.float32).reshape(B, H)

    # the binding's path on the same inputs: identical bytes
    path = make_path(to_device(wl, "cuda"))
    path.run()
    torch.cuda.synchronize()
    assert np.array_equal(topk, path.topk.cpu().numpy())
    assert np.array_equal(out_bits, path.out.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(lse, path.lse.cpu().numpy())

    # and the oracle gates
    o = torch.from_numpy(out_bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy().astype(np.float64)
    import oracle
    for t in range(B):
        P.check_topk_vs_oracle(topk[t], oracle.index_scores(wl, t), k)
        o_ref, l_ref = P.reference_attention_on(wl, t, topk[t])
        err, cos = P.check_attention(o[t], lse[t].astype(np.float64), o_ref, l_ref)
        print(f"  query {t}: max|err| {err:.3e} min cos {cos:.6f}", flush=True)
    sys.stdout.flush()
