"""The C ABI library loads, exports every entry point include/csa.h declares,
and rejects bad arguments on the host before any launch (CPU only: no call
here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import sparse_compressed_attention_amd as csa
from sparse_compressed_attention_amd import build as csa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa.library_path()):
        csa_build.build()
    return csa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_steps():
    names = declared_functions()
    for n in ["csa_index_scores", "csa_topk", "csa_decode_attn", "csa_prefill_attn"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_binding_names_match_header():
    for name in declared_functions():
        assert hasattr(csa, name), name


def test_status_strings(lib):
    assert csa.csa_status_string(0) == "ok"
    assert csa.csa_status_string(-1) == "invalid argument"
    assert csa.csa_status_string(-4) == "workspace missing or too small"
    assert csa.csa_version() >= 100


def test_workspace_sizes(lib):
    # rows that fit one chunk need no top-k workspace
    assert csa.csa_topk_workspace_size(64, 8192, 512) == 0
    # 131072-entry rows: 16 chunks of 8192, 512 candidates each
    assert csa.csa_topk_workspace_size(4, 131072, 512) == 4 * 16 * 512 * 8
    # 32 candidates per chunk: up to 512 chunks of 8192 fit the merge
    assert csa.csa_topk_workspace_size(2, 512 * 8192, 32) == 2 * 512 * 32 * 8
    # rows too long for two levels of 16384 candidates: "unsupported", told
    # apart from "no workspace needed" (0)
    assert lib.csa_topk_workspace_size(1, 1 << 22, 2048) == csa.CSA_WORKSPACE_UNSUPPORTED
    with pytest.raises(ValueError, match="unsupported"):
        csa.csa_topk_workspace_size(1, 1 << 22, 2048)
    assert lib.csa_topk_workspace_size(4, 8192, 4096) == csa.CSA_WORKSPACE_UNSUPPORTED   # k > 2048
    assert lib.csa_index_topk_workspace_size(64, 8192, 0) == csa.CSA_WORKSPACE_UNSUPPORTED
    # rows of one chunk: no candidates leave the chip (fewer than 16 queries)
    assert csa.csa_index_topk_workspace_size(8, 2048, 512) == 0
    # 64 queries of one sequence (eight blocks of 8) may cut 2048 entries into
    # 2 parts of 1024 with 512 candidates each; beyond 65536 entries or k > 1024
    # only the one-query plan applies
    assert csa.csa_index_topk_workspace_size(64, 2048, 512) == 64 * 2 * 512 * 8
    assert csa.csa_index_topk_workspace_size(64, 2048, 1025) == 0
    # 2048 queries over 16384 entries: the many-query plan needs none (256
    # query blocks, no split), the one-query plan 8 chunks of 2048
    assert csa.csa_index_topk_workspace_size(2048, 16384, 512) == 2048 * 8 * 512 * 8
    assert csa.csa_index_topk_workspace_size(40, 15000, 512) == 40 * 14 * 512 * 8
    # many queries: one workgroup per (query, 32 heads), no split
    assert csa.csa_attn_workspace_size(64, 128, 448, 64, 640) == 0
    # one query: split over workgroups, a partial row per head of 512 BF16
    # values plus (M, L) as floats, padded to 1040 bytes
    ws = csa.csa_attn_workspace_size(1, 128, 448, 64, 640)
    assert ws > 0 and ws % (128 * 1040) == 0
    # key ranges beyond 128 splits of 2048 slots are not supported
    assert lib.csa_attn_workspace_size(1, 128, 448, 64, 128 * 2048) == csa.CSA_WORKSPACE_UNSUPPORTED
    assert lib.csa_attn_workspace_size(1, 128, 100, 64, 640) == csa.CSA_WORKSPACE_UNSUPPORTED   # unsupported dims
    with pytest.raises(ValueError, match="unsupported"):
        csa.csa_attn_workspace_size(1, 128, 100, 64, 640)


def test_null_arguments_rejected_without_launch(lib):
    vp = ctypes.c_void_p
    rc = lib.csa_index_scores(None, 1.0, None, None, 1.0, None, None, 1, 64, 1, 1, None, None, 4, 64, 128, 4,
                              None, 64, None, None)
    assert rc == -1
    rc = lib.csa_topk(None, 64, None, 4, 16, None, None, 0, None)
    assert rc == -1
    rc = lib.csa_decode_attn(None, 512, None, None, 16, None, None, None, 1.0, 0.0, 2, 128, None, None, None, 0, None)
    assert rc == -1
    rc = lib.csa_prefill_attn(None, 512, None, 0, None, 16, None, None, 1.0, 0, 0, 128, None, 4, None, 1.0, 0.0, 128,
                              None, None, None, 0, None)
    assert rc == -1
    # zero-sized work is a no-op success
    assert lib.csa_topk(None, 64, None, 0, 16, None, None, 0, None) == 0
    assert lib.csa_index_scores(None, 1.0, None, None, 1.0, None, None, 1, 64, 1, 1, None, None, 0, 64, 128, 4,
                                None, 64, None, None) == 0


def test_unsupported_shapes_rejected(lib):
    fake = ctypes.c_void_p(1 << 20)   # 16-byte aligned host address, never dereferenced
    rc = lib.csa_index_scores(fake, 1.0, fake, fake, 1.0, fake, fake, 1, 64, 1, 1, fake, fake, 4, 65, 128, 4,
                              fake, 64, fake, None)
    assert rc == -2      # H_I > 64
    rc = lib.csa_index_scores(fake, 1.0, fake, fake, 1.0, fake, fake, 1, 64, 1, 1, fake, fake, 4, 64, 100, 4,
                              fake, 64, fake, None)
    assert rc == -2      # D_I not a multiple of 32
    rc = lib.csa_index_scores(fake, 1.0, fake, fake, 1.0, fake, fake, 1, 60, 1, 1, fake, fake, 4, 64, 128, 4,
                              fake, 64, fake, None)
    assert rc == -1      # page size not a multiple of 16
    rc = lib.csa_topk(fake, 64, fake, 4, 4096, fake, None, 0, None)
    assert rc == -2      # k > 2048
    rc = lib.csa_topk(fake, 131072, fake, 4, 512, fake, None, 0, None)
    assert rc == -4      # long rows need the workspace
    cache = csa._LatentCacheC(1 << 20, 1 << 20, 1.0, 1 << 20, 1 << 20, 2, 8, 64, 4, 100, 64, 4)
    ring = csa._SwaRingC(1 << 20, 1 << 20, 1.0, 1 << 20, 128)
    rc = lib.csa_decode_attn(fake, 512, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake, 1.0, 0.0, 2, 128,
                             fake, None, None, 0, None)
    assert rc == -2      # D_nope 100 has no kernel
    cache.D_nope = 448
    ring.W = 4096
    rc = lib.csa_decode_attn(fake, 512 * 128, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake, 1.0, 0.0, 2, 128,
                             fake, None, None, 0, None)
    assert rc == -2      # window too large
    ring.W = 128
    rc = lib.csa_decode_attn(fake, 100, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake, 1.0, 0.0, 2, 128,
                             fake, None, None, 0, None)
    assert rc == -1      # q stride below H*D
    misaligned = ctypes.c_void_p((1 << 20) + 4)
    rc = lib.csa_decode_attn(misaligned, 512 * 128, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake,
                             1.0, 0.0, 2, 128, fake, None, None, 0, None)
    assert rc == -1      # misaligned q
    rc = lib.csa_decode_attn(fake, 512 * 128, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake,
                             1.0, 0.0, 3, 128, fake, None, None, 0, None)
    assert rc == -1      # more queries than cached sequences
    rc = lib.csa_prefill_attn(fake, 512 * 128, ctypes.byref(cache), 2, fake, 16, fake, fake, 1.0, 0, 8, 128, fake,
                              4, fake, 1.0, 0.0, 128, fake, None, None, 0, None)
    assert rc == -1      # prefill sequence beyond the page table
    for theta in (-10000.0, float("nan"), float("inf")):
        rc = lib.csa_decode_attn(fake, 512 * 128, ctypes.byref(cache), fake, 16, ctypes.byref(ring), fake, fake,
                                 1.0, theta, 2, 128, fake, None, None, 0, None)
        assert rc == -1  # inverse-RoPE base must be 0 (off) or finite and > 0
        rc = lib.csa_prefill_attn(fake, 512 * 128, ctypes.byref(cache), 0, fake, 16, fake, fake, 1.0, 0, 8, 128,
                                  fake, 4, fake, 1.0, theta, 128, fake, None, None, 0, None)
        assert rc == -1


def test_binding_refuses_cpu_tensors(lib):
    import torch
    with pytest.raises(ValueError):
        csa.csa_topk(torch.zeros(4, 64), torch.zeros(4, dtype=torch.int32), 8, torch.zeros(4, 8, dtype=torch.int32))


def test_graph_calls_reject_null_handles_without_gpu_work(lib):
    # argument checks run before any HIP call
    h = ctypes.c_void_p()
    assert lib.csa_graph_capture_begin(None) == -1       # the legacy default stream cannot be captured
    assert lib.csa_graph_capture_end(None, ctypes.byref(h)) == -1
    assert lib.csa_graph_launch(None, None) == -1
    lib.csa_graph_destroy(None)                          # no-op


def test_attention_without_enough_workspace_is_rejected_before_launch(lib):
    # HCA over up to 6400 entries needs its key range split over workgroups
    # (at most 2048 slots each), so it needs the partial-result workspace
    fake = ctypes.c_void_p(1 << 20)
    cache = csa._LatentCacheC(1 << 20, 1 << 20, 1.0, 1 << 20, 1 << 20, 2, 8, 64, 100, 448, 64, 128)
    ring = csa._SwaRingC(1 << 20, 1 << 20, 1.0, 1 << 20, 128)
    need = lib.csa_attn_workspace_size(2, 128, 448, 64, 100 * 64 + 128)
    assert need > 0
    rc = lib.csa_decode_attn(fake, 512 * 128, ctypes.byref(cache), None, 0, ctypes.byref(ring), fake, fake,
                             1.0, 0.0, 2, 128, fake, None, None, 0, None)
    assert rc == -4      # no workspace
    rc = lib.csa_decode_attn(fake, 512 * 128, ctypes.byref(cache), None, 0, ctypes.byref(ring), fake, fake,
                             1.0, 0.0, 2, 128, fake, None, fake, 1024, None)
    assert rc == -4      # far too small


# ---------------------------------------------------------------- binding shape checks
def _decode_args(B=2, H=8, dn=48, dr=16, W=32, k=16):
    import torch
    D = dn + dr
    cache = csa.LatentCache(torch.zeros(4, 64, dn, dtype=torch.uint8), torch.zeros(4, 64, dr, dtype=torch.bfloat16),
                            1.0, torch.zeros(B, 2, dtype=torch.int32), torch.zeros(B, dtype=torch.int32), 4)
    swa = csa.SwaRing(torch.zeros(B, W, dn, dtype=torch.uint8), torch.zeros(B, W, dr, dtype=torch.bfloat16), 1.0,
                      torch.zeros(B, W, dtype=torch.int32))
    return dict(q=torch.zeros(B, H, D, dtype=torch.bfloat16), cache=cache, topk_idx=torch.zeros(B, k, dtype=torch.int32),
                k=k, swa=swa, q_pos=torch.zeros(B, dtype=torch.int32), sink=torch.zeros(H), softmax_scale=0.125,
                out=torch.zeros(B, H, D, dtype=torch.bfloat16), lse=torch.zeros(B, H))


@pytest.mark.parametrize("change,match", [
    (lambda a, t: a.update(out=t.zeros(2, 8, 63, dtype=t.bfloat16)), "out has shape"),
    (lambda a, t: a.update(out=t.zeros(3, 8, 64, dtype=t.bfloat16)), "out has shape"),
    (lambda a, t: a.update(lse=t.zeros(2, 7)), "lse has shape"),
    (lambda a, t: a.update(topk_idx=t.zeros(2, 15, dtype=t.int32)), "topk_idx has shape"),
    (lambda a, t: a.update(topk_idx=t.zeros(1, 16, dtype=t.int32)), "topk_idx has shape"),
    (lambda a, t: a.update(q_pos=t.zeros(3, dtype=t.int32)), "q_pos has shape"),
    (lambda a, t: a.update(sink=t.zeros(7)), "sink has shape"),
    (lambda a, t: a.update(q=t.zeros(2, 8, 60, dtype=t.bfloat16)), "dims per head"),
    (lambda a, t: a["swa"].__setattr__("nope", t.zeros(1, 32, 48, dtype=t.uint8)), "swa.nope has shape"),
    (lambda a, t: a["swa"].__setattr__("nope", t.zeros(2, 32, 40, dtype=t.uint8)), "swa.nope has shape"),
    (lambda a, t: a["swa"].__setattr__("rope", t.zeros(2, 32, 8, dtype=t.bfloat16)), "swa.rope has shape"),
    (lambda a, t: a["swa"].__setattr__("rope", t.zeros(2, 31, 16, dtype=t.bfloat16)), "swa.rope has shape"),
    (lambda a, t: a["swa"].__setattr__("pos", t.zeros(2, 16, dtype=t.int32)), "swa.pos has shape"),
    (lambda a, t: a["cache"].__setattr__("page_table", t.zeros(1, 2, dtype=t.int32)), "cache.page_table"),
])
def test_decode_binding_rejects_mismatched_shapes(change, match):
    import torch
    a = _decode_args()
    change(a, torch)
    with pytest.raises(ValueError, match=match):
        csa.csa_decode_attn(**a)


def test_decode_binding_shape_check_passes_consistent_shapes():
    # consistent shapes get past the shape checks and stop at the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        csa.csa_decode_attn(**_decode_args())


def _prefill_args(T=5, H=8, dn=48, dr=16, L=40, k=16):
    import torch
    a = _decode_args(B=1, H=H, dn=dn, dr=dr, k=k)
    D = dn + dr
    return dict(q=torch.zeros(T, H, D, dtype=torch.bfloat16), cache=a["cache"], seq=0,
                topk_idx=torch.zeros(T, k, dtype=torch.int32), k=k, swa_nope=torch.zeros(L, dn, dtype=torch.uint8),
                swa_rope=torch.zeros(L, dr, dtype=torch.bfloat16), swa_scale=1.0, swa_first_pos=0, W=32,
                q_pos=torch.zeros(T, dtype=torch.int32), sink=torch.zeros(H), softmax_scale=0.125,
                out=torch.zeros(T, H, D, dtype=torch.bfloat16), lse=torch.zeros(T, H))


@pytest.mark.parametrize("change,match", [
    (lambda a, t: a.update(swa_rope=t.zeros(39, 16, dtype=t.bfloat16)), "swa_rope has shape"),
    (lambda a, t: a.update(swa_nope=t.zeros(40, 32, dtype=t.uint8)), "swa_nope has shape"),
    (lambda a, t: a.update(seq=1), "page table"),
    (lambda a, t: a.update(topk_idx=t.zeros(4, 16, dtype=t.int32)), "topk_idx has shape"),
    (lambda a, t: a.update(lse=t.zeros(5, 8, 1)), "lse has shape"),
    (lambda a, t: a.update(q_pos=t.zeros(6, dtype=t.int32)), "q_pos has shape"),
])
def test_prefill_binding_rejects_mismatched_shapes(change, match):
    import torch
    a = _prefill_args()
    change(a, torch)
    with pytest.raises(ValueError, match=match):
        csa.csa_prefill_attn(**a)


def test_prefill_binding_shape_check_passes_consistent_shapes():
    with pytest.raises(ValueError, match="GPU tensor"):
        csa.csa_prefill_attn(**_prefill_args())


def test_topk_in_attention_rejects_long_rows_before_launch(lib):
    # one attention workgroup holds a row of at most 8192 scores
    fake = ctypes.c_void_p(1 << 20)
    cache = csa._LatentCacheC(1 << 20, 1 << 20, 1.0, 1 << 20, 1 << 20, 2, 8, 64, 4, 448, 64, 4)
    ring = csa._SwaRingC(1 << 20, 1 << 20, 1.0, 1 << 20, 128)
    args = (fake, 512 * 128, ctypes.byref(cache), ctypes.byref(ring), fake, fake, 1.0, 0.0, 2, 128, fake, None,
            None, 0, None)
    assert lib.csa_topk_decode_attn(fake, 8193, fake, 512, None, *args) == -2
    assert lib.csa_topk_decode_attn(fake, 8192, fake, 4096, None, *args) == -2     # k > 2048
    assert lib.csa_topk_decode_attn(None, 8192, fake, 512, None, *args) == -1      # no scores
    assert lib.csa_topk_decode_attn(fake, 8192, None, 512, None, *args) == -1      # no visible counts
