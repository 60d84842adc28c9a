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
    # rows too long for two levels of 16384 candidates
    assert csa.csa_topk_workspace_size(1, 1 << 22, 2048) == 0
    # many queries: one workgroup per (query, 32 heads), no split
    assert csa.csa_attn_workspace_size(64, 128, 448, 64, 640) == 0
    # one query: split over workgroups, partials of 512 + 2 floats per head
    # padded to 516 (16-byte rows)
    ws = csa.csa_attn_workspace_size(1, 128, 448, 64, 640)
    assert ws > 0 and ws % (128 * 516 * 4) == 0
    # key ranges beyond 128 splits of 2048 slots are not supported
    assert csa.csa_attn_workspace_size(1, 128, 448, 64, 128 * 2048) == 0
    assert csa.csa_attn_workspace_size(1, 128, 100, 64, 640) == 0   # unsupported dims


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
