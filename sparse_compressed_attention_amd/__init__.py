"""Python binding of libcsa.so, the MI355X (gfx950) CSA hot path.

Thin ctypes marshalling over the C ABI declared in include/csa.h: every
function below has the name of the C entry point it wraps, checks tensor
dtypes/devices/shapes, passes data_ptr()s and the current HIP stream, and
raises CsaError on a non-zero status.  All computation runs in the HIP
kernels of libcsa.so; torch only provides device memory and streams.  There
is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "CsaError", "LatentCache", "SwaRing", "DecodePath", "PrefillPath", "library_path", "load_library",
    "csa_index_scores", "csa_index_scores_mxfp4", "csa_index_topk", "csa_index_topk_workspace_size", "csa_topk", "csa_topk_workspace_size", "csa_attn_workspace_size",
    "csa_decode_attn", "csa_decode_attn_noalloc", "csa_topk_decode_attn", "csa_prefill_attn", "csa_status_string", "csa_version",
    "csa_graph_capture_begin", "csa_graph_capture_end", "csa_graph_launch", "csa_graph_destroy", "StepGraph",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None

CSA_OK = 0
CSA_WORKSPACE_UNSUPPORTED = (1 << (8 * ctypes.sizeof(ctypes.c_size_t))) - 1


class CsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed with status {code} ({_status(code)})")
        self.code = code


def library_path() -> str:
    return os.path.join(_PKG_DIR, "libcsa.so")


class _LatentCacheC(ctypes.Structure):
    _fields_ = [("nope", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("nope_scale", ctypes.c_float),
                ("page_table", ctypes.c_void_p), ("n_comp", ctypes.c_void_p),
                ("num_seqs", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("D_nope", ctypes.c_int32), ("D_rope", ctypes.c_int32), ("ratio_m", ctypes.c_int32)]


class _SwaRingC(ctypes.Structure):
    _fields_ = [("nope", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("nope_scale", ctypes.c_float),
                ("pos", ctypes.c_void_p), ("W", ctypes.c_int32)]


def load_library():
    """Load libcsa.so (built by __graft_entry__.build() / python -m
    sparse_compressed_attention_amd.build).  Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_compressed_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.csa_index_scores.argtypes = [vp, f32, vp, vp, f32, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, i32,
                                     vp, i64, vp, vp]
    lib.csa_index_scores.restype = ctypes.c_int
    lib.csa_index_scores_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, i32,
                                           vp, i64, vp, vp]
    lib.csa_index_scores_mxfp4.restype = ctypes.c_int
    lib.csa_index_topk_workspace_size.argtypes = [i32, i64, i32]
    lib.csa_index_topk_workspace_size.restype = sz
    lib.csa_index_topk.argtypes = [vp, f32, vp, vp, f32, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, i32, i32,
                                   vp, vp, vp, sz, vp]
    lib.csa_index_topk.restype = ctypes.c_int
    lib.csa_topk_workspace_size.argtypes = [i32, i64, i32]
    lib.csa_topk_workspace_size.restype = sz
    lib.csa_topk.argtypes = [vp, i64, vp, i32, i32, vp, vp, sz, vp]
    lib.csa_topk.restype = ctypes.c_int
    lib.csa_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.csa_attn_workspace_size.restype = sz
    lib.csa_decode_attn.argtypes = [vp, i64, ctypes.POINTER(_LatentCacheC), vp, i32, ctypes.POINTER(_SwaRingC),
                                    vp, vp, f32, f32, i32, i32, vp, vp, vp, sz, vp]
    lib.csa_decode_attn.restype = ctypes.c_int
    lib.csa_decode_attn_noalloc.argtypes = [vp, i64, ctypes.POINTER(_LatentCacheC), vp, i32,
                                            ctypes.POINTER(_SwaRingC), vp, vp, f32, f32, i32, i32, vp, vp, vp]
    lib.csa_decode_attn_noalloc.restype = ctypes.c_int
    lib.csa_topk_decode_attn.argtypes = [vp, i64, vp, i32, vp, vp, i64, ctypes.POINTER(_LatentCacheC),
                                         ctypes.POINTER(_SwaRingC), vp, vp, f32, f32, i32, i32, vp, vp, vp, sz, vp]
    lib.csa_topk_decode_attn.restype = ctypes.c_int
    lib.csa_prefill_attn.argtypes = [vp, i64, ctypes.POINTER(_LatentCacheC), i32, vp, i32, vp, vp, f32, i32, i32,
                                     i32, vp, i32, vp, f32, f32, i32, vp, vp, vp, sz, vp]
    lib.csa_prefill_attn.restype = ctypes.c_int
    lib.csa_status_string.argtypes = [ctypes.c_int]
    lib.csa_status_string.restype = ctypes.c_char_p
    lib.csa_version.argtypes = []
    lib.csa_version.restype = ctypes.c_int
    lib.csa_graph_capture_begin.argtypes = [vp]
    lib.csa_graph_capture_begin.restype = ctypes.c_int
    lib.csa_graph_capture_end.argtypes = [vp, ctypes.POINTER(vp)]
    lib.csa_graph_capture_end.restype = ctypes.c_int
    lib.csa_graph_launch.argtypes = [vp, vp]
    lib.csa_graph_launch.restype = ctypes.c_int
    lib.csa_graph_destroy.argtypes = [vp]
    lib.csa_graph_destroy.restype = None
    _LIB = lib
    return lib


def _status(code: int) -> str:
    try:
        return load_library().csa_status_string(code).decode()
    except Exception:  # noqa: BLE001 - only used to format an error message
        return "?"


def csa_status_string(code: int) -> str:
    return load_library().csa_status_string(int(code)).decode()


def csa_version() -> int:
    return int(load_library().csa_version())


# ---------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None, contiguous: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_U8 = (torch.uint8, torch.float8_e4m3fn)
_B16 = (torch.bfloat16, torch.int16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _stream(stream) -> ctypes.c_void_p:
    if isinstance(stream, ctypes.c_void_p):
        return stream
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, rc: int):
    if rc != CSA_OK:
        raise CsaError(fn, rc)


def _shape(t, name: str, want: tuple):
    """Exact shape check; None entries of `want` match any size."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        raise ValueError(f"{name} has shape {got}, expected {tuple('*' if w is None else w for w in want)}")


def _rows_at_least(t, name: str, n: int):
    if t.dim() < 1 or t.shape[0] < n:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs at least {n} rows")


def _attn_shapes(q, cache, topk_idx, k, q_pos, sink, out, lse):
    """Shapes shared by both attention calls: q [n][H][D] (D = the cache's
    D_nope + D_rope), out [n][H][D], lse [n][H], topk_idx [n][k], q_pos [n],
    sink with at least H entries.  Returns (n, H)."""
    if q.dim() != 3:
        raise ValueError(f"q has shape {tuple(q.shape)}, expected [queries][H][D]")
    n, H, D = q.shape
    dn, dr = cache.nope.shape[-1], cache.rope.shape[-1]
    if D != dn + dr:
        raise ValueError(f"q has {D} dims per head; the cache holds {dn} + {dr}")
    _shape(out, "out", (n, H, D))
    if lse is not None:
        _shape(lse, "lse", (n, H))
    if topk_idx is not None:
        _shape(topk_idx, "topk_idx", (n, int(k)))
    _shape(q_pos, "q_pos", (n,))
    if sink.dim() != 1 or sink.shape[0] < H:
        raise ValueError(f"sink has shape {tuple(sink.shape)}, needs one entry per head ({H})")
    return n, H


def _decode_shapes(q, cache, topk_idx, k, swa, q_pos, sink, out, lse):
    """Decode: the ring and the page table hold at least one row per query,
    with the cache's dims."""
    B, _ = _attn_shapes(q, cache, topk_idx, k, q_pos, sink, out, lse)
    _rows_at_least(cache.page_table, "cache.page_table", B)
    if swa.nope.dim() != 3:
        raise ValueError(f"swa.nope has shape {tuple(swa.nope.shape)}, expected [B][W][D_nope]")
    nb, W, dn = swa.nope.shape
    if nb < B or dn != cache.nope.shape[-1]:
        raise ValueError(f"swa.nope has shape {tuple(swa.nope.shape)}, expected [>= {B}][W][{cache.nope.shape[-1]}]")
    _shape(swa.rope, "swa.rope", (nb, W, cache.rope.shape[-1]))
    _shape(swa.pos, "swa.pos", (nb, W))


def _prefill_shapes(q, cache, seq, topk_idx, k, swa_nope, swa_rope, q_pos, sink, out, lse):
    """Prefill: the linear window buffer has as many rope rows as nope rows,
    with the cache's dims; `seq` is a row of the page table."""
    _attn_shapes(q, cache, topk_idx, k, q_pos, sink, out, lse)
    if not 0 <= int(seq) < cache.page_table.shape[0]:
        raise ValueError(f"seq {seq} is not a row of the page table ({cache.page_table.shape[0]} rows)")
    if swa_nope.dim() != 2 or swa_nope.shape[1] != cache.nope.shape[-1]:
        raise ValueError(f"swa_nope has shape {tuple(swa_nope.shape)}, expected [L][{cache.nope.shape[-1]}]")
    _shape(swa_rope, "swa_rope", (swa_nope.shape[0], cache.rope.shape[-1]))


@dataclass
class LatentCache:
    """Paged compressed-latent cache of one layer (see csa_latent_cache)."""
    nope: torch.Tensor        # [P][page][D_nope] uint8 (E4M3 bytes)
    rope: torch.Tensor        # [P][page][D_rope] bfloat16
    nope_scale: float
    page_table: torch.Tensor  # [B][max_pages] int32
    n_comp: torch.Tensor      # [B] int32
    ratio_m: int

    def as_c(self) -> _LatentCacheC:
        _need(self.nope, "cache.nope", _U8, 3)
        _need(self.rope, "cache.rope", _B16, 3)
        _need(self.page_table, "cache.page_table", _I32, 2)
        _need(self.n_comp, "cache.n_comp", _I32, 1)
        P, ps, dn = self.nope.shape
        if tuple(self.rope.shape[:2]) != (P, ps):
            raise ValueError(f"cache.rope has shape {tuple(self.rope.shape)}, expected [{P}][{ps}][D_rope] "
                             "like cache.nope")
        if self.n_comp.shape[0] != self.page_table.shape[0]:
            raise ValueError("cache.n_comp must have one entry per page-table row")
        return _LatentCacheC(self.nope.data_ptr(), self.rope.data_ptr(), float(self.nope_scale),
                             self.page_table.data_ptr(), self.n_comp.data_ptr(), self.page_table.shape[0], P, ps,
                             self.page_table.shape[1], dn, self.rope.shape[2], int(self.ratio_m))


@dataclass
class SwaRing:
    """Sliding-window ring of a decode batch (see csa_swa_ring)."""
    nope: torch.Tensor        # [B][W][D_nope] uint8
    rope: torch.Tensor        # [B][W][D_rope] bfloat16
    nope_scale: float
    pos: torch.Tensor         # [B][W] int32, -1 = empty

    def as_c(self) -> _SwaRingC:
        _need(self.nope, "swa.nope", _U8, 3)
        _need(self.rope, "swa.rope", _B16, 3)
        _need(self.pos, "swa.pos", _I32, 2)
        return _SwaRingC(self.nope.data_ptr(), self.rope.data_ptr(), float(self.nope_scale),
                         self.pos.data_ptr(), self.pos.shape[1])


# ---------------------------------------------------------------- entry points
def csa_index_scores(q_idx, q_idx_scale, w, k_idx, k_idx_scale, page_table, n_comp, q_pos, q_seq, ratio_m,
                     scores, n_visible, stream=None):
    _need(q_idx, "q_idx", _U8, 3)
    _need(w, "w", _F32, 2)
    _need(k_idx, "k_idx", _U8, 3)
    _need(page_table, "page_table", _I32, 2)
    _need(n_comp, "n_comp", _I32, 1)
    _need(q_pos, "q_pos", _I32, 1)
    if q_seq is not None:                  # None: query t belongs to sequence t
        _need(q_seq, "q_seq", _I32, 1)
    _need(scores, "scores", _F32, 2, contiguous=False)
    _need(n_visible, "n_visible", _I32, 1)
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    T, H_I, D_I = q_idx.shape
    P, ps, dk = k_idx.shape
    if dk != D_I or tuple(w.shape) != (T, H_I) or scores.shape[0] != T:
        raise ValueError("inconsistent indexer shapes")
    rc = load_library().csa_index_scores(
        _ptr(q_idx), float(q_idx_scale), _ptr(w), _ptr(k_idx), float(k_idx_scale), _ptr(page_table),
        _ptr(n_comp), P, ps, page_table.shape[1], page_table.shape[0], _ptr(q_pos), _ptr(q_seq), T, H_I, D_I,
        int(ratio_m), _ptr(scores), scores.stride(0), _ptr(n_visible), _stream(stream))
    _check("csa_index_scores", rc)


def csa_index_scores_mxfp4(q_idx, q_idx_sc, w, k_idx, k_idx_sc, page_table, n_comp, q_pos, q_seq, ratio_m,
                           scores, n_visible, stream=None):
    """MXFP4 indexer: q_idx [T][H_I][D_I/2] and k_idx [P][ps][D_I/2] packed
    E2M1 bytes, q_idx_sc [T][H_I][D_I/32] and k_idx_sc [P][ps][D_I/32] E8M0."""
    _need(q_idx, "q_idx", _U8, 3)
    _need(q_idx_sc, "q_idx_sc", _U8, 3)
    _need(w, "w", _F32, 2)
    _need(k_idx, "k_idx", _U8, 3)
    _need(k_idx_sc, "k_idx_sc", _U8, 3)
    _need(page_table, "page_table", _I32, 2)
    _need(n_comp, "n_comp", _I32, 1)
    _need(q_pos, "q_pos", _I32, 1)
    if q_seq is not None:                  # None: query t belongs to sequence t
        _need(q_seq, "q_seq", _I32, 1)
    _need(scores, "scores", _F32, 2, contiguous=False)
    _need(n_visible, "n_visible", _I32, 1)
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    T, H_I, DH = q_idx.shape
    D_I = 2 * DH
    P, ps, dk = k_idx.shape
    if (dk != DH or tuple(w.shape) != (T, H_I) or scores.shape[0] != T or D_I % 32
            or tuple(q_idx_sc.shape) != (T, H_I, D_I // 32) or tuple(k_idx_sc.shape) != (P, ps, D_I // 32)):
        raise ValueError("inconsistent MXFP4 indexer shapes")
    rc = load_library().csa_index_scores_mxfp4(
        _ptr(q_idx), _ptr(q_idx_sc), _ptr(w), _ptr(k_idx), _ptr(k_idx_sc), _ptr(page_table), _ptr(n_comp), P, ps,
        page_table.shape[1], page_table.shape[0], _ptr(q_pos), _ptr(q_seq), T, H_I, D_I, int(ratio_m),
        _ptr(scores), scores.stride(0), _ptr(n_visible), _stream(stream))
    _check("csa_index_scores_mxfp4", rc)


def _ws_bytes(fn: str, n: int) -> int:
    if n == CSA_WORKSPACE_UNSUPPORTED:
        raise ValueError(f"{fn}: unsupported arguments (the matching call would reject them)")
    return int(n)


def csa_index_topk_workspace_size(T: int, max_entries: int, k: int) -> int:
    return _ws_bytes("csa_index_topk_workspace_size",
                     load_library().csa_index_topk_workspace_size(int(T), int(max_entries), int(k)))


def csa_index_topk(q_idx, q_idx_scale, w, k_idx, k_idx_scale, page_table, n_comp, q_pos, q_seq, ratio_m, k,
                   topk_idx, n_visible, workspace=None, stream=None):
    """Steps 1+2 fused: the top-k of the indexer scores without writing them."""
    _need(q_idx, "q_idx", _U8, 3)
    _need(w, "w", _F32, 2)
    _need(k_idx, "k_idx", _U8, 3)
    _need(page_table, "page_table", _I32, 2)
    _need(n_comp, "n_comp", _I32, 1)
    _need(q_pos, "q_pos", _I32, 1)
    if q_seq is not None:                  # None: query t belongs to sequence t
        _need(q_seq, "q_seq", _I32, 1)
    _need(topk_idx, "topk_idx", _I32, 2)
    _need(n_visible, "n_visible", _I32, 1)
    T, H_I, D_I = q_idx.shape
    P, ps, dk = k_idx.shape
    if dk != D_I or tuple(w.shape) != (T, H_I) or tuple(topk_idx.shape) != (T, int(k)):
        raise ValueError("inconsistent indexer / top-k shapes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().csa_index_topk(
        _ptr(q_idx), float(q_idx_scale), _ptr(w), _ptr(k_idx), float(k_idx_scale), _ptr(page_table), _ptr(n_comp),
        P, ps, page_table.shape[1], page_table.shape[0], _ptr(q_pos), _ptr(q_seq), T, H_I, D_I, int(ratio_m),
        int(k), _ptr(topk_idx), _ptr(n_visible), _ptr(workspace), ws_bytes, _stream(stream))
    _check("csa_index_topk", rc)


def csa_topk_workspace_size(T: int, ld_scores: int, k: int) -> int:
    return _ws_bytes("csa_topk_workspace_size", load_library().csa_topk_workspace_size(int(T), int(ld_scores), int(k)))


def csa_topk(scores, n_visible, k, topk_idx, workspace=None, stream=None):
    _need(scores, "scores", _F32, 2, contiguous=False)
    _need(n_visible, "n_visible", _I32, 1)
    _need(topk_idx, "topk_idx", _I32, 2)
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    T = scores.shape[0]
    if tuple(topk_idx.shape) != (T, k):
        raise ValueError("topk_idx must be [T][k]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().csa_topk(_ptr(scores), scores.stride(0), _ptr(n_visible), T, int(k), _ptr(topk_idx),
                                 _ptr(workspace), ws_bytes, _stream(stream))
    _check("csa_topk", rc)


def csa_attn_workspace_size(n_queries: int, H: int, D_nope: int, D_rope: int, max_keys_per_query: int) -> int:
    return _ws_bytes("csa_attn_workspace_size",
                     load_library().csa_attn_workspace_size(int(n_queries), int(H), int(D_nope), int(D_rope),
                                                            int(max_keys_per_query)))


def csa_decode_attn(q, cache: LatentCache, topk_idx, k, swa: SwaRing, q_pos, sink, softmax_scale, out,
                    lse=None, workspace=None, stream=None, inv_rope_theta=0.0):
    _decode_shapes(q, cache, topk_idx, k, swa, q_pos, sink, out, lse)
    _need(q, "q", _B16, 3, contiguous=False)
    _need(q_pos, "q_pos", _I32, 1)
    _need(sink, "sink", _F32, 1)
    _need(out, "out", _B16, 3)
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", _I32, 2)
    if lse is not None:
        _need(lse, "lse", _F32, 2)
    if q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [.][H][D] with contiguous heads")
    B, H, _ = q.shape
    cc, sc = cache.as_c(), swa.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().csa_decode_attn(
        _ptr(q), q.stride(0), ctypes.byref(cc), _ptr(topk_idx), int(k), ctypes.byref(sc), _ptr(q_pos), _ptr(sink),
        float(softmax_scale), float(inv_rope_theta), B, H, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check("csa_decode_attn", rc)


def csa_decode_attn_noalloc(q, cache: LatentCache, topk_idx, k, swa: SwaRing, q_pos, sink, softmax_scale, out,
                            lse=None, stream=None, inv_rope_theta=0.0):
    """csa_decode_attn with the split partial results in the library's
    static scratch array (16 MiB per GPU) instead of a caller workspace:
    allocates nothing.  Calls that overlap on one GPU race on that array."""
    _decode_shapes(q, cache, topk_idx, k, swa, q_pos, sink, out, lse)
    _need(q, "q", _B16, 3, contiguous=False)
    _need(q_pos, "q_pos", _I32, 1)
    _need(sink, "sink", _F32, 1)
    _need(out, "out", _B16, 3)
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", _I32, 2)
    if lse is not None:
        _need(lse, "lse", _F32, 2)
    if q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [.][H][D] with contiguous heads")
    B, H, _ = q.shape
    cc, sc = cache.as_c(), swa.as_c()
    rc = load_library().csa_decode_attn_noalloc(
        _ptr(q), q.stride(0), ctypes.byref(cc), _ptr(topk_idx), int(k), ctypes.byref(sc), _ptr(q_pos), _ptr(sink),
        float(softmax_scale), float(inv_rope_theta), B, H, _ptr(out), _ptr(lse), _stream(stream))
    _check("csa_decode_attn_noalloc", rc)


def csa_topk_decode_attn(scores, n_visible, k, q, cache: LatentCache, swa: SwaRing, q_pos, sink, softmax_scale, out,
                         lse=None, topk_idx=None, workspace=None, stream=None, inv_rope_theta=0.0):
    """csa_topk followed by csa_decode_attn in one launch: the attention
    kernel selects each query's top-k from scores [B][ld] (rows up to 8192
    entries) itself; topk_idx [B][k], when given, receives the indices."""
    _need(scores, "scores", _F32, 2, contiguous=False)
    _need(n_visible, "n_visible", _I32, 1)
    if scores.stride(1) != 1:
        raise ValueError("scores rows must be contiguous")
    _decode_shapes(q, cache, topk_idx, k, swa, q_pos, sink, out, lse)
    B = q.shape[0]
    if scores.shape[0] != B or n_visible.shape[0] != B:
        raise ValueError(f"scores {tuple(scores.shape)} / n_visible {tuple(n_visible.shape)} need {B} rows")
    _need(q, "q", _B16, 3, contiguous=False)
    _need(q_pos, "q_pos", _I32, 1)
    _need(sink, "sink", _F32, 1)
    _need(out, "out", _B16, 3)
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", _I32, 2)
    if lse is not None:
        _need(lse, "lse", _F32, 2)
    if q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [.][H][D] with contiguous heads")
    H = q.shape[1]
    cc, sc = cache.as_c(), swa.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().csa_topk_decode_attn(
        _ptr(scores), scores.stride(0), _ptr(n_visible), int(k), _ptr(topk_idx), _ptr(q), q.stride(0),
        ctypes.byref(cc), ctypes.byref(sc), _ptr(q_pos), _ptr(sink), float(softmax_scale), float(inv_rope_theta), B,
        H, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check("csa_topk_decode_attn", rc)


def csa_prefill_attn(q, cache: LatentCache, seq, topk_idx, k, swa_nope, swa_rope, swa_scale, swa_first_pos, W,
                     q_pos, sink, softmax_scale, out, lse=None, workspace=None, stream=None, inv_rope_theta=0.0):
    _prefill_shapes(q, cache, seq, topk_idx, k, swa_nope, swa_rope, q_pos, sink, out, lse)
    _need(q, "q", _B16, 3, contiguous=False)
    _need(q_pos, "q_pos", _I32, 1)
    _need(sink, "sink", _F32, 1)
    _need(out, "out", _B16, 3)
    _need(swa_nope, "swa_nope", _U8, 2)
    _need(swa_rope, "swa_rope", _B16, 2)
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", _I32, 2)
    if lse is not None:
        _need(lse, "lse", _F32, 2)
    if q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [.][H][D] with contiguous heads")
    T, H, _ = q.shape
    cc = cache.as_c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().csa_prefill_attn(
        _ptr(q), q.stride(0), ctypes.byref(cc), int(seq), _ptr(topk_idx), int(k), _ptr(swa_nope), _ptr(swa_rope),
        float(swa_scale), int(swa_first_pos), swa_nope.shape[0], int(W), _ptr(q_pos), T, _ptr(sink),
        float(softmax_scale), float(inv_rope_theta), H, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check("csa_prefill_attn", rc)


# ---------------------------------------------------------------- whole path
class _Path:
    """Base of DecodePath / PrefillPath: the ABI calls of one step with their
    arguments marshalled once (pointers and host structs are fixed for the
    life of the object), so run() only issues the C calls."""

    stage_names: tuple = ()

    def _finalize(self):
        lib = load_library()
        self._stages = [(getattr(lib, fn), fn, args) for fn, args in self._plan()]

    def _index_stage(self):
        """The indexer call of the step: E4M3 with per-tensor scales, or
        MXFP4 when the block-scale tensors were given."""
        T, H_I, DQ = self.q_idx.shape
        P, ps, _ = self.k_idx.shape
        pt = self.cache.page_table
        tail = (_ptr(pt), _ptr(self.cache.n_comp), P, ps, pt.shape[1], pt.shape[0], _ptr(self.q_pos),
                _ptr(self.q_seq), T, H_I)
        if self.q_idx_sc is not None and self.k_idx_sc is not None:
            _need(self.q_idx_sc, "q_idx_sc", _U8, 3)
            _need(self.k_idx_sc, "k_idx_sc", _U8, 3)
            return ("csa_index_scores_mxfp4", (
                _ptr(self.q_idx), _ptr(self.q_idx_sc), _ptr(self.w), _ptr(self.k_idx), _ptr(self.k_idx_sc), *tail,
                2 * DQ, int(self.cache.ratio_m), _ptr(self.scores), self.ld, _ptr(self.n_vis)))
        return ("csa_index_scores", (
            _ptr(self.q_idx), float(self.q_idx_scale), _ptr(self.w), _ptr(self.k_idx), float(self.k_idx_scale),
            *tail, DQ, int(self.cache.ratio_m), _ptr(self.scores), self.ld, _ptr(self.n_vis)))

    def _index_topk_stage(self):
        """Steps 1+2 as one call (csa_index_topk, E4M3 operands)."""
        T, H_I, D_I = self.q_idx.shape
        P, ps, _ = self.k_idx.shape
        pt = self.cache.page_table
        tw = 0 if self.topk_ws is None else self.topk_ws.numel()
        return ("csa_index_topk", (
            _ptr(self.q_idx), float(self.q_idx_scale), _ptr(self.w), _ptr(self.k_idx), float(self.k_idx_scale),
            _ptr(pt), _ptr(self.cache.n_comp), P, ps, pt.shape[1], pt.shape[0], _ptr(self.q_pos), _ptr(self.q_seq),
            T, H_I, D_I, int(self.cache.ratio_m), self.k, _ptr(self.topk), _ptr(self.n_vis), _ptr(self.topk_ws),
            tw))

    def run_stage(self, i: int, stream=None):
        fn, name, args = self._stages[i]
        rc = fn(*args, _stream(stream))
        if rc != CSA_OK:
            raise CsaError(name, rc)

    def run(self, stream=None):
        st = _stream(stream)
        for fn, name, args in self._stages:
            rc = fn(*args, st)
            if rc != CSA_OK:
                raise CsaError(name, rc)
        return self.out, self.lse


class DecodePath(_Path):
    """One CSA decode step (indexer -> top-k -> gather + attention) with all
    buffers allocated once, so run() enqueues only the kernels.

    HCA layers (no indexer) pass q_idx=None: run() then attends every
    visible compressed entry."""

    def __init__(self, *, cache: LatentCache, swa: SwaRing, q, q_pos, sink, softmax_scale, k,
                 q_idx=None, q_idx_scale=1.0, w=None, k_idx=None, k_idx_scale=1.0, inv_rope_theta=0.0,
                 q_idx_sc=None, k_idx_sc=None, fused_topk=False, topk_in_attn=False):
        dev = q.device
        self.inv_rope_theta = float(inv_rope_theta)
        self.q_idx_sc, self.k_idx_sc = q_idx_sc, k_idx_sc   # both given: MXFP4 indexer inputs
        # steps 1+2 as one call that keeps the scores on chip (E4M3 only)
        self.fused_topk = bool(fused_topk) and q_idx is not None and q_idx_sc is None
        # steps 2-4 as one call (csa_topk_decode_attn): the attention kernel
        # selects the top-k from the scores (rows up to 8192 entries)
        self.topk_in_attn = bool(topk_in_attn) and q_idx is not None and not self.fused_topk
        self.cache, self.swa, self.q, self.q_pos, self.sink = cache, swa, q, q_pos, sink
        self.softmax_scale, self.k = float(softmax_scale), int(k)
        self.q_idx, self.q_idx_scale, self.w, self.k_idx, self.k_idx_scale = q_idx, q_idx_scale, w, k_idx, k_idx_scale
        _need(q, "q", _B16, 3)
        B, H, D = q.shape
        self.q_seq = None                  # the indexer's default: query b belongs to sequence b
        max_entries = cache.page_table.shape[1] * cache.nope.shape[1]
        self.ld = max(16, (max_entries + 15) // 16 * 16)
        self.out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        if q_idx is not None:
            self.n_vis = torch.empty((B,), dtype=torch.int32, device=dev)
            self.topk = torch.empty((B, self.k), dtype=torch.int32, device=dev)
            if self.topk_in_attn and self.ld > 8192:
                raise ValueError("the top-k inside the attention takes rows of at most 8192 entries")
            if self.topk_in_attn:
                self.scores = torch.empty((B, self.ld), dtype=torch.float32, device=dev)
                tw = 0
                self.stage_names = ("index_scores", "topk_decode_attn")
            elif self.fused_topk:
                self.scores = None
                tw = csa_index_topk_workspace_size(B, max_entries, self.k)
                self.stage_names = ("index_topk", "decode_attn")
            else:
                self.scores = torch.empty((B, self.ld), dtype=torch.float32, device=dev)
                tw = csa_topk_workspace_size(B, self.ld, self.k)
                self.stage_names = ("index_scores", "topk", "decode_attn")
            self.topk_ws = torch.empty((max(tw, 16),), dtype=torch.uint8, device=dev) if tw else None
            max_keys = self.k + swa.pos.shape[1]
        else:
            self.scores = self.n_vis = self.topk = self.topk_ws = None
            max_keys = max_entries + swa.pos.shape[1]
            self.stage_names = ("decode_attn",)
        aw = csa_attn_workspace_size(B, H, cache.nope.shape[2], cache.rope.shape[2], max_keys)
        self.attn_ws = torch.empty((max(aw, 16),), dtype=torch.uint8, device=dev) if aw else None
        self._finalize()

    def _plan(self):
        B, H, _ = self.q.shape
        self._cc, self._sc = self.cache.as_c(), self.swa.as_c()
        plan = []
        if self.q_idx is not None:
            _need(self.q_idx, "q_idx", _U8, 3)
            _need(self.k_idx, "k_idx", _U8, 3)
            _need(self.w, "w", _F32, 2)
            tw = 0 if self.topk_ws is None else self.topk_ws.numel()
            if self.fused_topk:
                plan.append(self._index_topk_stage())
            elif self.topk_in_attn:
                plan.append(self._index_stage())
            else:
                plan.append(self._index_stage())
                plan.append(("csa_topk", (_ptr(self.scores), self.ld, _ptr(self.n_vis), B, self.k, _ptr(self.topk),
                                          _ptr(self.topk_ws), tw)))
        _decode_shapes(self.q, self.cache, self.topk, self.k, self.swa, self.q_pos, self.sink, self.out, self.lse)
        _need(self.q_pos, "q_pos", _I32, 1)
        _need(self.sink, "sink", _F32, 1)
        aw = 0 if self.attn_ws is None else self.attn_ws.numel()
        if self.topk_in_attn:
            plan.append(("csa_topk_decode_attn", (
                _ptr(self.scores), self.ld, _ptr(self.n_vis), self.k, _ptr(self.topk), _ptr(self.q), self.q.stride(0),
                ctypes.byref(self._cc), ctypes.byref(self._sc), _ptr(self.q_pos), _ptr(self.sink),
                self.softmax_scale, self.inv_rope_theta, B, H, _ptr(self.out), _ptr(self.lse), _ptr(self.attn_ws),
                aw)))
            return plan
        plan.append(("csa_decode_attn", (
            _ptr(self.q), self.q.stride(0), ctypes.byref(self._cc), _ptr(self.topk), self.k, ctypes.byref(self._sc),
            _ptr(self.q_pos), _ptr(self.sink), self.softmax_scale, self.inv_rope_theta, B, H, _ptr(self.out),
            _ptr(self.lse),
            _ptr(self.attn_ws), aw)))
        return plan


class PrefillPath(_Path):
    """One CSA prefill chunk (T queries of one sequence) with buffers
    allocated once.  fused_topk runs steps 1+2 as one call that keeps the
    scores on chip (E4M3 indexer inputs)."""

    def __init__(self, *, cache: LatentCache, seq, q, q_pos, sink, softmax_scale, k, W, swa_nope, swa_rope,
                 swa_scale, swa_first_pos, q_idx, q_idx_scale, w, k_idx, k_idx_scale, inv_rope_theta=0.0,
                 q_idx_sc=None, k_idx_sc=None, fused_topk=False):
        dev = q.device
        self.inv_rope_theta = float(inv_rope_theta)
        self.q_idx_sc, self.k_idx_sc = q_idx_sc, k_idx_sc   # both given: MXFP4 indexer inputs
        self.fused_topk = bool(fused_topk) and q_idx_sc is None
        self.cache, self.seq, self.q, self.q_pos, self.sink = cache, int(seq), q, q_pos, sink
        self.softmax_scale, self.k, self.W = float(softmax_scale), int(k), int(W)
        self.swa_nope, self.swa_rope, self.swa_scale, self.swa_first_pos = swa_nope, swa_rope, swa_scale, swa_first_pos
        self.q_idx, self.q_idx_scale, self.w, self.k_idx, self.k_idx_scale = q_idx, q_idx_scale, w, k_idx, k_idx_scale
        _need(q, "q", _B16, 3)
        T, H, D = q.shape
        self.q_seq = torch.full((T,), self.seq, dtype=torch.int32, device=dev)
        max_entries = cache.page_table.shape[1] * cache.nope.shape[1]
        self.ld = max(16, (max_entries + 15) // 16 * 16)
        self.n_vis = torch.empty((T,), dtype=torch.int32, device=dev)
        self.topk = torch.empty((T, self.k), dtype=torch.int32, device=dev)
        if self.fused_topk:
            self.scores = None
            tw = csa_index_topk_workspace_size(T, max_entries, self.k)
            self.stage_names = ("index_topk", "prefill_attn")
        else:
            self.scores = torch.empty((T, self.ld), dtype=torch.float32, device=dev)
            tw = csa_topk_workspace_size(T, self.ld, self.k)
            self.stage_names = ("index_scores", "topk", "prefill_attn")
        self.topk_ws = torch.empty((max(tw, 16),), dtype=torch.uint8, device=dev) if tw else None
        self.out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        aw = csa_attn_workspace_size(T, H, cache.nope.shape[2], cache.rope.shape[2], self.k + self.W)
        self.attn_ws = torch.empty((max(aw, 16),), dtype=torch.uint8, device=dev) if aw else None
        self._finalize()

    def _plan(self):
        T, H, _ = self.q.shape
        _prefill_shapes(self.q, self.cache, self.seq, self.topk, self.k, self.swa_nope, self.swa_rope, self.q_pos,
                        self.sink, self.out, self.lse)
        _need(self.q_pos, "q_pos", _I32, 1)
        _need(self.sink, "sink", _F32, 1)
        self._cc = self.cache.as_c()
        _need(self.q_idx, "q_idx", _U8, 3)
        _need(self.k_idx, "k_idx", _U8, 3)
        _need(self.w, "w", _F32, 2)
        _need(self.swa_nope, "swa_nope", _U8, 2)
        _need(self.swa_rope, "swa_rope", _B16, 2)
        tw = 0 if self.topk_ws is None else self.topk_ws.numel()
        aw = 0 if self.attn_ws is None else self.attn_ws.numel()
        if self.fused_topk:
            steps = [self._index_topk_stage()]
        else:
            steps = [self._index_stage(),
                     ("csa_topk", (_ptr(self.scores), self.ld, _ptr(self.n_vis), T, self.k, _ptr(self.topk),
                                   _ptr(self.topk_ws), tw))]
        return steps + [
            ("csa_prefill_attn", (
                _ptr(self.q), self.q.stride(0), ctypes.byref(self._cc), self.seq, _ptr(self.topk), self.k,
                _ptr(self.swa_nope), _ptr(self.swa_rope), float(self.swa_scale), int(self.swa_first_pos),
                self.swa_nope.shape[0], self.W, _ptr(self.q_pos), T, _ptr(self.sink), self.softmax_scale,
                self.inv_rope_theta, H,
                _ptr(self.out), _ptr(self.lse), _ptr(self.attn_ws), aw)),
        ]


# ---------------------------------------------------------------- graph replay
def csa_graph_capture_begin(stream) -> None:
    _check("csa_graph_capture_begin", load_library().csa_graph_capture_begin(_stream(stream)))


def csa_graph_capture_end(stream) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check("csa_graph_capture_end", load_library().csa_graph_capture_end(_stream(stream), ctypes.byref(h)))
    return h


def csa_graph_launch(graph: ctypes.c_void_p, stream=None) -> None:
    _check("csa_graph_launch", load_library().csa_graph_launch(graph, _stream(stream)))


def csa_graph_destroy(graph: ctypes.c_void_p) -> None:
    load_library().csa_graph_destroy(graph)


class StepGraph:
    """One step of a DecodePath / PrefillPath recorded once with the library's
    graph calls and replayed with a single launch.  A replay reads the current
    contents of the path's buffers (refreshed q, positions, cache rows) and
    writes path.out / path.lse; shapes and pointers are those of the capture."""

    def __init__(self, path: "_Path"):
        self.path = path
        dev = path.out.device
        cur = torch.cuda.current_stream(dev)
        side = torch.cuda.Stream(device=dev)   # default priority
        side.wait_stream(cur)
        csa_graph_capture_begin(side)
        try:
            path.run(stream=side)
        except BaseException:
            h = ctypes.c_void_p()
            load_library().csa_graph_capture_end(_stream(side), ctypes.byref(h))
            if h.value:
                csa_graph_destroy(h)
            raise
        self._h = csa_graph_capture_end(side)
        cur.wait_stream(side)

    def replay(self, stream=None):
        if self._h is None:
            raise RuntimeError("graph already destroyed")
        csa_graph_launch(self._h, stream)
        return self.path.out, self.path.lse

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            csa_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
