"""Moves a seeded workload to GPU tensors and wires it to the HIP path
(DecodePath / PrefillPath of the binding).  Plumbing only: tensor copies and
views, no arithmetic of the method."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch


def _t(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def to_device(wl, device="cuda") -> SimpleNamespace:
    s = wl.spec
    d = SimpleNamespace(spec=s, T=wl.T, B=wl.B)
    d.lat_nope = _t(wl.lat_nope, device)
    d.lat_rope = _t(wl.lat_rope.view(np.int16), device).view(torch.bfloat16)
    d.lat_scale = float(wl.lat_scale)
    d.page_table = _t(wl.page_table, device)
    d.n_comp = _t(wl.n_comp, device)
    d.q_pos = _t(wl.q_pos, device)
    d.q_seq = _t(wl.q_seq, device)
    d.q = _t(wl.q.view(np.int16), device).view(torch.bfloat16)
    d.sink = _t(wl.sink, device)
    d.swa_nope = _t(wl.swa_nope, device)
    d.swa_rope = _t(wl.swa_rope.view(np.int16), device).view(torch.bfloat16)
    d.swa_scale = float(wl.swa_scale)
    d.swa_pos = None if wl.swa_pos is None else _t(wl.swa_pos, device)
    d.swa_first_pos, d.swa_len = int(wl.swa_first_pos), int(wl.swa_len)
    if wl.q_idx is not None:
        d.q_idx = _t(wl.q_idx, device)
        d.w = _t(wl.w, device)
        d.k_idx = _t(wl.k_idx, device)
    else:
        d.q_idx = d.w = d.k_idx = None
    d.q_idx4 = d.q_idx4_sc = d.k_idx4 = d.k_idx4_sc = None
    if wl.q_idx4 is not None:
        d.q_idx4, d.q_idx4_sc = _t(wl.q_idx4, device), _t(wl.q_idx4_sc, device)
        d.k_idx4, d.k_idx4_sc = _t(wl.k_idx4, device), _t(wl.k_idx4_sc, device)
    d.q_idx_scale, d.k_idx_scale = float(wl.q_idx_scale), float(wl.k_idx_scale)
    return d


def make_path(d, csa=None, inv_rope_theta=0.0, mxfp4=False, fused_topk=False, topk_in_attn=False):
    """DecodePath (decode workloads) or PrefillPath (prefill chunk); a
    nonzero inv_rope_theta turns on the inverse-RoPE epilogue; mxfp4 feeds
    the indexer the MXFP4 copy of its inputs; fused_topk runs steps 1+2 as
    one call (decode and prefill), topk_in_attn steps 2-4 (decode)."""
    if csa is None:
        import sparse_compressed_attention_amd as csa  # noqa: PLC0415
    s = d.spec
    idx = dict(q_idx=d.q_idx, q_idx_scale=d.q_idx_scale, w=d.w, k_idx=d.k_idx, k_idx_scale=d.k_idx_scale)
    if mxfp4:
        if d.q_idx4 is None:
            raise ValueError("the workload has no MXFP4 indexer inputs (generate it with mxfp4=True)")
        idx.update(q_idx=d.q_idx4, k_idx=d.k_idx4, q_idx_sc=d.q_idx4_sc, k_idx_sc=d.k_idx4_sc)
    cache = csa.LatentCache(d.lat_nope, d.lat_rope, d.lat_scale, d.page_table, d.n_comp, s.m)
    if s.kind == "decode":
        swa = csa.SwaRing(d.swa_nope, d.swa_rope, d.swa_scale, d.swa_pos)
        return csa.DecodePath(cache=cache, swa=swa, q=d.q, q_pos=d.q_pos, sink=d.sink, softmax_scale=s.sigma,
                              k=s.k, inv_rope_theta=inv_rope_theta, fused_topk=fused_topk,
                              topk_in_attn=topk_in_attn, **idx)
    return csa.PrefillPath(cache=cache, seq=0, q=d.q, q_pos=d.q_pos, sink=d.sink, softmax_scale=s.sigma, k=s.k,
                           W=s.W, swa_nope=d.swa_nope, swa_rope=d.swa_rope, swa_scale=d.swa_scale,
                           swa_first_pos=d.swa_first_pos, inv_rope_theta=inv_rope_theta, fused_topk=fused_topk,
                           **idx)
