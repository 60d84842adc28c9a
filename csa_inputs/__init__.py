"""Seeded synthetic inputs for the CSA hot path.

This module is shared by the FP64 oracle tests, the GPU parity tests and the
benchmark.  It draws random numbers and stores them in the formats the cache
uses (OCP E4M3FN bytes with a per-tensor dequant multiplier, BF16 bits); the
encoding is done by torch's own float8_e4m3fn / bfloat16 casts.  It holds none
of the method's arithmetic: no scoring, selection, gather or attention.

Shapes and distributions follow the workloads described on the pages' subject
(DSV4 Audit, Part B, B1/B2; DSV4 Inference Kernel README, Architecture):
a 512-d latent shared by all query heads, stored as FP8_E4M3 "nope" dims plus
BF16 rope dims, an FP8 indexer with one key per compressed entry, a
sliding-window ring, per-head sink logits.  Data: q, latents and keys N(0,1),
index-head weights U(0,1), sink N(0,1).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0


def e4m3_bytes(x: np.ndarray, scale: float) -> np.ndarray:
    """Store x / scale as OCP E4M3FN bytes (torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / np.float32(scale))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store x as BF16 bit patterns (torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_pack(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Store x [..., D] (D a multiple of 32) in the OCP MX FP4 format:
    E2M1 codes two per byte (element 2j in the low nibble) [..., D/2] and
    one E8M0 scale byte per block of 32 [..., D/32].  The block scale is
    2^(floor(log2 amax) - 2) (the MX rule: the largest E2M1 exponent is 2);
    elements are rounded to the nearest E2M1 value, ties to the even code,
    and saturate at 6."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % 32 == 0
    blk = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127).clip(-127, 127)
    y = blk / np.ldexp(1.0, e)[..., None]
    a = np.minimum(np.abs(y), 6.0)
    hi = np.searchsorted(_E2M1_GRID, a, side="left").clip(0, 7)
    lo = (hi - 1).clip(0, 7)
    dlo = a - _E2M1_GRID[lo]
    dhi = _E2M1_GRID[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = code | (((y < 0) & (code > 0)).astype(np.int64) << 3)
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def per_tensor_scale(x: np.ndarray, unit: bool) -> float:
    if unit:
        return 1.0
    amax = float(np.abs(x).max())
    return amax / E4M3_MAX if amax > 0 else 1.0


@dataclass
class Spec:
    """Everything that fixes one synthetic workload."""
    name: str
    kind: str                      # "decode" or "prefill"
    ctx_lens: list                 # context length per sequence (tokens)
    H: int = 128
    D_nope: int = 448
    D_rope: int = 64
    H_I: int = 64
    D_I: int = 128
    k: int = 512
    W: int = 128
    m: int = 4
    page_size: int = 64
    shuffle_pages: bool = False
    unit_scale: bool = False       # values already on the E4M3 grid (scale 1)
    with_indexer: bool = True      # False for the HCA layer (no indexer inputs)
    mxfp4: bool = False            # also store the indexer q/k in MXFP4 (same draws)
    keep_float: bool = False       # also keep the indexer q/k draws unquantised (float32)
    # plant this many indexer keys per sequence along its query's summed
    # index-head direction (gains U(plant_gain)), among the entries before the
    # newest stored one: a workload whose unquantised top-k stands apart
    plant_topk: int = 0
    plant_gain: tuple = (1.0, 2.0)
    # prefill only: number of query tokens at the end of the single sequence
    T_prefill: int = 0
    # decode: position of each sequence's query (default ctx_len - 1)
    q_pos: Optional[list] = None

    @property
    def D(self) -> int:
        return self.D_nope + self.D_rope

    @property
    def sigma(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


@dataclass
class Workload:
    spec: Spec
    seed: int
    B: int
    T: int
    # indexer
    q_idx: Optional[np.ndarray] = None     # u8 [T][H_I][D_I]
    q_idx_scale: float = 1.0
    w: Optional[np.ndarray] = None         # f32 [T][H_I]
    k_idx: Optional[np.ndarray] = None     # u8 [P][ps][D_I]
    k_idx_scale: float = 1.0
    # the same indexer draws in MXFP4 (spec.mxfp4): E2M1 pairs + E8M0 scales
    q_idx4: Optional[np.ndarray] = None    # u8 [T][H_I][D_I/2]
    q_idx4_sc: Optional[np.ndarray] = None # u8 [T][H_I][D_I/32]
    k_idx4: Optional[np.ndarray] = None    # u8 [P][ps][D_I/2]
    k_idx4_sc: Optional[np.ndarray] = None # u8 [P][ps][D_I/32]
    # the unquantised indexer draws (spec.keep_float): q [T][H_I][D_I], and
    # the keys in entry order [sum n_comp][D_I], sequence b's from entry_offset[b]
    q_idx_f32: Optional[np.ndarray] = None
    k_idx_f32: Optional[np.ndarray] = None
    entry_offset: Optional[np.ndarray] = None
    # compressed latent cache
    lat_nope: np.ndarray = None            # u8 [P][ps][D_nope]
    lat_rope: np.ndarray = None            # u16 [P][ps][D_rope]
    lat_scale: float = 1.0
    page_table: np.ndarray = None          # i32 [B][max_pages]
    n_comp: np.ndarray = None              # i32 [B]
    # queries
    q_pos: np.ndarray = None               # i32 [T]
    q_seq: np.ndarray = None               # i32 [T]
    q: np.ndarray = None                   # u16 [T][H][D] (bf16 bits)
    sink: np.ndarray = None                # f32 [H]
    # decode SWA ring
    swa_nope: np.ndarray = None            # u8 [B][W][D_nope] or [L][D_nope] (prefill)
    swa_rope: np.ndarray = None            # u16 [B][W][D_rope] or [L][D_rope]
    swa_scale: float = 1.0
    swa_pos: Optional[np.ndarray] = None   # i32 [B][W] (decode ring), -1 = empty
    swa_first_pos: int = 0                 # prefill linear buffer start position
    swa_len: int = 0                       # prefill linear buffer length

    @property
    def num_pages(self) -> int:
        return self.lat_nope.shape[0]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


def _draw_normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _plant_keys(ki, q_draws, s, n_comp, seed):
    """Adds gain x dir_b to plant_topk keys of each decode sequence b, where
    dir_b is the sum of query b's index-head vectors scaled to norm
    sqrt(D_I), and the gains are U(plant_gain).  The keys are drawn among the
    entries before the sequence's newest stored one (those a query at the
    sequence's last position sees).  A generator of its own (seed + 7919), so
    every other array keeps its draws."""
    if s.kind != "decode":
        raise ValueError("planted keys are defined for decode batches")
    prng = np.random.default_rng(seed + 7919)
    off = 0
    for b in range(len(n_comp)):
        n = int(n_comp[b])
        if s.plant_topk > n - 1:
            raise ValueError("more planted keys than entries")
        d = q_draws[b].astype(np.float64).sum(axis=0)
        d *= np.sqrt(s.D_I) / np.linalg.norm(d)
        rows = prng.choice(n - 1, size=s.plant_topk, replace=False)
        gains = prng.uniform(s.plant_gain[0], s.plant_gain[1], size=s.plant_topk)
        ki[off + rows] += (gains[:, None] * d[None, :]).astype(np.float32)
        off += n


def generate(spec: Spec, seed: int) -> Workload:
    """Draw one workload.  Draw order (PCG64 via numpy.default_rng(seed)):
    q_idx, w, k_idx, latents, SWA rows, q, sink, page permutation."""
    rng = np.random.default_rng(seed)
    s = spec
    ps = s.page_size
    if s.kind == "decode":
        B = len(s.ctx_lens)
        T = B
        ctx = np.asarray(s.ctx_lens, dtype=np.int64)
        q_pos = (np.asarray(s.q_pos, dtype=np.int64) if s.q_pos is not None else ctx - 1)
        q_seq = np.arange(B)
    elif s.kind == "prefill":
        assert len(s.ctx_lens) == 1 and s.T_prefill > 0
        B = 1
        T = s.T_prefill
        L = int(s.ctx_lens[0])
        ctx = np.asarray([L], dtype=np.int64)
        q_pos = np.arange(L - T, L, dtype=np.int64)
        q_seq = np.zeros(T, dtype=np.int64)
    else:
        raise ValueError(s.kind)
    n_comp = (ctx // s.m).astype(np.int64)
    pages_per_seq = (n_comp + ps - 1) // ps
    max_pages = int(max(1, pages_per_seq.max()))
    P = int(pages_per_seq.sum())
    n_entries = int(n_comp.sum())

    wl = Workload(spec=s, seed=seed, B=B, T=T)
    wl.q_pos = q_pos.astype(np.int32)
    wl.q_seq = q_seq.astype(np.int32)
    wl.n_comp = n_comp.astype(np.int32)

    # ---- indexer queries, weights and keys
    if s.with_indexer:
        qi = _draw_normal(rng, (T, s.H_I, s.D_I))
        wl.q_idx_scale = per_tensor_scale(qi, s.unit_scale)
        wl.q_idx = e4m3_bytes(qi, wl.q_idx_scale)
        if s.mxfp4:
            wl.q_idx4, wl.q_idx4_sc = mxfp4_pack(qi)
        if s.keep_float:
            wl.q_idx_f32 = qi
        q_draws = qi
        del qi
        wl.w = rng.random((T, s.H_I), dtype=np.float32)
        ki = _draw_normal(rng, (n_entries, s.D_I))
        if s.plant_topk:
            _plant_keys(ki, q_draws, s, n_comp, seed)
        del q_draws
        wl.k_idx_scale = per_tensor_scale(ki, s.unit_scale)
        ki_b = e4m3_bytes(ki, wl.k_idx_scale)
        if s.mxfp4:
            ki4, ki4_sc = mxfp4_pack(ki)
        if s.keep_float:
            wl.k_idx_f32 = ki
            wl.entry_offset = np.concatenate([[0], np.cumsum(n_comp)[:-1]]).astype(np.int64)
        del ki
    # ---- compressed latents
    lat = _draw_normal(rng, (n_entries, s.D))
    wl.lat_scale = per_tensor_scale(lat[:, :s.D_nope], s.unit_scale)
    lat_n = e4m3_bytes(lat[:, :s.D_nope], wl.lat_scale)
    lat_r = bf16_bits(lat[:, s.D_nope:])
    del lat
    # ---- SWA rows
    if s.kind == "decode":
        sw = _draw_normal(rng, (B, s.W, s.D))
        wl.swa_scale = per_tensor_scale(sw[..., :s.D_nope], s.unit_scale)
        wl.swa_nope = e4m3_bytes(sw[..., :s.D_nope], wl.swa_scale)
        wl.swa_rope = bf16_bits(sw[..., s.D_nope:])
        # ring slot of position p is p % W; slots outside [0, pos] stay empty
        swa_pos = np.full((B, s.W), -1, dtype=np.int32)
        for b in range(B):
            for p in range(max(0, int(q_pos[b]) - s.W + 1), int(q_pos[b]) + 1):
                swa_pos[b, p % s.W] = p
        wl.swa_pos = swa_pos
    else:
        first = max(0, int(q_pos[0]) - s.W + 1)
        last = int(q_pos[-1])
        Lb = last - first + 1
        sw = _draw_normal(rng, (Lb, s.D))
        wl.swa_scale = per_tensor_scale(sw[:, :s.D_nope], s.unit_scale)
        wl.swa_nope = e4m3_bytes(sw[:, :s.D_nope], wl.swa_scale)
        wl.swa_rope = bf16_bits(sw[:, s.D_nope:])
        wl.swa_first_pos = first
        wl.swa_len = Lb
    del sw
    # ---- queries and sinks
    wl.q = bf16_bits(_draw_normal(rng, (T, s.H, s.D)))
    wl.sink = _draw_normal(rng, (s.H,)).astype(np.float32)
    # ---- paging
    perm = rng.permutation(P) if s.shuffle_pages else np.arange(P)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    wl.lat_nope = np.zeros((P, ps, s.D_nope), dtype=np.uint8)
    wl.lat_rope = np.zeros((P, ps, s.D_rope), dtype=np.uint16)
    if s.with_indexer:
        wl.k_idx = np.zeros((P, ps, s.D_I), dtype=np.uint8)
        if s.mxfp4:
            wl.k_idx4 = np.zeros((P, ps, s.D_I // 2), dtype=np.uint8)
            wl.k_idx4_sc = np.zeros((P, ps, s.D_I // 32), dtype=np.uint8)
    logical = 0
    e0 = 0
    for b in range(B):
        for j in range(int(pages_per_seq[b])):
            phys = int(perm[logical])
            logical += 1
            page_table[b, j] = phys
            lo = e0 + j * ps
            hi = min(e0 + int(n_comp[b]), lo + ps)
            cnt = hi - lo
            wl.lat_nope[phys, :cnt] = lat_n[lo:hi]
            wl.lat_rope[phys, :cnt] = lat_r[lo:hi]
            if s.with_indexer:
                wl.k_idx[phys, :cnt] = ki_b[lo:hi]
                if s.mxfp4:
                    wl.k_idx4[phys, :cnt] = ki4[lo:hi]
                    wl.k_idx4_sc[phys, :cnt] = ki4_sc[lo:hi]
        e0 += int(n_comp[b])
    wl.page_table = page_table
    return wl


# ---------------------------------------------------------------------------
# The five configurations of the CSA workload (numbered 0..4), plus the HCA
# layer that configuration 3 pairs with its CSA layer.
# ---------------------------------------------------------------------------
BASE_SEED = 20260


def spec_for(name: str) -> Spec:
    if name == "c0":
        # tiny decode: pos 255, 8 heads x (48 FP8 + 16 BF16), 64 entries,
        # indexer 4 x 32, top-k 16, window 32, values on the E4M3 grid
        return Spec(name="c0", kind="decode", ctx_lens=[256], H=8, D_nope=48, D_rope=16,
                    H_I=4, D_I=32, k=16, W=32, m=4, unit_scale=True)
    if name == "c1":
        return Spec(name="c1", kind="decode", ctx_lens=[8192])
    if name == "c2":
        # 64 sequences; context lengths uniform over multiples of 4 in [4096, 32768]
        rng = np.random.default_rng(BASE_SEED + 1002)
        lens = (rng.integers(4096 // 4, 32768 // 4 + 1, size=64) * 4).tolist()
        return Spec(name="c2", kind="decode", ctx_lens=lens, shuffle_pages=True)
    if name == "c3_csa":
        return Spec(name="c3_csa", kind="decode", ctx_lens=[524288] * 4)
    if name == "c3_hca":
        return Spec(name="c3_hca", kind="decode", ctx_lens=[524288] * 4, m=128,
                    with_indexer=False)
    if name == "c4":
        return Spec(name="c4", kind="prefill", ctx_lens=[65536], T_prefill=2048)
    raise KeyError(name)


CONFIG_NAMES = ["c0", "c1", "c2", "c3_csa", "c3_hca", "c4"]
_CONFIG_INDEX = {"c0": 0, "c1": 1, "c2": 2, "c3_csa": 3, "c3_hca": 3, "c4": 4}


def make_config(name: str, seed: Optional[int] = None, mxfp4: bool = False) -> Workload:
    """One of the configurations; mxfp4 adds the MXFP4 copy of the indexer
    inputs (from the same draws, so every other array is unchanged)."""
    if seed is None:
        seed = BASE_SEED + _CONFIG_INDEX[name] + (100 if name == "c3_hca" else 0)
    spec = spec_for(name)
    if mxfp4:
        spec = dataclasses.replace(spec, mxfp4=True)
    return generate(spec, seed)


def small_spec(name: str = "small", **kw) -> Spec:
    """Production head/latent shapes at context sizes the oracle finishes in
    seconds (several KV tiles, ragged tails)."""
    base = dict(name=name, kind="decode", ctx_lens=[1500, 2400, 620])
    base.update(kw)
    return Spec(**base)


def with_ring_permuted(wl: Workload, seed: int) -> Workload:
    """Copy of a decode workload whose ring storage order is shuffled per
    sequence (membership is by stored position, so results must not change)."""
    out = dataclasses.replace(wl)
    rng = np.random.default_rng(seed)
    nope = wl.swa_nope.copy()
    rope = wl.swa_rope.copy()
    pos = wl.swa_pos.copy()
    for b in range(wl.B):
        p = rng.permutation(wl.spec.W)
        nope[b] = wl.swa_nope[b, p]
        rope[b] = wl.swa_rope[b, p]
        pos[b] = wl.swa_pos[b, p]
    out.swa_nope, out.swa_rope, out.swa_pos = nope, rope, pos
    return out


def with_fp8_scale(wl: Workload, source: str, factor: float) -> Workload:
    """Copy of a workload whose latent ("lat") or window ("swa") nope plane is
    stored with its per-tensor FP8 scale multiplied by `factor`: the stored
    values (codes x scale) are re-encoded to E4M3 under the new scale with
    torch's RNE cast (saturating), so the real values stay close while the
    two key sources' scales differ.  Encoding only."""
    out = dataclasses.replace(wl)
    codes = getattr(wl, f"{source}_nope")
    scale = float(getattr(wl, f"{source}_scale"))
    vals = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32) * scale
    new_scale = scale * float(factor)
    new = (vals / new_scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    setattr(out, f"{source}_nope", new)
    setattr(out, f"{source}_scale", new_scale)
    return out
