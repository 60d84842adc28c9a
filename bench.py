"""Benchmark of the CSA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
csa_index_scores -> csa_topk -> csa_decode_attn (or csa_prefill_attn).
Default workload: batched CSA decode (64 sequences, 4096..32768-token
contexts, paged FP8 cache with a shuffled page table, 128 heads x 512-d
latent, indexer 64 x 128, top-k 512, window 128).

Output: one JSON line with the throughput, a roofline object for the
dominant kernel (algorithmic bytes or FLOPs per launch / the kernel's
average duration measured with HIP events on its stream), and the FP64 CPU
oracle timed on a bounded sample of the same workload.  Inputs are rotated
over several device copies so that every step reads HBM, not the 256 MB
Infinity Cache.

Timed regions: the throughput comes from K whole steps back to back with no
event between the kernels (an event record between two kernels adds a few
microseconds of idle GPU); the per-kernel durations come from a second
region that launches each stage K times back to back between two events; a
third region brackets every step with events for the spread of step times
(median, p10, p90).  The roofline fractions are given against MI355X's
published peaks and against peaks measured on the same GPU by a plain copy
kernel and an FP8 MFMA loop (libcsa_peak.so).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BASE_METRIC = "CSA decode queries/s (indexer+top-k+FMHA); % of HBM & FP8-MFMA roofline"
PREFILL_METRIC = "CSA prefill tokens/s (indexer+top-k+FMHA); % of HBM & FP8-MFMA roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

WORKLOADS = {
    "c1": "single-sequence CSA decode: 1 query, 8192-token context (2048 entries, 2047 visible), 128 heads x "
          "(448 FP8 + 64 BF16), indexer 64x128 FP8, top-k 512, window 128",
    "c2": "batched CSA decode: 64 sequences, contexts uniform over multiples of 4 in [4096, 32768], page 64 "
          "with shuffled page table, 128 heads x (448 FP8 + 64 BF16), indexer 64x128 FP8, top-k 512, window 128",
    "c3_csa": "long-context CSA decode: 4 sequences x 524288 tokens (131072 entries), top-k 512, window 128",
    "c3_hca": "long-context HCA decode: 4 sequences x 524288 tokens, m'=128 (4096 entries, all visible ones "
              "attended), window 128, no indexer",
    "c4": "CSA prefill chunk: 2048 queries at positions 63488..65535 of a 65536-token context (16384 entries), "
          "top-k 512, window 128",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the oracle's CPU time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of the inputs (0 = enough that one pass over them touches >= 1 GiB)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / MFMA peaks")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured graph (csa_graph_*) instead of issuing its calls")
    ap.add_argument("--mxfp4", action="store_true",
                    help="indexer on MXFP4 inputs (csa_index_scores_mxfp4) instead of E4M3")
    ap.add_argument("--fused-topk", action="store_true",
                    help="steps 1+2 as one call (csa_index_topk: the scores stay on chip)")
    ap.add_argument("--topk-in-attn", action="store_true",
                    help="steps 2-4 as one call (csa_topk_decode_attn: the attention kernel selects the top-k; "
                         "decode rows up to 8192 entries)")
    ap.add_argument("--inv-rope-theta", type=float, default=0.0,
                    help="base of the inverse-RoPE epilogue on the output's rope dims (0 = off)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to calibrate HBM byte counters")
    return ap.parse_args()


def calibrate_copy(mib):
    """The plain copy probe of libcsa_peak.so over a buffer of known size,
    launched 5 times: its FETCH_SIZE / WRITE_SIZE counter readings give the
    factor between those counters and the bytes a kernel moves."""
    import ctypes
    import torch
    from sparse_compressed_attention_amd import build as csa_build
    lib = ctypes.CDLL(csa_build.PEAK_LIB_PATH)
    lib.csa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    nbytes = mib * (1 << 20)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(5):
        if lib.csa_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, 256 * 16, st):
            raise RuntimeError("csa_peak_copy failed")
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": nbytes, "calibrate_copy_bytes_written": nbytes}), flush=True)


# --------------------------------------------------------------- measured peaks
def measured_peaks(torch, stream, reps=5):
    """Copy bandwidth and FP8 MFMA rate measured on this GPU (median of
    `reps` timed launches each, after a warm-up launch), with the probes of
    libcsa_peak.so: a 16-byte-load grid-stride copy of 2 GiB (1 GiB read +
    1 GiB written, far beyond the 256 MB Infinity Cache) and a loop of
    independent v_mfma_scale_f32_16x16x128_f8f6f4 on every SIMD."""
    import ctypes
    import numpy as np
    from sparse_compressed_attention_amd import build as csa_build
    lib = ctypes.CDLL(csa_build.PEAK_LIB_PATH)
    lib.csa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.csa_peak_mfma_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.csa_peak_mfma_chains.restype = ctypes.c_int
    st = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)

    def copy(blocks):
        if lib.csa_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, blocks, st):
            raise RuntimeError("csa_peak_copy failed")
    # the fastest of three grid sizes (fewer, longer-lived workgroups leave
    # part of the bandwidth unused on this part)
    t_copy, blocks = min((timed(lambda b=b: copy(b)), b) for b in (256 * 16, 256 * 64, 256 * 256))
    if not torch.equal(src[:1024], dst[:1024]):
        raise RuntimeError("copy probe produced wrong bytes")
    del src, dst
    mblocks, iters = 256 * 8, 2048
    out = torch.empty(mblocks * 256, dtype=torch.float32, device="cuda:0")

    def mfma():
        if lib.csa_peak_mfma_fp8(ctypes.c_void_p(out.data_ptr()), iters, mblocks, st):
            raise RuntimeError("csa_peak_mfma_fp8 failed")
    t_mfma = timed(mfma)
    flops = mblocks * 4 * iters * lib.csa_peak_mfma_chains() * 2 * 16 * 16 * 128
    return dict(copy_GBps=round(2 * nbytes / t_copy / 1e9, 1), fp8_mfma_TFLOPs=round(flops / t_mfma / 1e12, 1),
                how=f"copy: {blocks} x 256 threads over 1 GiB -> 1 GiB (fastest of 4096, 16384, 65536 workgroups), "
                    f"median of {reps}; MFMA: {mblocks} x 4 "
                    f"waves x {iters} x {lib.csa_peak_mfma_chains()} independent 16x16x128 FP8, median of {reps}")


def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count(), len(os.sched_getaffinity(0))


# --------------------------------------------------------------- accounting
def accounting(wl, mxfp4=False):
    """Algorithmic bytes and FLOPs per launch of each step: only what the
    method must move (visible index keys once, q_idx, w, scores written and
    read back, selected + window latent rows once per query, q and o).  With
    the MXFP4 indexer an index row is D_I / 2 code bytes + D_I / 32 scale
    bytes instead of D_I E4M3 bytes."""
    import numpy as np
    s = wl.spec
    T = wl.T
    pos = wl.q_pos.astype(np.int64)
    seq = wl.q_seq.astype(np.int64)
    nv = np.minimum(pos // s.m, wl.n_comp[seq].astype(np.int64))
    n_sel = np.minimum(nv, s.k) if wl.q_idx is not None else nv
    if s.kind == "decode":
        lo = np.maximum(pos - s.W + 1, 0)
        n_win = np.array([int(((wl.swa_pos[b] >= lo[t]) & (wl.swa_pos[b] <= pos[t])).sum())
                          for t, b in enumerate(seq)])
    else:
        lo = np.maximum(np.maximum(pos - s.W + 1, 0), wl.swa_first_pos)
        hi = np.minimum(pos, wl.swa_first_pos + wl.swa_len - 1)
        n_win = np.maximum(hi - lo + 1, 0)
    row = s.D_nope + 2 * s.D_rope
    acc = {}
    if wl.q_idx is not None:
        idx_row = s.D_I // 2 + s.D_I // 32 if mxfp4 else s.D_I
        if s.kind == "decode":
            key_bytes = int(nv.sum()) * idx_row
        else:
            key_bytes = int(nv.max()) * idx_row   # one sequence: every key is read once per chunk
        acc["index_scores"] = dict(
            bytes=key_bytes + T * s.H_I * (idx_row + 4) + int(nv.sum()) * 4 + T * 4,
            flops=2.0 * s.H_I * s.D_I * float(nv.sum()))
        acc["topk"] = dict(bytes=int(nv.sum()) * 4 + T * s.k * 4 + T * 4, flops=0.0)
        # fused steps 1+2: the scores stay on chip
        acc["index_topk"] = dict(bytes=key_bytes + T * s.H_I * (idx_row + 4) + T * s.k * 4 + T * 4,
                                 flops=acc["index_scores"]["flops"])
    keys = n_sel + n_win
    if s.kind == "decode":
        lat_bytes = int(keys.sum()) * row
    else:
        lat_bytes = int(nv.max()) * row + wl.swa_len * row   # union of rows, counted once
    attn = "decode_attn" if s.kind == "decode" else "prefill_attn"
    acc[attn] = dict(
        bytes=lat_bytes + T * s.H * s.D * 2 * 2 + T * s.H * 4 + (T * s.k * 4 if wl.q_idx is not None else 0),
        flops=4.0 * s.H * s.D * float(keys.sum()))
    if wl.q_idx is not None and s.kind == "decode":
        # steps 2-4 in one call: the scores are read instead of the top-k
        # list, and the list is written once
        acc["topk_decode_attn"] = dict(bytes=acc[attn]["bytes"] + int(nv.sum()) * 4 + T * 4,
                                       flops=acc[attn]["flops"])
    return acc


def roofline_entry(name, a, ms, peaks=None):
    """Roofline of one kernel: algorithmic bytes (or FLOPs) per launch over
    its average duration, against MI355X's published peak (`frac`) and, when
    given, the peak measured on this GPU (`frac_measured`)."""
    sec = ms * 1e-3
    intensity = a["flops"] / max(a["bytes"], 1)
    gbs = a["bytes"] / sec / 1e9
    tfl = a["flops"] / sec / 1e12
    if a["flops"] > 0 and intensity >= RIDGE:
        e = dict(bound="mfma", achieved=round(tfl, 2), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                 frac=round(tfl / PEAK_FP8_TFLOPS, 4))
        if peaks:
            e["peak_measured"] = peaks["fp8_mfma_TFLOPs"]
            e["frac_measured"] = round(tfl / peaks["fp8_mfma_TFLOPs"], 4)
        return e
    e = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4))
    if peaks:
        e["peak_measured"] = peaks["copy_GBps"]
        e["frac_measured"] = round(gbs / peaks["copy_GBps"], 4)
    if a["flops"] > 0:
        e["mfma_frac"] = round(tfl / PEAK_FP8_TFLOPS, 4)
    return e


def kernel_source_sha(name):
    src = {"index_scores": "index_scores.hip", "topk": "topk.hip", "decode_attn": "attn.hip",
           "prefill_attn": "attn.hip", "index_topk": "index_scores.hip", "topk_decode_attn": "attn.hip"}[name]
    h = hashlib.sha256()
    for f in (src, "csa_device.h", "csa_internal.h", "topk_select.h"):
        with open(os.path.join(ROOT, "sparse_compressed_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, name):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(workload, {}).get(name)
        if ent and ent.get("source_sha") == kernel_source_sha(name):
            return int(ent["hbm_bytes_per_launch"])
    except (ValueError, KeyError, OSError):
        return None
    return None


# --------------------------------------------------------------- CPU oracle leg
def cpu_baseline(wl, gpu_res, seconds, is_prefill, inv_rope_theta=0.0):
    """The FP64 oracle timed on this host over a bounded sample of the
    workload's queries (random order; stops once `seconds` have elapsed).
    Only the oracle's own path is inside the clock; its results then check
    the GPU's outputs, outside the clock."""
    import numpy as np
    import oracle
    from tests import parity as P
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - informational only
        blas_threads = None
    model, n_cpu, n_aff = cpu_info()
    order = list(range(wl.T))
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    # passes over the shuffled queries until `seconds` have elapsed (small
    # workloads are repeated, so the rate comes from seconds of work); the
    # first pass's results are checked
    done = []
    n_runs = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= seconds:
        for t in order:
            if wl.q_idx is not None:
                res = oracle.run_decode_path(wl, queries=[t])
            else:
                res = oracle.run_attention(wl, None, queries=[t])
            if n_runs < len(order):
                done.append((t, res))
            n_runs += 1
            if time.perf_counter() - t0 > seconds:
                break
    el = time.perf_counter() - t0
    errs, overlap = [], []
    for t, res in done:
        if wl.q_idx is not None:
            o_ref, l_ref = P.reference_attention_on(wl, t, gpu_res["topk"][t])
            ref_set = set(int(i) for i in res["topk"][0] if i >= 0)
            got = set(int(i) for i in gpu_res["topk"][t] if i >= 0)
            overlap.append(len(ref_set & got) / max(1, len(ref_set)))
        else:
            o_ref, l_ref = res[0][0], res[1][0]
        if inv_rope_theta:
            o_ref = oracle.inverse_rope(o_ref, int(wl.q_pos[t]), wl.spec.D_nope, inv_rope_theta)
        errs.append(P.check_attention(gpu_res["o"][t], gpu_res["lse"][t], o_ref, l_ref))
    unit = "tokens/s" if is_prefill else "queries/s"
    cores = blas_threads or n_aff
    return dict(value=round(n_runs / el, 3), unit=unit, cores=int(cores), kind="oracle",
                cpu_model=model, cpu_count=n_cpu, affinity_cpus=n_aff, blas_threads=blas_threads,
                sample=f"{n_runs} query runs ({len(done)} distinct of {wl.T}, random order, seed 0, repeated "
                       f"until {seconds:g} s) through the FP64 NumPy oracle (indexer, top-k, attention), {el:.1f} s "
                       f"on {cores} threads; outside the clock the first pass's outputs checked the GPU's: "
                       f"max|o-ref| {max(e[0] for e in errs):.2e}, min per-head cos "
                       f"{min(e[1] for e in errs):.6f}"
                       + (f"; GPU top-k vs the oracle's (E4M3-input) top-k: mean overlap {np.mean(overlap):.4f}"
                          if overlap else ""))


# --------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the CSA path here is a single-GPU build with no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import csa_inputs as ci
    import sparse_compressed_attention_amd as csa
    from csa_inputs.device import to_device, make_path

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    csa.load_library()
    torch.cuda.set_device(0)
    dev = "cuda:0"
    name = args.workload
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    wl = ci.make_config(name, mxfp4=args.mxfp4)
    acc = accounting(wl, args.mxfp4)
    d0 = to_device(wl, dev)
    footprint = sum(t.numel() * t.element_size() for t in vars(d0).values() if isinstance(t, torch.Tensor))
    stage_keys = [k for k in ("index_scores", "topk", "decode_attn", "prefill_attn") if k in acc]
    touched = sum(acc[k]["bytes"] for k in stage_keys)
    # enough copies that one pass over them touches >= 1 GiB of algorithmic
    # bytes (4x the 256 MB Infinity Cache), within 64 GiB of device memory
    copies = args.copies or int(max(2, min(1024, math.ceil((1 << 30) / max(touched, 1)),
                                           (64 << 30) // max(footprint, 1))))
    theta = args.inv_rope_theta
    fp4 = args.mxfp4
    opts = dict(inv_rope_theta=theta, mxfp4=fp4, fused_topk=args.fused_topk, topk_in_attn=args.topk_in_attn)
    paths = [make_path(d0, **opts)] + [make_path(to_device(wl, dev), **opts) for _ in range(copies - 1)]
    del d0
    stages = paths[0].stage_names
    stream = torch.cuda.current_stream()
    st = csa._stream(stream)
    print(f"[bench] {copies} input copies of {footprint / 2**20:.1f} MiB ({touched / 2**20:.1f} MiB touched per "
          f"step); stages {stages}", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        paths[i % copies].run(st)
    torch.cuda.synchronize()
    graphs = [csa.StepGraph(p) for p in paths] if args.graph else None
    if graphs:
        for i in range(args.warmup):
            graphs[i % copies].replay(st)
        torch.cuda.synchronize()

    K = args.steps
    # Timed region 1, the headline: K whole steps back to back, nothing else
    # on the stream (an event record between two kernels adds a gap of a few
    # microseconds on this GPU, so per-kernel events stay out of this loop).
    e_begin = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_begin.record(stream)
    if graphs:
        for i in range(K):
            graphs[i % copies].replay(st)
    else:
        for i in range(K):
            paths[i % copies].run(st)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step = e_begin.elapsed_time(e_end) / K
    # Timed region 2, per-kernel durations: each stage launched K times back
    # to back (over the same rotating input copies, whose earlier stages ran
    # above) between two events on the launch stream.
    per_stage = []
    for j in range(len(stages)):
        ea = torch.cuda.Event(enable_timing=True)
        eb = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record(stream)
        for i in range(K):
            paths[i % copies].run_stage(j, st)
        eb.record(stream)
        torch.cuda.synchronize()
        per_stage.append(ea.elapsed_time(eb) / K)
    # Timed region 3, spread of step times: an event before every step (each
    # interval also holds one event record's gap)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    for i in range(K):
        evs[i].record(stream)
        if graphs:
            graphs[i % copies].replay(st)
        else:
            paths[i % copies].run(st)
    evs[K].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    spread = dict(p10=round(float(np.percentile(step_ms, 10)), 5), median=round(float(np.median(step_ms)), 5),
                  p90=round(float(np.percentile(step_ms, 90)), 5), how="per-step HIP events, one event gap each")
    ms_per_step = wall * 1e3 / K
    latency = None
    if graphs:
        # Single-step latency, the quantity graph replay is meant to cut: one
        # step issued and waited for, as when every decode step depends on
        # the previous one's output.  Median over 50 steps each way.
        def one_step(fn):
            ts = []
            for i in range(50):
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                fn(i % copies)
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t1) * 1e6)
            return round(float(np.median(ts)), 1)
        latency = dict(eager_us=one_step(lambda i: paths[i].run(st)),
                       graph_us=one_step(lambda i: graphs[i].replay(st)))
    n_items = wl.T
    value = n_items / (ms_per_step * 1e-3)

    peaks = None if args.no_peaks else measured_peaks(torch, stream)
    kernels = {}
    for nm, ms in zip(stages, per_stage):
        a = acc[nm]
        kernels[nm] = dict(ms=round(ms, 5), bytes=int(a["bytes"]), flops=a["flops"],
                           GBps=round(a["bytes"] / (ms * 1e-3) / 1e9, 1),
                           TFLOPs=round(a["flops"] / (ms * 1e-3) / 1e12, 2))
    traffic_key = name + ("_mxfp4" if fp4 else "")
    dom = max(range(len(stages)), key=lambda j: per_stage[j])
    dom_name = stages[dom]
    roof = roofline_entry(dom_name, acc[dom_name], per_stage[dom], peaks)
    roof["kernel"] = dom_name
    roof["traffic"] = measured_traffic(traffic_key, dom_name)
    # the two kernels the metric names: the indexer scan and the attention
    by_kernel = {}
    for role, nm in (("indexer", "index_scores"), ("indexer", "index_topk"), ("fmha", "decode_attn"),
                     ("fmha", "prefill_attn"), ("fmha", "topk_decode_attn")):
        if nm in kernels:
            e = roofline_entry(nm, acc[nm], kernels[nm]["ms"], peaks)
            e["kernel"] = nm
            e["traffic"] = measured_traffic(traffic_key, nm)
            by_kernel[role] = e

    out = dict(
        metric=PREFILL_METRIC if wl.spec.kind == "prefill" else BASE_METRIC,
        value=round(value, 2),
        unit="tokens/s" if wl.spec.kind == "prefill" else "queries/s",
        n_gpus=1, steps=K, warmup=args.warmup, ms_per_step=round(ms_per_step, 5),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="fp8", data="synthetic",
        config=dict(workload=f"{name}: {WORKLOADS[name]}", queries_per_step=n_items, input_copies=copies,
                    gpu_ms_per_step=round(gpu_step, 5), launch="graph replay" if graphs else "eager calls",
                    inv_rope_theta=theta or None, indexer="MXFP4" if fp4 else "E4M3",
                    fused_topk=bool(getattr(paths[0], "fused_topk", False)),
                    topk_in_attn=bool(getattr(paths[0], "topk_in_attn", False)),
                    synced_step_latency=latency, step_ms_spread=spread),
        roofline=roof,
        roofline_kernels=by_kernel,
        measured_peaks=peaks,
        kernels=kernels,
    )
    if not args.no_cpu_baseline:
        last = paths[(K - 1) % copies]
        res = dict(o=last.out.float().cpu().numpy().astype(np.float64),
                   lse=last.lse.cpu().numpy().astype(np.float64))
        if getattr(last, "topk", None) is not None:
            res["topk"] = last.topk.cpu().numpy()
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, res, args.cpu_seconds, wl.spec.kind == "prefill", theta)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
