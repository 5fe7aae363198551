#!/usr/bin/env python3
"""Benchmark of one chunk step of paged top-K chunk attention on one MI355X.

A step is the whole hot path of the OOMB page's method (technical summary,
section 2) for one attention layer and one chunk: representative vectors of the
chunk's new pages, chunk-mean-query page scores and top-K per kv-head, the fused
forward over the selected pages plus the causal chunk, and the fused backward
that reuses the selection and adds dK/dV in place into the paged fp32 gradient
pools.  Inputs are seeded synthetic tensors of the Qwen2.5-7B attention shape
(28 query heads, 4 kv heads, head dim 128, 128-token pages), resident in HBM
before the timed region; the rep vectors of the prior context are built once,
untimed.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sparse-256k]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk attn fwd+bwd tokens/s and MFMA util, Qwen2.5-7B shape, 256K ctx top-K"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def kernel_work(p, name):
    """Algorithmic work of one launch: (bound, amount, unit).  Attention flops
    count only visible (query-head row, key) pairs: forward 4*D per pair (QK^T,
    PV), backward 10*D per pair (QK^T, dO V^T, dV, dK, dQ).  The key-major
    dK/dV kernel is credited S, dP, dV, dK (8*D); the query-major dQ kernel is
    credited dQ only (2*D), its S and dP being recomputation."""
    pairs = p.pairs()
    eb = 2 if p.dtype == "bf16" else 4
    if name == "fwd_kernel":
        return "mfma", 4.0 * p.d * pairs, "flop"
    if name == "dkdv_kernel":
        return "mfma", 8.0 * p.d * pairs, "flop"
    if name == "dq_kernel":
        return "mfma", 2.0 * p.d * pairs, "flop"
    if name == "rep_update_kernel":     # the chunk's pages: read ps*D keys, write D floats, per (page, head)
        return "hbm", p.chunk_pages * p.hkv * (p.ps * p.d * eb + p.d * 4), "byte"
    if name == "qmean_partial_kernel":  # read Q
        return "hbm", p.c * p.hq * p.d * eb, "byte"
    if name == "scores_kernel":         # read the rep rows of the N prior pages, write N*Hkv scores
        return "hbm", p.n * p.hkv * p.d * 4 + p.n * p.hkv * 4, "byte"
    if name == "dt_kernel":             # read O and dO, write Dt
        return "hbm", 2 * p.c * p.hq * p.d * eb + p.c * p.hq * 4, "byte"
    return "hbm", 0.0, "byte"


class HipEvents:
    """hipEvent_t handles made and read through the process's HIP runtime."""

    def __init__(self, runtime_path, n):
        self.rt = ctypes.CDLL(runtime_path)
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            self._ok(self.rt.hipEventCreate(ctypes.byref(ev)), "hipEventCreate")
            self.handles[i] = ev.value

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with hipError {rc}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        self._ok(self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[a]),
                                             ctypes.c_void_p(self.handles[b])), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        for h in self.handles:
            if h:
                self.rt.hipEventDestroy(ctypes.c_void_p(h))


def host_cpu():
    """CPU model and logical CPU counts of this host (the oracle's machine)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "host_logical_cpus": os.cpu_count()}


def cpu_baseline(p, seed, x, tokens):
    """The fp64 oracle, as it stands, on the host cores: the selection over the
    whole chunk plus forward and backward of `tokens` chunk tokens (all heads),
    scaled to one chunk step."""
    import numpy as np
    import oracle
    oracle.build()
    ora = oracle.Oracle()
    pt = x["page_table"]
    t0 = time.perf_counter()
    rep = ora.rep(p, x["k_pool"], pt, 0, p.n)      # rep vectors of the prior context: setup, as on the GPU
    t_setup = time.perf_counter() - t0
    t0 = time.perf_counter()
    ora.rep(p, x["k_pool"], pt, p.n, p.chunk_pages)
    sel = ora.select(p, ora.scores(p, ora.qmean(p, x["q"]), rep))
    t_sel = time.perf_counter() - t0
    # rows of tokens spread over the chunk
    toks = np.linspace(0, p.c - 1, tokens).astype(np.int64)
    rows = (toks[:, None] * p.hq + np.arange(p.hq)[None, :]).reshape(-1)
    t0 = time.perf_counter()
    ora.bwd(p, x["q"], x["k_pool"], x["v_pool"], pt, sel, x["do"], rows=rows)
    t_rows = time.perf_counter() - t0
    t_step = t_sel + t_rows * (p.c / tokens)
    return {"value": p.c / t_step, "unit": "tokens/s", "cores": ora.threads(), **host_cpu(), "kind": "oracle",
            "sample": (f"rep vectors of the chunk's pages and selection over the full chunk ({t_sel:.2f} s) + "
                       f"forward and backward (dQ, and dK/dV of every key) of {tokens} of {p.c} chunk tokens "
                       f"x {p.hq} heads ({t_rows:.2f} s), "
                       f"scaled to {p.c} tokens; fp64"),
            "seconds": t_sel + t_rows, "rep_setup_seconds": t_setup}


def copy_calibration(mib):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings convert the attention kernels' readings to bytes."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)


def measured_peaks(P):
    """The part's sustained bf16 MFMA rate (the library's probe kernel: register
    operands, four independent chains per wave, 4 workgroups of 4 waves per CU)
    and its device-copy bandwidth (a 1 GiB copy, read plus write), each the best
    of five timed launches on the current stream."""
    import torch
    blocks, iters = 1024, 8192  # 4 workgroups per CU: the best of a sweep of grid sizes
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    P.oomb_probe_mfma_peak(blocks, iters // 8, out)  # warm-up
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        P.oomb_probe_mfma_peak(blocks, iters, out)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    if not bool((out == 4.0 * iters).all()):
        raise RuntimeError("MFMA probe returned a wrong check value")
    mfma_tflops = blocks * 4 * 4 * iters * 32768 / (best / 1e3) / 1e12
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return {"mfma_bf16_tflops": mfma_tflops, "hbm_copy_gbs": 2 * n / (best / 1e3) / 1e9}


SOURCE_DIRS = ("paged_sparse_attention_amd/csrc", "include")


def source_digest():
    """sha256 over the HIP sources and headers the library is built from."""
    import hashlib
    h = hashlib.sha256()
    for d in SOURCE_DIRS:
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            if name.endswith((".hip", ".h")):
                h.update(name.encode())
                with open(os.path.join(ROOT, d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the counter summary in profiles/,
    or None when there is none or the sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_digest():
        return None
    return t["traffic_bytes_per_launch"]


def _short_kernel_name(name):
    """liboomb kernel name out of a (mangled or demangled) symbol, else None."""
    import re
    m = re.search(r"oomb::(\w+)", name)
    if m:
        return m.group(1)
    m = re.search(r"4oomb(\d+)(\w+)", name)
    if m:
        return m.group(2)[: int(m.group(1))]
    return None


def _counter_per_dispatch(csv_dir, counter):
    """{kernel: [value per dispatch]} from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in sorted(per.items(), key=lambda kv: int(kv[0][1])):
        out.setdefault(name, []).append(v)
    return out


def record_traffic(dirs, kernel, workload, copy_mib, commands):
    """Write profiles/traffic_<kernel>_<workload>.json from four rocprofv3 runs
    (FETCH_SIZE and WRITE_SIZE of the step, then of the copy calibration) and
    print the per-kernel table.  Counter readings are KiB per dispatch; each is
    scaled by bytes moved / reading for the plain copy of copy_mib MiB."""
    fetch, write, cfetch, cwrite = (_counter_per_dispatch(d, c) for d, c in
                                    zip(dirs, ("FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE")))
    copy_bytes = copy_mib << 20

    def copy_reading(t):
        vals = [v for n, vs in t.items() if "copyBuffer" in n for v in vs]
        big = [v for v in vals if v * 1024 > copy_bytes / 8]  # the 1 GiB copies, not torch's fills
        return sum(big) / len(big)

    cf, cw = copy_reading(cfetch), copy_reading(cwrite)
    ff, fw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)

    def mean_by_kernel(t):
        out = {}
        for n, vs in t.items():
            k = _short_kernel_name(n)
            if k is None:
                continue
            if k == "rep_update_kernel":
                vs = vs[1:]  # the first call is the untimed set-up pass over the prior pages
            out[k] = sum(vs) / len(vs)
        return out

    mf, mw = mean_by_kernel(fetch), mean_by_kernel(write)
    rows = []
    for k in mf:
        rows.append((k, mf[k], mw.get(k, 0.0), mf[k] * 1024 * ff / 1e6, mw.get(k, 0.0) * 1024 * fw / 1e6))
    rec = {
        "kernel": kernel, "workload": workload, "source_sha256": source_digest(),
        "fetch_kib_per_dispatch": mf[kernel], "write_kib_per_dispatch": mw[kernel],
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_factor": ff, "write_factor": fw,
        "traffic_bytes_per_launch": (mf[kernel] * ff + mw[kernel] * fw) * 1024,
        "commands": commands,
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(f"wrote {path}: {rec['traffic_bytes_per_launch'] / 1e6:.1f} MB per launch; "
          f"factors fetch {ff:.4f}, write {fw:.4f}")
    print("| Kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (MB) | written (MB) |")
    print("|---|---|---|---|---|")
    for k, a, b, r, w in rows:
        print(f"| {k} | {a:.0f} | {b:.0f} | {r:.1f} | {w:.1f} |")


def _time_passes(args, fwd, bwd, hip_path):
    """W untimed, then K timed forward+backward passes on the current stream.
    Returns (ms per pass by the host clock, forward ms, backward ms by events)."""
    import torch
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    hip = HipEvents(hip_path, 3 * args.steps)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    t0 = time.perf_counter()
    for i in range(args.steps):
        hip.rt.hipEventRecord(ctypes.c_void_p(hip.handles[3 * i]), stream)
        fwd()
        hip.rt.hipEventRecord(ctypes.c_void_p(hip.handles[3 * i + 1]), stream)
        bwd()
        hip.rt.hipEventRecord(ctypes.c_void_p(hip.handles[3 * i + 2]), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    f = statistics.mean(hip.elapsed_ms(3 * i, 3 * i + 1) for i in range(args.steps))
    b = statistics.mean(hip.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(args.steps))
    return (t1 - t0) * 1e3 / args.steps, f, b


def layer_bench(args):
    """A Qwen2-style decoder layer (random weights) around the attention path,
    forward over all chunks then backward in reverse with each chunk's forward
    re-run (paged_sparse_attention_amd.layer); one JSON line with tokens/s, the
    attention kernels' share of the pass and the device memory it held."""
    import numpy as np
    import torch

    import synth
    import paged_sparse_attention_amd as P
    from paged_sparse_attention_amd.layer import WEIGHTS, ChunkedDecoderLayer

    seed, s = synth.LAYERS[args.layer]
    print(f"bench: layer {args.layer} {s}", file=sys.stderr, flush=True)
    # GEMM solutions: hipBLASLt/rocBLAS defaults, or a TunableOp table of the
    # layer's GEMM shapes tuned once on an MI355X (read only: nothing is tuned
    # or written here; its validators reject it under other library versions)
    gemm = "hipBLASLt/rocBLAS defaults"
    if args.gemm_table != "none":
        import tempfile
        torch.cuda.tunable.set_filename(os.path.join(tempfile.gettempdir(), "oomb_tunableop.csv"))
        torch.cuda.tunable.tuning_enable(False)
        torch.cuda.tunable.enable(True)
        ok = torch.cuda.tunable.read_file(args.gemm_table)
        gemm = "TunableOp table %s%s" % (os.path.relpath(args.gemm_table, ROOT), "" if ok else " (rejected: defaults used)")
    print(f"bench: GEMM selection: {gemm}", file=sys.stderr, flush=True)
    bits = synth.make_layer_inputs(s, seed)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    x, dy = dev(bits["x"]), dev(bits["dy"]).float()
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(s.pages).astype(np.int32))
    m0 = torch.cuda.memory_allocated()
    layer = ChunkedDecoderLayer(s.hidden, s.hq, s.hkv, s.d, s.inter, s.ps, s.c, s.chunks, s.k,
                                {n: dev(bits[n]) for n in WEIGHTS}, page_table=perm, rope_theta=s.rope_theta,
                                eps=s.eps)
    del bits
    layer_bytes = torch.cuda.memory_allocated() - m0
    nbytes = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
    # the parts of the layer that grow with the sequence: paged K/V and their
    # gradients, representative vectors, selections, page table, rotary tables
    seq_state = nbytes(layer.k_pool, layer.v_pool, layer.dk_pool, layer.dv_pool, layer.rep, layer.pt, layer.cos,
                       layer.sin, *layer.sel)
    held = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    hip = HipEvents(P.hip_runtimes_loaded()[0], 2 * 16 * s.chunks)  # per pass: at most 16 launches a chunk
    fwd_ms, bwd_ms, attn_ms = [], [], []
    for it in range(args.warmup + args.steps):
        timed = it >= args.warmup
        if timed:
            P.oomb_trace_events(hip.handles)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        layer.forward(x)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        layer.backward(x, dy)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        if timed:
            n = P.oomb_trace_count()
            if n <= 0:
                raise RuntimeError(f"kernel tracing recorded nothing (status {n})")
            attn_ms.append(sum(hip.elapsed_ms(2 * i, 2 * i + 1) for i in range(n)))
            P.oomb_trace_events(None)
            fwd_ms.append((t1 - t0) * 1e3)
            bwd_ms.append((t2 - t1) * 1e3)
    fwd, bwd, attn = statistics.median(fwd_ms), statistics.median(bwd_ms), statistics.median(attn_ms)
    ms = fwd + bwd
    tokens = s.tokens
    qd, kd = s.hq * s.d, s.hkv * s.d
    params = s.hidden * (qd + 2 * kd) + qd * s.hidden + 3 * s.hidden * s.inter
    # GEMM flops of the pass: forward 2*params per token, backward 4*params
    # per token plus the re-run forward 2*params per token
    gemm_flops = 8.0 * params * tokens
    cp = s.c // s.ps
    pairs = sum(s.hq * (s.c * min(s.k, i * cp) * s.ps + s.c * (s.c + 1) // 2) for i in range(s.chunks))
    out = {
        "metric": "decoder layer (random weights) chunk-recurrent fwd+bwd tokens/s, attention on the paged path",
        "value": tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "fwd_ms": fwd, "bwd_ms": bwd, "attention_kernels_ms": attn,
        "attention_share": attn / ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.layer, "hidden": s.hidden, "n_q_heads": s.hq, "n_kv_heads": s.hkv,
                   "head_dim": s.d, "intermediate": s.inter, "page_size": s.ps, "chunk_len": s.c,
                   "chunks": s.chunks, "tokens": tokens, "top_k": s.k, "seed": seed,
                   "activations": "one chunk, forward re-run in the backward", "gemm_selection": gemm},
        "gemm_tflops": gemm_flops / ((ms - attn) / 1e3) / 1e12,
        "attention_tflops": 14.0 * s.d * pairs / (attn / 1e3) / 1e12,
        # peak = what is held before the pass (inputs, layer) + the pass's
        # fp32 [tokens][hidden] result (y in the forward, dx in the backward)
        # + activations: one chunk's autograd graph and workspaces
        "device_bytes": {"layer": layer_bytes, "layer_sequence_state": seq_state,
                         "layer_fixed": layer_bytes - seq_state, "inputs_x_dy": x.numel() * 2 + dy.numel() * 4,
                         "pass_result": tokens * s.hidden * 4, "peak_allocated": torch.cuda.max_memory_allocated(),
                         "activation_peak": torch.cuda.max_memory_allocated() - held - tokens * s.hidden * 4},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def sequence_bench(args):
    """Chunk-recurrent forward (chunks in order) and backward (reverse order) of
    one layer over a whole synthetic sequence; one JSON line.  With --offload
    the K/V and dK/dV pools live in pinned host memory (OffloadedSequence) and
    the resident driver is timed in the same process for the overhead."""
    import numpy as np
    import torch

    import synth
    import paged_sparse_attention_amd as P
    from paged_sparse_attention_amd.sequence import ChunkedSequence

    seed, s = synth.SEQUENCES[args.sequence]
    print(f"bench: sequence {args.sequence} {s}", file=sys.stderr, flush=True)
    x = synth.make_sequence_inputs(s, seed)

    def dev(a, bf=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf else t).cuda()

    bf = s.dtype == "bf16"
    q, k, v, do = dev(x["q"], bf), dev(x["k_pool"], bf), dev(x["v_pool"], bf), dev(x["do"], bf)
    pt = dev(x["page_table"])
    dk = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    keep = not args.recompute
    nbytes = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
    m0 = torch.cuda.memory_allocated()
    drv = ChunkedSequence(s.hq, s.hkv, s.d, s.ps, s.c, s.chunks, s.k, n_initial_pages=s.n0, dtype=s.dtype,
                          softmax_scale=s.scale, keep_activations=keep)
    driver_bytes = torch.cuda.memory_allocated() - m0
    hip_path = P.hip_runtimes_loaded()[0]
    torch.cuda.reset_peak_memory_stats()
    ms, fwd_ms, bwd_ms = _time_passes(args, lambda: drv.forward(q, k, v, pt),
                                      lambda: drv.backward(q, k, v, pt, do, dk, dv), hip_path)
    # device memory: Q and dO of every chunk are inputs of this single-layer
    # driver (a model makes them chunk by chunk); dQ of every chunk is its output
    resident = {"ms_per_step": ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                "device_bytes": {"q_do_inputs": nbytes(q, do), "kv_pools": nbytes(k, v), "dkdv_pools": nbytes(dk, dv),
                                 "driver": driver_bytes, "driver_dq_output": nbytes(drv.dq),
                                 "peak_allocated": torch.cuda.max_memory_allocated()}}
    offload = None
    if args.offload:
        from paged_sparse_attention_amd.offload import OffloadedSequence
        pinned = lambda a, bf16: (torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16) if bf16
                                  else torch.from_numpy(np.ascontiguousarray(a))).pin_memory()
        host_k, host_v = pinned(x["k_pool"], bf), pinned(x["v_pool"], bf)
        host_dk = torch.zeros(k.shape, dtype=torch.float32).pin_memory()
        host_dv = torch.zeros(k.shape, dtype=torch.float32).pin_memory()
        # each chunk's own pages, as the layer's K/V projection would hand them over
        idx = torch.arange(s.chunk_pages, device="cuda")
        slots = torch.stack([pt[s.n0 + i * s.chunk_pages + idx].long() for i in range(s.chunks)])
        k_new, v_new = k[slots], v[slots]
        del k, v, dk, dv, drv
        torch.cuda.empty_cache()
        m0 = torch.cuda.memory_allocated()
        off = OffloadedSequence(s.hq, s.hkv, s.d, s.ps, s.c, s.chunks, s.k, n_initial_pages=s.n0, dtype=s.dtype,
                                softmax_scale=s.scale, keep_activations=keep, copy_cus=args.copy_cus,
                                host_accumulate=args.host_accumulate)
        off_driver_bytes = torch.cuda.memory_allocated() - m0
        torch.cuda.reset_peak_memory_stats()
        ms, fwd_ms, bwd_ms = _time_passes(
            args, lambda: off.forward(q, k_new, v_new, host_k, host_v, pt),
            lambda: off.backward(q, do, host_k, host_v, host_dk, host_dv, pt), hip_path)
        eb, blk = (2 if bf else 4), s.ps * s.d
        h2d = d2h = 0
        for i in range(s.chunks):
            ke, cp = off.keff(i), s.chunk_pages * s.hkv
            h2d += 2 * s.hkv * ke * blk * eb                          # forward: selected K/V blocks
            d2h += 2 * cp * blk * eb                                  # forward: the chunk's K/V pages
            h2d += 2 * (s.hkv * ke + cp) * blk * eb                   # backward: selected and chunk K/V
            if not args.host_accumulate:
                h2d += 2 * (s.hkv * ke + cp) * blk * 4                # backward: host dK/dV read ...
            d2h += 2 * (s.hkv * ke + cp) * blk * 4                    # ... and written back (or the deltas)
        offload = {"overhead_vs_resident": ms / resident["ms_per_step"] - 1.0, "copy_cus": args.copy_cus,
                   "gradient_adds": "host" if args.host_accumulate else "device, over the link",
                   "host_to_device_bytes_per_step": h2d, "device_to_host_bytes_per_step": d2h,
                   "host_pool_bytes": 2 * host_k.numel() * eb + 2 * host_dk.numel() * 4,
                   "device_staging_bytes": sum(t.numel() * t.element_size()
                                               for t in off.stage_k + off.stage_v + off.stage_dk + off.stage_dv),
                   "device_bytes": {"q_do_inputs": nbytes(q, do), "new_chunk_kv_inputs": nbytes(k_new, v_new),
                                    "driver": off_driver_bytes, "driver_dq_output": nbytes(off.dq),
                                    "peak_allocated": torch.cuda.max_memory_allocated()}}
    del x
    tokens = s.chunks * s.c
    flops = 14.0 * s.d * s.pairs()
    peak = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = flops / (ms / 1e3) / 1e12
    out = {
        "metric": "chunk-recurrent layer fwd+bwd tokens/s over a whole sequence, Qwen2.5-7B shape",
        "value": tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": args.sequence, "n_q_heads": s.hq, "n_kv_heads": s.hkv, "head_dim": s.d,
                   "page_size": s.ps, "chunk_len": s.c, "chunks": s.chunks, "tokens": tokens, "top_k": s.k,
                   "initial_pages": s.n0, "visible_pairs": s.pairs(), "seed": seed,
                   "activations": "two chunks' buffers, forward re-run alongside the next chunk's backward" if args.recompute else "every chunk kept",
                   "kv_cache": "pinned host memory, staged per chunk" if args.offload else "device"},
        "roofline": {"bound": "mfma", "kernel": "whole pass (every kernel of every chunk)", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "work_per_launch": flops},
        "cpu_baseline": None,
    }
    if offload is not None:
        out["resident"] = resident
        out["offload"] = offload
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sparse-256k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1536, help="chunk tokens in the oracle's timed sample")
    ap.add_argument("--sequence", default=None, metavar="NAME",
                    help="instead of one chunk step, time chunk-recurrent forward and backward over a whole "
                         "sequence (synth.SEQUENCES, e.g. seq-64k)")
    ap.add_argument("--layer", default=None, metavar="NAME",
                    help="instead of one chunk step, time a decoder layer with random weights around the path, "
                         "chunk by chunk, forward and backward (synth.LAYERS, e.g. layer-qwen-64k)")
    ap.add_argument("--gemm-table", default=os.path.join(ROOT, "paged_sparse_attention_amd", "tunableop_gfx950.csv"),
                    help="--layer: TunableOp table of the layer's GEMM shapes (read only), or 'none' for the defaults")
    ap.add_argument("--recompute", action="store_true",
                    help="with --sequence: keep one chunk's O/LSE and re-run each chunk's forward in the backward "
                         "(14*D flop per pair are still credited; the re-run forward is extra work)")
    ap.add_argument("--offload", action="store_true",
                    help="with --sequence: K/V and dK/dV pools in pinned host memory (OffloadedSequence); the "
                         "resident driver is timed too, for the overhead")
    ap.add_argument("--copy-cus", type=int, default=0,
                    help="with --offload: compute units reserved for the copy kernels (0: no partition)")
    ap.add_argument("--host-accumulate", action="store_true",
                    help="with --offload: add the gradients on the host CPU instead of on the device over the link")
    ap.add_argument("--record-traffic", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: turn the csv output of four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of "
                         "this benchmark, then of --copy-calibration) into profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--traffic-kernel", default="dkdv_kernel")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), the reference for HBM byte counters")
    args = ap.parse_args()
    if args.record_traffic:
        d = args.record_traffic
        cmds = [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d[0]} -o run -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d[1]} -o run -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline",
                f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d[2]} -o run -- python3 bench.py --copy-calibration 1024",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d[3]} -o run -- python3 bench.py --copy-calibration 1024"]
        record_traffic(d, args.traffic_kernel, args.workload, 1024, cmds)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.layer:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            sys.exit(2)
        layer_bench(args)
        return
    if args.sequence:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            sys.exit(2)
        sequence_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by kv-head across GPUs by design but no multi-GPU code is built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import paged_sparse_attention_amd as P
    from paged_sparse_attention_amd.step import ChunkStep

    seed, p = synth.WORKLOADS[args.workload]
    print(f"bench: workload {args.workload} {p}", file=sys.stderr, flush=True)
    x = synth.make_inputs(p, seed)
    tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float32

    def dev(a, bf=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf else t).cuda()

    bf = p.dtype == "bf16"
    q, k, v, do = dev(x["q"], bf), dev(x["k_pool"], bf), dev(x["v_pool"], bf), dev(x["do"], bf)
    pt = dev(x["page_table"])
    dk = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    st = ChunkStep(p.hq, p.hkv, p.d, p.ps, p.c, p.n, p.k, p.slots, dtype=p.dtype)
    st.rep_update(k, pt, 0, p.n)   # rep vectors of the prior context: setup, untimed
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        st.step(q, k, v, pt, do, dk, dv)
    torch.cuda.synchronize()

    def traced(steps, only=None):
        """`steps` chunk steps with HIP events that the library records on the
        launch stream around each kernel (every kernel, or only `only`).
        Returns (wall seconds, {kernel: [ms per launch]})."""
        hip = HipEvents(P.hip_runtimes_loaded()[0], 2 * 16 * steps)
        P.oomb_trace_only(only)
        P.oomb_trace_events(hip.handles)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.step(q, k, v, pt, do, dk, dv)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        n_traced = P.oomb_trace_count()
        names = [P.oomb_trace_kernel(i) for i in range(max(n_traced, 0))]
        P.oomb_trace_events(None)
        P.oomb_trace_only(None)
        if n_traced <= 0:
            raise RuntimeError(f"kernel tracing recorded nothing (status {n_traced})")
        durations = {}
        for i, name in enumerate(names):
            durations.setdefault(name, []).append(hip.elapsed_ms(2 * i, 2 * i + 1))
        return t1 - t0, durations

    # Events around every kernel would add twenty event records to every timed
    # step.  So two untimed steps with events around every kernel name the
    # dominant kernel; the timed steps record events around it alone (the
    # roofline line uses them); a pass after them with events around every
    # kernel gives the per-kernel breakdown.
    _, durations = traced(2)
    dominant = max(durations, key=lambda n: sum(durations[n]))
    seconds, dom = traced(args.steps, only=dominant)
    ms_per_step = seconds * 1e3 / args.steps
    if set(dom) != {dominant}:
        raise RuntimeError(f"filtered tracing recorded {sorted(dom)}, expected {dominant}")
    dominant_ms = statistics.mean(dom[dominant])
    profile_steps = max(4, args.steps // 4)
    _, durations = traced(profile_steps)
    kernels = {n: {"launches": len(v), "avg_ms": statistics.mean(v)} for n, v in durations.items()}
    print("bench: per-kernel ms " + json.dumps({n: [round(x, 4) for x in v[:4]] for n, v in durations.items()}),
          file=sys.stderr, flush=True)
    if not any(kv["avg_ms"] > 0 for kv in kernels.values()):
        raise RuntimeError("kernel events report zero durations")
    bound, work, unit = kernel_work(p, dominant)
    avg_s = dominant_ms / 1e3
    if bound == "mfma":
        peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = work / avg_s / 1e12
        roof = {"bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": measured_traffic(dominant, args.workload), "work_per_launch": work}
    else:
        achieved = work / avg_s / 1e9
        roof = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(dominant, args.workload),
                "work_per_launch": work}
    for n, kv in kernels.items():
        b, w, u = kernel_work(p, n)
        s = kv["avg_ms"] / 1e3
        kv["achieved"] = (w / s / 1e12) if b == "mfma" else (w / s / 1e9)
        kv["unit"] = "TFLOP/s" if b == "mfma" else "GB/s"
    attn_ms = sum(kernels[n]["avg_ms"] for n in ("fwd_kernel", "dt_kernel", "dkdv_kernel", "dq_kernel")
                  if n in kernels)
    attn_flops = 14.0 * p.d * p.pairs()
    peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_FP32_TFLOPS

    out = {
        "metric": METRIC,
        "value": p.c / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "n_q_heads": p.hq, "n_kv_heads": p.hkv, "head_dim": p.d,
                   "page_size": p.ps, "chunk_len": p.c, "prior_pages": p.n, "prior_tokens": p.n * p.ps,
                   "top_k": p.k, "visible_pairs": p.pairs(), "seed": seed},
        "roofline": roof,
        "attention_mfma_frac": attn_flops / (attn_ms / 1e3) / 1e12 / peak,
        "attention_ms": attn_ms,
        "kernels": kernels,
        "kernel_timing": {"roofline": f"HIP events around {dominant} in the {args.steps} timed steps (avg "
                                      f"{dominant_ms:.4f} ms)",
                          "kernels": f"HIP events around every kernel in {profile_steps} more steps, after the "
                                     f"timed ones; attention_ms and attention_mfma_frac use them"},
    }
    if p.dtype == "bf16":
        mp = measured_peaks(P)
        mp["attention_mfma_frac_of_measured"] = attn_flops / (attn_ms / 1e3) / 1e12 / mp["mfma_bf16_tflops"]
        if bound == "mfma":
            mp["dominant_frac_of_measured"] = roof["achieved"] / mp["mfma_bf16_tflops"]
        out["measured_peaks"] = mp
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(p, seed, x, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
