#!/usr/bin/env python3
"""Benchmark of the Lookahead Sparse Attention decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ctx1m] [--cold device|host]

A step is one decode step of the whole batch through the full path: on the
steps where the refresh cadence (every 64 steps) fires, the index refresh
(query encoder, block scoring, threshold, OR-union, compaction), the copy of
the selection to the host, the residency plan and the block gather; then the
sparse decode (window append, split-K attention, log-sum-exp merge).  W
untimed warm-up steps run first (they include the first refresh and the
initial load of every selected block), then K timed steps.

Default workload: 4 requests x 1,048,576-token contexts (16384 blocks of 64
tokens each), bf16, 3 indexers (d_model 4096, d_idx 256), 16 query heads
sharing one KV head of dim 128, an 8192-token window, 10% background + 10%
planted relevant blocks.  Inputs are seeded synthetic data with those shapes
and distributions.  With --cold device (default) the cold pool sits in HBM, so
the timed region moves no host data except the selected ids; --cold host puts
it in pinned host memory and the gather crosses the host link.  The residency
plan is made on the host (--plan host, the default) or on the device (--plan
device: no host round trip, the decode reads the counts on the device).

Prints one JSON line.  `value` is end-to-end decode tokens/s (requests x K /
wall time of the timed steps).  `roofline` describes the attention kernel
(the dominant kernel): algorithmic bytes per launch / mean launch time from
HIP events passed to the kernel's launch, on every --event-every-th timed step
(default 16), offset by half of that from the timed region's start so that the
event launch (~30 us of host time) does not follow a refresh, where the GPU
waits for the host.  The start event is the dispatch's own start stamp; the end event
lands a few microseconds after the kernel ends, so the figure is on the low
side, and the events cost stream time (the GPU idles ~10 us around each timed
launch).  `decode_steady` is the decode between refreshes, from the start
stamps of those launches; the refresh, gather and latent kernels are timed the
same way on at most 8 refreshes.  `cpu_baseline` times the CPU oracle on a
bounded sample.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "LSA decode tokens/s at 1M ctx + index-refresh µs; % of HBM roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12,
                    help="timed steps; a step is 64 decode steps of every request (one refresh interval)")
    ap.add_argument("--warmup", type=int, default=2, help="untimed steps before them")
    ap.add_argument("--workload", default="ctx1m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold", choices=("device", "host"), default="device")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the cold-read ceiling (read probe) measured after the timed region")
    ap.add_argument("--cpu-sample-steps", type=int, default=6, help="decode steps per request timed on the CPU")
    ap.add_argument("--tau", type=int, default=0,
                    help="refresh cadence in steps (default: the workload's, 64); 1 scores every step")
    ap.add_argument("--density", type=float, default=0.0,
                    help="union density the indexer biases are set for (default: the workload's)")
    ap.add_argument("--layers", type=int, default=1,
                    help="attention layers whose block loads each selection drives (own K/V and queries)")
    ap.add_argument("--hidden-rho", type=float, default=0.0,
                    help="correlation of successive refresh hidden states (0: independent)")
    ap.add_argument("--select", choices=("threshold", "all"), default="threshold",
                    help="all: every block selected at one refresh before the first step, i.e. dense "
                         "attention over the whole context through the same kernels (comparator)")
    ap.add_argument("--q-rank", type=int, default=0,
                    help="low-rank query projection: each refresh first forms the latents c_i = A_i h of "
                         "this rank (2048 on the pages), and the Query Encoder projects them")
    ap.add_argument("--denoise", action="store_true",
                    help="measure the indexer's label-denoising pipeline instead of the decode loop: 21 "
                         "layers x --denoise-windows windows x 16,384 blocks of synthetic logits per call")
    ap.add_argument("--denoise-windows", type=int, default=64)
    ap.add_argument("--read-ceiling", action="store_true",
                    help="measure the cold-read ceiling of one launch at the refresh's and the attention's "
                         "sizes with the read probe (libprobe.so) instead of the decode loop")
    ap.add_argument("--ceiling-reps", type=int, default=10)
    ap.add_argument("--latent-sweep", action="store_true",
                    help="measure the low-rank latent c_i = A_i h (3 indexers x rank 2048 x d_model 4096, bf16, "
                         "A cold) across batch sizes instead of the decode loop")
    ap.add_argument("--refresh-sweep", action="store_true",
                    help="measure one index refresh (3 indexers, d_model 4096, d_idx 256, bf16, 16,384 blocks "
                         "per request, keys cold) across the number of 1M-context requests per call instead "
                         "of the decode loop")
    ap.add_argument("--kernel-trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="no run: per kernel and grid size, the dispatch durations of a rocprofv3 "
                         "--kernel-trace CSV")
    ap.add_argument("--plan", choices=("device", "host"), default="device",
                    help="where the residency plan of a refresh is made: on the device "
                         "(lsa_gather_plan_device, the default: no host round trip, the decode reads the counts "
                         "on the device) or on the host (lsa_gather_blocks_batch: the ids come back to the host "
                         "and the stream waits for them)")
    ap.add_argument("--overlap", choices=("auto", "on", "off"), default="off",
                    help="staggered refreshes (some requests at a step): run their refresh, plan, copy and "
                         "attention on a second stream beside the other requests' attention (StaggeredLoop); "
                         "auto: with the device plan, one layer and a workload whose steps refresh some requests. "
                         "Off by default: on one MI355X any use of a second stream left every later kernel of "
                         "the decode stream ~3%% slower, and the ragged mix ran at 221K tokens/s against 248K")
    ap.add_argument("--reactive", action="store_true",
                    help="reactive comparator: every block resident in HBM, the index scored at every step "
                         "and the decode reading the selected blocks in place (refresh cadence 1, no "
                         "gathers, no host round trip)")
    ap.add_argument("--level", type=float, default=0.5,
                    help="selection level: keep a block when sigmoid(z) > level (0.5 on the pages; the "
                         "refresh's select_level)")
    ap.add_argument("--host-leg", type=int, default=2,
                    help="after the timed region, continue this many steps with the cold pool's pinned host "
                         "copy (gathers over the host link) and report that rate beside the HBM-pool one")
    ap.add_argument("--event-every", type=int, default=16,
                    help="time the attention kernel with HIP events on every N-th timed step (the events "
                         "take the dispatch's own stamps but still cost stream time)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no run: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 pass (both taken with --calib-copy-mib) into "
                         "profiles/<kernel>_<workload>_traffic.json")
    ap.add_argument("--traffic-kernel", default="attn_kernel", choices=sorted(KERNEL_SOURCES),
                    help="the kernel --traffic-summary summarises")
    return ap.parse_args()


def _bf16_to_f32(raw: np.ndarray) -> np.ndarray:
    return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _planting_query(dtype):
    """Query embeddings used only to place the planted keys (input construction)."""
    def fn(h, w):
        hf = _bf16_to_f32(h) if dtype == "bf16" else h
        wf = _bf16_to_f32(w) if dtype == "bf16" else w
        hs = [hf if hf.ndim == 1 else hf[i] for i in range(wf.shape[0])]  # one per indexer (latents)
        return np.stack([wf[i].astype(np.float64) @ hs[i].astype(np.float64) for i in range(wf.shape[0])])
    return fn


def _planting_latent(dtype):
    """Latents of a low-rank workload, used only to place the planted keys (input construction)."""
    from workloads import bf16_bits_from_f32

    def fn(h, w_down):
        hf = (_bf16_to_f32(h) if dtype == "bf16" else h).astype(np.float64)
        wf = _bf16_to_f32(w_down) if dtype == "bf16" else w_down
        c = np.stack([wf[i].astype(np.float64) @ hf for i in range(wf.shape[0])]).astype(np.float32)
        return bf16_bits_from_f32(c) if dtype == "bf16" else c
    return fn


KERNEL_SOURCES = {"attn_kernel": ("decode.hip", "lsa_internal.hpp"),
                  "refresh_kernel": ("refresh.hip", "lsa_internal.hpp")}


def kernel_hash(kernel: str = "attn_kernel") -> str:
    """Hash of the sources a kernel is built from (its counters stay valid while this is unchanged)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update((ROOT / "lookahead_block_sparse_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, calib_mib: int,
                    kernel: str = "attn_kernel") -> dict:
    """HBM bytes per launch of `kernel` from two rocprofv3 counter passes.  Each counter is scaled
    by what it reads for the plain device copy of calib_mib MiB in the same pass (read calib bytes,
    write calib bytes), which takes out the counters' units and any sampling of channels."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        calib = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        mine = [r for r in rows if kernel in r["Kernel_Name"]]
        # the launches over every request (the largest grid): a run also refreshes single requests
        # to recompute selections, and those launches read a quarter of the keys
        grid = max((int(r["Grid_Size"]) for r in mine), default=0)
        vals = [float(r["Counter_Value"]) for r in mine if int(r["Grid_Size"]) == grid]
        if not vals or not calib:
            raise SystemExit(f"{path}: no {kernel} or copy dispatches with {counter}")
        return float(np.mean(vals)), max(calib), len(vals)

    n = calib_mib << 20
    f_k, f_cal, n_f = per_kernel(fetch_csv, "FETCH_SIZE")
    w_k, w_cal, n_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = n / (f_cal * 1024.0), n / (w_cal * 1024.0)
    return {
        "kernel": kernel,
        "workload": workload,
        "dispatches": {"fetch_pass": n_f, "write_pass": n_w},
        "launch": "the launches of the largest grid (every request of the workload)",
        "fetch_size_kib_per_dispatch": f_k,
        "write_size_kib_per_dispatch": w_k,
        "calib_copy_bytes": n,
        "calib_fetch_size_kib": f_cal,
        "calib_write_size_kib": w_cal,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "fetch_bytes_per_launch": f_k * 1024.0 * f_scale,
        "write_bytes_per_launch": w_k * 1024.0 * w_scale,
        "traffic_bytes_per_launch": f_k * 1024.0 * f_scale + w_k * 1024.0 * w_scale,
        "kernel_sources_sha256_16": kernel_hash(kernel),
    }


def stored_traffic(workload: str, kernel: str = "attn_kernel"):
    """HBM traffic per launch of a kernel from the committed counter summary, if it was taken on the
    kernel's current sources; else None."""
    f = ROOT / "profiles" / f"{kernel}_{workload}_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("kernel_sources_sha256_16") != kernel_hash(kernel):
        return None
    return d.get("traffic_bytes_per_launch")


def host_link_peak(dev, mib: int = 512, reps: int = 5) -> float:
    """Pinned host -> device rate of one large asynchronous copy (the DMA engines), best of `reps`:
    the reference the gather's host-link rate is read against."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        b.synchronize()
        best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


def cpu_baseline(wl, sample_steps: int, seed: int):
    """Time the oracle on a bounded sample of the same workload: one refresh of every request and
    `sample_steps` decode steps per request with the BLAS threads it finds; then one refresh and
    `sample_steps` decode steps of one request on a single thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = 1
    cfg = wl.cfg
    dt = cfg.dtype
    w_q = oracle.decode_values(wl.w_q, dt)
    rng = np.random.default_rng(seed)
    steps = sorted(rng.choice(np.arange(1, min(cfg.steps, 64)), size=sample_steps, replace=False).tolist())

    def run(reqs):
        t_ref, t_dec, n = 0.0, 0.0, 0
        for r in reqs:
            t0 = time.perf_counter()
            keys = oracle.decode_values(wl.keys[r], dt)
            res = oracle.refresh(oracle.decode_values(wl.hidden[r][0], dt), w_q, keys, wl.bias[r])
            t_ref += time.perf_counter() - t0
            kp, vp = wl.kv_prefill(r)
            N = int(wl.ctx[r])
            for t in steps:
                t0 = time.perf_counter()
                pos = oracle.token_set(oracle.seq_len_at(N, t), cfg.window, res.ids, cfg.block)
                # only the attended prefill rows are decoded (the whole 1M-token prefill in float64
                # would be 1 GB per tensor): kv_rows reads them as a prefill of m rows, the new
                # tokens' positions shifted to follow it
                lo = pos < N
                m = int(lo.sum())
                rel = np.concatenate([np.arange(m), pos[~lo] - N + m])
                k = oracle.kv_rows(oracle.decode_values(kp[pos[lo]], dt), oracle.decode_values(wl.k_new[:, r], dt), m, rel)
                v = oracle.kv_rows(oracle.decode_values(vp[pos[lo]], dt), oracle.decode_values(wl.v_new[:, r], dt), m, rel)
                oracle.attention(oracle.decode_values(wl.q_dec[t, r], dt), k, v, cfg.head_dim ** -0.5)
                t_dec += time.perf_counter() - t0
                n += 1
        return t_ref, t_dec, n

    t_ref, t_dec, n = run(range(wl.n_req))
    out = {
        "value": n / t_dec,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} request-steps (steps {steps} of each of {wl.n_req} requests, selection of the "
                  f"first refresh) and one refresh per request; float64 NumPy",
        "refresh_us_per_request": 1e6 * t_ref / wl.n_req,
        "seconds": t_dec + t_ref,
    }
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1_ref, t1_dec, n1 = run([0])
        out["single_thread"] = {"value": n1 / t1_dec, "unit": "tokens/s", "cores": 1,
                                "refresh_us_per_request": 1e6 * t1_ref, "seconds": t1_ref + t1_dec,
                                "sample": f"{n1} request-steps of request 0 and its first refresh"}
    return out


def run_denoise(args) -> dict:
    """Label denoising (softmax, top-p 0.6, vote >= 3 of 21) over synthetic logits of 1M-context
    windows; one step = one call over every window."""
    import torch

    from lookahead_block_sparse_amd import lsa_label_denoise_workspace
    from workloads import build_denoise_workload

    W, K, Wu = args.denoise_windows, args.steps, args.warmup
    n_layers, n_blocks = 21, 16384
    dw = build_denoise_workload([n_blocks] * W, n_layers=n_layers, seed=args.seed)
    dev = torch.device("cuda")
    logits = torch.from_numpy(dw.logits).to(dev)
    n_blk_dev = torch.from_numpy(dw.n_blk).to(dev)
    words = (n_blocks + 63) // 64
    labels = torch.empty((W, words), dtype=torch.int64, device=dev)
    n_pos = torch.empty(W, dtype=torch.int32, device=dev)
    n_naive = torch.empty(W, dtype=torch.int32, device=dev)
    ws = torch.empty(lsa_label_denoise_workspace(n_layers=n_layers, n_blk=dw.n_blk), dtype=torch.uint8, device=dev)
    def mk_event():  # recorded once so torch treats it as recorded; the launch then takes its stamps
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    evs = [(mk_event(), mk_event()) for _ in range(K)]

    # the argument struct is built once; a call only swaps the timing events (as DecodeLoop does)
    import ctypes

    from lookahead_block_sparse_amd import LIB, _check, _denoise_args

    dargs, keep = _denoise_args(n_layers=n_layers, n_blk=dw.n_blk, top_p=0.6, min_votes=3, logits=logits,
                                logit_stride=logits.shape[2], n_blk_dev=n_blk_dev, labels=labels, n_pos=n_pos,
                                n_naive=n_naive, workspace=ws)
    dref = ctypes.byref(dargs)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(ev=(None, None)):
        dargs.ev_begin = ev[0].cuda_event if ev[0] is not None else None
        dargs.ev_end = ev[1].cuda_event if ev[1] is not None else None
        _check(LIB.lsa_label_denoise(dref, stream))

    for _ in range(Wu):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    topp_us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    # algorithmic bytes of the top-p kernel: every logit once, every layer's set word once
    topp_bytes = n_layers * W * n_blocks * 4 + n_layers * W * words * 8
    res = {
        "metric": "label-denoising token windows/s (21 layers x 16,384 blocks, top-p 0.6, vote >= 3)",
        "value": W * K / elapsed,
        "unit": "windows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 logits, fp64 exponentials in 48-bit fixed point",
        "data": "synthetic",
        "config": {"workload": f"label denoising: {W} windows x {n_blocks} blocks x {n_layers} layers, "
                               "300 relevant blocks per window (signal 4, noise 1)", "windows": W,
                   "blocks": n_blocks, "layers": n_layers, "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": "topp_kernel (softmax + top-p per layer and window)",
                     "achieved": topp_bytes / (topp_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": topp_bytes / (topp_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": topp_bytes, "timed_launches": K,
                     "mean_launch_us": topp_us},
        "labels_per_window": float(n_pos.float().mean().item()),
        "naive_positives_per_window": float(n_naive.float().mean().item()),
    }
    if not args.no_cpu_baseline:
        import oracle
        sample = min(2, W)
        t0 = time.perf_counter()
        for w in range(sample):
            oracle.denoise_window(dw.logits[:, w, :n_blocks].astype(np.float64), 0.6, 3)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": sample / dt, "unit": "windows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{sample} windows of the same workload through oracle.denoise_window"}
    return res


def _probe_lib():
    """The read probe (libprobe.so, built by __graft_entry__.build()), or None when it is not built."""
    import ctypes

    path = ROOT / "lookahead_block_sparse_amd" / "libprobe.so"
    if not path.exists():
        return None
    lib = ctypes.CDLL(str(path))
    lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p, ctypes.c_uint, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
    lib.probe_batches.argtypes = [ctypes.c_longlong, ctypes.c_int]
    lib.probe_batches.restype = ctypes.c_longlong
    lib.probe_groups_per_cu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    return lib


def _probe_rows(lib, name: str, size: int, variants, reps: int) -> list:
    """One row per (pattern, nontemporal, loads, persistent) variant: `reps` event-timed launches of
    the read probe over `size` bytes, each reading a region last read more than 1.2 GB earlier."""
    import torch

    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    stride = (size + (1 << 20) - 1) >> 20 << 20
    n_reg = max(3, -(-(1200 << 20) // stride))
    buf = torch.empty(n_reg * stride, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reg = 0
    rows = []
    for pattern, nt, loads, persistent in variants:
        per_cu = lib.probe_groups_per_cu(pattern, loads, nt)
        nb = lib.probe_batches(size, loads)
        groups = cus * per_cu if persistent else 0
        g_launch = groups if groups else (nb + 3) // 4
        if sink.numel() < 256 * g_launch:
            sink = torch.zeros(256 * g_launch, dtype=torch.int32, device=dev)
        evs = []
        for _ in range(reps + 1):  # the first launch of a variant loads its code
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            ptr = buf.data_ptr() + reg * stride
            reg = (reg + 1) % n_reg
            rc = lib.probe_read(ptr, size, pattern, loads, nt, groups, sink.data_ptr(),
                                0xDEADBEEF, e0.cuda_event, e1.cuda_event, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"probe_read returned {rc}")
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([1e3 * a.elapsed_time(b) for a, b in evs[1:]])
        read = nb * loads * 1024
        rows.append({"size": name, "bytes": int(read), "pattern": ("runs", "rows")[pattern],
                     "nontemporal": bool(nt), "loads_per_batch": loads,
                     "shape": "one-shot" if groups == 0 else f"persistent {per_cu}/CU",
                     "groups": int(g_launch), "median_us": float(np.median(us)),
                     "min_us": float(us.min()), "TB_per_s": read / (np.median(us) * 1e-6) / 1e12})
    del buf
    torch.cuda.empty_cache()
    return rows


def read_ceiling_best(size: int, reps: int = 5):
    """The measured cold-read ceiling for `size` bytes: the best median rate of the read probe over
    the load shapes the hot kernels use (whole 1 KiB runs, non-temporal loads; 48 loads per wave
    requested at once, or 16 per batch at as many groups as fit), or None without libprobe.so."""
    lib = _probe_lib()
    if lib is None:
        return None
    rows = _probe_rows(lib, "kernel", size, [(0, 1, 48, False), (0, 1, 16, True)], reps)
    best = max(rows, key=lambda r: r["TB_per_s"])
    return {"GB_per_s": best["TB_per_s"] * 1e3, "bytes": best["bytes"], "median_us": best["median_us"],
            "shape": f"{best['loads_per_batch']} loads per wave, {best['shape']}",
            "probe": "read probe (libprobe.so): a cold region read with whole 1 KiB runs and non-temporal loads"}


def run_read_ceiling(args) -> dict:
    """Cold-read ceilings for the two hot kernels' sizes: one launch of the read probe
    (libprobe.so) per size, access pattern, load hint, loads per batch and launch shape, each
    reading a region last touched more than 1 GB of reads earlier (past the 256 MB memory-side
    cache), timed with the dispatch's own start and end stamps."""
    import torch

    torch.cuda.init()
    lib = _probe_lib()
    if lib is None:
        raise SystemExit("libprobe.so is not built: run __graft_entry__.build()")
    # the refresh's bytes at 4 x 1M (W_q + keys) and the attention's (4 x ~206K tokens of K and V)
    sizes = {"refresh": 3 * 4096 * 256 * 2 + 4 * 3 * 16384 * 256 * 2, "attention": 416 << 20}
    reps = max(3, args.ceiling_reps)
    variants = [(pattern, nt, loads, persistent) for pattern in (0, 1) for nt in (1, 0) for loads in (16, 48)
                for persistent in (False, True)]
    rows = []
    for name, size in sizes.items():
        rows += _probe_rows(lib, name, size, variants, reps)
    return {"metric": "cold-read ceiling of one launch", "rows": rows, "reps": reps,
            "note": "event-timed dispatches; each launch reads a region last read more than 1 GB earlier"}


def run_latent_sweep(args) -> dict:
    """The latent projection of the low-rank Query Encoder (3 indexers x rank 2048 x d_model 4096,
    bf16) at batch sizes 1-64: each launch reads one of 8 copies of A (400 MB in all, past the
    256 MB memory-side cache, so A is cold), timed with the dispatch's own start and end stamps;
    algorithmic bytes = A + the hidden states + the latents.  Each size's result is checked
    against an fp32 product of the same bf16 values."""
    import torch

    from lookahead_block_sparse_amd import lsa_query_latent

    dev = torch.device("cuda")
    n_idx, rank, d = 3, 2048, 4096
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    copies = 8
    A = [(torch.randn(n_idx, rank, d, device=dev, generator=gen) / d ** 0.5).to(torch.bfloat16) for _ in range(copies)]
    reps = max(10, args.ceiling_reps * 4)
    rows = []
    for R in (1, 4, 8, 10, 12, 16, 32, 64):
        h = torch.randn(R, d, device=dev, generator=gen).to(torch.bfloat16)
        out = torch.empty(R, n_idx, rank, dtype=torch.int16, device=dev)
        evs = []
        for it in range(reps + copies):
            a = A[it % copies]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            lsa_query_latent(dtype="bf16", d_model=d, rank=rank, n_idx=n_idx, n_req=R, hidden=h.view(torch.int16),
                             w_down=a.view(torch.int16), latent=out, hidden_req_stride=d, hidden_idx_stride=0,
                             ev_begin=e0, ev_end=e1)
            if it == copies - 1:  # the latent of the last copy against an fp32 product
                got = out.view(torch.bfloat16).float()
                want = torch.stack([(a[i].float() @ h.float().T).T for i in range(n_idx)], 1)
                err = ((got - want).abs().max() / want.abs().max()).item()
                if not err < 1e-2:
                    raise RuntimeError(f"latent at {R} requests: relative error {err:.3g}")
            if it >= copies:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([1e3 * x.elapsed_time(y) for x, y in evs])
        nbytes = (n_idx * rank * d + R * d + R * n_idx * rank) * 2
        tbs = nbytes / (np.median(us) * 1e-6) / 1e12
        rows.append({"requests": R, "median_us": float(np.median(us)), "min_us": float(us.min()),
                     "bytes": int(nbytes), "TB_per_s": tbs, "frac": tbs * 1e3 / HBM_PEAK_GBS})
    return {"metric": "latent projection time across batch sizes", "rows": rows, "launches_per_size": reps,
            "shape": {"n_idx": n_idx, "rank": rank, "d_model": d, "dtype": "bf16"}}


def run_refresh_sweep(args) -> dict:
    """One index refresh of R requests of 16,384 blocks (1M tokens) each, 3 indexers, d_model 4096,
    d_idx 256, bf16, with the bit planes the device plan reads, at R = 1-16.  Before each timed
    launch a 1 GiB copy pushes the keys out of the 256 MB memory-side cache, so they are read cold;
    the launch is timed with the dispatch's own start and end stamps.  Algorithmic bytes as for the
    decode loop's refresh: W_q + keys + hidden states + ids + counts + bit planes.  Each size's
    counts are checked against an fp32 computation of the same bf16 values (equal up to the few
    blocks whose logits lie within rounding of the threshold)."""
    import torch

    from lookahead_block_sparse_amd import lsa_index_refresh, lsa_index_refresh_workspace

    dev = torch.device("cuda")
    n_idx, d_idx, d, B = 3, 256, 4096, 16384
    sizes = (1, 2, 4, 8, 16)
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    R_max = max(sizes)
    keys = (torch.randn(R_max * n_idx * B * d_idx, device=dev, generator=gen) / d_idx ** 0.5).to(torch.bfloat16)
    w_q = (torch.randn(n_idx * d_idx * d, device=dev, generator=gen) / d ** 0.5).to(torch.bfloat16)
    hid = torch.randn(R_max * d, device=dev, generator=gen).to(torch.bfloat16)
    bias_val = -1.8  # logits are ~N(0, 1): ~3.6% per indexer, ~10% union
    flush_src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush_dst = torch.empty_like(flush_src)
    reps = max(8, args.ceiling_reps)
    rows = []
    for R in sizes:
        blk = [B * r for r in range(R + 1)]
        words = R * B // 64
        bias = torch.full((R * n_idx,), bias_val, device=dev)
        sel = torch.zeros(R * B, dtype=torch.int32, device=dev)
        cnt = torch.zeros(R, dtype=torch.int32, device=dev)
        masks = torch.zeros(words * (n_idx + 1), dtype=torch.int64, device=dev)
        ws = torch.zeros(lsa_index_refresh_workspace(dtype="bf16", d_model=d, d_idx=d_idx, n_idx=n_idx, blk_off=blk),
                         dtype=torch.uint8, device=dev)
        evs = []
        for it in range(reps + 2):
            flush_dst.copy_(flush_src)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            lsa_index_refresh(dtype="bf16", d_model=d, d_idx=d_idx, n_idx=n_idx, hidden=hid.view(torch.int16),
                              w_q=w_q.view(torch.int16), keys=keys.view(torch.int16), blk_off=blk, bias=bias,
                              sel_ids=sel, sel_count=cnt, workspace=ws, masks=masks, ev_begin=e0, ev_end=e1)
            if it >= 2:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        # counts against fp32 logits of the same bf16 values
        wq = w_q.float().view(n_idx, d_idx, d)
        want = np.zeros(R, dtype=np.int64)
        for r in range(R):
            q = torch.bmm(wq, hid[r * d:(r + 1) * d].float().view(1, d, 1).expand(n_idx, d, 1).contiguous())
            kk = keys[r * n_idx * B * d_idx:(r + 1) * n_idx * B * d_idx].float().view(n_idx, B, d_idx)
            z = torch.bmm(kk, q).view(n_idx, B) + bias_val  # fp32 logits [n_idx][B]
            want[r] = int((z > 0).any(0).sum().item())
        got = cnt.cpu().numpy()
        if np.any(np.abs(got - want) > 0.001 * B):
            raise RuntimeError(f"refresh at {R} requests: counts {got.tolist()} against fp32 {want.tolist()}")
        us = np.array([1e3 * x.elapsed_time(y) for x, y in evs])
        nbytes = 2 * (n_idx * d_idx * d + R * n_idx * B * d_idx + R * d) + 4 * int(got.sum()) + 4 * R \
            + 8 * (n_idx + 1) * words
        tbs = nbytes / (np.median(us) * 1e-6) / 1e12
        rows.append({"requests": R, "median_us": float(np.median(us)), "min_us": float(us.min()),
                     "bytes": int(nbytes), "TB_per_s": tbs, "frac": tbs * 1e3 / HBM_PEAK_GBS,
                     "selected_per_request": float(got.mean())})
        del bias, sel, cnt, masks, ws
    return {"metric": "index refresh time across requests per call (1M context each)", "rows": rows,
            "launches_per_size": reps,
            "shape": {"n_idx": n_idx, "d_model": d, "d_idx": d_idx, "blocks_per_request": B, "dtype": "bf16"}}


def kernel_trace_summary(path: str) -> dict:
    """Per (kernel, grid size): dispatch count, mean and median duration in us, from the
    kernel_trace.csv of a rocprofv3 --kernel-trace run."""
    import csv

    groups = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        key = (name, int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    out = []
    for (name, grid), us in sorted(groups.items()):
        a = np.array(us)
        out.append({"kernel": name, "grid_x": grid, "dispatches": len(a), "mean_us": float(a.mean()),
                    "median_us": float(np.median(a)), "min_us": float(a.min())})
    return {"trace": path, "kernels": out}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the LSA decode path runs on one GPU only; --gpus must be 1 "
              "(sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        if args.calib_copy_mib <= 0:
            raise SystemExit("--traffic-summary needs the --calib-copy-mib the counter passes ran with")
        d = traffic_summary(*args.traffic_summary, workload=args.workload, calib_mib=args.calib_copy_mib,
                            kernel=args.traffic_kernel)
        out = ROOT / "profiles" / f"{args.traffic_kernel}_{args.workload}_traffic.json"
        out.write_text(json.dumps(d, indent=1) + "\n")
        print(json.dumps(d))
        return

    if args.denoise:
        print(json.dumps(run_denoise(args)), flush=True)
        return
    if args.kernel_trace_summary:
        print(json.dumps(kernel_trace_summary(args.kernel_trace_summary)), flush=True)
        return
    if args.read_ceiling:
        print(json.dumps(run_read_ceiling(args)), flush=True)
        return
    if args.latent_sweep:
        print(json.dumps(run_latent_sweep(args)), flush=True)
        return
    if args.refresh_sweep:
        print(json.dumps(run_refresh_sweep(args)), flush=True)
        return

    print(json.dumps(run_loop(args)), flush=True)


STEP_DECODE = 64  # decode steps per benchmark step: one refresh interval at the pages' cadence


def prologue_requests(wl):
    """Requests whose first refresh falls before step 0 (staggered phases): their selection at step
    0 comes from that prologue refresh, which the benchmark runs before the warm-up."""
    return [r for r in range(wl.n_req) if wl.refresh_steps[r][0] < 0]


def max_bench_steps(cfg) -> int:
    """Most steps (warm-up included) whose decode-time tokens all stay inside the window."""
    return cfg.window // STEP_DECODE


def run_loop(args) -> dict:
    """The decode loop: K timed steps of STEP_DECODE decode steps each (one refresh interval at
    tau = 64), after W untimed ones and the prologue refreshes of staggered requests."""
    import torch

    from lookahead_block_sparse_amd.session import DecodeLoop, LSASession, ResidentLoop, StaggeredLoop
    from workloads import build_workload, get_config

    def note(msg):
        print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)

    cfg = get_config(args.workload)
    W, K = args.warmup * STEP_DECODE, args.steps * STEP_DECODE  # in decode steps
    total_steps = W + K
    if args.warmup + args.steps > max_bench_steps(cfg):
        raise SystemExit(f"at most {max_bench_steps(cfg)} steps in all (warm-up included): decode-time "
                         f"tokens must stay inside the {cfg.window}-token window")
    if args.tau > 0:
        cfg = cfg.scaled(tau=args.tau)
    if args.density > 0:
        cfg = cfg.scaled(density=("fixed", args.density))
    if args.layers > 1 or args.hidden_rho:
        cfg = cfg.scaled(n_layers=args.layers, hidden_rho=args.hidden_rho)
    if args.select == "all":
        cfg = cfg.scaled(tau=max(cfg.tau, total_steps + 1), planted_frac=0.0, staggered=False)  # one refresh
    if args.q_rank > 0:
        cfg = cfg.scaled(q_rank=args.q_rank)
    if args.level != 0.5:
        cfg = cfg.scaled(level=args.level)
    if args.reactive:
        if args.select == "all" or cfg.n_layers > 1 or args.cold != "device":
            raise SystemExit("--reactive runs one layer with the default selection and the pool in HBM")
        cfg = cfg.scaled(tau=1, staggered=False)
    t_setup = time.perf_counter()
    wl = build_workload(cfg, seed=args.seed, steps=max(cfg.steps, total_steps))
    cfg = wl.cfg
    if cfg.planted_frac > 0:
        wl.condition(_planting_query(cfg.dtype), None, latent_fn=_planting_latent(cfg.dtype))
    if args.select == "all":
        wl.bias[:] = 1e4  # every logit above zero: every block selected
    note(f"workload {cfg.name}: {wl.n_req} requests, contexts {wl.ctx.tolist()[:4]}..., built")

    dev = torch.device("cuda")
    dplan = args.plan == "device" and not args.reactive
    host_leg = args.host_leg if (args.cold == "device" and not args.reactive and args.select != "all") else 0
    sess = LSASession(dtype=cfg.dtype, n_idx=cfg.n_idx, d_model=cfg.d_model, d_idx=cfg.d_idx,
                      n_heads=cfg.n_heads, head_dim=cfg.head_dim, win_cap=cfg.window, n_blocks=wl.n_blocks,
                      w_q=wl.w_q, keys=wl.keys, cold_on_device=(args.cold == "device"), with_masks=False,
                      n_layers=cfg.n_layers, w_down=wl.w_down, device_plan=dplan,
                      cold_host_mirror=host_leg > 0, select_level=cfg.level)
    for r in range(wl.n_req):
        k, v = wl.kv_prefill(r)
        sess.load_prefill(r, k, v)
        for layer in range(1, cfg.n_layers):
            kl, vl = wl.kv_prefill(r, layer)
            sess.load_prefill(r, kl, vl, layer=layer)
        if args.no_cpu_baseline:
            wl.drop_kv(r)
    if args.reactive:
        sess.make_resident()  # every block in the hot pool, block b of request r at slot base + b
    note(f"session ready in {time.perf_counter() - t_setup:.1f}s (cold pool on {args.cold}"
         + (", every block resident" if args.reactive else "") + ")")

    def dev_raw(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    # every refresh's hidden state and the biases are device-resident before the timed region
    # (stacked per refresh step, in request order); the prologue refreshes (staggered requests
    # whose first refresh falls before step 0) are keyed -1
    hid_at = {}
    prologue = prologue_requests(wl)
    if prologue:
        hid_at[-1] = dev_raw(np.stack([wl.hidden[r][0] for r in prologue]))
    for t in range(total_steps):
        reqs = wl.refreshes_at(t)
        if reqs:
            hid_at[t] = dev_raw(np.stack([wl.hidden[r][wl.refresh_index_at(r, t)] for r in reqs]))
    bias_dev = torch.from_numpy(np.ascontiguousarray(wl.bias, dtype=np.float32)).to(dev)
    q_all = dev_raw(wl.q_dec[:total_steps])
    kn_all = dev_raw(wl.k_new[:total_steps])
    vn_all = dev_raw(wl.v_new[:total_steps])
    # layers 1..: their own queries and new tokens (layer 0 is timed)
    layer_in = [tuple(dev_raw(a[:total_steps]) for a in (wl.q_dec_of(l), wl.k_new_of(l), wl.v_new_of(l)))
                for l in range(1, cfg.n_layers)]
    out = torch.empty((wl.n_req, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    window = np.full(wl.n_req, cfg.window, dtype=np.int32)

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    ev_every = max(1, args.event_every)
    # half a period in: with refreshes every 16 or 64 steps from the timed region's start, the
    # event-timed launches (a costlier launch) never come right after a refresh's host round trip
    att_ev = {i: (new_event(), new_event()) for i in range(ev_every // 2, K, ev_every)}
    ref_ev, lat_ev, gather_ev, copy_ev = {}, {}, {}, {}
    copied_at = {}  # device plan: blocks entered at an event-timed refresh (copied back after the run)
    slot_reqs = {}  # row of copied_hist -> the requests of that refresh (the other counts are stale)
    refresh_decode_steps = [t for t in range(total_steps) if wl.refreshes_at(t)]
    # the first refresh of a run loads every selected block (not so after a prologue refresh)
    first_refresh = refresh_decode_steps[0] if refresh_decode_steps and not prologue else None
    # the host-link leg replays the refresh states of the first decode steps of the timed region
    n_leg = host_leg * STEP_DECODE if total_steps + host_leg * STEP_DECODE <= cfg.window else 0
    leg_refreshes = [W + t for t in range(n_leg) if W + t < total_steps and wl.refreshes_at(W + t)]
    # the refreshes whose kernels are timed with events (every event costs stream time and host time
    # on the refresh's critical path): at most about 8, evenly spread over the timed steps
    timed_steps_with_refresh = [t for t in range(W, W + K) if wl.refreshes_at(t)]
    timed_refresh = set(timed_steps_with_refresh[::max(1, len(timed_steps_with_refresh) // 8)][:8])
    # the refreshes' events are made and recorded once before timing: made inside the loop they
    # cost ~60 us of host time per refresh while the GPU waits for the gather's launch
    ev_pool = [new_event() for _ in range(8 * len(timed_refresh) + 2 * len(leg_refreshes) + 8)]

    def mk_event():
        return ev_pool.pop() if ev_pool else new_event()

    first_copy_ev = (mk_event(), mk_event())  # the first refresh of a run loads every selected block
    first_blocks = []
    # the counts of blocks a refresh copied stay on the device while the loop runs: the plan writes
    # them into a row of this history, read after the run.  Sent to pinned host memory from a
    # stream of their own instead, even once in the warm-up, they left every later kernel of the
    # decode stream slower (attention 66.9 -> 69.6 us per launch, 70.0 -> 74.0 us per decode step)
    copied_hist = torch.zeros((len(timed_refresh) + len(leg_refreshes) + 2, wl.n_req), dtype=torch.int32,
                              device=dev)
    copied_host = []
    torch.cuda.synchronize()

    e = 2 if cfg.dtype == "bf16" else 4
    D, H = cfg.head_dim, cfg.n_heads
    partial_refresh = any(0 < len(wl.refreshes_at(t)) < wl.n_req for t in range(total_steps))
    overlap = dplan and cfg.n_layers == 1 and not args.reactive and (
        args.overlap == "on" or (args.overlap == "auto" and partial_refresh))
    if args.overlap == "on" and not overlap:
        raise SystemExit("--overlap on needs the device plan (--plan device), one layer and no --reactive")
    sloop = StaggeredLoop(sess, wl.ctx, window, out) if overlap else None
    loop = sloop.loop if overlap else DecodeLoop(sess, wl.ctx, window, out, device_counts=dplan)
    # the first launch of a kernel in the process loads its code, inside a timed dispatch's events:
    # the copy kernels run once before anything is timed
    if dplan:
        # a plan over the empty union planes the session starts with changes nothing
        import ctypes
        from lookahead_block_sparse_amd import LIB as _lib
        if _lib.lsa_gather_plan_device(ctypes.byref(sess._plan_args(0, wl.n_req)[0]),
                                       ctypes.c_void_p(sess.stream.cuda_stream)) != 0:
            raise RuntimeError(_lib.lsa_last_error().decode())
        torch.cuda.synchronize()
    elif not args.reactive:
        # one block into request 0's hot pool and out again
        sess.gather_many({0: np.zeros(1, dtype=np.int32)})
        sess.gather_many({0: np.zeros(0, dtype=np.int32)})
        torch.cuda.synchronize()
    rloop = ResidentLoop(sess, wl.ctx, window, out) if args.reactive else None
    outs_l = [torch.empty_like(out) for _ in range(1, cfg.n_layers)]
    loops_l = [DecodeLoop(sess, wl.ctx, window, outs_l[l - 1], layer=l, device_counts=dplan)
               for l in range(1, cfg.n_layers)]
    gather_host_s = []
    gather_blocks = []
    sel_hist = {}        # (request, selection version) -> ascending ids
    step_log = []        # (t, attended entries per request, selection version per request, event-timed)

    def refresh_group(t, reqs, hid, ev_ref=(None, None), ev_plan=(None, None), ev_copy=(None, None),
                      copy_slot=None):
        """One refresh of `reqs` and its gathers.  Returns the blocks copied (host plan) or None."""
        bias = bias_dev[reqs[0]:reqs[-1] + 1] if reqs == list(range(reqs[0], reqs[-1] + 1)) else \
            torch.stack([bias_dev[r] for r in reqs])
        if dplan:
            # refresh, plan and copy on the device: nothing comes back to the host
            sess.refresh_device(reqs, hid, bias, ev_begin=ev_ref[0], ev_end=ev_ref[1], ev_plan=ev_plan,
                                ev_latent=lat_ev.get(t, (None, None)),
                                copied_out=copied_hist[copy_slot] if copy_slot is not None else None)
            if copy_slot is not None:
                slot_reqs[copy_slot] = list(reqs)
            return None
        sel = sess.refresh(reqs, hid, bias, ev_begin=ev_ref[0], ev_end=ev_ref[1],
                           ev_latent=lat_ev.get(t, (None, None)))
        copied = 0
        for r, (c, _) in sess.gather_many(sel, ev_copy=ev_copy).items():
            copied += c
            sel_hist[(r, int(sess.sel_version[r]))] = sess.sel_host[r]
        return copied

    def reactive_step(t, timed_idx):
        evs = (None, None)
        ev = (None, None)
        if timed_idx is not None and timed_idx in att_ev:
            ref_ev[t] = evs = (mk_event(), mk_event())
            ev = att_ev[timed_idx]
        rloop.step(t, hid_at[t], bias_dev, q_all[t], kn_all[t], vn_all[t], ev_refresh=evs, ev_attn=ev)
        if timed_idx is not None:
            step_log.append((t, None, None, timed_idx in att_ev))

    def step(t, timed_idx):
        if rloop is not None:
            return reactive_step(t, timed_idx)
        reqs = wl.refreshes_at(t)
        ev = att_ev.get(timed_idx, (None, None)) if timed_idx is not None else (None, None)
        if (sloop is not None and 0 < len(reqs) < wl.n_req and not (timed_idx is not None and t in timed_refresh)
                and t != first_refresh and ev[0] is None):
            # the refreshing requests on the second stream, beside the others' attention
            bias = torch.stack([bias_dev[r] for r in reqs])
            sloop.step(t, q_all[t], kn_all[t], vn_all[t], refresh=reqs, hidden=hid_at[t], bias=bias)
            if timed_idx is not None:
                step_log.append((t, None, sess.sel_version.copy(), False))
            return
        if reqs:
            timed_ref = timed_idx is not None and t in timed_refresh
            if timed_ref:
                ref_ev[t] = (mk_event(), mk_event())
                gather_ev[t] = (mk_event(), mk_event())
                if sess.rank:
                    lat_ev[t] = (mk_event(), mk_event())
            evs = ref_ev.get(t, (None, None))
            if dplan:
                pev = gather_ev[t] if timed_ref else (first_copy_ev if t == first_refresh else (None, None))
                slot = None
                if timed_ref:
                    slot = copied_at[t] = len(copied_at)
                elif t == first_refresh:
                    slot = copied_at["first"] = len(copied_at)
                refresh_group(t, reqs, hid_at[t], ev_ref=evs, ev_plan=pev, copy_slot=slot)
            else:
                h0 = time.perf_counter()
                if timed_ref:
                    gather_ev[t][0].record(sess.stream)
                    cev = copy_ev[t] = (mk_event(), mk_event())
                elif t == first_refresh:
                    cev = first_copy_ev
                else:
                    cev = (None, None)
                copied = refresh_group(t, reqs, hid_at[t], ev_ref=evs, ev_copy=cev)
                if timed_ref:
                    gather_ev[t][1].record(sess.stream)
                    gather_host_s.append(time.perf_counter() - h0)
                    gather_blocks.append(copied)
                elif t == first_refresh:
                    first_blocks.append(copied)
        loop.step(t, q_all[t], kn_all[t], vn_all[t], ev[0], ev[1])
        for lp, (ql, kl, vl) in zip(loops_l, layer_in):
            lp.step(t, ql[t], kl[t], vl[t])
        if timed_idx is not None:
            step_log.append((t, None if dplan else loop.n_sel.copy(), sess.sel_version.copy(), timed_idx in att_ev))

    if prologue:
        note(f"prologue refresh of {len(prologue)} staggered requests")
        refresh_group(-1, prologue, hid_at[-1])
        torch.cuda.synchronize()
    note(f"warm-up {W // STEP_DECODE} steps ({W} decode steps)")
    for t in range(W):
        step(t, None)
    torch.cuda.synchronize()
    if dplan:
        sess.check_plan_status()
    note(f"timing {K // STEP_DECODE} steps ({K} decode steps)")
    # no garbage-collector pass inside the timed region: a full pass over this process's objects
    # stops the host for tens of milliseconds, which a loop whose steps take microseconds of GPU
    # time cannot hide (a serving loop would freeze its long-lived objects the same way)
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    note(f"timed region {elapsed * 1e3:.2f} ms")
    if dplan:
        sess.check_plan_status()  # any refresh of the run that gave up or did not fit raises here

    attn_ms = np.array([a.elapsed_time(b) for a, b in att_ev.values()])
    sel_at = {}
    if dplan:
        # the selections in force at the event-timed steps, recomputed after the timed region (the
        # refresh is deterministic): the governing refresh of each request
        cache = {}
        for t, _, _, timed_ev in step_log:
            if not timed_ev:
                continue
            sel_at[t] = {}
            for r in range(wl.n_req):
                k = max(i for i, tk in enumerate(wl.refresh_steps[r]) if tk <= t)
                if (r, k) not in cache:
                    hid_rk = dev_raw(wl.hidden[r][k][None])
                    cache[(r, k)] = sess.refresh([r], hid_rk, bias_dev[r:r + 1])[r]
                sel_at[t][r] = cache[(r, k)]
    if rloop is not None:
        # the selections of the event-timed steps, recomputed after the timed region (the refresh
        # is deterministic), give their attended bytes
        for t, _, _, timed_ev in step_log:
            if timed_ev:
                sel_at[t] = sess.refresh(list(range(wl.n_req)), hid_at[t], bias_dev)
        step_log = [(t, None, None, te) for t, _, _, te in step_log]
    # algorithmic bytes of every timed attention launch: window tokens + tokens of the attended
    # selected blocks (below the window start), K and V, plus q and the table entries
    attn_bytes, attn_tokens, with_ev = [], [], []
    for t, n_att, ver, timed_ev in step_log:
        if (rloop is not None or dplan) and not timed_ev:
            continue
        with_ev.append(timed_ev)
        toks = 0
        n_entries = 0
        for r in range(wl.n_req):
            L = int(wl.ctx[r]) + t + 1
            ws = max(0, L - cfg.window)
            toks += min(L, cfg.window)
            if rloop is not None or dplan:
                ids = sel_at[t][r]
            else:
                ids = sel_hist.get((r, int(ver[r])), np.zeros(0, dtype=np.int32))
            n_entries += len(ids)  # the decode reads every table entry (in-window blocks are skipped)
            n = int(np.searchsorted(ids, (ws + 63) // 64, side="left"))
            if n > 0:
                last = int(ids[n - 1])
                toks += 64 * (n - 1) + min(64, ws - 64 * last)
        attn_tokens.append(toks)
        attn_bytes.append(toks * 2 * D * e + wl.n_req * H * D * e + 8 * n_entries)
    ref_us = np.array([1e3 * a.elapsed_time(b) for a, b in ref_ev.values()])
    lat_us = np.array([1e3 * a.elapsed_time(b) for a, b in lat_ev.values()])
    gat_us = np.array([1e3 * a.elapsed_time(b) for a, b in gather_ev.values()])
    copy_us = np.array([1e3 * a.elapsed_time(b) for a, b in copy_ev.values()])
    # steady-state decode: between the start stamps of two event-timed attention launches lie the
    # steps from the first to the one before the second, and the refresh work of the second one's
    # step (a refresh precedes its step's decode), so windows with a refresh in (i1, i2] are left out
    idx = sorted(att_ev)
    steady = [(i2 - i1, 1e3 * att_ev[i1][0].elapsed_time(att_ev[i2][0])) for i1, i2 in zip(idx, idx[1:])
              if not any(wl.refreshes_at(W + i) for i in range(i1 + 1, i2 + 1))]
    attn_bytes = np.array(attn_bytes, dtype=np.float64)
    ev_bytes = attn_bytes[np.array(with_ev)]  # the launches the events timed, in the same order
    achieved = ev_bytes.sum() / (attn_ms.sum() * 1e-3) / 1e9  # GB/s

    # refresh algorithmic bytes: keys, W_q, the hidden states and the ids of the requests one
    # refresh serves (all of them when aligned; the staggered mix refreshes one request at a time)
    ref_reqs = wl.refreshes_at(sorted(ref_ev)[0]) if ref_ev else list(range(wl.n_req))
    n_blocks_ref = int(sum(int(wl.n_blocks[r]) for r in ref_reqs))
    q_in_bytes = (len(ref_reqs) * cfg.n_idx * cfg.q_rank * e) if cfg.q_rank else len(ref_reqs) * cfg.d_model * e
    ids_per_refresh = None
    if dplan and sel_at:
        ids_per_refresh = np.mean([sum(len(v) for r, v in s_.items() if r in ref_reqs) for s_ in sel_at.values()])
    elif rloop is not None and sel_at:
        ids_per_refresh = np.mean([sum(len(v) for v in s_.values()) for s_ in sel_at.values()])
    else:
        ids_per_refresh = sum(len(sess.sel_host[r]) for r in ref_reqs)
    ref_bytes = cfg.n_idx * cfg.q_in * cfg.d_idx * e + n_blocks_ref * cfg.n_idx * cfg.d_idx * e + q_in_bytes
    if dplan:  # the bit planes the device plan reads are the refresh's whole result (no ids, no counts)
        ref_bytes += 8 * (cfg.n_idx + 1) * int(sum(int(sess.word_off[r + 1] - sess.word_off[r]) for r in ref_reqs))
    else:  # the ids and counts
        ref_bytes += int(4 * ids_per_refresh) + 4 * len(ref_reqs)
    if rloop is not None:  # the table pairs the refresh writes for the resident pool
        ref_bytes += int(8 * ids_per_refresh)
    lat_bytes = (cfg.n_idx * cfg.q_rank * cfg.d_model * e + len(ref_reqs) * cfg.d_model * e
                 + len(ref_reqs) * cfg.n_idx * cfg.q_rank * e) if cfg.q_rank else 0

    bb = sess.block_bytes * cfg.n_layers
    torch.cuda.synchronize()

    def slot_blocks(slot):
        if not copied_host:
            copied_host.append(copied_hist.cpu().numpy())
        return int(copied_host[0][slot][slot_reqs[slot]].sum())

    gather_copy = None
    if dplan and len(gat_us):
        # plan + copy kernels (events on the plan's dispatch start and the copy's end)
        blocks = np.array([slot_blocks(copied_at[t]) for t in sorted(gather_ev)], dtype=np.float64)
        gather_copy = {"source": ("pinned host memory (host link)" if args.cold == "host" else "device memory (HBM)"),
                       "kernels": "plan_kernel + copy_kernel", "plan_and_copy_us": float(np.median(gat_us)),
                       "blocks_per_refresh": float(blocks.mean()), "bytes_per_refresh": float(blocks.mean() * bb),
                       "GB_per_s": float(np.median(blocks * bb / (gat_us * 1e-6) / 1e9))}
        if "first" in copied_at:
            fb = slot_blocks(copied_at["first"]) * bb
            fus = 1e3 * first_copy_ev[0].elapsed_time(first_copy_ev[1])
            gather_copy["first_refresh"] = {"blocks": fb // bb, "bytes": int(fb), "plan_and_copy_us": fus,
                                            "GB_per_s": fb / (fus * 1e-6) / 1e9}
        gather_blocks = blocks.tolist()
    if copy_ev and gather_blocks and not dplan:
        # cold-pool bytes each copy kernel reads (every layer's copy of every entering block); with
        # the cold pool in HBM the kernel writes as many again to the hot pool
        later = np.array(gather_blocks, dtype=np.float64) * bb
        gather_copy = {
            "source": "pinned host memory (host link)" if args.cold == "host" else "device memory (HBM)",
            "kernels": "gather_kernel (host plan)",
            "bytes_per_refresh": float(later.mean()),
            "copy_us": float(np.median(copy_us)),
            "GB_per_s": float(np.median(later / (copy_us * 1e-6) / 1e9)),
        }
        if first_blocks:
            fb = first_blocks[0] * bb
            fus = 1e3 * first_copy_ev[0].elapsed_time(first_copy_ev[1])
            gather_copy["first_refresh"] = {"blocks": int(first_blocks[0]), "bytes": int(fb), "copy_us": fus,
                                            "GB_per_s": fb / (fus * 1e-6) / 1e9}
    if gather_copy is not None and args.cold == "host":
        gather_copy["link_peak_GB_per_s"] = host_link_peak(dev)

    # the same loop continued with the cold pool's pinned host copy: every gather crosses the host
    # link (same blocks, same residency state); timed over whole steps by the wall clock
    host_cold = None
    if n_leg and leg_refreshes:
        sess.use_cold("host")
        leg_evs, leg_slots = [], []
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        tl0 = time.perf_counter()
        for t in range(n_leg):
            ts = W + t  # the refresh states and decode inputs of timed step ts, replayed
            reqs = wl.refreshes_at(ts) if ts < total_steps else []
            if reqs:
                ev = (mk_event(), mk_event())
                leg_evs.append(ev)
                if dplan:
                    slot = len(copied_at) + len(leg_slots)
                    leg_slots.append(slot)
                    refresh_group(ts, reqs, hid_at[ts], ev_plan=ev, copy_slot=slot)
                else:
                    leg_slots.append(refresh_group(ts, reqs, hid_at[ts], ev_copy=ev))
            tt = total_steps + t  # the window keeps growing: positions past the timed region
            loop.step(tt, q_all[ts], kn_all[ts], vn_all[ts])
            for lp, (ql, kl, vl) in zip(loops_l, layer_in):
                lp.step(tt, ql[ts], kl[ts], vl[ts])
        torch.cuda.synchronize()
        leg_s = time.perf_counter() - tl0
        gc.enable()
        if dplan:
            sess.check_plan_status()
        us = np.array([1e3 * a.elapsed_time(b) for a, b in leg_evs])
        copied_host.clear()  # the leg's refreshes wrote their rows since the last read
        blocks = (np.array([slot_blocks(s_) for s_ in leg_slots], dtype=np.float64) if dplan
                  else np.array(leg_slots, dtype=np.float64))
        host_cold = {
            "tokens_per_s": wl.n_req * n_leg / leg_s,
            "steps": host_leg, "decode_steps": n_leg, "seconds": leg_s,
            "gather_us": float(np.median(us)),
            "gather_kernels": "plan_kernel + copy_kernel" if dplan else "gather_kernel (host plan)",
            "gather_bytes_per_refresh": float(blocks.mean() * bb),
            "gather_GB_per_s": float(np.median(blocks * bb / (us * 1e-6) / 1e9)),
            "link_peak_GB_per_s": host_link_peak(dev),
            "note": "the loop continued over whole steps with the cold pool's pinned host copy (the refresh "
                    "states of the timed region's first steps replayed): every gather reads over the host link"}
        sess.use_cold("device")

    # recall of the planted relevant blocks (4 x 1M): the share of them in the selections in force at
    # the event-timed steps
    planted_recall = None
    if cfg.planted_frac > 0 and sel_at:
        rec = [np.isin(wl.planted[r], s_[r]).mean() for s_ in sel_at.values() for r in range(wl.n_req)
               if len(wl.planted[r])]
        planted_recall = float(np.mean(rec)) if rec else None
    elif cfg.planted_frac > 0 and sel_hist:
        rec = [np.isin(wl.planted[r], ids).mean() for (r, _), ids in sel_hist.items() if len(wl.planted[r])]
        planted_recall = float(np.mean(rec)) if rec else None

    khash = kernel_hash()
    res = {
        "metric": METRIC,
        "value": wl.n_req * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K // STEP_DECODE,
        "warmup": W // STEP_DECODE,
        "ms_per_step": elapsed * 1e3 / (K // STEP_DECODE),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {wl.n_req} requests x {int(wl.ctx[0])}-token context, {cfg.n_idx} indexers "
                         f"(d_model {cfg.d_model}, d_idx {cfg.d_idx}), {cfg.n_heads} q-heads / 1 kv-head x "
                         f"{cfg.head_dim}, window {cfg.window}, refresh every {cfg.tau} steps, "
                         f"{int(100 * cfg.planted_frac)}% planted + background density {cfg.density}"
                         + (", every block selected (dense comparator)" if args.select == "all" else "")
                         + (f", {cfg.n_layers} attention layers per selection" if cfg.n_layers > 1 else "")
                         + (f", hidden-state correlation {cfg.hidden_rho}" if cfg.hidden_rho else "")
                         + (", reactive comparator: every block resident, scored every step" if args.reactive
                            else "")
                         + (f", low-rank query projection r={cfg.q_rank}" if cfg.q_rank else "")
                         + (f", selection level sigmoid > {args.level}" if args.level != 0.5 else "")),
            "step": f"{STEP_DECODE} decode steps of every request (one refresh interval at tau = 64): refreshes, "
                    "gathers and sparse decode",
            "cold_pool": args.cold,
            "tau": cfg.tau,
            "layers": cfg.n_layers,
            "hidden_rho": cfg.hidden_rho,
            "select": args.select,
            "level": args.level,
            "reactive": bool(args.reactive),
            "q_rank": cfg.q_rank,
            "residency_plan": "device" if dplan else ("none (resident)" if args.reactive else "host"),
            "staggered_overlap": bool(overlap),
            "requests": wl.n_req,
            "context_tokens": int(wl.ctx[0]) if len(set(wl.ctx.tolist())) == 1 else wl.ctx.tolist(),
            "seed": args.seed,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_kernel (split-K block-sparse flash-decode)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": stored_traffic(cfg.name),
            "algorithmic_bytes_per_launch": float(ev_bytes.mean()),
            "timed_launches": int(len(attn_ms)),
            "mean_launch_us": float(attn_ms.mean() * 1e3),
        },
        "decode_steps_timed": K,
        "decode_attn_us": float(attn_ms.mean() * 1e3),
        "attended_tokens_per_step": float(np.mean(attn_tokens)),
        "planted_recall": planted_recall,
        "refresh_us": float(np.median(ref_us)) if len(ref_us) else None,
        "refresh_us_p90": float(np.percentile(ref_us, 90)) if len(ref_us) else None,
        "refresh_timed": int(len(ref_us)),
        "refreshes_in_timed_region": int(sum(len(wl.refreshes_at(t)) > 0 for t in range(W, W + K))),
        "decode_steady": ({"tokens_per_s": wl.n_req * sum(n for n, _ in steady) / (sum(u for _, u in steady) * 1e-6),
                           "us_per_step": sum(u for _, u in steady) / sum(n for n, _ in steady),
                           "steps": int(sum(n for n, _ in steady))} if steady else None),
        "refresh_roofline": ({"kernel": ("refresh_kernel (encode + score + threshold + union bit planes, one launch; "
                                         "the device plan ranks the selected blocks)" if dplan else
                                         "refresh_kernel (encode + score + compaction, one launch)"),
                              "achieved": ref_bytes / (np.median(ref_us) * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": ref_bytes / (np.median(ref_us) * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "algorithmic_bytes": ref_bytes, "requests_per_refresh": len(ref_reqs),
                              "traffic": stored_traffic(cfg.name, "refresh_kernel")}
                             if len(ref_us) else None),
        "latent_us": float(np.median(lat_us)) if len(lat_us) else None,
        "latent_roofline": ({"achieved": lat_bytes / (np.median(lat_us) * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": lat_bytes / (np.median(lat_us) * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": lat_bytes} if len(lat_us) else None),
        "gather_us": float(np.median(gat_us)) if len(gat_us) else None,
        "gather_blocks_per_refresh": float(np.mean(gather_blocks)) if gather_blocks else None,
        "gather_host_plan_ms": float(np.median(gather_host_s) * 1e3) if gather_host_s else None,
        "gather_copy": gather_copy,
        "cold_pool_in_pinned_host_memory": host_cold,
        "kernel_sources_sha256_16": khash,
        "refresh_sources_sha256_16": kernel_hash("refresh_kernel"),
    }
    if not args.no_ceiling:
        # the same byte counts read by the read probe: the kernels' fraction of what the memory
        # delivers to a plain cold read (measured after the timed region, outside it)
        note("measuring the cold-read ceiling of the kernels' byte counts (read probe)")
        c = read_ceiling_best(int(ev_bytes.mean()))
        if c is not None:
            c["frac"] = achieved / c["GB_per_s"]
            res["roofline"]["measured_ceiling"] = c
        if res["refresh_roofline"] is not None:
            c = read_ceiling_best(int(ref_bytes))
            if c is not None:
                c["frac"] = res["refresh_roofline"]["achieved"] / c["GB_per_s"]
                res["refresh_roofline"]["measured_ceiling"] = c
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = n
    if not args.no_cpu_baseline:
        note("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_steps, args.seed)
    return res


if __name__ == "__main__":
    main()
