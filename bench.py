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
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="ctx1m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold", choices=("device", "host"), default="device")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    ap.add_argument("--plan", choices=("device", "host"), default="host",
                    help="where the residency plan of a refresh is made: on the host "
                         "(lsa_gather_blocks_batch; the default, and always with --cold host, as the device "
                         "plan copies within device memory) or on the device (lsa_gather_plan_device, no host "
                         "round trip)")
    ap.add_argument("--reactive", action="store_true",
                    help="reactive comparator: every block resident in HBM, the index scored at every step "
                         "and the decode reading the selected blocks in place (refresh cadence 1, no "
                         "gathers, no host round trip)")
    ap.add_argument("--event-every", type=int, default=16,
                    help="time the attention kernel with HIP events on every N-th timed step (the events "
                         "take the dispatch's own stamps but still cost stream time)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no run: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 pass (both taken with --calib-copy-mib) into "
                         "profiles/attn_kernel_<workload>_traffic.json")
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


def kernel_hash() -> str:
    """Hash of the sources the attention kernel is built from (its counters stay valid while this
    is unchanged)."""
    h = hashlib.sha256()
    for name in ("decode.hip", "lsa_internal.hpp"):
        h.update((ROOT / "lookahead_block_sparse_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, calib_mib: int) -> dict:
    """HBM bytes per attn_kernel launch from two rocprofv3 counter passes.  Each counter is scaled
    by what it reads for the plain device copy of calib_mib MiB in the same pass (read calib bytes,
    write calib bytes), which takes out the counters' units and any sampling of channels."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        calib = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        attn = [float(r["Counter_Value"]) for r in rows if "attn_kernel" in r["Kernel_Name"]]
        if not attn or not calib:
            raise SystemExit(f"{path}: no attn_kernel or copy dispatches with {counter}")
        return float(np.mean(attn)), max(calib), len(attn)

    n = calib_mib << 20
    f_attn, f_cal, n_f = per_kernel(fetch_csv, "FETCH_SIZE")
    w_attn, w_cal, n_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = n / (f_cal * 1024.0), n / (w_cal * 1024.0)
    return {
        "kernel": "attn_kernel",
        "workload": workload,
        "dispatches": {"fetch_pass": n_f, "write_pass": n_w},
        "fetch_size_kib_per_dispatch": f_attn,
        "write_size_kib_per_dispatch": w_attn,
        "calib_copy_bytes": n,
        "calib_fetch_size_kib": f_cal,
        "calib_write_size_kib": w_cal,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "traffic_bytes_per_launch": f_attn * 1024.0 * f_scale + w_attn * 1024.0 * w_scale,
        "kernel_sources_sha256_16": kernel_hash(),
    }


def stored_traffic(workload: str, khash: str):
    """HBM traffic of the attention kernel from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    f = ROOT / "profiles" / f"attn_kernel_{workload}_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("kernel_sources_sha256_16") != khash:
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
    `sample_steps` decode steps per request."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cfg = wl.cfg
    dt = cfg.dtype
    w_q = oracle.decode_values(wl.w_q, dt)
    t_ref = 0.0
    refs = {}
    for r in range(wl.n_req):
        t0 = time.perf_counter()
        keys = oracle.decode_values(wl.keys[r], dt)
        res = oracle.refresh(oracle.decode_values(wl.hidden[r][0], dt), w_q, keys, wl.bias[r])
        t_ref += time.perf_counter() - t0
        refs[r] = res
    rng = np.random.default_rng(seed)
    steps = sorted(rng.choice(np.arange(1, min(cfg.steps, 64)), size=sample_steps, replace=False).tolist())
    t_dec = 0.0
    n = 0
    for r in range(wl.n_req):
        kp, vp = wl.kv_prefill(r)
        N = int(wl.ctx[r])
        for t in steps:
            t0 = time.perf_counter()
            L = N + t + 1
            pos = oracle.token_set(L, cfg.window, refs[r].ids, cfg.block)
            lo = pos < N
            k = np.empty((len(pos), cfg.head_dim))
            v = np.empty((len(pos), cfg.head_dim))
            k[lo] = oracle.decode_values(kp[pos[lo]], dt)
            v[lo] = oracle.decode_values(vp[pos[lo]], dt)
            k[~lo] = oracle.decode_values(wl.k_new[pos[~lo] - N, r], dt)
            v[~lo] = oracle.decode_values(wl.v_new[pos[~lo] - N, r], dt)
            oracle.attention(oracle.decode_values(wl.q_dec[t, r], dt), k, v, cfg.head_dim ** -0.5)
            t_dec += time.perf_counter() - t0
            n += 1
    return {
        "value": n / t_dec,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} request-steps (steps {steps} of each of {wl.n_req} requests, selection of the "
                  f"first refresh) and one refresh per request; float64 NumPy",
        "refresh_us_per_request": 1e6 * t_ref / wl.n_req,
        "seconds": t_dec + t_ref,
    }


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
        d = traffic_summary(*args.traffic_summary, workload=args.workload, calib_mib=args.calib_copy_mib)
        out = ROOT / "profiles" / f"attn_kernel_{args.workload}_traffic.json"
        out.write_text(json.dumps(d, indent=1) + "\n")
        print(json.dumps(d))
        return

    if args.denoise:
        print(json.dumps(run_denoise(args)), flush=True)
        return

    import torch

    from lookahead_block_sparse_amd.session import DecodeLoop, LSASession, ResidentLoop
    from workloads import build_workload, get_config

    def note(msg):
        print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)

    cfg = get_config(args.workload)
    W, K = args.warmup, args.steps
    total_steps = W + K
    if args.tau > 0:
        cfg = cfg.scaled(tau=args.tau)
    if args.density > 0:
        cfg = cfg.scaled(density=("fixed", args.density))
    if args.layers > 1 or args.hidden_rho:
        cfg = cfg.scaled(n_layers=args.layers, hidden_rho=args.hidden_rho)
    if args.select == "all":
        cfg = cfg.scaled(tau=max(cfg.tau, total_steps + 1), planted_frac=0.0)  # one refresh, at step 0
    if args.q_rank > 0:
        cfg = cfg.scaled(q_rank=args.q_rank)
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
    sess = LSASession(dtype=cfg.dtype, n_idx=cfg.n_idx, d_model=cfg.d_model, d_idx=cfg.d_idx,
                      n_heads=cfg.n_heads, head_dim=cfg.head_dim, win_cap=cfg.window, n_blocks=wl.n_blocks,
                      w_q=wl.w_q, keys=wl.keys, cold_on_device=(args.cold == "device"), with_masks=False,
                      n_layers=cfg.n_layers, w_down=wl.w_down,
                      device_plan=(args.plan == "device" and not args.reactive and args.cold == "device"))
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
    # (stacked per refresh step, in request order)
    hid_at = {}
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
    ref_ev = {}
    lat_ev = {}
    gather_ev = {}
    copy_ev = {}  # the copy kernel alone (host plan)
    first_refresh = min(t for t in range(total_steps) if wl.refreshes_at(t))
    # the refreshes whose kernels are timed with events (every event costs stream time and host time
    # on the refresh's critical path): at most about 8, evenly spread over the timed steps
    refresh_steps = [t for t in range(W, W + K) if wl.refreshes_at(t)]
    timed_refresh = set(refresh_steps[::max(1, len(refresh_steps) // 8)])
    # the refreshes' events are made and recorded once before timing: made inside the loop they
    # cost ~60 us of host time per refresh while the GPU waits for the gather's launch
    ev_pool = [new_event() for _ in range(8 * len(timed_refresh) + 8)]

    def mk_event():
        return ev_pool.pop() if ev_pool else new_event()

    first_copy_ev = (mk_event(), mk_event())  # the first refresh loads every selected block
    first_blocks = []
    torch.cuda.synchronize()

    e = 2 if cfg.dtype == "bf16" else 4
    D, H = cfg.head_dim, cfg.n_heads
    dplan = sess.device_plan
    loop = DecodeLoop(sess, wl.ctx, window, out, device_counts=dplan)
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
    step_log = []        # (t, attended entries per request, selection version per request)

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
        timed_ref = timed_idx is not None and t in timed_refresh
        if reqs:
            if timed_ref:
                ref_ev[t] = (mk_event(), mk_event())
                gather_ev[t] = (mk_event(), mk_event())
                if sess.rank:
                    lat_ev[t] = (mk_event(), mk_event())
            hid = hid_at[t]
            bias = bias_dev[reqs[0]:reqs[-1] + 1] if reqs == list(range(reqs[0], reqs[-1] + 1)) else \
                torch.stack([bias_dev[r] for r in reqs])
            evs = ref_ev.get(t, (None, None)) if timed_ref else (None, None)
            if dplan:
                # refresh, plan and copy on the device: nothing comes back to the host
                pev = gather_ev.get(t, (None, None)) if timed_ref else \
                    (first_copy_ev if t == first_refresh else (None, None))
                sess.refresh_device(reqs, hid, bias, ev_begin=evs[0], ev_end=evs[1], ev_plan=pev)
            else:
                sel = sess.refresh(reqs, hid, bias, ev_begin=evs[0], ev_end=evs[1],
                                   ev_latent=lat_ev.get(t, (None, None)))
        if reqs and not dplan:
            h0 = time.perf_counter()
            if timed_ref:
                gather_ev[t][0].record(sess.stream)
                cev = copy_ev[t] = (mk_event(), mk_event())
            elif t == first_refresh:
                cev = first_copy_ev
            else:
                cev = (None, None)
            copied = 0
            for r, (c, _) in sess.gather_many(sel, ev_copy=cev).items():
                copied += c
                sel_hist[(r, int(sess.sel_version[r]))] = sess.sel_host[r]
            if timed_ref:
                gather_ev[t][1].record(sess.stream)
                gather_host_s.append(time.perf_counter() - h0)
                gather_blocks.append(copied)
            elif t == first_refresh:
                first_blocks.append(copied)
        if timed_idx is None:
            loop.step(t, q_all[t], kn_all[t], vn_all[t])
            for lp, (ql, kl, vl) in zip(loops_l, layer_in):
                lp.step(t, ql[t], kl[t], vl[t])
        else:
            ev = att_ev.get(timed_idx, (None, None))
            loop.step(t, q_all[t], kn_all[t], vn_all[t], ev[0], ev[1])
            for lp, (ql, kl, vl) in zip(loops_l, layer_in):
                lp.step(t, ql[t], kl[t], vl[t])
            step_log.append((t, None if dplan else loop.n_sel.copy(), sess.sel_version.copy(), timed_idx in att_ev))

    note(f"warm-up {W} steps")
    for t in range(W):
        step(t, None)
    torch.cuda.synchronize()
    if dplan and [t for t in range(W) if wl.refreshes_at(t)] == [first_refresh]:
        first_blocks.append(int(sess.copied_dev.sum().item()))  # the one warm-up refresh
    note(f"timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    note(f"timed region {elapsed * 1e3:.2f} ms")

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
        # the table entries the decode reads: every selected block of the step
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
                n_entries += len(ids)  # the decode reads every table entry (in-window ones masked)
                n = int(np.searchsorted(ids, (ws + 63) // 64, side="left"))
            else:
                ids = sel_hist[(r, int(ver[r]))] if n_att[r] > 0 else None
                n = int(n_att[r])
                n_entries += n
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

    # refresh algorithmic bytes for one group of all requests
    n_blocks_total = int(wl.n_blocks.sum())
    # (low rank: the Query Encoder reads B and the latents of every indexer instead of W_q and h)
    q_in_bytes = (wl.n_req * cfg.n_idx * cfg.q_rank * e) if cfg.q_rank else wl.n_req * cfg.d_model * e
    ref_bytes = (cfg.n_idx * cfg.q_in * cfg.d_idx * e + n_blocks_total * cfg.n_idx * cfg.d_idx * e
                 + q_in_bytes + 4 * sum(len(x) for x in sess.sel_host) + 4 * wl.n_req)
    lat_bytes = (cfg.n_idx * cfg.q_rank * cfg.d_model * e + wl.n_req * cfg.d_model * e
                 + wl.n_req * cfg.n_idx * cfg.q_rank * e) if cfg.q_rank else 0
    if dplan and sel_at:  # ids of the recomputed selections, plus the bit planes the plan reads
        n_ids = np.mean([sum(len(v) for v in s_.values()) for s_ in sel_at.values()])
        ref_bytes = (cfg.n_idx * cfg.q_in * cfg.d_idx * e + n_blocks_total * cfg.n_idx * cfg.d_idx * e
                     + q_in_bytes + int(4 * n_ids) + 8 * (cfg.n_idx + 1) * int(sess.word_off[-1]) + 4 * wl.n_req)
    if rloop is not None:  # ids and table pairs of the recomputed selections
        n_ids = np.mean([sum(len(v) for v in s.values()) for s in sel_at.values()]) if sel_at else 0.0
        ref_bytes = (cfg.n_idx * cfg.q_in * cfg.d_idx * e + n_blocks_total * cfg.n_idx * cfg.d_idx * e
                     + q_in_bytes + int(12 * n_ids) + 4 * wl.n_req)

    gather_copy = None
    if dplan and len(gat_us):
        # plan + copy kernels (events on the plan's dispatch start and the copy's end)
        bb = sess.block_bytes * cfg.n_layers
        gather_copy = {"source": "device memory (HBM)", "kernels": "plan_kernel + copy_kernel",
                       "plan_and_copy_us": float(np.median(gat_us)),
                       "bytes_last_refresh": int(sess.copied_dev.sum().item()) * bb}
        if first_blocks:
            fb = first_blocks[0] * bb
            fus = 1e3 * first_copy_ev[0].elapsed_time(first_copy_ev[1])
            gather_copy["first_refresh"] = {"blocks": int(first_blocks[0]), "bytes": int(fb), "plan_and_copy_us": fus,
                                            "GB_per_s": fb / (fus * 1e-6) / 1e9}
    if copy_ev and gather_blocks:
        # cold-pool bytes each copy kernel reads (every layer's copy of every entering block); with
        # the cold pool in HBM the kernel writes as many again to the hot pool
        bb = sess.block_bytes * cfg.n_layers
        later = np.array(gather_blocks, dtype=np.float64) * bb
        gather_copy = {
            "source": "pinned host memory (host link)" if args.cold == "host" else "device memory (HBM)",
            "bytes_per_refresh": float(later.mean()),
            "copy_us": float(np.median(copy_us)),
            "GB_per_s": float(np.median(later / (copy_us * 1e-6) / 1e9)),
        }
        if first_blocks:
            fb = first_blocks[0] * bb
            fus = 1e3 * first_copy_ev[0].elapsed_time(first_copy_ev[1])
            gather_copy["first_refresh"] = {"blocks": int(first_blocks[0]), "bytes": int(fb), "copy_us": fus,
                                            "GB_per_s": fb / (fus * 1e-6) / 1e9}
        if args.cold == "host":
            gather_copy["link_peak_GB_per_s"] = host_link_peak(dev)
    khash = kernel_hash()
    res = {
        "metric": METRIC,
        "value": wl.n_req * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": elapsed * 1e3 / K,
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
                         + (f", low-rank query projection r={cfg.q_rank}" if cfg.q_rank else "")),
            "cold_pool": args.cold,
            "tau": cfg.tau,
            "layers": cfg.n_layers,
            "hidden_rho": cfg.hidden_rho,
            "select": args.select,
            "reactive": bool(args.reactive),
            "q_rank": cfg.q_rank,
            "residency_plan": "device" if dplan else ("none (resident)" if args.reactive else "host"),
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
            "traffic": stored_traffic(cfg.name, khash),
            "algorithmic_bytes_per_launch": float(ev_bytes.mean()),
            "timed_launches": int(len(attn_ms)),
            "mean_launch_us": float(attn_ms.mean() * 1e3),
        },
        "decode_attn_us": float(attn_ms.mean() * 1e3),
        "attended_tokens_per_step": float(np.mean(attn_tokens)),
        "refresh_us": float(np.median(ref_us)) if len(ref_us) else None,
        "refresh_us_p90": float(np.percentile(ref_us, 90)) if len(ref_us) else None,
        "decode_steady": ({"tokens_per_s": wl.n_req * sum(n for n, _ in steady) / (sum(u for _, u in steady) * 1e-6),
                           "us_per_step": sum(u for _, u in steady) / sum(n for n, _ in steady),
                           "steps": int(sum(n for n, _ in steady))} if steady else None),
        "refresh_roofline": ({"achieved": ref_bytes / (np.median(ref_us) * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": ref_bytes / (np.median(ref_us) * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "algorithmic_bytes": ref_bytes} if len(ref_us) else None),
        "latent_us": float(np.median(lat_us)) if len(lat_us) else None,
        "latent_roofline": ({"achieved": lat_bytes / (np.median(lat_us) * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": lat_bytes / (np.median(lat_us) * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": lat_bytes} if len(lat_us) else None),
        "gather_us": float(np.median(gat_us)) if len(gat_us) else None,
        "gather_blocks_per_refresh": float(np.mean(gather_blocks)) if gather_blocks else None,
        "gather_host_plan_ms": float(np.median(gather_host_s) * 1e3) if gather_host_s else None,
        "gather_copy": gather_copy,
        "kernel_sources_sha256_16": khash,
    }
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
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
