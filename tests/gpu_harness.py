"""Helpers for the GPU parity tests: run a workload through the library and through the oracle.

Inputs come from the seeded generators (workloads/), conditioned with the oracle (planted keys,
logits moved off the decision boundary).  Nothing here computes any step of the method on the
GPU side except through liblsa.so.
"""

from __future__ import annotations

import os
import sys
import time
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np
import torch

import oracle
from workloads import build_workload


def log(msg: str) -> None:
    """Print a progress line (and append it to $LSA_TEST_REPORT when set)."""
    line = f"[{time.strftime('%H:%M:%S')}] {msg}"
    print(line, flush=True)
    sys.stdout.flush()
    path = os.environ.get("LSA_TEST_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def oracle_query_fn(dtype):
    return lambda h, w: oracle.query_encoder(oracle.decode_values(h, dtype), oracle.decode_values(w, dtype))


def oracle_latent_fn(dtype):
    """Latents of a low-rank workload as stored activations (raw), from the oracle."""
    from workloads import bf16_bits_from_f32

    def fn(h, w_down):
        c = oracle.query_latent(oracle.decode_values(h, dtype), oracle.decode_values(w_down, dtype), dtype)
        c32 = c.astype(np.float32)  # exact: the values are already bf16 / f32 values
        return bf16_bits_from_f32(c32) if dtype == "bf16" else c32
    return fn


def oracle_logits_fn(dtype, level=0.5):
    """Logits relative to the selection level's logit (the decision point the margin keeps away from)."""
    off = oracle.level_logit(level)
    return lambda q, keys, bias: oracle.block_logits(q, oracle.decode_values(keys, dtype), bias) - off


def conditioned_workload(name_or_cfg, seed=0, steps=None):
    wl = build_workload(name_or_cfg, seed=seed, steps=steps)
    dt = wl.cfg.dtype
    rep = wl.condition(oracle_query_fn(dt), oracle_logits_fn(dt, wl.cfg.level), latent_fn=oracle_latent_fn(dt))
    assert rep.min_abs_logit >= 2e-3, rep
    return wl


def raw_to_torch(arr: np.ndarray, device="cuda") -> torch.Tensor:
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device)
    return torch.from_numpy(arr.astype(np.float32, copy=False)).to(device)


def make_session(wl, capacity=None, cold_on_device=False, with_masks=True, max_groups=0, device_plan=False,
                 cold_host_mirror=False):
    from lookahead_block_sparse_amd.session import LSASession

    cfg = wl.cfg
    sess = LSASession(dtype=cfg.dtype, n_idx=cfg.n_idx, d_model=cfg.d_model, d_idx=cfg.d_idx,
                      n_heads=cfg.n_heads, head_dim=cfg.head_dim, win_cap=cfg.window, n_blocks=wl.n_blocks,
                      w_q=wl.w_q, keys=wl.keys, capacity=capacity, cold_on_device=cold_on_device,
                      with_masks=with_masks, max_groups=max_groups, w_down=wl.w_down, device_plan=device_plan,
                      n_layers=wl.cfg.n_layers, cold_host_mirror=cold_host_mirror, select_level=wl.cfg.level)
    for r in range(wl.n_req):
        k, v = wl.kv_prefill(r)
        sess.load_prefill(r, k, v)
    for layer in range(1, wl.cfg.n_layers):
        for r in range(wl.n_req):
            k, v = wl.kv_prefill(r, layer)
            sess.load_prefill(r, k, v, layer=layer)
    return sess


def refresh_requests(wl, sess, reqs: Sequence[int], k_of: Dict[int, int]):
    """Refresh requests `reqs` with their k-th hidden state (k_of[r]); gather; return ids."""
    hid = np.stack([wl.hidden[r][k_of[r]] for r in reqs])
    bias = np.stack([wl.bias[r] for r in reqs])
    sel = sess.refresh(reqs, hid, bias)
    for r in reqs:
        sess.gather(r, sel[r])
    return sel


def run_loop(wl, sess, steps: Iterable[int], record: Optional[Iterable[int]] = None, on_refresh=None,
             max_groups=None):
    """Run decode steps in order (refreshing where the schedule says).  Returns
    ({t: out [R][H][D] float64}, {(r, k): ids})."""
    cfg = wl.cfg
    steps = list(steps)
    record = set(steps if record is None else record)
    R = wl.n_req
    selections = {}
    # prologue refreshes (before step 0)
    pro = [r for r in range(R) if wl.refresh_steps[r][0] < 0]
    if pro:
        sel = refresh_requests(wl, sess, pro, {r: 0 for r in pro})
        for r in pro:
            selections[(r, 0)] = sel[r]
            if on_refresh:
                on_refresh(r, 0, sel[r])
    dev = sess.device
    out = torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    outs = {}
    for t in steps:
        reqs = wl.refreshes_at(t)
        if reqs:
            k_of = {r: wl.refresh_index_at(r, t) for r in reqs}
            sel = refresh_requests(wl, sess, reqs, k_of)
            for r in reqs:
                selections[(r, k_of[r])] = sel[r]
                if on_refresh:
                    on_refresh(r, k_of[r], sel[r])
        q = raw_to_torch(wl.q_dec[t], dev)
        kn = raw_to_torch(wl.k_new[t], dev)
        vn = raw_to_torch(wl.v_new[t], dev)
        seq_len = (wl.ctx + t + 1).astype(np.int32)
        window = np.full(R, cfg.window, dtype=np.int32)
        sess.decode(q, seq_len, window, out, k_new=kn, v_new=vn, max_groups=max_groups)
        if t in record:
            outs[t] = out.double().cpu().numpy()
    torch.cuda.synchronize()
    return outs, selections


def attention_errors(gpu: np.ndarray, ref: np.ndarray):
    """(max abs error, max abs error / max |ref|, L2-relative error)."""
    d = np.abs(gpu - ref)
    return float(d.max()), float(d.max() / np.abs(ref).max()), float(np.linalg.norm(gpu - ref) / np.linalg.norm(ref))


ABS_TOL = 2e-2
REL_TOL = 1e-2
