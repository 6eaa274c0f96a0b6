"""Parity at the full workload sizes, in the benchmark's launch configuration.

Each workload runs its whole decode loop through the C-ABI: with the residency plan on the host
(cold pool in HBM, no bit planes, a work-group per CU slot, DecodeLoop's per-step call), and in the
benchmark's default path, the residency plan on the device with device-side counts, the cold pool
in pinned host memory (4 x 1M, 8 x 512K) or in HBM (the ragged mix).  Every refresh of every request
is compared with the oracle bit for bit; the attention outputs of sampled steps (the device-plan
runs: every refresh step, the step before it, 8 seeded steps and the last) within the fp tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, make_session, raw_to_torch

pytestmark = pytest.mark.gpu

# (workload, sampled steps besides the last one)
FULL = [("ctx128k", [0, 63, 64, 200]), ("ctx512k", [0, 64]), ("ctx1m", [64, 191]), ("ragged", [100])]


def _run_bench_style(wl, sess, record):
    """The benchmark's per-step path: refreshes and gathers where the schedule says, then one
    DecodeLoop step.  Returns ({t: out float64}, {(r, k): ids})."""
    from lookahead_block_sparse_amd.session import DecodeLoop

    cfg = wl.cfg
    R, T = wl.n_req, cfg.steps
    dev = sess.device
    sels = {}

    def refresh(reqs, k_of):
        hid = torch.from_numpy(np.stack([wl.hidden[r][k_of[r]] for r in reqs]).view(np.int16)).to(dev)
        bias = torch.from_numpy(np.stack([wl.bias[r] for r in reqs]).astype(np.float32)).to(dev)
        got = sess.refresh(reqs, hid, bias)
        sess.gather_many(got)
        for r in reqs:
            sels[(r, k_of[r])] = got[r]

    pro = [r for r in range(R) if wl.refresh_steps[r][0] < 0]
    if pro:
        refresh(pro, {r: 0 for r in pro})
    out = torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    loop = DecodeLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), out)
    outs = {}
    for t in range(T):
        reqs = wl.refreshes_at(t)
        if reqs:
            refresh(reqs, {r: wl.refresh_index_at(r, t) for r in reqs})
        loop.step(t, raw_to_torch(wl.q_dec[t], dev), raw_to_torch(wl.k_new[t], dev), raw_to_torch(wl.v_new[t], dev))
        if t in record:
            outs[t] = out.double().cpu().numpy()
    torch.cuda.synchronize()
    return outs, sels


@pytest.mark.parametrize("name,steps", FULL, ids=[n for n, _ in FULL])
def test_full_size_loop_matches_oracle(name, steps):
    wl = conditioned_workload(name, seed=11)
    assert wl.cfg.dtype == "bf16"
    T = wl.cfg.steps
    sample = sorted(set([t for t in steps if t < T] + [T - 1]))
    log(f"full size {name}: {wl.n_req} requests, {int(wl.ctx.sum())} context tokens, {T} steps, sampled {sample}")
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    gpu, sels = _run_bench_style(wl, sess, set(sample))
    log(f"  {name}: GPU loop done, {len(sels)} refreshes")
    refs, outs = oracle.simulate(wl, steps=sample)
    n_ref = 0
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k, len(ids), len(refs[r][k].ids))
        n_ref += 1
    assert n_ref == sum(len(s) for s in wl.refresh_steps), (n_ref, [len(s) for s in wl.refresh_steps])
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        e = attention_errors(gpu[t], ref)
        worst = tuple(max(a, b) for a, b in zip(worst, e))
    log(f"  {name}: {n_ref} selections bit-exact; attention max abs {worst[0]:.3e} rel {worst[1]:.3e} "
        f"l2 {worst[2]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def test_full_size_lowrank_matches_oracle():
    """4 x 1M context with the rank-2048 query projection, as bench.py --q-rank 2048 runs it: every
    refresh bit-exact, sampled outputs within tolerance."""
    from workloads import get_config

    cfg = get_config("ctx1m").scaled(q_rank=2048, steps=130)
    wl = conditioned_workload(cfg, seed=12)
    sample = [64, 129]
    log(f"full size low-rank ctx1m: rank {cfg.q_rank}, {cfg.steps} steps, sampled {sample}")
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    assert sess.rank == 2048
    gpu, sels = _run_bench_style(wl, sess, set(sample))
    refs, outs = oracle.simulate(wl, steps=sample)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (r, k, len(ids), len(refs[r][k].ids))
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  low-rank ctx1m: {len(sels)} selections bit-exact; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def test_full_size_reactive_matches_oracle():
    """4 x 1M context through the reactive comparator as bench.py --reactive runs it (every block
    resident, a refresh at every step writing the block table, device-side counts): six steps, every
    selection bit-exact, outputs of the first and last step within tolerance."""
    from lookahead_block_sparse_amd.session import ResidentLoop
    from workloads import get_config

    steps = 6
    cfg = get_config("ctx1m").scaled(tau=1, steps=steps, staggered=False)
    wl = conditioned_workload(cfg, seed=13)
    R = wl.n_req
    log(f"full size reactive ctx1m: {steps} steps")
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    sess.make_resident()
    dev = sess.device
    out = torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    loop = ResidentLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), out)
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    sels, gpu = {}, {}
    for t in range(steps):
        hid = raw_to_torch(np.stack([wl.hidden[r][wl.refresh_index_at(r, t)] for r in range(R)]), dev)
        loop.step(t, hid, bias, raw_to_torch(wl.q_dec[t], dev), raw_to_torch(wl.k_new[t], dev),
                  raw_to_torch(wl.v_new[t], dev))
        counts = sess.sel_count.cpu().numpy()
        ids = sess.sel_ids.cpu().numpy()
        for r in range(R):
            b0 = int(sess.blk_off[r])
            sels[(r, wl.refresh_index_at(r, t))] = ids[b0:b0 + counts[r]].copy()
        if t in (0, steps - 1):
            gpu[t] = out.double().cpu().numpy()
    refs, outs = oracle.simulate(wl, steps=[0, steps - 1])
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (r, k)
    worst = (0.0, 0.0, 0.0)
    for t in (0, steps - 1):
        ref = np.stack([outs[(r, t)] for r in range(R)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  reactive ctx1m: {len(sels)} selections bit-exact; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def _sampled_steps(wl, seed, n_random=8):
    """Every refresh step, the step before it and n_random seeded steps (each sampled step holds the
    outputs of every request), plus the last step."""
    T = wl.cfg.steps
    s = {T - 1}
    for r in range(wl.n_req):
        for tk in wl.refresh_steps[r]:
            if 0 <= tk < T:
                s.add(tk)
                if tk > 0:
                    s.add(tk - 1)
    rng = np.random.default_rng(seed)
    s.update(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    return sorted(s)


FULL_DEVICE_PLAN = [("ctx1m", "host"), ("ctx512k", "host"), ("ragged", "device")]


@pytest.mark.parametrize("name,cold", FULL_DEVICE_PLAN, ids=[f"{n}-{c}" for n, c in FULL_DEVICE_PLAN])
def test_full_size_device_plan_matches_oracle(name, cold):
    """The benchmark's default path at full size: refresh, residency plan and copy on the device,
    device-side counts in the decode; the cold pool in pinned host memory (4 x 1M, 8 x 512K: every
    gather reads over the host link) or in HBM (the 32-request ragged mix).  Every refresh of every
    request bit-exact, the hot pool holding each request's selection after every refresh, and the
    outputs of every refresh step, the step before it, 8 seeded steps and the last step within the
    tolerance."""
    from test_gpu_device_plan import _run

    wl = conditioned_workload(name, seed=14)
    sample = _sampled_steps(wl, seed=14)
    if name == "ragged":  # 287 refresh steps: keep every refresh check, sample a bounded set of steps
        rng = np.random.default_rng(15)
        keep = set(rng.choice(sample, size=24, replace=False).tolist()) | {wl.cfg.steps - 1}
        sample = sorted(keep)
    log(f"full size device plan {name}, cold pool {cold}: {wl.n_req} requests, {wl.cfg.steps} steps, "
        f"{len(sample)} sampled steps")
    sess = make_session(wl, cold_on_device=(cold == "device"), with_masks=False, device_plan=True)
    gpu, sels = _run(wl, sess, set(sample))
    log(f"  {name}: GPU loop done, {len(sels)} refreshes")
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    refs, outs = oracle.simulate(wl, steps=sample)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k, len(ids), len(refs[r][k].ids))
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[(0, t)], ref)))
    log(f"  {name}: {len(sels)} selections bit-exact; {len(sample)} steps, max abs {worst[0]:.3e} "
        f"rel {worst[1]:.3e} l2 {worst[2]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


@pytest.mark.parametrize("name", ["tiny", "ctx128k_s", "ctx512k_s", "ctx1m"])
def test_refresh_logits_match_oracle(name):
    """The fp32 logits the refresh thresholds (its optional logits output) against the oracle's
    float64 logits of the same stored inputs, on every block of every request of the first refresh
    (4 x 1M: 196,608 logits).  Bit-exact selection rests on this error staying far below the 2e-3
    margin the generators keep around the threshold; the bound asserted is a tenth of it."""
    from lookahead_block_sparse_amd import lsa_index_refresh, lsa_index_refresh_workspace

    wl = conditioned_workload(name, steps=1)
    cfg, R, dev = wl.cfg, wl.n_req, "cuda"
    blk = np.concatenate([[0], np.cumsum(wl.n_blocks)]).astype(np.int64)
    n_blk = int(blk[-1])
    keys = raw_to_torch(np.concatenate([np.ascontiguousarray(wl.keys[r]).reshape(-1) for r in range(R)]), dev)
    w_q = raw_to_torch(np.ascontiguousarray(wl.w_q).reshape(-1), dev)
    hid = raw_to_torch(np.stack([wl.hidden[r][0] for r in range(R)]).reshape(-1), dev)
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32).reshape(-1)).to(dev)
    sel = torch.zeros(n_blk, dtype=torch.int32, device=dev)
    cnt = torch.zeros(R, dtype=torch.int32, device=dev)
    logits = torch.full((cfg.n_idx * n_blk,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.zeros(lsa_index_refresh_workspace(dtype=cfg.dtype, d_model=cfg.d_model, d_idx=cfg.d_idx,
                                                 n_idx=cfg.n_idx, blk_off=blk), dtype=torch.uint8, device=dev)
    lsa_index_refresh(dtype=cfg.dtype, d_model=cfg.d_model, d_idx=cfg.d_idx, n_idx=cfg.n_idx, hidden=hid, w_q=w_q,
                      keys=keys, blk_off=blk, bias=bias, sel_ids=sel, sel_count=cnt, workspace=ws, logits=logits,
                      select_level=cfg.level)
    torch.cuda.synchronize()
    z_gpu = logits.cpu().numpy().astype(np.float64)
    counts = cnt.cpu().numpy()
    w_q64 = oracle.decode_values(wl.w_q, cfg.dtype)
    worst, worst_rel = 0.0, 0.0
    for r in range(R):
        ref = oracle.refresh(oracle.decode_values(wl.hidden[r][0], cfg.dtype), w_q64,
                             oracle.decode_values(wl.keys[r], cfg.dtype), wl.bias[r].astype(np.float64), cfg.level)
        z_ref = ref.z
        got = z_gpu[cfg.n_idx * blk[r]: cfg.n_idx * blk[r + 1]].reshape(cfg.n_idx, -1)
        assert np.all(np.isfinite(got)), f"request {r}: logits not written"
        err = np.abs(got - z_ref)
        worst = max(worst, float(err.max()))
        worst_rel = max(worst_rel, float((err / np.maximum(np.abs(z_ref), 1.0)).max()))
        assert counts[r] == ref.count
        assert np.array_equal(got > oracle.level_logit(cfg.level), ref.s)
    log(f"{name}: max |z_gpu - z_oracle| = {worst:.3g} (relative to max(|z|, 1): {worst_rel:.3g}) "
        f"over {cfg.n_idx * n_blk} logits")
    assert worst <= 2e-4
