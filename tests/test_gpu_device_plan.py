"""The gather planned on the device (lsa_gather_plan_device) against the oracle: a decode loop whose
refreshes never return to the host.  After every refresh the selection is the oracle's (bit for bit),
the table is that selection with every slot holding its cold block (every layer), the device state
is consistent (free stack + resident slots = the request's slots), and sampled outputs match the
oracle; a selection that does not fit changes nothing and reports status 1."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, make_session, raw_to_torch

pytestmark = pytest.mark.gpu


def _check_state(sess, r, ids):
    """Table == ids with slots holding their cold blocks (every layer); free + used slots = all."""
    s0, s1 = int(sess.slot_base[r]), int(sess.slot_base[r + 1])
    assert int(sess.plan_status[r].item()) == 0
    cnt = int(sess.table_count[r].item())
    table = sess.table.view(-1, 2)[s0:s0 + cnt].cpu().numpy()
    assert cnt == len(ids) and np.array_equal(table[:, 0], ids), (r, cnt, len(ids))
    slots = table[:, 1]
    nf = int(sess.n_free_dev[r].item())
    free = sess.free_dev[s0:s0 + nf].cpu().numpy()
    assert sorted(np.concatenate([slots, free]).tolist()) == list(range(s0, s1)), r
    sob = sess.slot_of_block_dev[int(sess.blk_off[r]):int(sess.blk_off[r + 1])].cpu().numpy()
    assert np.array_equal(np.flatnonzero(sob >= 0), ids) and np.array_equal(sob[ids], slots)
    bb = sess.block_bytes
    lb = int(sess.n_blocks[r]) * bb
    st = torch.as_tensor(slots, dtype=torch.long, device=sess.device)
    bt = torch.as_tensor(ids, dtype=torch.long, device=sess.device)
    for layer in range(sess.n_layers):
        hot, _ = sess.layer_views(layer)
        cold = sess.cold[r][layer * lb:(layer + 1) * lb]  # HBM or pinned host memory
        want = cold.view(-1, bb)[bt.to(cold.device)].to(sess.device)
        assert torch.equal(hot.view(-1, bb)[st], want), (r, layer)


def _run(wl, sess, sample, check=True, switch_at=None):
    """The benchmark's device-planned loop (refresh_device + DecodeLoop with device counts): returns
    ({(layer, t): outputs}, {(r, k): ids}); with check, every refresh's table, device state and hot
    pool are checked against its selection."""
    from lookahead_block_sparse_amd.session import DecodeLoop

    cfg = wl.cfg
    R = wl.n_req
    dev = sess.device
    bias_all = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    sels, gpu = {}, {}

    prev = {r: np.zeros(0, dtype=np.int64) for r in range(R)}  # each request's resident blocks

    def refresh(reqs, k_of):
        hid = raw_to_torch(np.stack([wl.hidden[r][k_of[r]] for r in reqs]), dev)
        copied = torch.full((R,), -1, dtype=torch.int32, device=dev)  # the plan's count of copied blocks
        sess.refresh_device(reqs, hid, torch.stack([bias_all[r] for r in reqs]), copied_out=copied)
        if check:
            # the refresh wrote bit planes only; the plan rewrote the counts
            counts = sess.sel_count.cpu().numpy()
            got_copied = copied.cpu().numpy()
            for r in reqs:
                ids = sess.union_ids(r)
                assert counts[r] == len(ids), (r, counts[r], len(ids))
                sels[(r, k_of[r])] = ids
                _check_state(sess, r, ids)
                # the blocks that entered: selected now, not resident before
                assert got_copied[r] == len(np.setdiff1d(ids, prev[r])), (r, got_copied[r])
                prev[r] = ids
            assert all(got_copied[r] == -1 for r in range(R) if r not in reqs), got_copied

    pro = [r for r in range(R) if wl.refresh_steps[r][0] < 0]
    if pro:
        refresh(pro, {r: 0 for r in pro})
    outs = [torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev) for _ in range(cfg.n_layers)]
    loops = [DecodeLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), outs[l], layer=l, device_counts=True)
             for l in range(cfg.n_layers)]
    for t in range(cfg.steps):
        if switch_at is not None and t == switch_at:
            sess.use_cold("host")  # the same blocks from the pinned host copy from here on
        reqs = wl.refreshes_at(t)
        if reqs:
            refresh(reqs, {r: wl.refresh_index_at(r, t) for r in reqs})
        for l in range(cfg.n_layers):
            loops[l].step(t, raw_to_torch(wl.q_dec_of(l)[t], dev), raw_to_torch(wl.k_new_of(l)[t], dev),
                          raw_to_torch(wl.v_new_of(l)[t], dev))
        if t in sample:
            for l in range(cfg.n_layers):
                gpu[(l, t)] = outs[l].double().cpu().numpy()
    torch.cuda.synchronize()
    sess.check_plan_status()
    return gpu, sels


@pytest.mark.parametrize("name,layers", [("ctx128k_s", 1), ("ragged_s", 1), ("ctx512k_s", 2)])
def test_device_planned_loop_matches_oracle(name, layers):
    from workloads import get_config

    cfg = get_config(name).scaled(n_layers=layers, hidden_rho=0.9 if layers > 1 else 0.0)
    wl = conditioned_workload(cfg, seed=41)
    log(f"device-planned loop {name}, {layers} layer(s), {cfg.steps} steps")
    sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True)
    sample = sorted({0, 63, 64, cfg.steps - 1})
    gpu, sels = _run(wl, sess, sample)
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    worst = (0.0, 0.0, 0.0)
    for layer in range(layers):
        refs, outs = oracle.simulate(wl, steps=sample, layer=layer)
        for (r, k), ids in sels.items():
            assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
        for t in sample:
            ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
            worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[(layer, t)], ref)))
    log(f"  {name}: {len(sels)} device-planned refreshes; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def test_device_plan_overflow_changes_nothing():
    """With too few slots for the second refresh's selection, that refresh's plan reports status 1 and
    the table, the resident set and the free stack stay those of the first refresh."""
    from workloads import get_config

    cfg = get_config("ctx128k_s").scaled(steps=70)
    wl = conditioned_workload(cfg, seed=42)
    R = wl.n_req
    dt = cfg.dtype
    w_q = oracle.decode_values(wl.w_q, dt)
    counts = [[oracle.refresh(oracle.decode_values(wl.hidden[r][k], dt), w_q, oracle.decode_values(wl.keys[r], dt),
                              wl.bias[r]).count for k in range(len(wl.refresh_steps[r]))] for r in range(R)]
    # the refresh with the smallest selection first, the largest second; slots for the first only
    ks = [(int(np.argmin(c)), int(np.argmax(c))) for c in counts]
    first = [counts[r][ks[r][0]] for r in range(R)]
    second = [counts[r][ks[r][1]] for r in range(R)]
    cap = [max(first[r], 1) for r in range(R)]
    assert any(second[r] > cap[r] for r in range(R)), counts
    sess = make_session(wl, capacity=cap, cold_on_device=True, with_masks=False, device_plan=True)
    dev = sess.device
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    sess.refresh_device(list(range(R)), raw_to_torch(np.stack([wl.hidden[r][ks[r][0]] for r in range(R)]), dev), bias)
    torch.cuda.synchronize()
    before = (sess.table.clone(), sess.table_count.clone(), sess.resident_dev.clone(), sess.free_dev.clone(),
              sess.n_free_dev.clone(), sess.slot_of_block_dev.clone())
    sess.refresh_device(list(range(R)), raw_to_torch(np.stack([wl.hidden[r][ks[r][1]] for r in range(R)]), dev), bias)
    torch.cuda.synchronize()
    status = sess.plan_status.cpu().numpy()
    for r in range(R):
        assert status[r] == (1 if second[r] > cap[r] else 0), (r, status[r], second[r], cap[r])
    over = [r for r in range(R) if second[r] > cap[r]]
    for r in over:
        s0, s1 = int(sess.slot_base[r]), int(sess.slot_base[r + 1])
        assert torch.equal(sess.table.view(-1, 2)[s0:s1], before[0].view(-1, 2)[s0:s1])
        assert int(sess.table_count[r]) == int(before[1][r]) == first[r]
        w0, w1 = int(sess.word_off[r]), int(sess.word_off[r + 1])
        assert torch.equal(sess.resident_dev[w0:w1], before[2][w0:w1])
        assert int(sess.n_free_dev[r]) == int(before[4][r])


def test_device_counts_split_invariance():
    """With the counts on the device the kernels compute the split of the tiles themselves (at most
    half as many groups as tiles, groups on odd XCDs taking a smaller share); every group count gives
    the oracle's outputs, and the same ones up to the rounding of the bf16 softmax weights."""
    from workloads import get_config

    cfg = get_config("ctx128k_s").scaled(steps=3)
    wl = conditioned_workload(cfg, seed=43)
    log("device-count split invariance")
    outs = []
    for mg in (1, 2, 5, 0):
        sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True, max_groups=mg)
        gpu, _ = _run(wl, sess, [2], check=False)
        outs.append(gpu[(0, 2)])
    refs, oref = oracle.simulate(wl, steps=[2])
    ref = np.stack([oref[(r, 2)] for r in range(wl.n_req)])
    for o in outs:
        e = attention_errors(o, ref)
        assert e[0] <= ABS_TOL and e[1] <= REL_TOL, e
        assert np.abs(o - outs[-1]).max() <= 5e-3 * np.abs(outs[-1]).max()


def test_device_plan_events_change_nothing():
    """Events passed to the refresh and to the device plan (launches that record dispatch stamps)
    time the kernels and leave every result (table, counts, resident set, free stack, hot pool) as
    the plain launches give it, over two refreshes."""
    from workloads import get_config

    cfg = get_config("ctx128k_s").scaled(steps=70)
    wl = conditioned_workload(cfg, seed=42)
    R = wl.n_req
    results = []
    for timed in (False, True):
        log(f"device plan, events={timed}")
        sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True)
        dev = sess.device
        bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
        pairs = []
        for k in (0, 1):
            hid = raw_to_torch(np.stack([wl.hidden[r][min(k, len(wl.hidden[r]) - 1)] for r in range(R)]), dev)
            if timed:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                for e in ev:
                    e.record()  # torch creates the HIP event at its first record
                sess.refresh_device(list(range(R)), hid, bias, ev_begin=ev[0], ev_end=ev[1], ev_plan=(ev[2], ev[3]))
                pairs += [(ev[0], ev[1]), (ev[2], ev[3])]
            else:
                sess.refresh_device(list(range(R)), hid, bias)
        torch.cuda.synchronize()
        for a, b in pairs:
            assert a.elapsed_time(b) > 0
        # the hot pool is not initialised: compare the slots the tables name
        tbl, cnt = sess.table.view(-1, 2).cpu().numpy(), sess.table_count.cpu().numpy()
        slots = np.concatenate([tbl[int(sess.slot_base[r]):int(sess.slot_base[r]) + int(cnt[r]), 1] for r in range(R)])
        assert len(slots) > 0
        hot = sess.hot[:sess.n_slots * sess.block_bytes].view(sess.n_slots, sess.block_bytes)
        used = hot[torch.from_numpy(slots.astype(np.int64)).to(dev)]
        results.append([t.clone() for t in (sess.table, sess.table_count, sess.resident_dev, sess.free_dev,
                                            sess.n_free_dev, sess.slot_of_block_dev, sess.copied_dev,
                                            sess.plan_status)] + [used])
        del sess
    for x, y in zip(*results):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,mode", [("ctx1m_s", "host"), ("ragged_s", "host"), ("ctx128k_s", "switch")])
def test_device_plan_with_pinned_host_pool_matches_oracle(name, mode):
    """The device plan copying from a cold pool in pinned host memory (its copy kernel reads over
    the host link), or switching from the HBM pool to its pinned host copy between refreshes: every
    refresh bit-exact, every slot holding its block, outputs within tolerance."""
    from workloads import get_config

    cfg = get_config(name)
    wl = conditioned_workload(cfg, seed=44)
    log(f"device plan, cold pool {mode}, {name}")
    if mode == "host":
        sess = make_session(wl, cold_on_device=False, with_masks=False, device_plan=True)
        switch = None
    else:
        sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True, cold_host_mirror=True)
        switch = 64
    sample = sorted({0, 63, 64, cfg.steps - 1})
    gpu, sels = _run(wl, sess, sample, switch_at=switch)
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    refs, outs = oracle.simulate(wl, steps=sample)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[(0, t)], ref)))
    log(f"  {len(sels)} refreshes; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def test_refresh_that_gave_up_is_reported():
    """A refresh whose compaction gave up writes its count as -1; the device plan then changes
    nothing for that request and records status 2, which check_plan_status turns into an error.
    The -1 is written from the host (no kernel is made to fail)."""
    import ctypes

    from lookahead_block_sparse_amd import LIB
    from workloads import get_config

    cfg = get_config("ctx512k_s").scaled(steps=70)
    wl = conditioned_workload(cfg, seed=45)
    R = wl.n_req
    sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True)
    dev = sess.device
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    sess.refresh_device(list(range(R)), raw_to_torch(np.stack([wl.hidden[r][0] for r in range(R)]), dev), bias)
    sess.check_plan_status()  # a good refresh reports nothing
    before = (sess.table.clone(), sess.table_count.clone(), sess.resident_dev.clone())
    sess.sel_count[1] = -1  # request 1's refresh "gave up"
    a = sess._plan_args(0, R)[0]
    a.ev_begin = a.ev_end = None
    assert LIB.lsa_gather_plan_device(ctypes.byref(a), ctypes.c_void_p(sess.stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert sess.plan_status.cpu().tolist() == [0, 2, 0]
    with pytest.raises(RuntimeError, match="request 1 gave up"):
        sess.check_plan_status()
    sess.check_plan_status()  # the record was cleared
    s0, s1 = int(sess.slot_base[1]), int(sess.slot_base[2])
    assert torch.equal(sess.table.view(-1, 2)[s0:s1], before[0].view(-1, 2)[s0:s1])
    assert int(sess.table_count[1]) == int(before[1][1])
    w0, w1 = int(sess.word_off[1]), int(sess.word_off[2])
    assert torch.equal(sess.resident_dev[w0:w1], before[2][w0:w1])


@pytest.mark.parametrize("name", ["ragged_s"])
def test_staggered_overlap_matches_oracle(name):
    """Staggered refreshes overlapped with the other requests' decode (StaggeredLoop): at a step
    where some requests refresh, their refresh, plan, copy and attention run on a second stream
    beside the others' attention.  Every refresh selects the oracle's blocks and leaves the tables,
    device state and hot pool of its selection; the outputs at refresh steps and the steps after
    them match the oracle."""
    from workloads import get_config
    from lookahead_block_sparse_amd.session import StaggeredLoop

    cfg = get_config(name)
    wl = conditioned_workload(cfg, seed=47)
    R = wl.n_req
    sess = make_session(wl, cold_on_device=True, with_masks=False, device_plan=True)
    dev = sess.device
    bias_all = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    ref_steps = [t for t in range(cfg.steps) if 0 < len(wl.refreshes_at(t)) < R]
    assert ref_steps, "the workload has no staggered refresh"
    sample = sorted({0, cfg.steps - 1} | set(ref_steps[:4]) | {t + 1 for t in ref_steps[:4] if t + 1 < cfg.steps})
    log(f"staggered overlap {name}: {R} requests, {cfg.steps} steps, refresh steps {ref_steps[:6]}..., sample {sample}")
    pro = [r for r in range(R) if wl.refresh_steps[r][0] < 0]
    sels = {}
    if pro:
        sess.refresh_device(pro, raw_to_torch(np.stack([wl.hidden[r][0] for r in pro]), dev),
                            torch.stack([bias_all[r] for r in pro]))
        torch.cuda.synchronize()
        for r in pro:
            sels[(r, 0)] = sess.union_ids(r)
            assert int(sess.sel_count[r]) == len(sels[(r, 0)])
    out = torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    loop = StaggeredLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), out)
    gpu = {}
    for t in range(cfg.steps):
        reqs = wl.refreshes_at(t)
        hid = raw_to_torch(np.stack([wl.hidden[r][wl.refresh_index_at(r, t)] for r in reqs]), dev) if reqs else None
        bias = torch.stack([bias_all[r] for r in reqs]) if reqs else None
        loop.step(t, raw_to_torch(wl.q_dec[t], dev), raw_to_torch(wl.k_new[t], dev), raw_to_torch(wl.v_new[t], dev),
                  refresh=reqs, hidden=hid, bias=bias)
        if reqs:
            torch.cuda.synchronize()
            counts = sess.sel_count.cpu().numpy()
            for r in reqs:
                ids = sess.union_ids(r)
                assert counts[r] == len(ids), (r, counts[r], len(ids))
                sels[(r, wl.refresh_index_at(r, t))] = ids
                _check_state(sess, r, ids)
        if t in sample:
            gpu[t] = out.double().cpu().numpy()
    torch.cuda.synchronize()
    sess.check_plan_status()
    refs, outs = oracle.simulate(wl, steps=sample)
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(R)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  {name}: {len(sels)} refreshes ({len(ref_steps)} overlapped steps); max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst
