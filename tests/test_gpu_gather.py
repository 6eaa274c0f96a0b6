"""Cold pool -> hot pool gather on the GPU: copied bytes, residency delta, slot reuse under the
smallest capacity, and the device-memory cold pool."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, make_session, run_loop

pytestmark = pytest.mark.gpu


def _check_pool(sess, r, ids):
    bb = sess.block_bytes
    base = int(sess.slot_base[r])
    table = sess.table[2 * base: 2 * (base + len(ids))].view(-1, 2).cpu().numpy()
    assert np.array_equal(table[:, 0], ids)
    slots = table[:, 1]
    assert len(set(slots.tolist())) == len(slots)
    assert ((slots >= base) & (slots < base + sess.capacity[r])).all()
    hot = sess.hot.view(-1, bb)
    cold = sess.cold[r].view(-1, bb)
    got = hot[torch.as_tensor(slots, dtype=torch.long, device=hot.device)].cpu()
    want = cold[torch.as_tensor(ids, dtype=torch.long, device=cold.device)].cpu()
    assert torch.equal(got, want)
    # host state agrees with the device table
    assert np.array_equal(sess.slot_of_block[r][ids], slots)
    assert (sess.slot_of_block[r] >= 0).sum() == len(ids)
    return dict(zip(ids.tolist(), slots.tolist()))


@pytest.mark.parametrize("cold_on_device", [False, True])
def test_gather_contents_and_delta(cold_on_device):
    log(f"gather contents cold_on_device={cold_on_device}")
    wl = conditioned_workload("ctx1m_s", seed=11)
    sess = make_session(wl, cold_on_device=cold_on_device, with_masks=False)
    prev = {}
    for r in range(wl.n_req):
        prev[r] = {}
    for k in range(len(wl.refresh_steps[0])):
        reqs = list(range(wl.n_req))
        sel = sess.refresh(reqs, np.stack([wl.hidden[r][k] for r in reqs]), wl.bias)
        for r in reqs:
            copied, kept = sess.gather(r, sel[r])
            torch.cuda.synchronize()
            old = set(prev[r])
            new = set(sel[r].tolist())
            assert copied == len(new - old) and kept == len(new & old)
            cur = _check_pool(sess, r, sel[r])
            for b in new & old:
                assert cur[b] == prev[r][b], "a block that stayed moved"
            prev[r] = cur


def test_gather_slot_reuse_minimal_capacity():
    """Capacity = the largest selection: every refresh reuses freed slots.  Outputs still match
    the oracle around every refresh."""
    log("gather WAR stress")
    wl = conditioned_workload("ctx128k_s", seed=12, steps=4 * 64 + 2)
    cfg = wl.cfg
    refs, _ = oracle.simulate(wl, steps=[])
    cap = [max(len(x.ids) for x in refs[r]) for r in range(wl.n_req)]
    sess = make_session(wl, capacity=cap, with_masks=False)
    T = cfg.steps
    sample = sorted({t for t in range(T) if t % 64 in (0, 1, 63)})
    gpu, sels = run_loop(wl, sess, range(T), record=sample)
    _, outs = oracle.simulate(wl, steps=sample)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        e = attention_errors(gpu[t], ref)
        assert e[0] <= ABS_TOL and e[1] <= REL_TOL, (t, e)


def test_gather_capacity_overflow_is_an_error():
    import lookahead_block_sparse_amd as L
    log("gather overflow")
    wl = conditioned_workload("ctx128k_s", seed=13, steps=1)
    refs, _ = oracle.simulate(wl, steps=[])
    n = len(refs[0][0].ids)
    sess = make_session(wl, capacity=[n - 1], with_masks=False)
    sel = sess.refresh([0], wl.hidden[0][:1], wl.bias[:1])
    before = sess.slot_of_block[0].copy()
    with pytest.raises(L.LSAError) as e:
        sess.gather(0, sel[0])
    assert e.value.status == L.LSA_ERR_CAPACITY
    assert np.array_equal(before, sess.slot_of_block[0])


def test_gather_batch_matches_one_request_at_a_time():
    """One batched call for all requests of a refresh leaves the same pools, tables and residency
    state as one call per request, over refreshes that move blocks in and out."""
    log("gather batch vs single")
    wl = conditioned_workload("ctx512k_s", seed=14)
    one = make_session(wl, cold_on_device=True, with_masks=False)
    many = make_session(wl, cold_on_device=True, with_masks=False)
    reqs = list(range(wl.n_req))
    for k in range(len(wl.refresh_steps[0])):
        hid = np.stack([wl.hidden[r][k] for r in reqs])
        sel = one.refresh(reqs, hid, wl.bias)
        sel_b = many.refresh(reqs, hid, wl.bias)
        got_one = {r: one.gather(r, sel[r]) for r in reqs}
        got_many = many.gather_many(sel_b)
        torch.cuda.synchronize()
        assert got_one == got_many, (k, got_one, got_many)
        for r in reqs:
            assert np.array_equal(one.slot_of_block[r], many.slot_of_block[r]), (k, r)
            assert np.array_equal(one.free_slots[r][:one.n_free[r][0]], many.free_slots[r][:many.n_free[r][0]])
            _check_pool(many, r, sel_b[r])
        n = 2 * int(one.slot_base[-1])
        assert torch.equal(one.table[:n], many.table[:n])


def test_gather_batch_overflow_changes_no_request():
    """A batch whose second request overflows its hot pool fails as a whole: the first request's
    state and pool are untouched too."""
    import lookahead_block_sparse_amd as L
    log("gather batch overflow")
    wl = conditioned_workload("ctx512k_s", seed=15, steps=1)
    refs, _ = oracle.simulate(wl, steps=[])
    cap = [int(wl.n_blocks[r]) for r in range(wl.n_req)]
    cap[1] = len(refs[1][0].ids) - 1
    sess = make_session(wl, capacity=cap, with_masks=False)
    reqs = list(range(wl.n_req))
    sel = sess.refresh(reqs, np.stack([wl.hidden[r][0] for r in reqs]), wl.bias)
    before = [sess.slot_of_block[r].copy() for r in reqs]
    with pytest.raises(L.LSAError) as e:
        sess.gather_many(sel)
    assert e.value.status == L.LSA_ERR_CAPACITY
    for r in reqs:
        assert np.array_equal(before[r], sess.slot_of_block[r]), r
        assert sess.n_free[r][0] == sess.capacity[r]


def test_gather_events_time_the_copy_kernel():
    """Events passed to the gather take the copy kernel's dispatch stamps: the contents are those
    of an untimed gather, the elapsed time is positive, and with nothing to copy or list the events
    are still recorded."""
    log("gather events")
    wl = conditioned_workload("ctx1m_s", seed=16)
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    reqs = list(range(wl.n_req))
    sel = sess.refresh(reqs, np.stack([wl.hidden[r][0] for r in reqs]), wl.bias)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record(sess.stream)  # torch reads only events it has seen recorded
    res = sess.gather_many(sel, ev_copy=ev)
    torch.cuda.synchronize()
    assert sum(c for c, _ in res.values()) == sum(len(sel[r]) for r in reqs) > 0
    assert ev[0].elapsed_time(ev[1]) > 0.0
    for r in reqs:
        _check_pool(sess, r, sel[r])
    # the same selection again: nothing enters, only the tables are rewritten
    res = sess.gather_many(sel, ev_copy=ev)
    torch.cuda.synchronize()
    assert all(c == 0 for c, _ in res.values())
    assert ev[0].elapsed_time(ev[1]) >= 0.0
    # an empty selection for one request: no copy and no table entry, events recorded at the call
    empty = {0: np.zeros(0, dtype=np.int32)}
    res = sess.gather_many(empty, ev_copy=ev)
    torch.cuda.synchronize()
    assert res[0] == (0, 0)
    assert ev[0].elapsed_time(ev[1]) >= 0.0
    for r in reqs[1:]:
        _check_pool(sess, r, sel[r])
