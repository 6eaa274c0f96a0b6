"""GPU path vs the CPU oracle on the same seeded inputs (small workloads that still span many
64-token tiles, several requests, ragged contexts and staggered refreshes).

Selections must be bit-exact (inputs keep every logit at least 2e-3 away from 0); attention must
be within max-abs 2e-2 and max-abs / max|ref| 1e-2 (fp32 accumulation from bf16 inputs).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import (
    ABS_TOL,
    REL_TOL,
    attention_errors,
    conditioned_workload,
    log,
    make_session,
    raw_to_torch,
    run_loop,
)

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "ctx128k_s", "ctx512k_s", "ctx1m_s", "ragged_s"]


def _bits_of(ids, n_blocks):
    u = np.zeros(n_blocks, dtype=bool)
    u[ids] = True
    return u


def _unpack(words, n_blocks):
    bits = np.unpackbits(np.ascontiguousarray(words).view(np.uint8), bitorder="little")
    return bits[:n_blocks].astype(bool)


@pytest.mark.parametrize("name", SMALL)
def test_refresh_selection_bit_exact(name):
    log(f"refresh selection {name}")
    wl = conditioned_workload(name, seed=1)
    cfg = wl.cfg
    sess = make_session(wl, with_masks=True)
    w = oracle.decode_values(wl.w_q, cfg.dtype)
    for r in range(wl.n_req):
        keys = oracle.decode_values(wl.keys[r], cfg.dtype)
        for k in range(len(wl.refresh_steps[r])):
            ref = oracle.refresh(oracle.decode_values(wl.hidden[r][k], cfg.dtype), w, keys, wl.bias[r])
            got = sess.refresh([r], wl.hidden[r][k][None], wl.bias[r][None])[r]
            assert np.array_equal(got, ref.ids), (name, r, k, len(got), len(ref.ids))
            planes = sess.masks_of(r)
            B = int(wl.n_blocks[r])
            for i in range(cfg.n_idx):
                assert np.array_equal(_unpack(planes[i], B), ref.s[i]), (name, r, k, i)
            assert np.array_equal(_unpack(planes[cfg.n_idx], B), ref.u)
            if len(wl.planted[r]):
                assert set(wl.planted[r].tolist()) <= set(got.tolist())


# every key-row width the score role has a shape for: 256-byte rows (bf16, d_idx 128: four rows
# per 1 KiB run), 512-byte rows (the SMALL configs) and 1 KiB rows (fp32, d_idx 256: one per run)
# and hidden sizes whose rows end inside an encode chunk: 768 bf16 (96 pieces of 16 bytes: the
# last 64-lane load half in range) and 1280 fp32 (320 pieces)
# the hidden sizes the refresh accepts at both ends: 256 (the smallest: a fraction of one encode
# chunk per row) and 16,384 bf16 (the largest: four encode chunks per row)
WIDTHS = [("ctx128k_s", 128, 0), ("ragged_s", 128, 0), ("tiny", 256, 0), ("ctx128k_s", 256, 768), ("tiny", 128, 1280),
          ("tiny", 128, 256), ("ctx128k_s", 256, 16384)]


@pytest.mark.parametrize("name,d_idx,d_model", WIDTHS, ids=[f"{n}-didx{d}-d{m}" for n, d, m in WIDTHS])
def test_refresh_key_row_widths(name, d_idx, d_model):
    from workloads import get_config

    cfg = get_config(name).scaled(d_idx=d_idx, steps=130, **({"d_model": d_model} if d_model else {}))
    log(f"refresh {name} {cfg.dtype} d_idx {d_idx} d_model {cfg.d_model}")
    wl = conditioned_workload(cfg, seed=2)
    sess = make_session(wl, with_masks=True)
    w = oracle.decode_values(wl.w_q, cfg.dtype)
    reqs = list(range(wl.n_req))
    for k in range(min(len(s) for s in wl.refresh_steps)):
        got = sess.refresh(reqs, np.stack([wl.hidden[r][k] for r in reqs]), wl.bias)
        for r in reqs:
            keys = oracle.decode_values(wl.keys[r], cfg.dtype)
            ref = oracle.refresh(oracle.decode_values(wl.hidden[r][k], cfg.dtype), w, keys, wl.bias[r])
            assert np.array_equal(got[r], ref.ids), (name, d_idx, r, k, len(got[r]), len(ref.ids))
            planes = sess.masks_of(r)
            B = int(wl.n_blocks[r])
            for i in range(cfg.n_idx):
                assert np.array_equal(_unpack(planes[i], B), ref.s[i]), (name, d_idx, r, k, i)


LEVELS = [("ctx128k_s", 0.3), ("ragged_s", 0.7), ("tiny", 0.62)]


@pytest.mark.parametrize("name,level", LEVELS, ids=[f"{n}-{l}" for n, l in LEVELS])
def test_selection_level_matches_oracle(name, level):
    """Other selection levels (the explainer's section 7 calls 0.5 a preliminary choice): the
    refresh keeps sigmoid(z) > level (select_level of the C-ABI); every refresh's ids and every
    per-indexer and union bit plane equal the oracle's at that level (inputs conditioned 2e-3 away
    from the level's logit), and a decode loop over the selections is within tolerance."""
    from workloads import get_config

    cfg = get_config(name).scaled(level=level)
    wl = conditioned_workload(cfg, seed=5)
    log(f"selection level {level}, {name}")
    sess = make_session(wl, with_masks=True)
    assert sess.select_level == level
    w = oracle.decode_values(wl.w_q, cfg.dtype)
    dens = []
    for r in range(wl.n_req):
        keys = oracle.decode_values(wl.keys[r], cfg.dtype)
        for k in range(len(wl.refresh_steps[r])):
            ref = oracle.refresh(oracle.decode_values(wl.hidden[r][k], cfg.dtype), w, keys, wl.bias[r], level)
            got = sess.refresh([r], wl.hidden[r][k][None], wl.bias[r][None])[r]
            assert np.array_equal(got, ref.ids), (name, r, k, len(got), len(ref.ids))
            planes = sess.masks_of(r)
            B = int(wl.n_blocks[r])
            for i in range(cfg.n_idx):
                assert np.array_equal(_unpack(planes[i], B), ref.s[i]), (name, r, k, i)
            assert np.array_equal(_unpack(planes[cfg.n_idx], B), ref.u)
            dens.append(len(got) / B)
            # the same inputs at 0.5 select a superset (level < 0.5) or a subset (level > 0.5)
            half = set(oracle.refresh(oracle.decode_values(wl.hidden[r][k], cfg.dtype), w, keys, wl.bias[r]).ids.tolist())
            assert (set(got.tolist()) >= half) if level < 0.5 else (set(got.tolist()) <= half)
    T = min(cfg.steps, 70)
    sample = sorted({0, 1, min(T - 1, 64), T - 1})
    sess2 = make_session(wl, with_masks=False)
    gpu, sels = run_loop(wl, sess2, range(T), record=sample)
    refs, outs = oracle.simulate(wl, steps=sample)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  level {level}: mean density {np.mean(dens):.3f}; decode max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


@pytest.mark.parametrize("name", ["ctx512k_s", "ragged_s"])
def test_refresh_batched_requests_match_single(name):
    """One call for all requests equals one call per request."""
    log(f"refresh batched {name}")
    wl = conditioned_workload(name, seed=2)
    sess = make_session(wl)
    reqs = list(range(wl.n_req))
    hid = np.stack([wl.hidden[r][0] for r in reqs])
    bias = np.stack([wl.bias[r] for r in reqs])
    batched = sess.refresh(reqs, hid, bias)
    for r in reqs:
        single = sess.refresh([r], hid[r:r + 1], bias[r:r + 1])[r]
        assert np.array_equal(batched[r], single)


def test_refresh_run_to_run_deterministic():
    log("refresh determinism")
    wl = conditioned_workload("ctx1m_s", seed=3)
    sess = make_session(wl)
    a = sess.refresh([0, 1], np.stack([wl.hidden[0][1], wl.hidden[1][1]]), wl.bias[:2])
    for _ in range(3):
        b = sess.refresh([0, 1], np.stack([wl.hidden[0][1], wl.hidden[1][1]]), wl.bias[:2])
        for r in (0, 1):
            assert np.array_equal(a[r], b[r])


@pytest.mark.parametrize("name", SMALL)
def test_decode_loop_matches_oracle(name):
    """The whole loop: refreshes on schedule, gathers, window appends, sparse decode."""
    log(f"decode loop {name}")
    _check_decode_loop(conditioned_workload(name, seed=4), name)


def test_decode_loop_largest_call():
    """The most requests one lsa_sparse_decode call takes (64), contexts log-uniform in [64, 8192]
    tokens (single-block requests among them), a 64-token window and staggered refreshes: every
    refresh and the sampled steps' outputs against the oracle."""
    from lookahead_block_sparse_amd import MAX_DECODE_REQ
    from workloads.configs import CONFIGS

    cfg = CONFIGS["ragged"].scaled(name="ragged_max_call", n_req=MAX_DECODE_REQ, ctx=("loguniform", 64, 8192),
                                   window=64, steps=66, tag=15)
    wl = conditioned_workload(cfg, seed=3)
    log(f"decode loop, {wl.n_req} requests of {int(np.min(wl.n_blocks))}..{int(np.max(wl.n_blocks))} blocks")
    _check_decode_loop(wl, cfg.name)


def _check_decode_loop(wl, name):
    cfg = wl.cfg
    T = cfg.steps
    rng = np.random.default_rng(0)
    sample = sorted(set([0, 1, T - 1] + [t for t in range(T) if t % 64 in (0, 63)] +
                        rng.choice(T, size=min(T, 6), replace=False).tolist()))
    sess = make_session(wl, with_masks=False)
    gpu, sels = run_loop(wl, sess, range(T), record=sample)
    refs, outs = oracle.simulate(wl, steps=sample)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        e = attention_errors(gpu[t], ref)
        worst = tuple(max(a, b) for a, b in zip(worst, e))
    log(f"  {name}: max abs {worst[0]:.3e}  rel {worst[1]:.3e}  l2 {worst[2]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst
    if cfg.dtype == "f32":
        assert worst[1] <= 1e-4, worst


def test_split_count_invariance():
    """One work-group per step gives the same result as the full split, and so does every group
    count in between (odd and even counts: groups on odd XCDs take a smaller share of the tiles).
    The partition changes the running max each tile's bf16 softmax weights are rounded against, so
    the results differ by that rounding (relative ~2^-9 per weight), far below the parity tolerance."""
    log("split invariance")
    wl = conditioned_workload("ctx512k_s", seed=5, steps=3)
    outs = []
    for mg in (1, 2, 3, 7, 9, 64, 255, 0):
        sess = make_session(wl, with_masks=False, max_groups=mg)
        o, _ = run_loop(wl, sess, range(3))
        outs.append(o[2])
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 5e-3 * np.abs(outs[0]).max()


@pytest.mark.parametrize("name", ["tiny", "ctx128k_s"])
@pytest.mark.parametrize("mode", ["all", "none"])
def test_all_and_none_selected(name, mode):
    """bias +1e4: every block loaded -> dense attention; bias -1e4: window only."""
    log(f"all/none {name} {mode}")
    wl = conditioned_workload(name, seed=6, steps=5)
    wl.bias[:] = 1e4 if mode == "all" else -1e4
    cfg = wl.cfg
    sess = make_session(wl, with_masks=False)
    gpu, sels = run_loop(wl, sess, range(5))
    for (r, k), ids in sels.items():
        want = np.arange(wl.n_blocks[r]) if mode == "all" else np.zeros(0)
        assert np.array_equal(ids, want)
    dt = cfg.dtype
    for t in (0, 4):
        for r in range(wl.n_req):
            kp, vp = wl.kv_prefill(r)
            n = int(wl.ctx[r])
            K = np.concatenate([oracle.decode_values(kp, dt), oracle.decode_values(wl.k_new[:t + 1, r], dt)])
            V = np.concatenate([oracle.decode_values(vp, dt), oracle.decode_values(wl.v_new[:t + 1, r], dt)])
            L = n + t + 1
            lo = 0 if mode == "all" else L - cfg.window
            ref = oracle.attention(oracle.decode_values(wl.q_dec[t, r], dt), K[lo:L], V[lo:L], cfg.head_dim ** -0.5)
            e = attention_errors(gpu[t][r], ref)
            assert e[0] <= ABS_TOL and e[1] <= REL_TOL, (t, r, e)


@pytest.mark.parametrize("where", ["ws-1", "ws", "cur", "blk_first", "blk_last", "unselected"])
def test_needles(where):
    """One key scoring far above the rest: the output is its value iff it is attended."""
    log(f"needle {where}")
    name = "ctx128k_s"
    wl = conditioned_workload(name, seed=7, steps=2)
    cfg = wl.cfg
    dt = cfg.dtype
    sel = oracle.simulate(wl, steps=[])[0][0][0].ids
    t = 1
    L = int(wl.ctx[0]) + t + 1
    ws = L - cfg.window
    sel_set = set(sel.tolist())
    chosen = [b for b in sel.tolist() if 64 * b + 64 <= ws]
    unsel = [b for b in range(ws // 64) if b not in sel_set]
    p = {"ws-1": ws - 1, "ws": ws, "cur": L - 1, "blk_first": 64 * chosen[len(chosen) // 2],
         "blk_last": 64 * chosen[len(chosen) // 3] + 63, "unselected": 64 * unsel[len(unsel) // 2] + 17}[where]
    attended = p >= ws or (p // 64) in sel_set
    # make q_t head 0 = e_0 * 8, and key p = e_0 * 30*sqrt(D)/8 (bf16-exact powers of two approx.)
    q = oracle.decode_values(wl.q_dec[t, 0], dt).copy()
    D = cfg.head_dim
    q[:] = 0.0
    q[:, 0] = 1.0
    big = np.float32(32.0 * np.sqrt(D))  # score +32 after the 1/sqrt(D) scale
    kp, vp = wl.kv_prefill(0)
    kp = kp.copy()
    k_new = wl.k_new.copy()
    if dt == "bf16":
        from workloads import bf16_bits_from_f32
        enc = lambda x: bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    else:
        enc = lambda x: np.asarray(x, dtype=np.float32)
    row = np.zeros(D, dtype=np.float32)
    row[0] = big
    if p >= int(wl.ctx[0]):
        k_new[p - int(wl.ctx[0]), 0] = enc(row)
    else:
        kp[p] = enc(row)
    wl.set_kv_prefill(0, kp, vp)
    wl.k_new = k_new
    planted = wl.kv_prefill(0)[0][p] if p < int(wl.ctx[0]) else wl.k_new[p - int(wl.ctx[0]), 0]
    assert np.array_equal(planted, enc(row)), "the needle key was not planted"
    assert abs(oracle.decode_values(planted, dt)[0] - big) <= 1e-2 * big
    wl.q_dec = wl.q_dec.copy()
    wl.q_dec[t, 0] = enc(q)
    sess = make_session(wl, with_masks=False)
    gpu, _ = run_loop(wl, sess, range(t + 1))
    if p >= int(wl.ctx[0]):
        v_star = oracle.decode_values(wl.v_new[p - int(wl.ctx[0]), 0], dt)
    else:
        v_star = oracle.decode_values(vp[p], dt)
    o = gpu[t][0]
    close = np.allclose(o, v_star[None, :], atol=2e-2)
    assert close == attended, (where, p, ws, attended, np.abs(o - v_star).max())


@pytest.mark.parametrize("tau,steps", [(1, 24), (16, 70)])
def test_decode_loop_other_cadences(tau, steps):
    """The refresh cadence is a parameter of the method (64 on the pages): refreshing every step
    (the per-step, reactive extreme) or every 16 steps gives the oracle's selections and outputs."""
    from workloads import get_config

    cfg = get_config("ctx128k_s").scaled(tau=tau, steps=steps)
    log(f"cadence tau={tau}, {steps} steps")
    wl = conditioned_workload(cfg, seed=21)
    sample = sorted({0, steps - 1} | {t for t in range(steps) if t % tau in (0, tau - 1)} if tau > 1 else set(range(steps)))
    sess = make_session(wl, with_masks=False)
    gpu, sels = run_loop(wl, sess, range(steps), record=sample)
    refs, outs = oracle.simulate(wl, steps=sample)
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (tau, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  tau={tau}: {len(sels)} refreshes bit-exact; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


@pytest.mark.parametrize("name", ["tiny", "ctx128k_s", "ragged_s"])
def test_resident_reactive_loop_matches_oracle(name):
    """The reactive comparator: every step refreshes with that step's hidden state, the refresh
    writes the block table of a fully resident pool and the decode reads the counts on the device.
    Every step's selection is the oracle's (cadence 1), bit for bit, the table pairs are
    (id, slot of id), and the outputs match the oracle's within tolerance."""
    import torch

    from lookahead_block_sparse_amd.session import ResidentLoop
    from workloads import get_config

    steps = 10
    cfg = get_config(name).scaled(tau=1, steps=steps, staggered=False)
    log(f"resident reactive loop {name}, {steps} steps")
    wl = conditioned_workload(cfg, seed=23)
    R = wl.n_req
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    sess.make_resident()
    dev = sess.device
    out = torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    loop = ResidentLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), out)
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32)).to(dev)
    gpu, sels = {}, {}
    for t in range(steps):
        assert wl.refreshes_at(t) == list(range(R))
        hid = raw_to_torch(np.stack([wl.hidden[r][wl.refresh_index_at(r, t)] for r in range(R)]), dev)
        loop.step(t, hid, bias, raw_to_torch(wl.q_dec[t], dev), raw_to_torch(wl.k_new[t], dev),
                  raw_to_torch(wl.v_new[t], dev))
        counts = sess.sel_count.cpu().numpy()
        ids = sess.sel_ids.cpu().numpy()
        table = sess.table.view(-1, 2).cpu().numpy()
        for r in range(R):
            b0 = int(sess.blk_off[r])
            assert counts[r] >= 0
            sel = ids[b0:b0 + counts[r]].copy()
            sels[(r, wl.refresh_index_at(r, t))] = sel
            assert np.array_equal(table[b0:b0 + counts[r], 0], sel)
            assert np.array_equal(table[b0:b0 + counts[r], 1], sess.slot_base[r] + sel)
        gpu[t] = out.double().cpu().numpy()
    refs, outs = oracle.simulate(wl, steps=list(range(steps)))
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in range(steps):
        ref = np.stack([outs[(r, t)] for r in range(R)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  {name}: {len(sels)} selections bit-exact; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst


def test_refresh_largest_call_ragged_to_single_blocks():
    """The largest call lsa_index_refresh takes, 64 requests, with contexts log-uniform in
    [64, 8192] tokens (1 to 128 blocks: single-block requests, words that end mid-way and tiles of
    several requests in one launch, with more encode groups than fit on the device at once), in one
    launch: every request's ids, count, per-indexer and union bit planes bit-exact against the
    oracle, and its fp32 logits within 2e-4 of the oracle's."""
    from lookahead_block_sparse_amd import MAX_REFRESH_REQ, lsa_index_refresh, lsa_index_refresh_workspace
    from workloads.configs import CONFIGS

    R = MAX_REFRESH_REQ
    cfg = CONFIGS["ragged"].scaled(name="ragged_max_call", n_req=R, ctx=("loguniform", 64, 8192), window=64,
                                   steps=1, tag=15)
    wl = conditioned_workload(cfg, seed=2)
    dev = "cuda"
    nb = np.asarray(wl.n_blocks, dtype=np.int64)
    blk = np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)
    words = (nb + 63) // 64
    word_off = np.concatenate([[0], np.cumsum(words)]).astype(np.int64)
    n_blk = int(blk[-1])
    keys = raw_to_torch(np.concatenate([np.ascontiguousarray(wl.keys[r]).reshape(-1) for r in range(R)]), dev)
    w_q = raw_to_torch(np.ascontiguousarray(wl.w_q).reshape(-1), dev)
    hid = raw_to_torch(np.stack([wl.hidden[r][0] for r in range(R)]).reshape(-1), dev)
    bias = torch.from_numpy(np.stack([wl.bias[r] for r in range(R)]).astype(np.float32).reshape(-1)).to(dev)
    sel = torch.full((n_blk,), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((R,), -7, dtype=torch.int32, device=dev)
    masks = torch.zeros(int(word_off[-1]) * (cfg.n_idx + 1), dtype=torch.int64, device=dev)
    logits = torch.full((cfg.n_idx * n_blk,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.zeros(lsa_index_refresh_workspace(dtype=cfg.dtype, d_model=cfg.d_model, d_idx=cfg.d_idx,
                                                 n_idx=cfg.n_idx, blk_off=blk), dtype=torch.uint8, device=dev)
    lsa_index_refresh(dtype=cfg.dtype, d_model=cfg.d_model, d_idx=cfg.d_idx, n_idx=cfg.n_idx, hidden=hid, w_q=w_q,
                      keys=keys, blk_off=blk, bias=bias, sel_ids=sel, sel_count=cnt, workspace=ws, masks=masks,
                      logits=logits)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    masks_h = masks.cpu().numpy().view(np.uint64)
    z_h = logits.cpu().numpy().astype(np.float64)
    w64 = oracle.decode_values(wl.w_q, cfg.dtype)
    worst = 0.0
    for r in range(R):
        B = int(nb[r])
        ref = oracle.refresh(oracle.decode_values(wl.hidden[r][0], cfg.dtype), w64,
                             oracle.decode_values(wl.keys[r], cfg.dtype), wl.bias[r].astype(np.float64))
        assert cnt_h[r] == ref.count, (r, B, cnt_h[r], ref.count)
        assert np.array_equal(sel_h[blk[r]:blk[r] + ref.count], ref.ids), (r, B)
        planes = masks_h[int(word_off[r]) * (cfg.n_idx + 1):int(word_off[r + 1]) * (cfg.n_idx + 1)]
        planes = planes.reshape(cfg.n_idx + 1, int(words[r]))
        for i in range(cfg.n_idx):
            assert np.array_equal(_unpack(planes[i], B), ref.s[i]), (r, B, i)
        assert np.array_equal(_unpack(planes[cfg.n_idx], B), ref.u), (r, B)
        got_z = z_h[cfg.n_idx * blk[r]:cfg.n_idx * blk[r + 1]].reshape(cfg.n_idx, B)
        worst = max(worst, float(np.abs(got_z - ref.z).max()))
    log(f"64-request refresh: blocks per request {int(nb.min())}..{int(nb.max())} "
        f"({int((nb == 1).sum())} single-block), max |dz| {worst:.3g}")
    assert worst <= 2e-4


def test_decode_contexts_shorter_than_the_window():
    """Requests whose whole context fits in the window (seq_len < window: the ring holds every token
    and every table entry lies inside the window) beside one that does not, through refreshes and
    decode steps: selections exact and outputs within tolerance against the oracle, which then
    attends over the whole context of the short requests."""
    from workloads.configs import CONFIGS

    cfg = CONFIGS["ctx512k"].scaled(name="short_contexts", n_req=4, ctx=("loguniform", 64, 32768), window=2048,
                                    density=("uniform", 0.2, 0.5), steps=70, tag=16)
    wl = conditioned_workload(cfg, seed=3)  # contexts of 320, 26,496, 832 and 64 tokens
    short = int((np.asarray(wl.ctx) + cfg.steps < cfg.window).sum())
    log(f"contexts {np.asarray(wl.ctx).tolist()} tokens, window {cfg.window}: {short} shorter throughout")
    assert short >= 1 and short < wl.n_req
    _check_decode_loop(wl, cfg.name)
