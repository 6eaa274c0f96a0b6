"""Seeded workload generator: determinism, bf16 rounding, calibration, margin and planting."""

import numpy as np
import pytest

import oracle
import workloads
from workloads import bf16_bits_from_f32, build_workload, get_config


def oracle_query_fn(dtype):
    return lambda h, w: oracle.query_encoder(oracle.decode_values(h, dtype), oracle.decode_values(w, dtype))


def oracle_logits_fn(dtype):
    return lambda q, keys, bias: oracle.block_logits(q, oracle.decode_values(keys, dtype), bias)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is exactly halfway between 1 and 1 + 2^-7: ties to even (1.0)
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_same_seed_same_bytes():
    a = build_workload("ragged_s", seed=3)
    b = build_workload("ragged_s", seed=3)
    c = build_workload("ragged_s", seed=4)
    assert np.array_equal(a.ctx, b.ctx)
    assert np.array_equal(a.w_q, b.w_q)
    for r in range(a.n_req):
        assert np.array_equal(a.keys[r], b.keys[r])
        ka, va = a.kv_prefill(r)
        kb, vb = b.kv_prefill(r)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert not np.array_equal(a.w_q, c.w_q)


def test_shapes_and_schedule():
    wl = build_workload("ragged_s", seed=0)
    cfg = wl.cfg
    assert (wl.ctx % 64 == 0).all()
    assert len(set(wl.phase.tolist())) == cfg.n_req
    for r in range(cfg.n_req):
        steps = wl.refresh_steps[r]
        assert steps == sorted(steps)
        in_range = [t for t in steps if t >= 0]
        assert all((t + wl.phase[r]) % 64 == 0 for t in in_range)
        # at step 0 some refresh is in force
        assert steps[0] <= 0
        assert wl.hidden[r].shape == (len(steps), cfg.d_model)
        assert wl.keys[r].shape == (cfg.n_idx, wl.n_blocks[r], cfg.d_idx)
    # staggered: at most one request refreshes per step
    for t in range(cfg.steps):
        assert len(wl.refreshes_at(t)) <= 1


def test_tiny_is_fp32_and_calibrated():
    wl = build_workload("tiny", seed=0)
    assert wl.w_q.dtype == np.float32 and wl.keys[0].dtype == np.float32
    assert wl.refresh_steps == [[0]]


@pytest.mark.parametrize("name", ["ctx128k_s", "ctx512k_s", "ragged_s"])
def test_margin_conditioning(name):
    wl = build_workload(name, seed=1)
    dt = wl.cfg.dtype
    rep = wl.condition(oracle_query_fn(dt), oracle_logits_fn(dt))
    assert rep.min_abs_logit >= 2e-3
    # recompute independently: no logit within the margin at any refresh
    w = oracle.decode_values(wl.w_q, dt)
    for r in range(wl.n_req):
        keys = oracle.decode_values(wl.keys[r], dt)
        for k in range(len(wl.refresh_steps[r])):
            res = oracle.refresh(oracle.decode_values(wl.hidden[r][k], dt), w, keys, wl.bias[r])
            assert np.abs(res.z).min() >= 2e-3


def test_realised_density_near_target():
    wl = build_workload(get_config("ctx128k").scaled(name="dens", ctx=("fixed", 262144), steps=64), seed=2)
    dt = wl.cfg.dtype
    w = oracle.decode_values(wl.w_q, dt)
    res = oracle.refresh(oracle.decode_values(wl.hidden[0][0], dt), w, oracle.decode_values(wl.keys[0], dt),
                         wl.bias[0])
    frac = res.count / wl.n_blocks[0]
    assert abs(frac - 0.10) < 0.02, frac


def test_planted_blocks_recalled_small():
    wl = build_workload("ctx1m_s", seed=5)
    dt = wl.cfg.dtype
    rep = wl.condition(oracle_query_fn(dt), oracle_logits_fn(dt))
    assert rep.planted_rows == wl.cfg.n_idx * sum(len(p) for p in wl.planted)
    assert rep.min_planted_logit >= 1.0, rep.min_planted_logit
    w = oracle.decode_values(wl.w_q, dt)
    for r in range(wl.n_req):
        keys = oracle.decode_values(wl.keys[r], dt)
        for k in range(len(wl.refresh_steps[r])):
            res = oracle.refresh(oracle.decode_values(wl.hidden[r][k], dt), w, keys, wl.bias[r])
            assert set(wl.planted[r].tolist()) <= set(res.ids.tolist())
            # every indexer keeps every planted block
            assert res.s[:, wl.planted[r]].all()
        assert (wl.planted[r] < (wl.ctx[r] - wl.cfg.window) // 64).all()


def test_layers_have_their_own_streams_and_layer0_is_unchanged():
    from workloads import build_workload, get_config

    base = build_workload("tiny", seed=3)
    cfg = get_config("tiny").scaled(n_layers=3)
    wl = build_workload(cfg, seed=3)
    assert np.array_equal(wl.q_dec, base.q_dec) and np.array_equal(wl.k_new, base.k_new)
    assert np.array_equal(wl.kv_prefill(0)[0], base.kv_prefill(0)[0])
    assert len(wl.layer_dec) == 2
    for layer in (1, 2):
        assert wl.q_dec_of(layer).shape == wl.q_dec.shape
        assert not np.array_equal(wl.q_dec_of(layer), wl.q_dec)
        assert not np.array_equal(wl.kv_prefill(0, layer)[1], wl.kv_prefill(0)[1])
    assert not np.array_equal(wl.kv_prefill(0, 1)[0], wl.kv_prefill(0, 2)[0])


def test_correlated_hidden_states():
    """h_k = rho h_(k-1) + sqrt(1 - rho^2) eps_k: unit variance, lag-1 correlation rho; rho = 0 is
    the independent draw."""
    from workloads import build_workload, get_config
    from workloads.gen import Workload  # noqa: F401

    cfg = get_config("ctx128k").scaled(steps=64 * 40, hidden_rho=0.8)
    wl = build_workload(cfg, seed=5)
    h = (wl.hidden[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(h.var() - 1.0) < 0.02
    c = np.mean([np.corrcoef(h[k], h[k + 1])[0, 1] for k in range(len(h) - 1)])
    assert abs(c - 0.8) < 0.02, c
    wl0 = build_workload(get_config("ctx128k").scaled(steps=64 * 40), seed=5)
    assert np.array_equal((wl0.hidden[0][0].astype(np.uint32) << 16).view(np.float32), h[0].astype(np.float32))


def test_planted_prefill_is_what_oracle_and_session_read():
    """A test that replaces a prefill (a planted needle) must change what kv_prefill returns for that
    request and layer, and nothing else; a wrong shape is refused."""
    from workloads import build_workload, get_config

    wl = build_workload(get_config("tiny").scaled(n_layers=2), seed=4)
    k, v = wl.kv_prefill(0)
    k2 = k.copy()
    k2[5] = 0
    other = wl.kv_prefill(0, 1)[0].copy()
    wl.set_kv_prefill(0, k2, v)
    assert np.array_equal(wl.kv_prefill(0)[0], k2)
    assert np.array_equal(wl.kv_prefill(0, 1)[0], other)
    with pytest.raises(ValueError):
        wl.set_kv_prefill(0, k2[:-1], v)


@pytest.mark.parametrize("name", ["ragged", "ctx1m", "ragged_s", "ctx512k"])
def test_every_request_has_a_selection_before_its_first_step(name):
    """The selection in force at step 0 comes from a refresh at step 0 or from the prologue refresh
    before it (staggered phases): the benchmark runs the prologue refreshes of exactly the requests
    whose first refresh step is negative, so no request decodes window-only at the start."""
    import bench

    cfg = get_config(name)
    wl = build_workload(cfg.scaled(steps=min(cfg.steps, 128)), seed=3)
    pro = bench.prologue_requests(wl)
    for r in range(wl.n_req):
        first = wl.refresh_steps[r][0]
        assert first <= 0, (r, first)
        assert (first < 0) == (r in pro)
        assert sum(1 for t in wl.refresh_steps[r] if t <= 0) == 1  # exactly one governs step 0
    if cfg.staggered:
        assert len(pro) >= wl.n_req - 1  # at most one phase is 0


def test_benchmark_refuses_more_steps_than_the_window_holds():
    """Decode-time tokens never leave the window (they belong to no scored block), so the benchmark
    refuses a run whose decode steps exceed it."""
    import bench

    cfg = get_config("ctx1m")
    assert bench.max_bench_steps(cfg) == cfg.window // bench.STEP_DECODE


def _write_csv(path, header, rows):
    import csv

    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_traffic_summary_scales_counters_by_the_copy_in_the_same_pass(tmp_path):
    """The traffic figure the benchmark reports: per pass, the kernel's mean counter value over its
    largest-grid launches (smaller launches of the same kernel are single-request recomputations),
    scaled by what the counter read for the plain copy of known size in the same pass."""
    import bench

    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    calib_mib = 1024
    # the copy reads 2^30 bytes; FETCH_SIZE reports half of that in KiB (a factor of 2 to take out),
    # WRITE_SIZE all of it
    fetch = [["__amd_rocclr_copyBuffer", 4096, "FETCH_SIZE", 2 ** 30 / 1024 / 2],
             ["lsa::refresh_kernel<unsigned short, 256>", 159744, "FETCH_SIZE", 50000.0],
             ["lsa::refresh_kernel<unsigned short, 256>", 159744, "FETCH_SIZE", 52000.0],
             ["lsa::refresh_kernel<unsigned short, 256>", 58368, "FETCH_SIZE", 13000.0],
             ["lsa::attn_kernel<x>", 131072, "FETCH_SIZE", 1.0]]
    write = [["__amd_rocclr_copyBuffer", 4096, "WRITE_SIZE", 2 ** 30 / 1024],
             ["lsa::refresh_kernel<unsigned short, 256>", 159744, "WRITE_SIZE", 200.0],
             ["lsa::refresh_kernel<unsigned short, 256>", 58368, "WRITE_SIZE", 50.0]]
    _write_csv(tmp_path / "f.csv", hdr, fetch)
    _write_csv(tmp_path / "w.csv", hdr, write)
    d = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), workload="ctx1m",
                              calib_mib=calib_mib, kernel="refresh_kernel")
    assert d["dispatches"] == {"fetch_pass": 2, "write_pass": 1}
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_bytes_per_launch"] == pytest.approx(51000.0 * 1024 * 2)
    assert d["write_bytes_per_launch"] == pytest.approx(200.0 * 1024)
    assert d["traffic_bytes_per_launch"] == pytest.approx(51000.0 * 2048 + 200.0 * 1024)
    assert d["kernel_sources_sha256_16"] == bench.kernel_hash("refresh_kernel")


def test_kernel_trace_summary_groups_dispatches_by_kernel_and_grid(tmp_path):
    """Per (kernel, grid) dispatch count and durations from a kernel-trace CSV (ns stamps -> us)."""
    import bench

    hdr = ["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"]
    rows = [["void lsa::(anonymous namespace)::attn_kernel<A>(P)", 131072, 0, 66000],
            ["void lsa::(anonymous namespace)::attn_kernel<A>(P)", 131072, 100000, 168000],
            ["void lsa::(anonymous namespace)::refresh_kernel<B>(Q)", 159744, 200000, 227000],
            ["void lsa::(anonymous namespace)::refresh_kernel<B>(Q)", 58368, 300000, 316000]]
    _write_csv(tmp_path / "t.csv", hdr, rows)
    d = bench.kernel_trace_summary(str(tmp_path / "t.csv"))
    got = {(k["kernel"], k["grid_x"]): k for k in d["kernels"]}
    a = got[("lsa::attn_kernel<A>", 131072)]
    assert a["dispatches"] == 2 and a["mean_us"] == pytest.approx(67.0) and a["min_us"] == pytest.approx(66.0)
    assert got[("lsa::refresh_kernel<B>", 159744)]["mean_us"] == pytest.approx(27.0)
    assert got[("lsa::refresh_kernel<B>", 58368)]["dispatches"] == 1
