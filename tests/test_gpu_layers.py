"""One selection driving the block loads of several attention layers.

The pages' indexers feed the block loads of the whole model; here each layer has its own K/V, decode
queries and new tokens, and shares the session's hot slots, block table and selection.  Every
refresh must match the oracle bit for bit, every layer's hot pool must hold that layer's cold
blocks, and every layer's attention output must match the oracle for that layer.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, raw_to_torch

pytestmark = pytest.mark.gpu


def _session(wl, cold_on_device):
    from lookahead_block_sparse_amd.session import LSASession

    cfg = wl.cfg
    sess = LSASession(dtype=cfg.dtype, n_idx=cfg.n_idx, d_model=cfg.d_model, d_idx=cfg.d_idx,
                      n_heads=cfg.n_heads, head_dim=cfg.head_dim, win_cap=cfg.window, n_blocks=wl.n_blocks,
                      w_q=wl.w_q, keys=wl.keys, cold_on_device=cold_on_device, n_layers=cfg.n_layers)
    for r in range(wl.n_req):
        for layer in range(cfg.n_layers):
            k, v = wl.kv_prefill(r, layer)
            sess.load_prefill(r, k, v, layer=layer)
    return sess


def _check_layers(sess, r, ids):
    bb = sess.block_bytes
    base = int(sess.slot_base[r])
    table = sess.table[2 * base: 2 * (base + len(ids))].view(-1, 2).cpu().numpy()
    assert np.array_equal(table[:, 0], ids)
    slots = torch.as_tensor(table[:, 1], dtype=torch.long, device=sess.hot.device)
    lb = int(sess.n_blocks[r]) * bb
    for layer in range(sess.n_layers):
        hot, _ = sess.layer_views(layer)
        cold = sess.cold[r][layer * lb:(layer + 1) * lb]
        got = hot.view(-1, bb)[slots].cpu()
        want = cold.view(-1, bb)[torch.as_tensor(ids, dtype=torch.long, device=cold.device)].cpu()
        assert torch.equal(got, want), (r, layer)


@pytest.mark.parametrize("cold_on_device", [True, False])
def test_multi_layer_loop_matches_oracle(cold_on_device):
    from lookahead_block_sparse_amd.session import DecodeLoop
    from workloads import get_config

    cfg = get_config("ctx512k_s").scaled(n_layers=3, hidden_rho=0.9, steps=140)
    log(f"{cfg.n_layers} layers, hidden rho {cfg.hidden_rho}, cold on device {cold_on_device}")
    wl = conditioned_workload(cfg, seed=31)
    R, T, L = wl.n_req, cfg.steps, cfg.n_layers
    sess = _session(wl, cold_on_device)
    dev = sess.device
    outs_dev = [torch.empty((R, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev) for _ in range(L)]
    loops = [DecodeLoop(sess, wl.ctx, np.full(R, cfg.window, dtype=np.int32), outs_dev[layer], layer=layer)
             for layer in range(L)]
    sample = sorted({0, 63, 64, 127, 128, T - 1})
    gpu = {}
    sels = {}
    copied = []
    for t in range(T):
        reqs = wl.refreshes_at(t)
        if reqs:
            k_of = {r: wl.refresh_index_at(r, t) for r in reqs}
            got = sess.refresh(reqs, np.stack([wl.hidden[r][k_of[r]] for r in reqs]), wl.bias[reqs])
            res = sess.gather_many(got)
            torch.cuda.synchronize()
            copied.append(sum(c for c, _ in res.values()))
            for r in reqs:
                sels[(r, k_of[r])] = got[r]
                _check_layers(sess, r, got[r])
        for layer in range(L):
            loops[layer].step(t, raw_to_torch(wl.q_dec_of(layer)[t], dev), raw_to_torch(wl.k_new_of(layer)[t], dev),
                              raw_to_torch(wl.v_new_of(layer)[t], dev))
        if t in sample:
            for layer in range(L):
                gpu[(layer, t)] = outs_dev[layer].double().cpu().numpy()
    torch.cuda.synchronize()
    worst = (0.0, 0.0, 0.0)
    for layer in range(L):
        refs, outs = oracle.simulate(wl, steps=sample, layer=layer)
        for (r, k), ids in sels.items():
            assert np.array_equal(ids, refs[r][k].ids), (layer, r, k)
        for t in sample:
            ref = np.stack([outs[(r, t)] for r in range(R)])
            worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[(layer, t)], ref)))
    log(f"  blocks copied per refresh {copied}; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst
    # correlated hidden states keep most of the selection between refreshes
    assert copied[1] < copied[0] / 2, copied
