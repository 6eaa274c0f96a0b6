"""The low-rank query projection on the GPU: the latent kernel against the oracle's latent, and a
decode loop whose refreshes go through the latent (selections bit for bit, outputs within the
tolerance)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, make_session, raw_to_torch, run_loop

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d_model,rank,n_req,shared", [
    ("bf16", 4096, 2048, 4, True), ("bf16", 1024, 512, 5, False), ("f32", 512, 256, 3, False),
    ("bf16", 4096, 2048, 16, True), ("bf16", 1280, 256, 37, False), ("f32", 1024, 256, 20, False),
    ("bf16", 2048, 512, 9, False), ("bf16", 2048, 512, 10, True)])
def test_latent_matches_oracle(dtype, d_model, rank, n_req, shared):
    """c_i = A_i h: bf16 latents are the oracle's (exact sum rounded to bfloat16) up to a rounding
    decision taken on an fp32 sum instead of the exact one: equal almost everywhere over the
    batch, and elsewhere apart by at most one bfloat16 unit plus the fp32 sum's error.  That error
    is bounded by height x 2^-24 x sum_j |A_ij h_j| for a summation tree of that height (the
    recursive-summation bound); at these sizes every kernel sums a row in a tree of height below
    64.  Where cancellation leaves a small latent, that error can exceed the latent's own bfloat16
    unit.  fp32 latents agree to fp32 accumulation error.  Batches of 10 or more bf16 requests take
    the matrix-core kernel (9 and 10: either side of the switch; 10, 16 and 37: partial, whole and
    ragged request blocks; 1280 elements: a row ending inside a slice)."""
    from lookahead_block_sparse_amd import lsa_query_latent
    from workloads import bf16_bits_from_f32

    log(f"latent {dtype} d_model {d_model} rank {rank} requests {n_req} shared hidden {shared}")
    rng = np.random.default_rng(7)
    n_idx = 3
    a32 = (rng.standard_normal((n_idx, rank, d_model)) / np.sqrt(d_model)).astype(np.float32)
    h32 = rng.standard_normal((n_req, 1 if shared else n_idx, d_model)).astype(np.float32)
    enc = (lambda x: bf16_bits_from_f32(x)) if dtype == "bf16" else (lambda x: x)
    a_raw, h_raw = enc(a32), enc(h32)
    dev = torch.device("cuda")
    st = torch.int16 if dtype == "bf16" else torch.float32
    out = torch.empty((n_req, n_idx, rank), dtype=st, device=dev)
    lsa_query_latent(dtype=dtype, d_model=d_model, rank=rank, n_idx=n_idx, n_req=n_req,
                     hidden=raw_to_torch(h_raw, dev), w_down=raw_to_torch(a_raw, dev), latent=out,
                     hidden_req_stride=h_raw.shape[1] * d_model, hidden_idx_stride=0 if shared else d_model)
    got_raw = out.cpu().numpy()
    got = oracle.decode_values(got_raw.view(np.uint16) if dtype == "bf16" else got_raw, dtype)
    A = oracle.decode_values(a_raw, dtype)
    exact_frac, worst = [], 0.0
    for r in range(n_req):
        h = oracle.decode_values(h_raw[r, 0] if shared else h_raw[r], dtype)
        want = oracle.query_latent(h, A, dtype)
        if dtype == "bf16":
            hh = np.broadcast_to(h, (n_idx, d_model))
            mass = np.stack([np.abs(A[i]) @ np.abs(hh[i]) for i in range(n_idx)])
            ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(want), np.abs(got[r])))[1] - 8)
            diff = np.abs(got[r] - want)
            bound = ulp + 64 * 2.0 ** -24 * mass
            worst = max(worst, float((diff / bound).max()))
            assert (diff <= bound).all(), (r, diff.max())
            exact_frac.append((diff == 0).mean())
        else:
            exact = np.stack([A[i] @ (h if h.ndim == 1 else h[i]) for i in range(n_idx)])
            assert np.allclose(got[r], want, rtol=1e-5, atol=1e-5 * np.abs(exact).max())
    if exact_frac:
        log(f"  exact fraction {np.mean(exact_frac):.5f}; worst difference / bound {worst:.3f}")
        assert np.mean(exact_frac) >= 0.999, np.mean(exact_frac)


@pytest.mark.parametrize("name", ["ctx128k_s", "ragged_s"])
def test_lowrank_loop_matches_oracle(name):
    """Every refresh of a low-rank workload (rank 512) selects the oracle's blocks, bit for bit, and
    the attention outputs at sampled steps match the oracle."""
    from workloads import get_config

    cfg = get_config(name).scaled(q_rank=512, steps=70)
    log(f"low-rank loop {name}, rank {cfg.q_rank}")
    wl = conditioned_workload(cfg, seed=29)
    sess = make_session(wl, with_masks=False)
    assert sess.rank == 512
    sample = [0, 63, 64, 69]
    gpu, sels = run_loop(wl, sess, range(cfg.steps), record=sample)
    refs, outs = oracle.simulate(wl, steps=sample)
    assert len(sels) == sum(len(s) for s in wl.refresh_steps)
    for (r, k), ids in sels.items():
        assert np.array_equal(ids, refs[r][k].ids), (name, r, k)
    worst = (0.0, 0.0, 0.0)
    for t in sample:
        ref = np.stack([outs[(r, t)] for r in range(wl.n_req)])
        worst = tuple(max(a, b) for a, b in zip(worst, attention_errors(gpu[t], ref)))
    log(f"  {name}: {len(sels)} low-rank refreshes bit-exact; max abs {worst[0]:.3e} rel {worst[1]:.3e}")
    assert worst[0] <= ABS_TOL and worst[1] <= REL_TOL, worst
