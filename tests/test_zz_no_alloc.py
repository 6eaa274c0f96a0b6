"""lsa_sparse_decode_noalloc (partials in the library's static per-device array, no workspace, no
allocation) against lsa_sparse_decode through the C-ABI: two calls in a row on the same inputs,
the second smaller (fewer requests, shorter contexts, fewer selected blocks), each compared with
the workspace entry point's output on the same inputs to the parity bar (max abs 2e-2, max abs /
max |ref| 1e-2) and, as both run the same kernels, to the rounding of the bf16 softmax weights;
and a call needing more partials than the array holds is refused with nothing enqueued."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_harness import ABS_TOL, REL_TOL, attention_errors, conditioned_workload, log, make_session, refresh_requests

pytestmark = pytest.mark.gpu


def _decode_args(sess, wl, t, out, reqs_limit=None):
    """lsa_decode_args of decode step t for the first reqs_limit requests (all by default); the
    window already holds the step's token (k_new / v_new not given, so both calls read the same ring)."""
    from lookahead_block_sparse_amd import DecodeArgs

    R = sess.n_req if reqs_limit is None else reqs_limit
    keep = []
    a = DecodeArgs()
    a.n_req, a.n_heads, a.head_dim = R, sess.n_heads, sess.head_dim
    a.dtype = 1 if sess.dtype == "bf16" else 0
    a.win_cap = sess.win_cap
    a.scale = float(1.0 / np.sqrt(sess.head_dim))
    pool, ring = sess.layer_views(0)
    q = torch.from_numpy(np.ascontiguousarray(wl.q_dec[t][:R]).view(np.int16) if sess.dtype == "bf16"
                         else np.ascontiguousarray(wl.q_dec[t][:R])).to(sess.device)
    seq_len = (wl.ctx[:R] + t + 1).astype(np.int32)
    window = np.full(R, wl.cfg.window, dtype=np.int32)
    n_sel = np.ascontiguousarray(sess.n_sel[:R], dtype=np.int32)  # whole tables: the kernel skips in-window blocks
    tbl_off = np.ascontiguousarray(sess.slot_base[:R], dtype=np.int32)
    keep += [q, seq_len, window, n_sel, tbl_off]
    a.q, a.ring, a.pool, a.table = q.data_ptr(), ring.data_ptr(), pool.data_ptr(), sess.table.data_ptr()
    a.n_slots_total = sess.n_slots
    a.tbl_off, a.n_sel = tbl_off.ctypes.data, n_sel.ctypes.data
    a.seq_len, a.window = seq_len.ctypes.data, window.ctypes.data
    a.out = out.data_ptr()
    a.workspace, a.workspace_bytes = sess.decode_ws.data_ptr(), sess.decode_ws.numel()
    return a, keep


def _append_tokens(sess, wl, steps):
    """Run decode steps 0..steps-1 through the session (writing their tokens into the window)."""
    from gpu_harness import raw_to_torch

    out = torch.empty((sess.n_req, sess.n_heads, sess.head_dim), dtype=torch.float32, device=sess.device)
    for t in range(steps):
        sess.decode(raw_to_torch(wl.q_dec[t], sess.device), (wl.ctx + t + 1).astype(np.int32),
                    np.full(sess.n_req, wl.cfg.window, dtype=np.int32), out,
                    k_new=raw_to_torch(wl.k_new[t], sess.device), v_new=raw_to_torch(wl.v_new[t], sess.device))
    torch.cuda.synchronize()


def test_noalloc_decode_matches_workspace_decode():
    from lookahead_block_sparse_amd import LIB
    from workloads import get_config

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = []
    # first call: 3 requests x 24K context; second: 1 request of a 4K fp32 workload, fewer blocks
    for name, steps, limit in (("ctx512k_s", 3, None), ("tiny", 2, 1)):
        cfg = get_config(name).scaled(steps=max(steps, 2))
        wl = conditioned_workload(cfg, seed=51)
        sess = make_session(wl, cold_on_device=True, with_masks=False)
        refresh_requests(wl, sess, list(range(wl.n_req)), {r: 0 for r in range(wl.n_req)})
        _append_tokens(sess, wl, steps)
        cases.append((name, sess, wl, steps - 1, limit))
    # the two calls of the entry point that allocates nothing back to back (the second smaller),
    # then the workspace entry point on the same inputs
    runs = []
    for name, sess, wl, t, limit in cases:
        R = sess.n_req if limit is None else limit
        out_na = torch.full((R, sess.n_heads, sess.head_dim), float("nan"), device=sess.device)
        a, keep = _decode_args(sess, wl, t, out_na, limit)
        a.workspace, a.workspace_bytes = None, 0  # ignored by the entry point that allocates nothing
        assert LIB.lsa_sparse_decode_noalloc(ctypes.byref(a), stream) == 0, LIB.lsa_last_error()
        runs.append((name, sess, wl, t, limit, R, out_na, keep))
    for name, sess, wl, t, limit, R, out_na, _ in runs:
        out_ws = torch.full_like(out_na, float("nan"))
        a, keep = _decode_args(sess, wl, t, out_ws, limit)
        assert LIB.lsa_sparse_decode(ctypes.byref(a), stream) == 0, LIB.lsa_last_error()
        torch.cuda.synchronize()
        ref = out_ws.double().cpu().numpy()
        got = out_na.double().cpu().numpy()
        assert np.isfinite(ref).all() and np.isfinite(got).all()
        e = attention_errors(got, ref)
        log(f"no-alloc decode {name}: {R} request(s), step {t}; vs workspace entry max abs {e[0]:.3e} rel {e[1]:.3e}")
        assert e[0] <= ABS_TOL and e[1] <= REL_TOL, e
        # the same kernels; which tiles a wave takes varies from run to run, and the bf16 softmax
        # weights of P.V are rounded relative to each wave's running maximum
        assert e[1] <= 5e-3, e


def test_noalloc_decode_validates_before_enqueueing():
    """An invalid call of the entry point that allocates nothing returns its status and enqueues
    nothing (the output stays untouched).  (A call needing more partials than the array holds is
    refused the same way; that needs a device with more than 320 compute units.)"""
    from lookahead_block_sparse_amd import LIB, LSA_ERR_INVALID
    from workloads import get_config

    wl = conditioned_workload(get_config("tiny").scaled(steps=2), seed=52)
    sess = make_session(wl, cold_on_device=True, with_masks=False)
    out = torch.zeros((1, sess.n_heads, sess.head_dim), dtype=torch.float32, device=sess.device)
    a, keep = _decode_args(sess, wl, 0, out)
    a.reserved0 = 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert LIB.lsa_sparse_decode_noalloc(ctypes.byref(a), stream) == LSA_ERR_INVALID
    assert b"reserved" in LIB.lsa_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
