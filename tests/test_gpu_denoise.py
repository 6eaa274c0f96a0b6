"""Label denoising on the GPU against the oracle: every layer's top-p set, the voted labels and the
per-window counts, bit for bit (all three are index work; the kernel decides "reaches top_p" on
exact fixed-point sums of fp64 exponentials, the oracle on float64 running sums, and the two can
only disagree when a running sum lies within ~1e-11 of top_p, which these seeded inputs do not
reach: the test checks that margin on the oracle side)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import log

pytestmark = pytest.mark.gpu


def _bits_to_ids(words, n):
    bits = np.unpackbits(words.view(np.uint8), bitorder="little")
    return np.flatnonzero(bits[:n]).astype(np.int32), bits[n:].any()


def _run(dw, top_p, min_votes, with_sets=True):
    from lookahead_block_sparse_amd import lsa_label_denoise, lsa_label_denoise_workspace

    dev = torch.device("cuda")
    L_, W = dw.n_layers, dw.n_windows
    words = (int(dw.n_blk.max()) + 63) // 64
    logits = torch.from_numpy(dw.logits).to(dev)
    n_blk_dev = torch.from_numpy(dw.n_blk).to(dev)
    labels = torch.full((W, words), -1, dtype=torch.int64, device=dev)
    n_pos = torch.full((W,), -1, dtype=torch.int32, device=dev)
    n_naive = torch.full((W,), -1, dtype=torch.int32, device=dev)
    sets = torch.full((L_, W, words), -1, dtype=torch.int64, device=dev) if with_sets else None
    ws_bytes = lsa_label_denoise_workspace(n_layers=L_, n_blk=dw.n_blk, top_p=top_p, min_votes=min_votes,
                                           with_layer_sets=with_sets)
    ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    lsa_label_denoise(logits=logits, n_blk=dw.n_blk, n_blk_dev=n_blk_dev, labels=labels, n_pos=n_pos,
                      top_p=top_p, min_votes=min_votes, n_naive=n_naive, layer_sets=sets, workspace=ws)
    torch.cuda.synchronize()
    return (labels.cpu().numpy(), n_pos.cpu().numpy(), n_naive.cpu().numpy(),
            sets.cpu().numpy() if with_sets else None)


def _check(dw, top_p, min_votes, with_sets=True):
    labels, n_pos, n_naive, sets = _run(dw, top_p, min_votes, with_sets)
    for w in range(dw.n_windows):
        n = int(dw.n_blk[w])
        x = dw.logits[:, w, :n].astype(np.float64)
        lab, naive, osets = oracle.denoise_window(x, top_p, min_votes)
        # the decision margin the comparison relies on
        for l in range(dw.n_layers):
            p = oracle.layer_softmax(x[l])
            order = np.lexsort((np.arange(n), -x[l]))
            c = np.cumsum(p[order])
            assert np.abs(c - top_p).min() > 1e-9 or top_p == 1.0, (w, l)
        if with_sets:
            for l in range(dw.n_layers):
                ids, stray = _bits_to_ids(sets[l, w], n)
                assert not stray
                assert np.array_equal(ids, osets[l]), (w, l, len(ids), len(osets[l]))
        ids, stray = _bits_to_ids(labels[w], n)
        assert not stray
        assert np.array_equal(ids, np.flatnonzero(lab)), (w, len(ids), int(lab.sum()))
        assert n_pos[w] == int(lab.sum()) and n_naive[w] == int(naive.sum()), (w, n_pos[w], n_naive[w])
    return n_pos, n_naive


def test_denoise_matches_oracle():
    from workloads import build_denoise_workload

    dw = build_denoise_workload([16384, 9000, 4113, 100, 1, 64, 65], seed=3)
    n_pos, n_naive = _check(dw, 0.6, 3)
    log(f"denoise 21 layers x {dw.n_windows} windows: labels {n_pos.tolist()}, naive {n_naive.tolist()}")
    assert n_naive[0] > 5000 and 100 <= n_pos[0] <= 1000  # the magnitudes the pages report


def test_denoise_ties_taken_by_block_id():
    """Integer logits: long runs of equal logits straddle the top-p boundary.  The run of equal
    logits at a row's cut (computed here in float64) is ranked in one wave when it has at most 64
    blocks, by the whole group up to 256, and by the bisection kernel beyond; the two workloads'
    rows cover all three."""
    from workloads import build_denoise_workload

    def cut_runs(dw):
        runs = []
        for l in range(dw.n_layers):
            for w in range(dw.n_windows):
                x = dw.row(l, w).astype(np.float64)
                o = np.argsort(-x, kind="stable")
                pr = np.exp(x[o] - x.max())
                cut = int(np.searchsorted(np.cumsum(pr), 0.6 * pr.sum()))
                runs.append(int((x == x[o][cut]).sum()))
        return runs

    wide = build_denoise_workload([16384, 5000, 777], seed=4, integer_logits=True, noise=1.5)
    narrow = build_denoise_workload([16384, 3000], seed=7, integer_logits=True, noise=0.5, n_layers=5)
    runs = np.array(cut_runs(wide) + cut_runs(narrow))
    assert (runs <= 64).any() and ((runs > 64) & (runs <= 256)).any() and (runs > 256).any(), np.unique(runs)
    _check(wide, 0.6, 3)
    _check(narrow, 0.6, 3)


@pytest.mark.parametrize("top_p,min_votes", [(0.3, 1), (0.9, 21), (1.0, 3), (0.6, 11)])
def test_denoise_other_parameters(top_p, min_votes):
    from workloads import build_denoise_workload

    dw = build_denoise_workload([3000, 128, 16384], n_layers=21, seed=5)
    _check(dw, top_p, min_votes)


def test_denoise_without_layer_sets_output():
    """The layer sets kept in the workspace give the same labels."""
    from workloads import build_denoise_workload

    dw = build_denoise_workload([2048, 700], n_layers=7, seed=6)
    a = _run(dw, 0.6, 3, with_sets=True)
    b = _run(dw, 0.6, 3, with_sets=False)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3]))
    _check(dw, 0.6, 3, with_sets=False)
