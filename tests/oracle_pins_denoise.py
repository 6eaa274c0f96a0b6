"""Checks that pin the label-denoising oracle (oracle/denoise_ref.py) to facts other than itself:
a library softmax, hand-derived top-p fixtures (tests/golden/top_p_sets.json, with the page's
citation), closed forms for uniform rows, brute force over every subset of small rows, and explicit
vote counts.  Each pin takes the module `D` so that planted mistakes can be shown to be caught."""

from __future__ import annotations

import itertools
import json
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


def pin_softmax_is_the_library_softmax(D):
    """Step 1 equals scipy's softmax, sums to one, and ignores a constant shift of the logits."""
    from scipy.special import softmax

    rng = np.random.default_rng(51)
    for n in (1, 5, 300):
        x = rng.standard_normal(n) * 3
        p = D.layer_softmax(x)
        assert np.allclose(p, softmax(x), rtol=1e-13, atol=0)
        assert abs(p.sum() - 1.0) < 1e-12
        assert np.allclose(D.layer_softmax(x + 100.0), p, rtol=1e-12, atol=0)


def pin_top_p_fixture(D):
    """The hand-derived cases of top_p_sets.json."""
    g = json.loads((GOLDEN / "top_p_sets.json").read_text())
    for c in g["cases"]:
        x = np.log(np.asarray(c["logits_ln"], dtype=np.float64)) if "logits_ln" in c else \
            np.asarray(c["logits"], dtype=np.float64)
        got = D.top_p_set(x, g["p"])
        assert got.tolist() == c["set"], (c, got.tolist())


def pin_top_p_uniform_rows(D):
    """Uniform logits: every block has probability 1/n, so the set is the first ceil(p n) ids
    (n and p chosen so that p n is not an integer); with p = 0.6 and n = 10 the running sum of six
    tenths is 0.6 itself in float64, and 'reaches' keeps exactly six."""
    for n in (3, 7, 11, 33):
        for p in (0.3, 0.6, 0.95):
            k = int(np.ceil(p * n))
            assert not np.isclose(p * n, round(p * n))
            assert D.top_p_set(np.zeros(n), p).tolist() == list(range(k)), (n, p)
    assert D.top_p_set(np.zeros(10), 0.6).tolist() == list(range(6))


def pin_top_p_brute_force(D):
    """On rows of up to 9 blocks: no subset with probability >= p is smaller than the set, the set
    reaches p, and it is the highest-probability prefix (ties in increasing id)."""
    rng = np.random.default_rng(52)
    for trial in range(200):
        n = int(rng.integers(1, 10))
        x = np.round(rng.standard_normal(n) * 2, 1)  # rounded: ties occur
        p_target = float(rng.choice([0.3, 0.6, 0.9]))
        prob = np.exp(x - x.max())
        prob /= prob.sum()
        got = D.top_p_set(x, p_target)
        best = min(len(s) for k in range(1, n + 1) for s in itertools.combinations(range(n), k)
                   if prob[list(s)].sum() >= p_target - 1e-12)
        assert len(got) == best, (x, p_target, got, best)
        assert prob[got].sum() >= p_target - 1e-12
        out = np.setdiff1d(np.arange(n), got)
        for a in got:
            for b in out:
                assert x[a] > x[b] or (x[a] == x[b] and a < b), (x, got)


def pin_vote_counts(D):
    """Step 3 by explicit counting: a block is positive with at least min_votes layers, not with one
    fewer; min_votes = 1 is the union."""
    rng = np.random.default_rng(53)
    n = 50
    sets = [np.sort(rng.choice(n, size=int(rng.integers(0, 30)), replace=False)) for _ in range(21)]
    count = [sum(1 for s in sets if b in set(s.tolist())) for b in range(n)]
    for m in (1, 2, 3, 5, 21, 22):
        got = D.vote(sets, n, m)
        assert got.tolist() == [c >= m for c in count], m
    assert D.vote(sets, n, 1).tolist() == [any(b in set(s.tolist()) for s in sets) for b in range(n)]


def pin_denoise_window_special_cases(D):
    """Identical layers vote together: the labels are that layer's set when there are at least
    min_votes layers and empty when there are fewer; naive labels are the union of the layers'
    sets; one dominant block per layer gives each layer a singleton set."""
    rng = np.random.default_rng(54)
    row = rng.standard_normal(40)
    x = np.stack([row] * 5)
    labels, naive, sets = D.denoise_window(x, 0.6, 3)
    s0 = D.top_p_set(row, 0.6)
    assert np.flatnonzero(labels).tolist() == s0.tolist() == np.flatnonzero(naive).tolist()
    labels2, _, _ = D.denoise_window(x[:2], 0.6, 3)
    assert not labels2.any()
    # layer l's dominant block is l % 4: blocks 0..3 get 2, 2, 1, 1 votes of 6 layers
    x = np.zeros((6, 12))
    for l in range(6):
        x[l, l % 4] = 30.0
    labels, naive, sets = D.denoise_window(x, 0.6, 2)
    assert [s.tolist() for s in sets] == [[l % 4] for l in range(6)]
    assert np.flatnonzero(labels).tolist() == [0, 1]
    assert np.flatnonzero(naive).tolist() == [0, 1, 2, 3]


DENOISE_PINS = [
    pin_softmax_is_the_library_softmax,
    pin_top_p_fixture,
    pin_top_p_uniform_rows,
    pin_top_p_brute_force,
    pin_vote_counts,
    pin_denoise_window_special_cases,
]
