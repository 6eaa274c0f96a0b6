"""The label-denoising oracle against its pins (oracle_pins_denoise.py), and planted mistakes in
it (on the CPU), each of which some pin must catch."""

import numpy as np
import pytest

import oracle.denoise_ref as D
from oracle_pins_denoise import DENOISE_PINS

_orig = {name: getattr(D, name) for name in dir(D) if not name.startswith("_")}


@pytest.mark.parametrize("pin", DENOISE_PINS, ids=[p.__name__ for p in DENOISE_PINS])
def test_pin(pin):
    pin(D)


def _m_softmax_no_norm(x):
    x = np.asarray(x, dtype=np.float64)
    return np.exp(x - x.max())


def _m_softmax_of_negated(x):
    return _orig["layer_softmax"](-np.asarray(x, dtype=np.float64))


def _top_p_variant(x, p, order_fn, k_fn):
    x = np.asarray(x, dtype=np.float64)
    prob = _orig["layer_softmax"](x)
    order = order_fn(x)
    csum = np.cumsum(prob[order])
    return np.sort(order[:k_fn(csum, p, len(x))]).astype(np.int32)


def _m_top_p_strict(x, p=0.6):
    return _top_p_variant(x, p, lambda x: np.lexsort((np.arange(len(x)), -x)),
                          lambda c, p, n: min(int(np.searchsorted(c, p, side="right")) + 1, n))


def _m_top_p_below(x, p=0.6):
    return _top_p_variant(x, p, lambda x: np.lexsort((np.arange(len(x)), -x)),
                          lambda c, p, n: max(1, int(np.searchsorted(c, p, side="left"))))


def _m_top_p_ascending(x, p=0.6):
    return _top_p_variant(x, p, lambda x: np.lexsort((np.arange(len(x)), x)),
                          lambda c, p, n: min(int(np.searchsorted(c, p, side="left")) + 1, n))


def _m_top_p_ties_high_id(x, p=0.6):
    return _top_p_variant(x, p, lambda x: np.lexsort((-np.arange(len(x)), -x)),
                          lambda c, p, n: min(int(np.searchsorted(c, p, side="left")) + 1, n))


def _m_top_p_fixed_k(x, p=0.6):
    x = np.asarray(x, dtype=np.float64)
    k = max(1, int(round(p * len(x))))
    return np.sort(np.lexsort((np.arange(len(x)), -x))[:k]).astype(np.int32)


def _m_vote_strict(sets, n_blocks, min_votes=3):
    return _orig["vote"](sets, n_blocks, min_votes + 1)


def _m_vote_union(sets, n_blocks, min_votes=3):
    return _orig["vote"](sets, n_blocks, 1)


def _m_denoise_first_layer_only(x, p=0.6, min_votes=3):
    x = np.asarray(x, dtype=np.float64)
    s = D.top_p_set(x[0], p)
    lab = np.zeros(x.shape[1], dtype=bool)
    lab[s] = True
    return lab, lab.copy(), [s] * x.shape[0]


MUTATIONS = [
    ("layer_softmax", _m_softmax_no_norm),
    ("layer_softmax", _m_softmax_of_negated),
    ("top_p_set", _m_top_p_strict),
    ("top_p_set", _m_top_p_below),
    ("top_p_set", _m_top_p_ascending),
    ("top_p_set", _m_top_p_ties_high_id),
    ("top_p_set", _m_top_p_fixed_k),
    ("vote", _m_vote_strict),
    ("vote", _m_vote_union),
    ("denoise_window", _m_denoise_first_layer_only),
]


@pytest.mark.parametrize("target,mutant", MUTATIONS, ids=[m.__name__ for _, m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(D, target, mutant)
    caught = []
    for pin in DENOISE_PINS:
        try:
            pin(D)
        except Exception as e:  # an exception is a caught mistake too
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {mutant.__name__} of {target} passes every pin"
