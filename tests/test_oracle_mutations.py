"""Planted mistakes in the oracle (on the CPU) must each be caught by at least one pin.

Each mutation replaces one oracle function with a plausible wrong version (a
dropped term, a wrong sign, an off-by-one index, a transposed operand, the
wrong combination rule) and re-runs every pin of oracle_pins.py.  A mutation
that no pin catches means the pins do not fix that part of the oracle.
"""

import math

import numpy as np
import pytest

import oracle.lsa_ref as ref
from oracle_pins import PINS

_orig = {name: getattr(ref, name) for name in dir(ref) if not name.startswith("_")}


def _m_threshold_ge(z, level=0.5):
    return np.asarray(z, dtype=np.float64) >= ref.level_logit(level)


def _m_threshold_prob(z, level=0.5):
    return np.asarray(z, dtype=np.float64) > level


def _m_threshold_ignores_level(z, level=0.5):
    return np.asarray(z, dtype=np.float64) > 0.0


def _m_level_logit_flipped(level):
    level = float(level)
    return float(np.log((1.0 - level) / level))


def _m_union_and(s):
    return np.all(np.asarray(s, dtype=bool), axis=0)


def _m_union_first(s):
    return np.asarray(s, dtype=bool)[0]


def _m_compact_desc(u):
    return np.flatnonzero(np.asarray(u, dtype=bool))[::-1].astype(np.int32)


def _m_logits_no_bias(q, keys, bias):
    return _orig["block_logits"](q, keys, np.zeros_like(np.asarray(bias, dtype=np.float64)))


def _m_logits_neg_bias(q, keys, bias):
    return _orig["block_logits"](q, keys, -np.asarray(bias, dtype=np.float64))


def _m_logits_wrong_indexer(q, keys, bias):
    q = np.asarray(q, dtype=np.float64)
    return _orig["block_logits"](np.stack([q[0]] * q.shape[0]), keys, bias)


def _m_query_transposed(h, w_q):
    w_q = np.asarray(w_q, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    return np.stack([w_q[i].T @ (h if h.ndim == 1 else h[i]) for i in range(w_q.shape[0])])


def _m_query_one_matrix(h, w_q):
    w_q = np.asarray(w_q, dtype=np.float64)
    return _orig["query_encoder"](h, np.stack([w_q[0]] * w_q.shape[0]))


def _m_window_plus1(seq_len, window):
    return max(0, int(seq_len) - int(window) + 1)


def _m_window_minus1(seq_len, window):
    return max(0, int(seq_len) - int(window) - 1)


def _m_token_set_block_off_by_one(seq_len, window, sel_ids, block=64):
    L = int(seq_len)
    ws = ref.window_start(L, window)
    before = np.arange(ws, dtype=np.int64)
    keep = np.isin(before // block + 1, np.asarray(sel_ids, dtype=np.int64))
    return np.concatenate([before[keep], np.arange(ws, L, dtype=np.int64)])


def _m_token_set_no_window(seq_len, window, sel_ids, block=64):
    L = int(seq_len)
    pos = np.arange(L, dtype=np.int64)
    keep = np.isin(pos // block, np.asarray(sel_ids, dtype=np.int64))
    out = pos[keep]
    return out if len(out) else np.array([L - 1])


def _m_token_set_duplicates(seq_len, window, sel_ids, block=64):
    # selected-block tokens inside the window counted a second time
    L = int(seq_len)
    ws = ref.window_start(L, window)
    allpos = np.arange(L, dtype=np.int64)
    in_sel = allpos[np.isin(allpos // block, np.asarray(sel_ids, dtype=np.int64))]
    return np.sort(np.concatenate([in_sel, np.arange(ws, L, dtype=np.int64)]))


def _m_attention_no_scale(q, k, v, scale):
    return _orig["attention"](q, k, v, 1.0)


def _m_attention_scale_1_over_d(q, k, v, scale):
    D = np.asarray(q).shape[-1]
    return _orig["attention"](q, k, v, float(scale) ** 2 if D > 1 else scale)


def _m_attention_k_for_v(q, k, v, scale):
    return _orig["attention"](q, k, k, scale)


def _m_governing_next(t, refresh_steps):
    for k, tk in enumerate(refresh_steps):
        if tk >= t:
            return k
    return len(refresh_steps) - 1


def _m_governing_strict(t, refresh_steps):
    best = 0
    for k, tk in enumerate(refresh_steps):
        if tk < t:
            best = k
    return best


def _m_decode_bf16_shift(raw, dtype):
    raw = np.asarray(raw)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _orig["decode_values"](raw, dtype)


def _m_simulate_ignores_layer(wl, steps=None, requests=None, layer=0):
    return _orig["simulate"](wl, steps, requests, 0)


def _m_round_bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _m_round_bf16_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.floor(m * 256.0 + 0.5), e - 8)


def _m_latent_no_rounding(h, w_down, dtype):
    return _orig["query_latent"](h, w_down, "f32") if dtype == "bf16" else _orig["query_latent"](h, w_down, dtype)


def _m_latent_transposed(h, w_down, dtype):
    w = np.asarray(w_down, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    c = np.stack([w[i].T @ (h if h.ndim == 1 else h[i]) for i in range(w.shape[0])])
    return _orig["round_bf16"](c) if dtype == "bf16" else c.astype(np.float32).astype(np.float64)


def _m_latent_shared_hidden(h, w_down, dtype):
    h = np.asarray(h, dtype=np.float64)
    return _orig["query_latent"](h if h.ndim == 1 else h[0], w_down, dtype)


def _m_simulate_ignores_latent(wl, steps=None, requests=None, layer=0):
    """The latent skipped: the first r elements of the hidden state stand in for it."""
    import copy
    if getattr(wl, "w_down", None) is None:
        return _orig["simulate"](wl, steps, requests, layer)
    moved = copy.copy(wl)
    rank = wl.w_down.shape[1]
    moved.w_down = None
    moved.hidden = [np.ascontiguousarray(h[:, :rank]) for h in wl.hidden]
    return _orig["simulate"](moved, steps, requests, layer)

def _m_kv_rows_off_by_one(prefill, new_rows, n_prefill, positions):
    """Decode-time rows shifted by one: position p reads the token of step p - N - 1."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((len(positions), prefill.shape[1]), dtype=np.float64)
    lo = positions < n_prefill
    out[lo] = prefill[positions[lo]]
    out[~lo] = new_rows[positions[~lo] - n_prefill - 1]
    return out


def _m_seq_len_no_current(n_prefill, t):
    """The step attends to the tokens before it but not to its own."""
    return int(n_prefill) + int(t)


MUTATIONS = [
    ("threshold", _m_threshold_ge),
    ("threshold", _m_threshold_prob),
    ("threshold", _m_threshold_ignores_level),
    ("level_logit", _m_level_logit_flipped),
    ("union", _m_union_and),
    ("union", _m_union_first),
    ("compact", _m_compact_desc),
    ("block_logits", _m_logits_no_bias),
    ("block_logits", _m_logits_neg_bias),
    ("block_logits", _m_logits_wrong_indexer),
    ("query_encoder", _m_query_transposed),
    ("query_encoder", _m_query_one_matrix),
    ("window_start", _m_window_plus1),
    ("window_start", _m_window_minus1),
    ("token_set", _m_token_set_block_off_by_one),
    ("token_set", _m_token_set_no_window),
    ("token_set", _m_token_set_duplicates),
    ("attention", _m_attention_no_scale),
    ("attention", _m_attention_scale_1_over_d),
    ("attention", _m_attention_k_for_v),
    ("governing_refresh", _m_governing_next),
    ("governing_refresh", _m_governing_strict),
    ("decode_values", _m_decode_bf16_shift),
    ("simulate", _m_simulate_ignores_layer),
    ("round_bf16", _m_round_bf16_truncate),
    ("round_bf16", _m_round_bf16_half_up),
    ("query_latent", _m_latent_no_rounding),
    ("query_latent", _m_latent_transposed),
    ("query_latent", _m_latent_shared_hidden),
    ("simulate", _m_simulate_ignores_latent),
    ("kv_rows", _m_kv_rows_off_by_one),
    ("seq_len_at", _m_seq_len_no_current),
]


@pytest.mark.parametrize("target,mutant", MUTATIONS, ids=[m.__name__ for _, m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(ref, target, mutant)
    caught = []
    for pin in PINS:
        try:
            pin(ref)
        except Exception as e:  # an exception is a caught mistake too
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {mutant.__name__} of {target} passes every pin"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin(ref)
