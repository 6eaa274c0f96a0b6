"""Checks that pin the CPU oracle to facts other than itself.

Each pin takes the oracle module `O` and raises AssertionError when the oracle
disagrees with a closed form, a library routine, a hand-derived fixture under
tests/golden/ (each with its citation of the pages), or a brute-force
evaluation written in a different formulation.  They are functions of `O` so
that tests/test_oracle_mutations.py can re-run them against an oracle with a
planted mistake and show that every such mistake is caught.
"""

from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


def _golden(name):
    with open(GOLDEN / name) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------
def pin_bf16_decode(O):
    """bf16 bit patterns decode to the values the format defines (fixture bf16_values.json)."""
    g = _golden("bf16_values.json")
    bits = np.array([int(c["bits"], 16) for c in g["cases"]], dtype=np.uint16)
    want = np.array([c["value"] for c in g["cases"]], dtype=np.float64)
    got = O.decode_values(bits, "bf16")
    assert np.array_equal(got, want), (got, want)
    f = np.array([1.5, -3.25, 1e-20], dtype=np.float32)
    assert np.array_equal(O.decode_values(f, "f32"), f.astype(np.float64))


def pin_query_encoder_columns(O):
    """A one-hot hidden state e_m picks column m of every projection matrix."""
    rng = _rng(1)
    w = rng.standard_normal((3, 5, 7))
    for m in range(7):
        h = np.zeros(7)
        h[m] = 1.0
        q = O.query_encoder(h, w)
        assert q.shape == (3, 5)
        assert np.array_equal(q, w[:, :, m])
    # per-indexer hidden states: indexer i sees its own one-hot
    hs = np.zeros((3, 7))
    hs[0, 1] = hs[1, 4] = hs[2, 6] = 1.0
    q = O.query_encoder(hs, w)
    assert np.array_equal(q, np.stack([w[0, :, 1], w[1, :, 4], w[2, :, 6]]))


def pin_query_encoder_brute(O):
    """q[i][j] = sum_m W[i][j][m] h[m], by explicit loops (square matrices so a transposed
    operand would not even change the shape)."""
    rng = _rng(2)
    for d in (6, 9):
        w = rng.standard_normal((3, d, d))
        h = rng.standard_normal(d)
        want = np.zeros((3, d))
        for i in range(3):
            for j in range(d):
                want[i, j] = math.fsum(w[i, j, m] * h[m] for m in range(d))
        got = O.query_encoder(h, w)
        assert np.allclose(got, want, rtol=0, atol=1e-12), np.abs(got - want).max()


def pin_block_logits(O):
    """z = q.k + bias: brute force, a key orthogonal to q scores exactly the bias, and a
    key c q/|q|^2 scores c + bias."""
    rng = _rng(3)
    q = rng.standard_normal((3, 8))
    keys = rng.standard_normal((3, 5, 8))
    bias = np.array([0.25, -1.5, 2.0])
    want = np.zeros((3, 5))
    for i in range(3):
        for b in range(5):
            want[i, b] = math.fsum(q[i, j] * keys[i, b, j] for j in range(8)) + bias[i]
    got = O.block_logits(q, keys, bias)
    assert got.shape == (3, 5)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    # orthogonal keys and keys along q
    q = np.array([[1.0, 0, 0, 0], [0, 2.0, 0, 0], [0, 0, 0, 4.0]])
    k = np.zeros((3, 2, 4))
    k[0, 0] = [0, 3, -1, 2]          # orthogonal to q0
    k[1, 0] = [5, 0, 7, 1]           # orthogonal to q1
    k[2, 0] = [1, 1, 1, 0]           # orthogonal to q2
    for i in range(3):
        k[i, 1] = 1.75 * q[i] / (q[i] @ q[i])
    z = O.block_logits(q, k, bias)
    assert np.array_equal(z[:, 0], bias)
    assert np.allclose(z[:, 1], 1.75 + bias, rtol=0, atol=1e-15)


def pin_threshold_is_sigmoid_half(O):
    """Selection is sigmoid(z) > 0.5 computed with math.exp, over magnitudes 1e-6 .. 50."""
    mags = np.concatenate([np.logspace(-6, np.log10(50), 200)])
    z = np.concatenate([mags, -mags, [0.0]])
    want = np.array([1.0 / (1.0 + math.exp(-v)) > 0.5 for v in z])
    got = O.threshold(z)
    assert np.array_equal(got, want)


def pin_threshold_levels(O):
    """At other selection levels the rule is still sigmoid(z) > level, computed with math.exp, on
    logits on either side of the level's logit (offsets 1e-6 .. 30) and at a few fixed values; the
    default level is 0.5."""
    for level in (0.1, 0.3, 0.5, 0.7, 0.9):
        lg = math.log(level / (1.0 - level))
        mags = np.logspace(-6, np.log10(30), 120)
        z = np.concatenate([lg + mags, lg - mags, [-3.0, -0.5, 0.0, 0.4, 2.5]])
        want = np.array([1.0 / (1.0 + math.exp(-v)) > level for v in z])
        assert np.array_equal(O.threshold(z, level), want), level
    z = np.linspace(-4, 4, 81)
    assert np.array_equal(O.threshold(z), O.threshold(z, 0.5))
    # a higher level keeps fewer blocks: the selections are nested
    rng = _rng(13)
    z = rng.standard_normal((3, 400))
    sets = [O.threshold(z, lv) for lv in (0.2, 0.5, 0.8)]
    assert (sets[1] <= sets[0]).all() and (sets[2] <= sets[1]).all() and sets[0].sum() > sets[2].sum()


def pin_union_is_set_union(O):
    """Loaded ids = sorted(set union of the per-indexer selections)."""
    rng = _rng(4)
    for trial in range(20):
        n_idx = 1 + trial % 4
        s = rng.random((n_idx, 97)) < rng.uniform(0.0, 0.3)
        want = sorted(set().union(*[set(np.flatnonzero(s[i]).tolist()) for i in range(n_idx)]))
        got = O.compact(O.union(s))
        assert got.dtype == np.int32
        assert got.tolist() == want


def pin_golden_or_union(O):
    """Hand-applied threshold and OR rule (fixture or_union.json)."""
    g = _golden("or_union.json")
    z = np.array(g["logits"])
    s = O.threshold(z)
    for i, ids in enumerate(g["expected_per_indexer"]):
        assert np.flatnonzero(s[i]).tolist() == ids
    assert O.compact(O.union(s)).tolist() == g["expected_ids"]


def pin_golden_cadence(O):
    """Which refresh governs which step (fixture refresh_cadence.json)."""
    g = _golden("refresh_cadence.json")
    for case in g["cases"]:
        for t, k in zip(case["steps"], case["expected"]):
            assert O.governing_refresh(t, case["refresh_steps"]) == k, (case, t)


def pin_golden_token_set(O):
    """Window plus selected-block positions (fixture token_set.json)."""
    g = _golden("token_set.json")
    for case in g["cases"]:
        want = np.concatenate([np.arange(a, b) for a, b in case["expected_ranges"]])
        got = O.token_set(case["seq_len"], case["window"], case["sel_ids"], g["block"])
        assert len(got) == case["expected_count"]
        assert np.array_equal(np.asarray(got), want), case


def pin_golden_attention(O):
    """Rational softmax weights (fixture attention.json)."""
    g = _golden("attention.json")
    p = np.arange(4)
    k = np.stack([math.sqrt(2) * np.log(p + 1.0), math.sqrt(2) * np.log(4.0 - p)], axis=1)
    o = O.attention(np.array(g["q"]), k, np.array(g["v"]), 1.0 / math.sqrt(2.0))
    assert np.allclose(o, np.array(g["expected"]), rtol=0, atol=1e-12), o
    # decode_step applies 1/sqrt(D) by default
    o2 = O.decode_step(np.array(g["q"]), k, np.array(g["v"]), seq_len=4, window=4, sel_ids=[])
    assert np.allclose(o2, np.array(g["expected"]), rtol=0, atol=1e-12), o2


def _sdpa(q, k, v):
    """Library softmax attention (PyTorch CPU, float64), all heads sharing k and v."""
    import torch
    import torch.nn.functional as F

    H, D = q.shape
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).view(1, H, 1, D)
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).view(1, 1, -1, D).expand(1, H, -1, D)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).view(1, 1, -1, D).expand(1, H, -1, D)
    return F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous()).view(H, D).numpy()


def _tiny_case(seed, n_blocks=6, d=8, d_idx=4, H=2, D=4):
    rng = _rng(seed)
    N = 64 * n_blocks
    return dict(
        w=rng.standard_normal((3, d_idx, d)) / math.sqrt(d),
        h=rng.standard_normal(d),
        keys=rng.standard_normal((3, n_blocks, d_idx)) / math.sqrt(d_idx),
        K=rng.standard_normal((N + 8, D)),
        V=rng.standard_normal((N + 8, D)),
        q=rng.standard_normal((H, D)),
        N=N,
    )


def pin_all_selected_is_dense(O):
    """All blocks selected (bias +1e4) => LSA attention equals full softmax attention over
    [0, L), computed by PyTorch's scaled_dot_product_attention."""
    c = _tiny_case(5)
    res = O.refresh(c["h"], c["w"], c["keys"], np.full(3, 1e4))
    assert res.ids.tolist() == list(range(c["keys"].shape[1]))
    # decode-time tokens (positions >= N) belong to no scored block, so the identity needs
    # them inside the window: W > t
    for t, W in ((0, 1), (3, 4), (3, 70), (7, 8), (7, 200)):
        L = c["N"] + t + 1
        o = O.decode_step(c["q"], c["K"], c["V"], L, W, res.ids)
        ref = _sdpa(c["q"], c["K"][:L], c["V"][:L])
        assert np.allclose(o, ref, rtol=0, atol=1e-12), (t, W)


def pin_none_selected_is_window(O):
    """No block selected (bias -1e4) => attention over the window [L-W, L) only."""
    c = _tiny_case(6)
    res = O.refresh(c["h"], c["w"], c["keys"], np.full(3, -1e4))
    assert res.count == 0
    for t in (0, 5):
        L = c["N"] + t + 1
        for W in (1, 70, 130):
            o = O.decode_step(c["q"], c["K"], c["V"], L, W, res.ids)
            ref = _sdpa(c["q"], c["K"][L - W:L], c["V"][L - W:L])
            assert np.allclose(o, ref, rtol=0, atol=1e-12), (t, W)


def pin_brute_force_tiny(O):
    """Whole refresh + decode on tiny inputs against an independent formulation:
    per-block sigmoid via math.exp in Python loops, then attention as a dense 0/1 mask
    over every position with -inf fill and a log-sum-exp normaliser."""
    for seed in (7, 8, 9):
        c = _tiny_case(seed)
        n_blocks = c["keys"].shape[1]
        bias = np.array([-0.3, 0.1, -0.8])
        # brute-force selection
        q = [[math.fsum(c["w"][i, j, m] * c["h"][m] for m in range(c["w"].shape[2]))
              for j in range(c["w"].shape[1])] for i in range(3)]
        keep = set()
        per = []
        for i in range(3):
            ki = set()
            for b in range(n_blocks):
                z = math.fsum(q[i][j] * c["keys"][i, b, j] for j in range(len(q[i]))) + bias[i]
                if 1.0 / (1.0 + math.exp(-z)) > 0.5:
                    ki.add(b)
            per.append(ki)
            keep |= ki
        res = O.refresh(c["h"], c["w"], c["keys"], bias)
        assert res.ids.tolist() == sorted(keep)
        for i in range(3):
            assert np.flatnonzero(res.s[i]).tolist() == sorted(per[i])
        # brute-force attention with a dense mask
        D = c["q"].shape[1]
        for t in (0, 4):
            L = c["N"] + t + 1
            for W in (1, 65, 100):
                ws = max(0, L - W)
                mask = np.array([(p >= ws) or (p // 64 in keep) for p in range(L)])
                scores = (c["q"] @ c["K"][:L].T) / math.sqrt(D)
                scores = np.where(mask[None, :], scores, -np.inf)
                lse = np.logaddexp.reduce(scores, axis=1, keepdims=True)
                ref = np.exp(scores - lse) @ c["V"][:L]
                o = O.decode_step(c["q"], c["K"], c["V"], L, W, res.ids)
                assert np.allclose(o, ref, rtol=0, atol=1e-12), (seed, t, W)


def pin_uniform_scores_count(O):
    """K = 0 gives equal weights, so o = mean of V over the attended set; a one-hot V
    column then reads back 1/|T| at the marked position iff it is attended, pinning
    both the size of T and membership at window and block edges."""
    N, D = 64 * 8, 4
    L, W = N + 3, 100
    ws = L - W
    sel = [1, 3, 6, 7]   # block 7 straddles the window start (ws = 415 -> block 6 = [384,448))
    count = W + sum(max(0, min(64 * b + 64, ws) - 64 * b) for b in sel)
    K = np.zeros((L, D))
    q = np.ones((2, D))
    for p_star, inside in ((ws - 1, True), (ws, True), (L - 1, True), (64, True), (127, True),
                           (63, False), (128, False), (191 + 64, False), (64 * 7, False)):
        inside = (p_star >= ws) or (p_star // 64 in sel)
        V = np.zeros((L, D))
        V[p_star, 0] = 1.0
        o = O.decode_step(q, K, V, L, W, sel)
        want = 1.0 / count if inside else 0.0
        assert abs(o[0, 0] - want) < 1e-15 and abs(o[1, 0] - want) < 1e-15, (p_star, o[0, 0], want)
    V = np.full((L, D), 0.375)
    assert np.allclose(O.decode_step(q, K, V, L, W, sel), 0.375, rtol=0, atol=1e-15)


def pin_needles(O):
    """A single key with a score far above the rest dominates iff it is attended."""
    N, D = 64 * 10, 8
    L, W = N + 1, 130
    ws = L - W   # 511: block 7 = [448, 512) straddles it
    sel = [2, 7]
    rng = _rng(10)
    base_K = rng.standard_normal((L, D)) * 0.01
    V = rng.standard_normal((L, D))
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    for p_star in (ws - 1, ws, L - 1, 128, 191, 448, 510, 127, 192, 64 * 9):
        K = base_K.copy()
        K[p_star, 0] = 30.0 * math.sqrt(D)   # scaled score +30
        o = O.decode_step(q, K, V, L, W, sel)
        inside = (p_star >= ws) or (p_star // 64 in sel)
        close = np.allclose(o[0], V[p_star], atol=1e-6)
        assert close == inside, (p_star, inside)


def pin_bias_monotone(O):
    """Raising any indexer's bias can only add blocks."""
    rng = _rng(11)
    w = rng.standard_normal((3, 6, 12)) / math.sqrt(12)
    h = rng.standard_normal(12)
    keys = rng.standard_normal((3, 200, 6)) / math.sqrt(6)
    b0 = np.array([-1.0, -1.2, -0.9])
    base = set(O.refresh(h, w, keys, b0).ids.tolist())
    for i in range(3):
        b1 = b0.copy()
        b1[i] += 0.7
        up = set(O.refresh(h, w, keys, b1).ids.tolist())
        assert base <= up and len(up) > len(base)


def pin_block_permutation(O):
    """Permuting the order of block keys permutes the selected ids accordingly."""
    rng = _rng(12)
    w = rng.standard_normal((3, 6, 12)) / math.sqrt(12)
    h = rng.standard_normal(12)
    keys = rng.standard_normal((3, 150, 6)) / math.sqrt(6)
    bias = np.array([-1.0, -1.1, -0.8])
    ids = O.refresh(h, w, keys, bias).ids
    perm = rng.permutation(150)
    ids_p = O.refresh(h, w, keys[:, perm], bias).ids
    assert sorted(perm[ids_p].tolist()) == ids.tolist()



def pin_simulate_layer_uses_its_own_inputs(O):
    """simulate(layer=l) attends with layer l's queries, new tokens and prefill K/V and with the
    selection every layer shares: moving layer 1's arrays into layer 0's places gives the same
    outputs at layer 0, and they differ from layer 0's own."""
    import copy

    from workloads import build_workload, get_config

    wl = build_workload(get_config("tiny").scaled(n_layers=2), seed=2)
    steps = [0, 5, 63]
    refs1, out1 = O.simulate(wl, steps=steps, layer=1)
    refs0, out0 = O.simulate(wl, steps=steps, layer=0)
    moved = copy.copy(wl)
    moved.q_dec, moved.k_new, moved.v_new = wl.q_dec_of(1), wl.k_new_of(1), wl.v_new_of(1)
    moved._kv = {(0, 0): wl.kv_prefill(0, 1)}
    refsm, outm = O.simulate(moved, steps=steps, layer=0)
    for t in steps:
        assert np.array_equal(outm[(0, t)], out1[(0, t)])
        assert not np.allclose(out0[(0, t)], out1[(0, t)])
    assert all(np.array_equal(a.ids, b.ids) for a, b in zip(refs0[0], refs1[0]))


def _tiny_decode_workload(seed, steps=12, bias=None):
    """The fp32 tiny workload cut to a few steps (one refresh at step 0), optionally with every
    indexer's bias replaced."""
    from workloads import build_workload, get_config

    wl = build_workload(get_config("tiny").scaled(steps=steps), seed=seed)
    if bias is not None:
        wl.bias = np.full_like(wl.bias, bias)
    return wl


def pin_simulate_is_decode_over_grown_cache(O):
    """simulate() at step t equals one decode step over caches built by hand as the prefill
    rows followed by the rows of the tokens of steps 0..t, with L = N + t + 1 positions: the
    token being produced at step t is position N + t and attends to itself ([Explained] section 2
    step 4; the recent window holds the newest tokens)."""
    wl = _tiny_decode_workload(seed=21)
    steps = [0, 1, 5, 11]
    refs, out = O.simulate(wl, steps=steps)
    ids = refs[0][0].ids
    assert 0 < len(ids) < wl.n_blocks[0]
    kp, vp = wl.kv_prefill(0)
    N = int(wl.ctx[0])
    for t in steps:
        k_cache = np.concatenate([kp, wl.k_new[: t + 1, 0]]).astype(np.float64)
        v_cache = np.concatenate([vp, wl.v_new[: t + 1, 0]]).astype(np.float64)
        assert k_cache.shape[0] == N + t + 1
        want = O.decode_step(wl.q_dec[t, 0].astype(np.float64), k_cache, v_cache, N + t + 1,
                             wl.cfg.window, ids)
        assert np.allclose(out[(0, t)], want, rtol=0, atol=1e-13), (t, np.abs(out[(0, t)] - want).max())


def pin_simulate_decode_positions_closed_form(O):
    """All keys zero (prefill and new tokens) gives equal weights, so o = mean of V over the
    attended set.  V is one-hot in column 0 at one token appended during decode (step t0, position
    N + t0), zero elsewhere.  At step t the output is 1/|T_t| in column 0 when t >= t0 (the token
    is in the window; at t = t0 it is the current token) and exactly 0 for t < t0, where
    |T_t| = W + (tokens of selected blocks below the window start L - W) is counted by hand."""
    for bias, expect_all in ((-1e4, False), (1e4, True), (None, None)):
        wl = _tiny_decode_workload(seed=22, bias=bias)
        N, W, T = int(wl.ctx[0]), wl.cfg.window, wl.cfg.steps
        kp, vp = wl.kv_prefill(0)
        wl.set_kv_prefill(0, np.zeros_like(kp), np.zeros_like(vp))
        wl.k_new = np.zeros_like(wl.k_new)
        refs, _ = O.simulate(wl, steps=[])
        sel = refs[0][0].ids.tolist()
        if expect_all is not None:
            assert len(sel) == (wl.n_blocks[0] if expect_all else 0)
        for t0 in (0, 4, T - 1):
            v_new = np.zeros_like(wl.v_new)
            v_new[t0, 0, 0] = 1.0
            wl.v_new = v_new
            steps = sorted({0, max(0, t0 - 1), t0, min(T - 1, t0 + 3), T - 1})
            _, out = O.simulate(wl, steps=steps)
            for t in steps:
                L = N + t + 1
                ws = L - W
                count = W + sum(max(0, min(64 * b + 64, ws) - 64 * b) for b in sel)
                want = 1.0 / count if t >= t0 else 0.0
                o = out[(0, t)]
                assert np.all(np.abs(o[:, 0] - want) < 1e-15), (bias, t0, t, o[0, 0], want)
                assert np.all(o[:, 1:] == 0.0)


# ------------------------------------------------------------------------------------------
def _bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with integer arithmetic on the binary32 bits: add 0x7FFF
    plus the lowest kept bit, then drop the low 16 bits (round to nearest, ties to even)."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def pin_round_bf16(O):
    """Rounding to bfloat16: the hand-derived cases of bf16_rounding.json; every bfloat16 value
    (bf16_values.json) is a fixed point; and on random values the result is the nearest of the
    two bfloat16 neighbours, found by enumerating bit patterns, with ties to the even pattern."""
    g = _golden("bf16_rounding.json")
    x = np.array([c["x"] for c in g["cases"]], dtype=np.float64)
    want = np.array([c["rounded"] for c in g["cases"]], dtype=np.float64)
    got = O.round_bf16(x)
    assert np.array_equal(got, want), (x[got != want], got[got != want])
    vals = np.array([c["value"] for c in _golden("bf16_values.json")["cases"]], dtype=np.float64)
    normal = np.abs(vals) >= 2.0 ** -126
    assert np.array_equal(O.round_bf16(vals[normal]), vals[normal])
    rng = _rng(41)
    xs = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    got = O.round_bf16(xs)
    lo_bits = (xs.astype(np.float32).view(np.uint32) >> 16).astype(np.uint32)   # truncation toward zero
    for x, g1, lb in zip(xs, got, lo_bits):
        cands = [(int(b) << 16) for b in (lb - 1, lb, lb + 1)]
        cv = np.array(cands, dtype=np.uint32).view(np.float32).astype(np.float64)
        dist = np.abs(cv - x)
        best = dist.min()
        ok = [i for i in range(3) if dist[i] == best]
        pick = ok[0] if len(ok) == 1 else [i for i in ok if (cands[i] >> 16) % 2 == 0][0]
        assert g1 == cv[pick], (x, g1, cv)


def pin_query_latent(O):
    """The low-rank latent c_i = A_i h: explicit sums with rectangular and square A_i, per-indexer
    hidden states; for bf16 the exact sums are rounded as the binary32 bit trick rounds them (the
    sums are integers times 2^-6, exact in binary32); for f32 the sums are kept."""
    rng = _rng(42)
    for r, d in ((5, 7), (6, 6)):
        A = rng.integers(-100, 101, (3, r, d)).astype(np.float64)
        h = rng.integers(-100, 101, (3, d)).astype(np.float64) / 64.0  # sums: up to 17-bit integers / 64
        want = np.zeros((3, r))
        for i in range(3):
            for k in range(r):
                want[i, k] = math.fsum(A[i, k, m] * h[i, m] for m in range(d))
        assert np.array_equal(O.query_latent(h, A, "f32"), want)
        bits = _bf16_rne_bits(want.astype(np.float32))
        want16 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        got16 = O.query_latent(h, A, "bf16")
        assert np.array_equal(got16, want16), np.abs(got16 - want16).max()
        assert not np.array_equal(want16, want)  # the case does exercise rounding
    # one hidden state shared by the indexers
    A = rng.integers(-4, 5, (2, 3, 4)).astype(np.float64)
    h = rng.integers(-4, 5, 4).astype(np.float64)
    assert np.array_equal(O.query_latent(h, A, "f32"), np.stack([A[0] @ h, A[1] @ h]))


def pin_lowrank_query_is_product(O):
    """Without rounding (small integers, f32 storage exact) the chain B_i (A_i h) is the Query
    Encoder of the product matrix W_i = B_i A_i, and the refresh selects the same blocks."""
    rng = _rng(43)
    A = rng.integers(-3, 4, (3, 4, 9)).astype(np.float64)
    B = rng.integers(-3, 4, (3, 5, 4)).astype(np.float64)
    h = rng.integers(-3, 4, 9).astype(np.float64)
    W = np.stack([B[i] @ A[i] for i in range(3)])
    c = O.query_latent(h, A, "f32")
    assert np.array_equal(O.query_encoder(c, B), O.query_encoder(h, W))
    keys = rng.integers(-3, 4, (3, 40, 5)).astype(np.float64)
    bias = np.array([0.5, -0.5, 0.25])
    assert np.array_equal(O.refresh(c, B, keys, bias).ids, O.refresh(h, W, keys, bias).ids)


def pin_simulate_lowrank_uses_the_latent(O):
    """simulate() on a workload with a low-rank query projection selects what the chain selects:
    each refresh's ids equal a direct evaluation of B_i round(A_i h) . key + bias > 0."""
    from workloads import build_workload, get_config

    wl = build_workload(get_config("tiny").scaled(q_rank=96, steps=70), seed=4)
    assert wl.w_down is not None and wl.w_q.shape[2] == 96
    refs, _ = O.simulate(wl, steps=[])
    A = wl.w_down.astype(np.float64)
    B = wl.w_q.astype(np.float64)
    for r in range(wl.n_req):
        keys = wl.keys[r].astype(np.float64)
        for k, res in enumerate(refs[r]):
            h = wl.hidden[r][k].astype(np.float64)
            c = np.stack([(A[i] @ h).astype(np.float32).astype(np.float64) for i in range(A.shape[0])])
            z = np.stack([keys[i] @ (B[i] @ c[i]) + float(wl.bias[r][i]) for i in range(A.shape[0])])
            assert np.array_equal(res.ids, np.flatnonzero((z > 0).any(axis=0))), (r, k)


PINS = [
    pin_bf16_decode,
    pin_query_encoder_columns,
    pin_query_encoder_brute,
    pin_block_logits,
    pin_threshold_is_sigmoid_half,
    pin_threshold_levels,
    pin_union_is_set_union,
    pin_golden_or_union,
    pin_golden_cadence,
    pin_golden_token_set,
    pin_golden_attention,
    pin_all_selected_is_dense,
    pin_none_selected_is_window,
    pin_brute_force_tiny,
    pin_uniform_scores_count,
    pin_needles,
    pin_bias_monotone,
    pin_block_permutation,
    pin_simulate_layer_uses_its_own_inputs,
    pin_simulate_is_decode_over_grown_cache,
    pin_simulate_decode_positions_closed_form,
    pin_round_bf16,
    pin_query_latent,
    pin_lowrank_query_is_product,
    pin_simulate_lowrank_uses_the_latent,
]
