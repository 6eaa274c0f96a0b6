"""Plain float64 oracle of the Lookahead Sparse Attention (LSA) decode path.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.  It is slow on purpose: every step is the
definition written out with NumPy, with no blocking, fusion or reordering.

Sources (the web pages describing "FlashMemory-DeepSeek-V4: Lightning Index
Ultra-Long Context via Lookahead Sparse Attention"):

  [Explained]  "FlashMemory-DeepSeek-V4 Explained: Replacing Memory Sponge with a
               Fortune Teller via Lookahead Sparse Attention" (zhichai.net):
               section 2 "Core Idea of LSA" (the five-step decode loop),
               section 3 "Training the Indexer" (frozen KIComp block keys, a Query
               Encoder of three small projection matrices), section 4
               "Architecture" (three independent indexers, OR-mode union),
               section 5 "Results" (threshold recall at sigmoid 0.5).
  [1kpapers]   the 1kpapers.com page of the report, "01 In brief / Summary"
               (fetch critical KV chunks every 64 steps; dual-encoder indexer).

What the pages leave open and how it is read here:
  * score: a dual-encoder dot product of the query embedding with the frozen
    block key plus a per-indexer bias, z = q.k + beta; no extra scale.
  * threshold: sigmoid(z) > 0.5 is decided as z > 0 (identical in exact
    arithmetic; the sigmoid itself is never evaluated, so fp rounding of
    sigmoid near 0.5 cannot flip a decision).  Section 2 writes "> 0.5",
    section 5 writes ">= 0.5"; the strict form is used.
  * one hidden state per request per refresh, shared by the indexers; one set
    of block keys per indexer.
  * low-rank query projection ([Explained] section 4, training tricks: rank
    r = 2048, reusing the backbone's MLA/MQA bottleneck): indexer i first forms
    the latent c_i = A_i h (A_i is [r][d_model]), which, like any activation of
    the backbone, is stored in the input precision (rounded to the nearest
    bfloat16, ties to even, for bf16 inputs); the Query Encoder then projects
    the latent, q_i = B_i c_i.  The backbone's normalisation of the latent is
    not part of the path.
  * a refresh taken at step t_k governs steps t_k .. t_k + 63 (inclusive of t_k).
  * attended tokens: the last W tokens (the recent window, including the
    current token) plus every token of a selected block that lies before the
    window; each position once.
  * block list order: ascending block id.
  * softmax scale 1/sqrt(D); all query heads share the single KV head.

Every function below is pinned by tests against closed forms, library
routines, hand-derived fixtures or brute force; none is "parity unpinned".
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

BLOCK = 64  # tokens per KV block (the unit that is scored, selected and moved)


# ------------------------------------------------------------------------------------------
# input decoding
# ------------------------------------------------------------------------------------------
def decode_values(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs.

    bf16 tensors arrive as uint16 bit patterns: a bfloat16 is the top half of an
    IEEE-754 single, so the value is the single whose high 16 bits are the pattern
    and whose low 16 bits are zero.  float32 tensors are widened as they are.
    """
    raw = np.asarray(raw)
    if dtype == "bf16":
        if raw.dtype != np.uint16:
            raise TypeError("bf16 input must be given as uint16 bit patterns")
        as_u32 = raw.astype(np.uint32) << np.uint32(16)
        return as_u32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return raw.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64 (ties to even), as float64.

    A bfloat16 keeps 8 significant bits (the top half of an IEEE-754 single): x = m 2^e with
    m in [0.5, 1) is rounded to round_half_even(m 2^8) 2^(e-8).  Values stay within the single's
    normal range here (no subnormal or overflow handling).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


# ------------------------------------------------------------------------------------------
# index refresh: Query Encoder -> block scores -> threshold -> OR-union -> block list
# ------------------------------------------------------------------------------------------
def query_latent(h: np.ndarray, w_down: np.ndarray, dtype: str) -> np.ndarray:
    """Latent of the low-rank query projection, one per indexer.

    [Explained] section 4 (training tricks): the query projection is low-rank, r = 2048, using the
    backbone's MLA/MQA bottleneck.  w_down is [n_idx][r][d_model], h is [d_model] (shared) or
    [n_idx][d_model].  Returns c [n_idx][r]:
        c[i][k] = sum_m w_down[i][k][m] * h[m]
    computed exactly, then stored like an activation of the backbone: rounded to bfloat16 for
    bf16 inputs, to float32 for f32 inputs.  query_encoder(c, B) then gives q_i = B_i c_i.
    """
    w_down = np.asarray(w_down, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    n_idx = w_down.shape[0]
    c = np.stack([w_down[i] @ (h if h.ndim == 1 else h[i]) for i in range(n_idx)])
    if dtype == "bf16":
        return round_bf16(c)
    if dtype == "f32":
        return c.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def query_encoder(h: np.ndarray, w_q: np.ndarray) -> np.ndarray:
    """Query embeddings of the current hidden state, one per indexer.

    [Explained] section 3: the trained part of the indexer is a Query Encoder made
    of small projection matrices; section 2 step 2: the indexer looks at the
    current hidden state.  w_q is [n_idx][d_idx][d_model] (row j of matrix i
    projects onto output j), h is [d_model] (shared by the indexers) or
    [n_idx][d_model] (one per indexer).  Returns q [n_idx][d_idx]:
        q[i][j] = sum_m w_q[i][j][m] * h[m]
    """
    w_q = np.asarray(w_q, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    n_idx = w_q.shape[0]
    hs = [h if h.ndim == 1 else h[i] for i in range(n_idx)]
    return np.stack([w_q[i] @ hs[i] for i in range(n_idx)])


def block_logits(q: np.ndarray, keys: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Dual-encoder block scores (logits), one row per indexer.

    [Explained] section 3: historical KV blocks are represented by precomputed,
    frozen compressed keys (KIComp) and scored against the query embedding;
    [1kpapers] Summary: the indexer is a dual encoder.  keys is
    [n_idx][B][d_idx], q is [n_idx][d_idx], bias is [n_idx].  Returns z [n_idx][B]:
        z[i][b] = sum_j q[i][j] * keys[i][b][j] + bias[i]
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    return np.stack([keys[i] @ q[i] + bias[i] for i in range(keys.shape[0])])


def level_logit(level: float) -> float:
    """The logit at which sigmoid equals `level`: log(level / (1 - level)); 0 for the pages' 0.5."""
    level = float(level)
    if not 0.0 < level < 1.0:
        raise ValueError("the selection level lies strictly between 0 and 1")
    return float(np.log(level / (1.0 - level)))


def threshold(z: np.ndarray, level: float = 0.5) -> np.ndarray:
    """Per-indexer selection: keep block b iff sigmoid(z) > level, i.e. iff z > logit(level).

    [Explained] section 2 step 3 (blocks with sigmoid score above 0.5 are loaded); section 7 calls
    the 0.5 a preliminary choice, so the level is a parameter.  The sigmoid is monotone, so the
    comparison is made on the logit.
    """
    return np.asarray(z, dtype=np.float64) > level_logit(level)


def union(s: np.ndarray) -> np.ndarray:
    """OR-mode union over indexers: a block is loaded if any indexer selects it.

    [Explained] section 4 (the three indexers are combined with a union / OR rule).
    """
    return np.any(np.asarray(s, dtype=bool), axis=0)


def compact(u: np.ndarray) -> np.ndarray:
    """Ids of the loaded blocks, ascending, without duplicates (int32)."""
    return np.flatnonzero(np.asarray(u, dtype=bool)).astype(np.int32)


@dataclass
class RefreshResult:
    q: np.ndarray      # [n_idx][d_idx]
    z: np.ndarray      # [n_idx][B]
    s: np.ndarray      # [n_idx][B] bool, per-indexer selection
    u: np.ndarray      # [B] bool, union
    ids: np.ndarray    # ascending int32 ids of loaded blocks

    @property
    def count(self) -> int:
        return int(len(self.ids))


def refresh(h: np.ndarray, w_q: np.ndarray, keys: np.ndarray, bias: np.ndarray,
            level: float = 0.5) -> RefreshResult:
    """One index refresh: [Explained] section 2 steps 2-3 with section 4's union."""
    q = query_encoder(h, w_q)
    z = block_logits(q, keys, bias)
    s = threshold(z, level)
    u = union(s)
    return RefreshResult(q=q, z=z, s=s, u=u, ids=compact(u))


def governing_refresh(t: int, refresh_steps: Sequence[int]) -> int:
    """Index of the refresh whose selection is in force at decode step t.

    [Explained] section 2 steps 1, 4 and 5: a refresh predicts the blocks the next
    64 steps need, those steps attend over them, then the set is refreshed.  The
    selection in force at t is the one of the latest refresh taken at or before t.
    """
    best = -1
    for k, tk in enumerate(refresh_steps):
        if tk <= t:
            best = k
    if best < 0:
        raise ValueError(f"no refresh at or before step {t}")
    return best


# ------------------------------------------------------------------------------------------
# sparse decode
# ------------------------------------------------------------------------------------------
def window_start(seq_len: int, window: int) -> int:
    """First position of the recent window [ws, L): the last `window` tokens."""
    return max(0, int(seq_len) - int(window))


def token_set(seq_len: int, window: int, sel_ids: Sequence[int], block: int = BLOCK) -> np.ndarray:
    """Positions one decode step attends to, ascending.

    [Explained] section 2 step 4: attention runs only over the loaded blocks; the
    recent window (section 1: the last 8K tokens answer most requests) is always
    attended.  T = [ws, L) united with {p < ws : p // block is a selected block}.
    """
    L = int(seq_len)
    ws = window_start(L, window)
    before = np.arange(ws, dtype=np.int64)
    in_selected = np.isin(before // block, np.asarray(sel_ids, dtype=np.int64))
    return np.concatenate([before[in_selected], np.arange(ws, L, dtype=np.int64)])


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of H query rows over one shared K/V head.

    q [H][D], k and v [n][D] (the attended tokens).  For each head h:
        a_p = scale * q_h . k_p,   o_h = sum_p exp(a_p - m) v_p / sum_p exp(a_p - m)
    with m = max_p a_p.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = (q @ k.T) * float(scale)
    m = a.max(axis=1, keepdims=True)
    w = np.exp(a - m)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def seq_len_at(n_prefill: int, t: int) -> int:
    """Tokens in the cache at decode step t: the prefill plus the tokens of steps 0..t.

    [Explained] section 2 step 4: each decode step attends with the token it is producing; that
    token (the one of step t) sits at position n_prefill + t, so the step sees L = n_prefill + t + 1
    positions, the last of which is its own (it is in the recent window, section 1).
    """
    return int(n_prefill) + int(t) + 1


def kv_rows(prefill: np.ndarray, new_rows: np.ndarray, n_prefill: int, positions: np.ndarray) -> np.ndarray:
    """Rows of the K (or V) cache at `positions`: prefill rows below n_prefill,
    decode-time rows (new_rows[p - n_prefill]) at and above it."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((len(positions), prefill.shape[1]), dtype=np.float64)
    lo = positions < n_prefill
    out[lo] = prefill[positions[lo]]
    out[~lo] = new_rows[positions[~lo] - n_prefill]
    return out


def decode_step(q_t: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, seq_len: int,
                window: int, sel_ids: Sequence[int], scale: Optional[float] = None,
                block: int = BLOCK) -> np.ndarray:
    """One decode step over the window and the selected blocks (caches are
    indexed by position and hold at least seq_len rows)."""
    D = np.asarray(q_t).shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pos = token_set(seq_len, window, sel_ids, block)
    return attention(q_t, np.asarray(k_cache)[pos], np.asarray(v_cache)[pos], scale)


# ------------------------------------------------------------------------------------------
# driver over a whole workload (small sizes)
# ------------------------------------------------------------------------------------------
def simulate(wl, steps: Optional[Sequence[int]] = None, requests: Optional[Sequence[int]] = None,
             layer: int = 0):
    """Run the decode loop of a workload: the refreshes and the decode steps.

    `wl` supplies the raw inputs (see workloads.Workload).  Returns
    (refreshes, outputs): refreshes[r] is the list of RefreshResult in refresh order,
    outputs[(r, t)] is o [H][D] for every requested step t (default: all steps).

    `layer` picks the attention layer whose K/V, decode queries and new tokens are used.  The
    selection is the same for every layer: the indexers' loads serve the whole model
    ([1kpapers Summary]; [Explained] section 4, indexers at three layers, one OR-union).
    """
    cfg = wl.cfg
    dt = cfg.dtype
    w_q = decode_values(wl.w_q, dt)
    w_down = decode_values(wl.w_down, dt) if getattr(wl, "w_down", None) is not None else None
    req = range(wl.n_req) if requests is None else requests
    step_list = range(cfg.steps) if steps is None else steps
    refreshes = {}
    outputs = {}
    scale = 1.0 / np.sqrt(cfg.head_dim)
    for r in req:
        keys = decode_values(wl.keys[r], dt)
        bias = np.asarray(wl.bias[r], dtype=np.float64)
        hs = [decode_values(wl.hidden[r][k], dt) for k in range(len(wl.refresh_steps[r]))]
        if w_down is not None:  # low-rank query projection: the Query Encoder reads the latents
            hs = [query_latent(h, w_down, dt) for h in hs]
        res = [refresh(h, w_q, keys, bias, getattr(cfg, "level", 0.5)) for h in hs]
        refreshes[r] = res
        if not step_list:
            continue
        kp, vp = wl.kv_prefill(r, layer) if layer else wl.kv_prefill(r)
        kp = decode_values(kp, dt)
        vp = decode_values(vp, dt)
        n = int(wl.ctx[r])
        k_new = decode_values(wl.k_new_of(layer)[:, r] if layer else wl.k_new[:, r], dt)
        v_new = decode_values(wl.v_new_of(layer)[:, r] if layer else wl.v_new[:, r], dt)
        q_all = wl.q_dec_of(layer) if layer else wl.q_dec
        for t in step_list:
            L = seq_len_at(n, t)
            k_idx = governing_refresh(t, wl.refresh_steps[r])
            pos = token_set(L, cfg.window, res[k_idx].ids, cfg.block)
            kk = kv_rows(kp, k_new, n, pos)
            vv = kv_rows(vp, v_new, n, pos)
            outputs[(r, t)] = attention(decode_values(q_all[t, r], dt), kk, vv, scale)
    return refreshes, outputs
