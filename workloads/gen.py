"""Seeded draws for LSA workloads.

Every tensor comes from its own NumPy PCG64 stream keyed by
(seed, workload tag, tensor id, request, index, ...), so any piece can be
regenerated alone and the result never depends on thread count.  bf16
tensors are stored as their uint16 bit patterns, rounded to nearest-even
from float32 draws; float32 tensors are stored as float32.

What is drawn (all iid):
  * W_q[i] ~ N(0, 1/d_model), stored [n_idx][d_idx][d_model] (row j projects
    the hidden state onto output j);
  * block keys ~ N(0, 1/d_idx), per request [n_idx][B_r][d_idx];
  * hidden states ~ N(0, 1), one per request per refresh;
  * decode queries ~ N(0, 1) [H][D], new-token K and V ~ N(0, 1) [D], one per
    request per step;
  * prefill K and V ~ N(0, 1), per request [N_r][D].

The per-indexer bias is set analytically: with the distributions above the
logit q.k has standard deviation close to 1, so a per-indexer keep rate p
needs bias = -Phi^-1(1 - p), and a union density rho over three independent
indexers needs p = 1 - (1 - rho)^(1/3).  No logit is evaluated for this.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from statistics import NormalDist
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .configs import LSAConfig, get_config

# tensor ids used in stream keys
_T_CTX, _T_DENS, _T_PHASE, _T_WQ, _T_KEYS, _T_HID, _T_QDEC, _T_KPRE, _T_VPRE, \
    _T_KNEW, _T_VNEW, _T_PLANT_IDS, _T_PLANT, _T_REDRAW, _T_LAYER, _T_WDOWN = range(1, 17)

_KV_CHUNK = 1 << 16  # tokens per independent prefill K/V stream


def rng_for(seed: int, *key: int) -> np.random.Generator:
    """Independent generator for (seed, key...)."""
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    return x


def _storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


@dataclass
class ConditionReport:
    redrawn_rows: int = 0
    rounds: int = 0
    min_abs_logit: float = float("inf")
    min_planted_logit: float = float("inf")
    planted_rows: int = 0


@dataclass
class Workload:
    cfg: LSAConfig
    seed: int
    ctx: np.ndarray                 # [R] int64 prefill lengths N_r (multiples of 64)
    density: np.ndarray             # [R] union density targets
    phase: np.ndarray               # [R] refresh phase phi_r
    bias: np.ndarray                # [R][n_idx] float32
    w_q: np.ndarray                 # [n_idx][d_idx][d_model], or B [n_idx][d_idx][q_rank] (low rank)
    keys: List[np.ndarray]          # per request [n_idx][B_r][d_idx]
    refresh_steps: List[List[int]]  # per request, ascending; a negative entry is the prologue refresh
    hidden: List[np.ndarray]        # per request [n_refresh_r][d_model]
    planted: List[np.ndarray]       # per request ascending planted block ids (may be empty)
    q_dec: np.ndarray               # [T][R][H][D]   (layer 0)
    k_new: np.ndarray               # [T][R][D]      (layer 0)
    v_new: np.ndarray               # [T][R][D]      (layer 0)
    layer_dec: List[Tuple[np.ndarray, np.ndarray, np.ndarray]] = field(default_factory=list)  # layers 1..
    w_down: Optional[np.ndarray] = None  # low rank: A [n_idx][q_rank][d_model], latent c_i = A_i h
    _kv: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict, repr=False)
    report: Optional[ConditionReport] = None

    # ---- shapes -------------------------------------------------------------------------
    @property
    def n_req(self) -> int:
        return self.cfg.n_req

    @property
    def n_blocks(self) -> np.ndarray:
        return self.ctx // self.cfg.block

    def blk_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.n_blocks)]).astype(np.int64)

    # ---- prefill K/V ----------------------------------------------------------------------
    @property
    def n_layers(self) -> int:
        return self.cfg.n_layers

    def q_dec_of(self, layer: int) -> np.ndarray:
        return self.q_dec if layer == 0 else self.layer_dec[layer - 1][0]

    def k_new_of(self, layer: int) -> np.ndarray:
        return self.k_new if layer == 0 else self.layer_dec[layer - 1][1]

    def v_new_of(self, layer: int) -> np.ndarray:
        return self.v_new if layer == 0 else self.layer_dec[layer - 1][2]

    def kv_prefill(self, r: int, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Prefill K and V of request r in one layer, token-major [N_r][D] (generated on first use)."""
        if (r, layer) in self._kv:
            return self._kv[(r, layer)]
        cfg = self.cfg
        n, d = int(self.ctx[r]), cfg.head_dim
        st = _storage_dtype(cfg.dtype)
        k = np.empty((n, d), dtype=st)
        v = np.empty((n, d), dtype=st)
        chunks = [(c0, min(n, c0 + _KV_CHUNK)) for c0 in range(0, n, _KV_CHUNK)]

        def fill(ci: int) -> None:
            c0, c1 = chunks[ci]
            for arr, tid in ((k, _T_KPRE), (v, _T_VPRE)):
                rng = (rng_for(self.seed, cfg.tag, tid, r, ci) if layer == 0 else
                       rng_for(self.seed, cfg.tag, _T_LAYER, layer, tid, r, ci))
                arr[c0:c1] = _normal(rng, (c1 - c0, d), 1.0, cfg.dtype)

        if len(chunks) == 1:
            fill(0)
        else:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(len(chunks))))
        self._kv[(r, layer)] = (k, v)
        return k, v

    def set_kv_prefill(self, r: int, k: np.ndarray, v: np.ndarray, layer: int = 0) -> None:
        """Replace request r's prefill K and V in one layer (tests plant keys this way)."""
        n, d = int(self.ctx[r]), self.cfg.head_dim
        if k.shape != (n, d) or v.shape != (n, d):
            raise ValueError(f"prefill of request {r} is [{n}][{d}], got {k.shape} and {v.shape}")
        self._kv[(r, layer)] = (k, v)

    def drop_kv(self, r: Optional[int] = None) -> None:
        if r is None:
            self._kv.clear()
        else:
            for key in [key for key in self._kv if key[0] == r]:
                self._kv.pop(key)

    # ---- schedule -------------------------------------------------------------------------
    def refreshes_at(self, t: int) -> List[int]:
        """Requests that refresh at decode step t (0 <= t < steps)."""
        return [r for r in range(self.n_req) if t in self.refresh_steps[r]]

    def refresh_index_at(self, r: int, t: int) -> int:
        """Index (into refresh_steps[r]) of refresh k with t_k == t, or -1."""
        try:
            return self.refresh_steps[r].index(t)
        except ValueError:
            return -1

    # ---- conditioning -----------------------------------------------------------------------
    def condition(
        self,
        query_fn: Callable[[np.ndarray, np.ndarray], np.ndarray],
        logits_fn: Optional[Callable[[np.ndarray, np.ndarray, np.ndarray], np.ndarray]] = None,
        margin: float = 2e-3,
        max_rounds: int = 32,
        plant_logit: float = 2.0,
        latent_fn: Optional[Callable[[np.ndarray, np.ndarray], np.ndarray]] = None,
    ) -> ConditionReport:
        """Place planted keys and move keys away from the decision boundary.

        query_fn(h_raw[d], w_raw[n_idx][d_idx][d]) -> q float64 [n_idx][d_idx]
        logits_fn(q [n_idx][d_idx], keys_raw [n_idx][B][d_idx], bias [n_idx]) -> float64 [n_idx][B]
        latent_fn(h_raw[d], w_down_raw[n_idx][r][d]) -> latent raw [n_idx][r] (low-rank workloads
        only: query_fn then receives the latents in place of h)

        Both functions come from the caller; this module evaluates neither.

        Planted blocks: for every indexer, the key row is rebuilt so that its dot product
        with each of the request's refresh queries equals plant_logit - bias (plant_logit
        is in units of the logit's nominal standard deviation, 1), plus a fresh component
        orthogonal to all of those queries.  Margin: any (indexer, block) row whose logit
        at some refresh lies within `margin` of zero is redrawn from a fresh stream, until
        none is left.
        """
        cfg = self.cfg
        rep = ConditionReport()
        queries: List[np.ndarray] = []  # per request [n_ref][n_idx][d_idx]
        if self.w_down is not None and latent_fn is None:
            raise ValueError("a low-rank workload needs latent_fn to condition")
        for r in range(self.n_req):
            ins = [self.hidden[r][k] if self.w_down is None else latent_fn(self.hidden[r][k], self.w_down)
                   for k in range(len(self.refresh_steps[r]))]
            qs = np.stack([np.asarray(query_fn(h, self.w_q), dtype=np.float64) for h in ins])
            queries.append(qs)
        for r in range(self.n_req):
            if len(self.planted[r]) == 0:
                continue
            rep.planted_rows += self._plant(r, queries[r], plant_logit)
        if logits_fn is None:
            self.report = rep
            return rep
        for r in range(self.n_req):
            planted_mask = np.zeros(int(self.n_blocks[r]), dtype=bool)
            planted_mask[self.planted[r]] = True
            for attempt in range(max_rounds + 1):
                near = np.zeros((cfg.n_idx, int(self.n_blocks[r])), dtype=bool)
                min_abs, min_planted = float("inf"), float("inf")
                for k in range(len(self.refresh_steps[r])):
                    z = np.asarray(logits_fn(queries[r][k], self.keys[r], self.bias[r].astype(np.float64)))
                    az = np.abs(z)
                    near |= az < margin
                    min_abs = min(min_abs, float(az.min()))
                    if planted_mask.any():
                        min_planted = min(min_planted, float(z[:, planted_mask].min()))
                if not near.any():
                    rep.min_abs_logit = min(rep.min_abs_logit, min_abs)
                    rep.min_planted_logit = min(rep.min_planted_logit, min_planted)
                    break
                if attempt == max_rounds:
                    raise RuntimeError(f"margin conditioning did not converge for request {r}")
                if (near & planted_mask[None, :]).any():
                    raise RuntimeError("a planted key lies near the decision boundary")
                rows = np.argwhere(near)
                for i, b in rows:
                    rng = rng_for(self.seed, cfg.tag, _T_REDRAW, r, int(i), int(b), attempt)
                    self.keys[r][i, b] = _normal(rng, (cfg.d_idx,), cfg.k_std, cfg.dtype)
                rep.redrawn_rows += len(rows)
                rep.rounds = max(rep.rounds, attempt + 1)
        self.report = rep
        return rep

    def _plant(self, r: int, qs: np.ndarray, plant_logit: float) -> int:
        cfg = self.cfg
        ids = self.planted[r]
        n = 0
        for i in range(cfg.n_idx):
            Q = qs[:, i, :].T  # [d_idx][n_ref]
            gram_inv = np.linalg.inv(Q.T @ Q)
            proj = Q @ gram_inv  # [d_idx][n_ref]
            target = np.full(Q.shape[1], plant_logit - float(self.bias[r, i]), dtype=np.float64)
            rng = rng_for(self.seed, cfg.tag, _T_PLANT, r, i)
            perp = rng.standard_normal(size=(len(ids), cfg.d_idx)) * cfg.k_std
            perp -= (perp @ Q) @ proj.T  # remove the component in span(Q)
            rows = perp + (proj @ target)[None, :]
            rows32 = rows.astype(np.float32)
            self.keys[r][i, ids] = bf16_bits_from_f32(rows32) if cfg.dtype == "bf16" else rows32
            n += len(ids)
        return n


def _union_to_bias(rho: float) -> float:
    p = 1.0 - (1.0 - rho) ** (1.0 / 3.0)
    return -NormalDist().inv_cdf(1.0 - p)


def build_workload(cfg: LSAConfig | str, seed: int = 0, steps: Optional[int] = None) -> Workload:
    """Draw every input of a workload except the prefill K/V (drawn lazily per request)."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    if steps is not None:
        cfg = cfg.scaled(steps=steps)
    R, T = cfg.n_req, cfg.steps
    blk = cfg.block

    # context lengths
    if cfg.ctx[0] == "fixed":
        ctx = np.full(R, int(cfg.ctx[1]) // blk * blk, dtype=np.int64)
    else:
        lo, hi = cfg.ctx[1], cfg.ctx[2]
        u = rng_for(seed, cfg.tag, _T_CTX).random(R)
        ctx = (np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.int64) // blk) * blk
    if cfg.planted_frac > 0 and (ctx < cfg.window).any():
        # the planted blocks are drawn among the blocks wholly before the window
        raise ValueError("a workload with planted blocks needs every context to hold at least one window")

    # densities and bias
    if cfg.density[0] == "fixed":
        dens = np.full(R, float(cfg.density[1]))
    elif cfg.density[0] == "uniform":
        dens = rng_for(seed, cfg.tag, _T_DENS).uniform(cfg.density[1], cfg.density[2], R)
    else:
        lo, hi = cfg.density[1], cfg.density[2]
        u = rng_for(seed, cfg.tag, _T_DENS).random(R)
        dens = np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))
    bias = np.array([[_union_to_bias(float(d))] * cfg.n_idx for d in dens], dtype=np.float32)

    # refresh phases: refreshes happen at steps t with (t + phase) % tau == 0
    if cfg.staggered:
        if R > cfg.tau:
            raise ValueError("staggered phases need at most tau requests")
        phase = rng_for(seed, cfg.tag, _T_PHASE).permutation(cfg.tau)[:R].astype(np.int64)
    else:
        phase = np.zeros(R, dtype=np.int64)
    refresh_steps: List[List[int]] = []
    for r in range(R):
        first = (-int(phase[r])) % cfg.tau
        steps_r = list(range(first, T, cfg.tau))
        if first > 0:
            steps_r = [first - cfg.tau] + steps_r  # prologue: the refresh before step 0
        refresh_steps.append(steps_r)

    w_q = _normal(rng_for(seed, cfg.tag, _T_WQ), (cfg.n_idx, cfg.d_idx, cfg.q_in), cfg.w_std, cfg.dtype)
    # low rank: latents of unit variance from unit-variance hidden states
    w_down = (_normal(rng_for(seed, cfg.tag, _T_WDOWN), (cfg.n_idx, cfg.q_rank, cfg.d_model), cfg.d_model ** -0.5,
                      cfg.dtype) if cfg.q_rank > 0 else None)
    n_blocks = ctx // blk
    keys = [
        _normal(rng_for(seed, cfg.tag, _T_KEYS, r), (cfg.n_idx, int(n_blocks[r]), cfg.d_idx), cfg.k_std, cfg.dtype)
        for r in range(R)
    ]
    if cfg.hidden_rho == 0.0:
        hidden = [
            _normal(rng_for(seed, cfg.tag, _T_HID, r), (len(refresh_steps[r]), cfg.d_model), 1.0, cfg.dtype)
            for r in range(R)
        ]
    else:
        # an AR(1) sequence of unit-variance states: consecutive refreshes see related contexts
        rho = float(cfg.hidden_rho)
        hidden = []
        for r in range(R):
            eps = _normal(rng_for(seed, cfg.tag, _T_HID, r), (len(refresh_steps[r]), cfg.d_model), 1.0, "f32")
            h = np.empty(eps.shape, dtype=np.float64)
            h[0] = eps[0]
            for k in range(1, len(h)):
                h[k] = rho * h[k - 1] + np.sqrt(1.0 - rho * rho) * eps[k]
            h32 = h.astype(np.float32)
            hidden.append(bf16_bits_from_f32(h32) if cfg.dtype == "bf16" else h32)

    planted: List[np.ndarray] = []
    for r in range(R):
        if cfg.planted_frac <= 0:
            planted.append(np.zeros(0, dtype=np.int64))
            continue
        n_plant = int(round(cfg.planted_frac * int(n_blocks[r])))
        eligible = (int(ctx[r]) - cfg.window) // blk  # blocks wholly before the window at step 0
        ids = rng_for(seed, cfg.tag, _T_PLANT_IDS, r).choice(eligible, size=n_plant, replace=False)
        planted.append(np.sort(ids).astype(np.int64))

    q_dec = _normal(rng_for(seed, cfg.tag, _T_QDEC), (T, R, cfg.n_heads, cfg.head_dim), 1.0, cfg.dtype)
    k_new = _normal(rng_for(seed, cfg.tag, _T_KNEW), (T, R, cfg.head_dim), 1.0, cfg.dtype)
    v_new = _normal(rng_for(seed, cfg.tag, _T_VNEW), (T, R, cfg.head_dim), 1.0, cfg.dtype)

    layer_dec = []
    for layer in range(1, cfg.n_layers):
        layer_dec.append(tuple(
            _normal(rng_for(seed, cfg.tag, _T_LAYER, layer, tid), shape, 1.0, cfg.dtype)
            for tid, shape in ((_T_QDEC, (T, R, cfg.n_heads, cfg.head_dim)), (_T_KNEW, (T, R, cfg.head_dim)),
                               (_T_VNEW, (T, R, cfg.head_dim)))))

    return Workload(
        cfg=cfg, seed=seed, ctx=ctx, density=dens, phase=phase, bias=bias, w_q=w_q, keys=keys,
        refresh_steps=refresh_steps, hidden=hidden, planted=planted, q_dec=q_dec, k_new=k_new,
        v_new=v_new, layer_dec=layer_dec, w_down=w_down,
    )
