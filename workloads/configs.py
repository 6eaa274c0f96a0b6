"""Workload shapes for the LSA decode path.

The five full-size workloads follow the shapes and distributions of the
pages' setting: one attention layer, 64-token KV blocks, three indexers
refreshed every tau = 64 decode steps, a recent local window, and a cold
pool of blocks in host memory.  The pages run their system on evaluation
suites and a trained model; these seeded synthetic inputs stand in for them.

Density is the *union* density (fraction of blocks loaded), which is what
the pages measure as the physical KV share.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Tuple


@dataclass(frozen=True)
class LSAConfig:
    name: str
    n_req: int
    # context spec: ("fixed", N) or ("loguniform", lo, hi); N is rounded down to a multiple of 64
    ctx: Tuple = ("fixed", 4096)
    dtype: str = "bf16"  # element type of hidden, W_q, keys, decode q and K/V: "f32" or "bf16"
    d_model: int = 4096
    d_idx: int = 256
    n_idx: int = 3
    n_heads: int = 16
    head_dim: int = 128
    window: int = 8192
    steps: int = 256
    tau: int = 64
    block: int = 64
    # union density spec: ("fixed", rho) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    density: Tuple = ("fixed", 0.10)
    # fraction of blocks planted as relevant (keys placed above threshold along every refresh's query)
    planted_frac: float = 0.0
    # staggered refresh phases (at most one request refreshes per step)
    staggered: bool = False
    # attention layers whose block loads one selection drives (each with its own K/V, decode
    # queries and new tokens; the selection and the hidden states are shared)
    n_layers: int = 1
    # correlation of successive refresh hidden states: h_k = rho h_{k-1} + sqrt(1 - rho^2) eps_k
    hidden_rho: float = 0.0
    # selection level: a block is kept when sigmoid(logit) > level (0.5 on the pages)
    level: float = 0.5
    # low-rank query projection: 0 = full rank (W_q [n_idx][d_idx][d_model]); r > 0 = each indexer
    # projects the latent c_i = A_i h (A_i [r][d_model]) with B_i [d_idx][r] (w_q holds B)
    q_rank: int = 0
    # std of the drawn tensors
    wq_std: float = field(default=0.0)  # 0 => 1/sqrt(input size of W_q: d_model, or q_rank)
    key_std: float = field(default=0.0)  # 0 => 1/sqrt(d_idx)
    tag: int = 0  # distinguishes the random streams of different workloads

    @property
    def q_in(self) -> int:
        """Input size of the Query Encoder's matrices: the hidden size, or the latent rank."""
        return self.q_rank if self.q_rank > 0 else self.d_model

    @property
    def w_std(self) -> float:
        return self.wq_std if self.wq_std > 0 else self.q_in ** -0.5

    @property
    def k_std(self) -> float:
        return self.key_std if self.key_std > 0 else self.d_idx ** -0.5

    def scaled(self, **kw) -> "LSAConfig":
        return replace(self, **kw)


_BASE = LSAConfig(name="base", n_req=1)

CONFIGS: Dict[str, LSAConfig] = {
    # 1 request, 4096 tokens (64 blocks), fp32, d=512, d_idx=128, 8 q-heads / 1 kv-head, D=64,
    # ~20% of blocks selected, window 256, 64 decode steps with one refresh.
    "tiny": LSAConfig(
        name="tiny", n_req=1, ctx=("fixed", 4096), dtype="f32", d_model=512, d_idx=128,
        n_heads=8, head_dim=64, window=256, steps=64, density=("fixed", 0.20), tag=0,
    ),
    # 128K context, batch 1, bf16, ~10% selection, 8192 window, 256 steps (4 refreshes).
    "ctx128k": LSAConfig(
        name="ctx128k", n_req=1, ctx=("fixed", 131072), density=("fixed", 0.10), steps=256, tag=1,
    ),
    # 512K context, batch 8, per-request density uniform in 5..15%, 128 steps (2 refreshes).
    "ctx512k": LSAConfig(
        name="ctx512k", n_req=8, ctx=("fixed", 524288), density=("uniform", 0.05, 0.15),
        steps=128, tag=2,
    ),
    # 1M context, batch 4, 10% background + 10% planted relevant blocks, 256 steps.
    "ctx1m": LSAConfig(
        name="ctx1m", n_req=4, ctx=("fixed", 1048576), density=("fixed", 0.10),
        planted_frac=0.10, steps=256, tag=3,
    ),
    # 32 requests, context log-uniform 64K..1M, density log-uniform 1..50%, staggered phases,
    # 512 steps.
    "ragged": LSAConfig(
        name="ragged", n_req=32, ctx=("loguniform", 65536, 1048576),
        density=("loguniform", 0.01, 0.50), staggered=True, steps=512, tag=4,
    ),
}

# Reduced versions with the same structure, small enough for the oracle to finish in
# seconds while still spanning many tiles and ragged tails.
SMALL: Dict[str, LSAConfig] = {
    "tiny": CONFIGS["tiny"],
    "ctx128k_s": CONFIGS["ctx128k"].scaled(name="ctx128k_s", ctx=("fixed", 16384), window=2048,
                                          steps=130, tag=11),
    "ctx512k_s": CONFIGS["ctx512k"].scaled(name="ctx512k_s", n_req=3, ctx=("fixed", 24576),
                                          window=1024, steps=66, tag=12),
    "ctx1m_s": CONFIGS["ctx1m"].scaled(name="ctx1m_s", n_req=2, ctx=("fixed", 32768), window=2048,
                                      steps=70, tag=13),
    "ragged_s": CONFIGS["ragged"].scaled(name="ragged_s", n_req=5, ctx=("loguniform", 4096, 40960),
                                        window=1024, steps=80, tag=14),
}


def get_config(name: str) -> LSAConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in SMALL:
        return SMALL[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS) + sorted(SMALL)}")
