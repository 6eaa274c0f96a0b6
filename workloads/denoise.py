"""Seeded synthetic logits for the indexer's label-denoising pipeline.

The pages' input is the raw Lightning Indexer logits of 21 CSA layers for each token window of an
inference log (a public log is not available here, and none is written out).  The stand-in draws,
per window w, a set of relevant blocks (a fixed fraction of the window's history) and, per layer
l and block b, the logit
    x[l][w][b] = signal * [b relevant for w] + noise * eps[l][w][b],   eps ~ N(0, 1) iid,
so the layers agree on the relevant blocks and disagree on the rest.  With 16,384 blocks, 300
relevant, signal 4 and noise 1, a layer's top-60% set holds ~800 blocks, the layers' union ~8,000
and the 3-of-21 vote ~750, the magnitudes the pages report (~10,000 naive positives per window,
100-1,000 after denoising).  Nothing here evaluates the pipeline.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

from .gen import rng_for

_TAG = 21  # stream namespace of the denoising inputs
_T_REL, _T_EPS = 1, 2


@dataclass
class DenoiseWorkload:
    logits: np.ndarray          # float32 [n_layers][n_windows][stride]; row (l, w) holds n_blk[w] logits first
    n_blk: np.ndarray           # int32 [n_windows]
    relevant: List[np.ndarray]  # per window, ascending relevant block ids

    @property
    def n_layers(self) -> int:
        return self.logits.shape[0]

    @property
    def n_windows(self) -> int:
        return self.logits.shape[1]

    def row(self, l: int, w: int) -> np.ndarray:
        return self.logits[l, w, : int(self.n_blk[w])]


def build_denoise_workload(n_blk: Sequence[int], n_layers: int = 21, relevant: int = 300, signal: float = 4.0,
                           noise: float = 1.0, seed: int = 0, integer_logits: bool = False) -> DenoiseWorkload:
    """Logits for len(n_blk) windows (window w sees n_blk[w] blocks).  integer_logits rounds every
    logit to an integer (many equal logits: exercises the ordering of ties)."""
    n_blk = np.asarray(n_blk, dtype=np.int32)
    W = len(n_blk)
    stride = int((n_blk.max() + 3) // 4 * 4)
    x = np.zeros((n_layers, W, stride), dtype=np.float32)
    rel = []
    for w in range(W):
        n = int(n_blk[w])
        ids = np.sort(rng_for(seed, _TAG, _T_REL, w).choice(n, size=min(relevant, n), replace=False))
        rel.append(ids.astype(np.int32))
        base = np.zeros(n, dtype=np.float64)
        base[ids] = signal
        eps = rng_for(seed, _TAG, _T_EPS, w).standard_normal((n_layers, n))
        row = base[None, :] + noise * eps
        x[:, w, :n] = (np.rint(row) if integer_logits else row).astype(np.float32)
    return DenoiseWorkload(logits=x, n_blk=n_blk, relevant=rel)
