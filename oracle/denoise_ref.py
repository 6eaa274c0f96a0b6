"""Plain float64 oracle of the indexer's label-denoising pipeline.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  Every step is the definition written out with NumPy.

Source: the zhichai.net explainer of "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context
via Lookahead Sparse Attention", section 3 "Training the Indexer", the three-step label denoising
pipeline (and the Key Terms entry for top-p): the raw Lightning Indexer logits of each CSA layer
are softmax-normalised; each layer keeps the smallest set of entries whose cumulative probability
reaches 60% (top-p instead of a fixed top-k); across the 21 CSA layers a block is labelled positive
when at least 3 layers keep it.

What the page leaves open and how it is read here:
  * the unit is a (layer, token window) row of logits, one per history block the window can see;
    the softmax runs over that row's blocks.
  * "the smallest set whose cumulative probability reaches p": blocks are taken in decreasing
    probability (equal logits in increasing block id) until the running sum is >= p; that prefix is
    the set (a smallest one: any set reaching p has at least as many blocks).
  * "naive labels" are the blocks any layer keeps (the union), reported for comparison.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def layer_softmax(x: np.ndarray) -> np.ndarray:
    """Step 1: p_b = exp(x_b - max x) / sum_c exp(x_c - max x) over one row of block logits."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def top_p_set(x: np.ndarray, p: float = 0.6) -> np.ndarray:
    """Step 2: ascending ids of the smallest set of blocks whose probabilities sum to >= p.

    Blocks are ranked by logit, highest first (the softmax is monotone), equal logits by block id;
    the set is the shortest prefix of that ranking whose cumulative probability reaches p.
    """
    x = np.asarray(x, dtype=np.float64)
    prob = layer_softmax(x)
    order = np.lexsort((np.arange(len(x)), -x))  # by -x, then by id
    csum = np.cumsum(prob[order])
    k = int(np.searchsorted(csum, p, side="left")) + 1  # first prefix with csum >= p
    k = min(k, len(x))
    return np.sort(order[:k]).astype(np.int32)


def vote(sets: Sequence[np.ndarray], n_blocks: int, min_votes: int = 3) -> np.ndarray:
    """Step 3: block b is positive when at least min_votes layers' sets contain it."""
    counts = np.zeros(n_blocks, dtype=np.int64)
    for s in sets:
        counts[np.asarray(s, dtype=np.int64)] += 1
    return counts >= min_votes


def denoise_window(x: np.ndarray, p: float = 0.6, min_votes: int = 3) -> Tuple[np.ndarray, np.ndarray, List[np.ndarray]]:
    """The pipeline for one token window: x is [n_layers][n_blocks] raw logits.

    Returns (labels bool [n_blocks], naive bool [n_blocks] = kept by any layer, per-layer sets).
    """
    x = np.asarray(x, dtype=np.float64)
    sets = [top_p_set(x[l], p) for l in range(x.shape[0])]
    labels = vote(sets, x.shape[1], min_votes)
    naive = vote(sets, x.shape[1], 1)
    return labels, naive, sets
