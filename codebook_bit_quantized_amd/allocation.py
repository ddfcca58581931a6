"""Adaptive cluster allocation: choose a codebook width per weight matrix.

CodeQuant2, Figure 3 (left): importance scores and kernel latency guide how many
clusters each part of the model gets; Table 5 lists the allocation as one of the
method's steps.  Reading taken here: every weight matrix i gets bits b_i in a small
set (2, 3 or 4 bits: 4, 8 or 16 centroids per row); the choice minimises the total
importance-weighted clustering error sum_i err_i(b_i) subject to the measured kernel
latency sum_i lat_i(b_i) staying within a budget.  This is a multiple-choice knapsack,
solved exactly by dynamic programming over latency rounded up to a grid (the grid
only makes the budget test conservative).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def allocate_bits(latency: np.ndarray, error: np.ndarray, budget: float, choices: Sequence[int] = (2, 3, 4),
                  grid: int = 0) -> np.ndarray:
    """latency, error: [M][len(choices)] per matrix and choice; budget in the latency
    unit.  Returns the chosen bits per matrix (int array [M]) minimising the summed
    error with summed (grid-rounded-up) latency <= budget; the default grid keeps the
    rounding within 0.5 % of the budget.  Raises ValueError when even
    the fastest choice per matrix exceeds the budget."""
    lat = np.asarray(latency, dtype=np.float64)
    err = np.asarray(error, dtype=np.float64)
    M, C = lat.shape
    if err.shape != (M, C) or C != len(choices):
        raise ValueError("latency and error must be [M][len(choices)]")
    if grid <= 0:
        grid = max(4000, 200 * M)        # rounding up costs at most M cells: 0.5 % of the budget
    if lat.min(axis=1).sum() > budget:
        raise ValueError("budget below the fastest allocation")
    unit = budget / grid if budget > 0 else 1.0
    cost = np.ceil(lat / unit - 1e-9).astype(np.int64)      # rounded up: never over budget
    INF = np.inf
    best = np.full(grid + 1, INF)
    best[0] = 0.0
    pick = np.zeros((M, grid + 1), dtype=np.int8)
    for i in range(M):
        nxt = np.full(grid + 1, INF)
        arg = np.zeros(grid + 1, dtype=np.int8)
        for c in range(C):
            k = int(cost[i, c])
            if k > grid:
                continue
            cand = np.full(grid + 1, INF)
            cand[k:] = best[:grid + 1 - k] + err[i, c]
            better = cand < nxt
            nxt[better] = cand[better]
            arg[better] = c
        best, pick[i] = nxt, arg
    if not np.isfinite(best).any():
        raise ValueError("no allocation fits the budget on the latency grid")
    b = int(np.argmin(best))                                  # total cost with the least error
    out = np.empty(M, dtype=np.int64)
    for i in range(M - 1, -1, -1):
        c = int(pick[i, b])
        out[i] = choices[c]
        b -= int(cost[i, c])
    return out


def clustering_error(w_rows: np.ndarray, codebook: np.ndarray, idx: np.ndarray) -> float:
    """Sum of squared differences between weight rows (float [R][K]) and their
    dequantised codebook approximation (codebook float [R][L], idx int [R][K])."""
    approx = np.take_along_axis(codebook, idx, axis=1)
    return float(np.square(w_rows - approx).sum())
