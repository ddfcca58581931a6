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


# ---------------------------------------------------------------------------
# Inputs of the allocation, computed from the library's own results: routing counts
# from cbq_moe_route_gather and clusterings from cbq_kmeans_codebooks, decoded here.

def unpack_indices(packed: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Indices [..., K] (int64) of rows stored as the cbq_weights bitstream [..., K*bits/8]:
    index k occupies bits [k*bits, (k+1)*bits) counted from bit 0 of byte 0 (bits <= 4,
    so an index spans at most two bytes)."""
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    rows = p.reshape(-1, p.shape[-1]).astype(np.uint16)
    rows = np.concatenate([rows, np.zeros((rows.shape[0], 1), dtype=np.uint16)], axis=1)
    start = np.arange(K, dtype=np.int64) * bits
    byte, shift = start >> 3, (start & 7).astype(np.uint16)
    pair = rows[:, byte] | (rows[:, byte + 1] << np.uint16(8))
    out = (pair >> shift) & np.uint16((1 << bits) - 1)
    return out.astype(np.int64).reshape(*lead, K)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (a bf16 value is the high half of an fp32)."""
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def dequantize_rows(idx_packed: np.ndarray, codebook_bits: np.ndarray, K: int, bits: int) -> np.ndarray:
    """The weights [R][K] (float64) a clustered matrix stands for: row r's centroid at each
    of its K indices (idx_packed [R][K*bits/8] as the cbq_weights bitstream, codebook_bits
    [R][2^bits] fp16 patterns)."""
    idx = unpack_indices(idx_packed, K, bits)
    cb = f16_bits_to_float(np.asarray(codebook_bits).reshape(idx.shape[0], -1))
    return np.take_along_axis(cb, idx, axis=1)


def output_error(w_bits: np.ndarray, idx_packed: np.ndarray, codebook_bits: np.ndarray,
                 x_bits: np.ndarray, K: int, bits: int) -> float:
    """Relative error of a clustered matrix on the layer output: ||X (W - W')^T||_F /
    ||X W^T||_F for tokens X [n][K] (bf16 patterns), rows W [R][K] (bf16 patterns) and their
    clustering W' (CodeQuant2, Figure 3 right: the centroids are refit to the output error)."""
    W = bf16_bits_to_float(w_bits)
    Wc = dequantize_rows(idx_packed, codebook_bits, K, bits)
    X = bf16_bits_to_float(x_bits)
    return float(np.linalg.norm(X @ (W - Wc).T) / np.linalg.norm(X @ W.T))


def expert_share(offsets: np.ndarray, T: int, n_routed: int, n_shared: int) -> np.ndarray:
    """Importance proxy per expert from the router's row offsets [E + S + 1]: the share of
    the T tokens routed to each of the E routed experts, and 1 for each shared expert
    (they see every token)."""
    off = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(off[:n_routed + 1]).astype(np.float64)
    return np.concatenate([counts / float(T), np.ones(n_shared)])


def route_share(cbq, logits, topk: int, n_shared: int) -> np.ndarray:
    """expert_share of the routing that cbq.moe_route_gather gives device logits [T][E]."""
    T, E = int(logits.shape[0]), int(logits.shape[1])
    rt = cbq.moe_route_gather(logits, topk, True, n_shared)
    return expert_share(rt["offsets"].cpu().numpy(), T, E, n_shared)


def clustering_errors(cbq, torch, w_bits: np.ndarray, groups: int, choices: Sequence[int] = (2, 3, 4),
                      max_iters: int = 30, device: str = "cuda:0") -> np.ndarray:
    """Per-row K-means (cbq.kmeans_codebooks, on the GPU) of bf16 rows w_bits [groups*r][K]
    at every width in choices; returns [groups][len(choices)], the summed squared
    clustering error of each group of r consecutive rows."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    R, K = w_bits.shape
    if R % groups:
        raise ValueError("rows must split evenly into groups")
    wf = bf16_bits_to_float(w_bits)
    w = torch.from_numpy(w_bits.view(np.int16)).to(device)
    out = np.zeros((groups, len(choices)))
    for c, bits in enumerate(choices):
        cw = cbq.kmeans_codebooks(w, bits, max_iters)
        idx = unpack_indices(cw.idx.reshape(R, -1).cpu().numpy(), K, bits)
        cb = f16_bits_to_float(cw.codebook.reshape(R, -1).cpu().numpy().view(np.uint16))
        sq = np.square(wf - np.take_along_axis(cb, idx, axis=1)).sum(axis=1)
        out[:, c] = sq.reshape(groups, -1).sum(axis=1)
    return out
