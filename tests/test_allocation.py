"""Adaptive cluster allocation (CodeQuant2, Figure 3 left): the dynamic programme is
checked against exhaustive search on small instances, and for the properties any
optimum has (budget respected, error non-increasing as the budget grows)."""
import itertools

import numpy as np
import pytest

from codebook_bit_quantized_amd.allocation import allocate_bits


def _brute(lat, err, budget, grid):
    unit = budget / grid
    cost = np.ceil(lat / unit - 1e-9)
    best, arg = np.inf, None
    for combo in itertools.product(range(lat.shape[1]), repeat=lat.shape[0]):
        c = sum(cost[i, j] for i, j in enumerate(combo))
        e = sum(err[i, j] for i, j in enumerate(combo))
        if c <= grid and e < best - 1e-12:
            best, arg = e, combo
    return best, arg


@pytest.mark.parametrize("seed", range(8))
def test_dp_matches_exhaustive_search(seed):
    g = np.random.default_rng(seed)
    M = 6
    lat = np.sort(g.uniform(1, 10, (M, 3)), axis=1)          # more bits: slower
    err = -np.sort(-g.uniform(0, 5, (M, 3)), axis=1)         # more bits: less error
    budget = float(lat.mean(axis=1).sum())
    bits = allocate_bits(lat, err, budget, grid=400)
    chosen = bits - 2
    e = err[np.arange(M), chosen].sum()
    best, _ = _brute(lat, err, budget, 400)
    assert e == pytest.approx(best, abs=1e-12)
    assert lat[np.arange(M), chosen].sum() <= budget + 1e-9


def test_more_budget_never_more_error():
    g = np.random.default_rng(11)
    M = 30
    lat = np.sort(g.uniform(1, 10, (M, 3)), axis=1)
    err = -np.sort(-g.uniform(0, 5, (M, 3)), axis=1)
    lo, hi = lat[:, 0].sum(), lat[:, 2].sum()
    prev = np.inf
    for f in np.linspace(0.05, 1, 9):   # the grid rounds latencies up: start above the minimum
        budget = lo + f * (hi - lo) + 1e-6
        bits = allocate_bits(lat, err, budget)
        e = err[np.arange(M), bits - 2].sum()
        assert e <= prev + 1e-9
        prev = e
    assert np.all(allocate_bits(lat, err, hi * 1.01) == 4)   # everything fits (grid slack < 1%)


def test_budget_below_fastest_raises():
    lat = np.array([[1.0, 2.0, 3.0]])
    with pytest.raises(ValueError):
        allocate_bits(lat, np.zeros((1, 3)), 0.5)


def test_library_index_decoding_matches_the_oracle():
    # the allocation inputs decode the library's clusterings with their own helpers;
    # the oracle's bit unpacking and fp16 / bf16 conversions are the reference
    import oracle
    from codebook_bit_quantized_amd.allocation import (bf16_bits_to_float, f16_bits_to_float,
                                                       unpack_indices)
    g = np.random.default_rng(5)
    for bits in (2, 3, 4):
        for K in (32, 96, 1408):
            p = g.integers(0, 256, (2, 3, K * bits // 8), dtype=np.uint8)
            assert np.array_equal(unpack_indices(p, K, bits), oracle.unpack_indices(p, K, bits))
    h = g.integers(0, 1 << 16, 4096, dtype=np.uint16)
    h = h[(h & 0x7C00) != 0x7C00]                      # finite fp16 patterns
    assert np.array_equal(f16_bits_to_float(h), oracle.f16_bits_to_f64(h))
    b = g.integers(0, 1 << 16, 4096, dtype=np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]                      # finite bf16 patterns
    assert np.array_equal(bf16_bits_to_float(b), oracle.bf16_bits_to_f64(b))


def test_expert_share_from_offsets():
    from codebook_bit_quantized_amd.allocation import expert_share
    import oracle
    lg = np.random.default_rng(3).standard_normal((40, 8)).astype(np.float32)
    rt = oracle.route(lg, 2, True, 1)
    share = expert_share(rt["offsets"], 40, 8, 1)
    assert np.array_equal(share[:8], rt["counts"] / 40.0)
    assert share[8] == 1.0 and share[:8].sum() == 2.0   # top-2: every token counted twice
