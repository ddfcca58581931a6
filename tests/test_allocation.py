"""Adaptive cluster allocation (CodeQuant2, Figure 3 left): the dynamic programme is
checked against exhaustive search on small instances, and for the properties any
optimum has (budget respected, error non-increasing as the budget grows)."""
import itertools

import numpy as np
import pytest

import oracle
from codebook_bit_quantized_amd import allocation
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


def test_dequantize_rows_and_output_error_match_the_oracle():
    # the allocation module's own decoding (used by the benchmark's quality figures) against
    # the oracle's definitions, on random packed rows of every width
    rng = np.random.default_rng(11)
    for bits in (2, 3, 4):
        R, K, n = 6, 96, 5
        idx = rng.integers(0, 1 << bits, (R, K))
        packed = np.zeros((R, K * bits // 8), dtype=np.uint8)
        for r in range(R):
            v = 0
            for k in range(K):
                v |= int(idx[r, k]) << (k * bits)
            packed[r] = np.frombuffer(v.to_bytes(K * bits // 8, "little"), dtype=np.uint8)
        cb = rng.standard_normal((R, 1 << bits)).astype(np.float16).view(np.uint16)
        w = (rng.standard_normal((R, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        x = (rng.standard_normal((n, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        want_w = oracle.dequantize(oracle.unpack_indices(packed, K, bits), cb)
        assert np.array_equal(allocation.dequantize_rows(packed, cb, K, bits), want_w)
        got = allocation.output_error(w, packed, cb, x, K, bits)
        want = oracle.output_error(w, oracle.unpack_indices(packed, K, bits), cb, x)
        assert abs(got - want) <= 1e-12 * max(1.0, want)
