"""Pins for the oracle's offline codebook construction (CPU only).

CodeQuant2, Figure 3 (right): K-means initialises the centroid matrix and the per-row
assignments.  The oracle's per-row K-means is tied to: a worked example derived by
hand (tests/golden), exact rational arithmetic for the fp16 rounding and the final
nearest-centroid assignment, the fixed-point property of converged Lloyd centroids,
closed forms (rows of L distinct values), and invariances the definition implies
(permuting a row, scaling it by a power of two)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def _bf16(x):
    return datagen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _f16_exact_round(x: float) -> int:
    """fp16 pattern nearest to x (ties to even) by exhaustive comparison with the
    neighbouring fp16 values, in exact rational arithmetic."""
    fx = Fraction(x)
    if fx == 0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if fx < 0 else 0
    a = abs(fx)
    # all finite positive fp16 values are k * 2^-24 (k < 2^11) or m * 2^(e-10)
    best, best_d = None, None
    for h in range(0x0000, 0x7C00):
        v = Fraction(float(np.uint16(h).view(np.float16)))
        d = abs(v - a)
        if best is None or d < best_d or (d == best_d and (h & 1) == 0):
            best, best_d = h, d
    # beyond the largest finite value: inf once at least half an ulp (16) above 65504
    if a >= Fraction(65520):
        best = 0x7C00
    return sign | best


def test_round_f64_to_f16_against_exhaustive():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(60) * np.exp2(rng.integers(-28, 17, 60)))
    # ties between neighbours, subnormals, the overflow boundary, signed zero
    xs += [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -24 * 1.5,
           65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -26, -0.0, 0.0, 6.1e-5, -1.0009765625]
    got = oracle.round_f64_to_f16_bits(np.array(xs, dtype=np.float64))
    for x, g in zip(xs, got):
        assert int(g) == _f16_exact_round(float(x)), (x, hex(int(g)), hex(_f16_exact_round(float(x))))


def test_order_keys_sort_like_values():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(500) * 10, [0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40]])
    bits = _bf16(vals)
    order = np.argsort(oracle.bf16_order_keys(bits), kind="stable")
    v = oracle.bf16_bits_to_f64(bits[order])
    assert np.all(np.diff(v) >= 0)
    zeros = bits[order][v == 0]
    assert list(zeros) == sorted(zeros, key=lambda b: 0 if b == 0x8000 else 1)   # -0 first


def test_golden_worked_example():
    g = _golden("kmeans_worked_example.txt")
    row = _bf16([float(t) for t in g["values"].split()])
    idx, cb, upd = oracle.kmeans_row(row, int(g["bits"]), 10)
    assert list(idx) == [int(t) for t in g["indices"].split()]
    assert [int(c) for c in cb] == [int(t, 16) for t in g["codebook"].split()]
    assert upd == int(g["updates"])


def _nearest_exact(w_bits, cb_bits):
    """Nearest fp16 centroid of each weight in exact arithmetic, ties to the lower index."""
    cs = [Fraction(float(c)) for c in oracle.f16_bits_to_f64(cb_bits)]
    out = []
    for v in oracle.bf16_bits_to_f64(w_bits):
        fv = Fraction(float(v))
        d = [abs(fv - c) for c in cs]
        out.append(d.index(min(d)))
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_final_assignment_is_nearest_and_rows_meet_precondition(bits):
    w = datagen.weights_bf16(1000 + bits, datagen.TAG_W_FULL, 0, 3, 256)
    for r in range(w.shape[0]):
        assert oracle.kmeans_precondition(w[r])
        idx, cb, _ = oracle.kmeans_row(w[r], bits, 30)
        assert list(idx) == _nearest_exact(w[r], cb)
        c = oracle.f16_bits_to_f64(cb)
        assert np.all(np.diff(c) >= 0)               # 1-D Lloyd keeps centroids ordered


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_converged_centroids_are_fixed_points(bits):
    """At convergence every non-empty cluster's fp64 centroid is the correctly rounded
    mean of the weights nearest to it (exact rational check)."""
    w = datagen.weights_bf16(2000 + bits, datagen.TAG_W_FULL, 0, 2, 192)
    for r in range(w.shape[0]):
        _, _, upd, c64 = oracle.kmeans_row(w[r], bits, 200, return_f64=True)
        assert upd < 200
        vals = [Fraction(float(v)) for v in oracle.bf16_bits_to_f64(w[r])]
        cs = [Fraction(float(c)) for c in c64]
        members = [[] for _ in cs]
        for v in vals:
            d = [abs(v - c) for c in cs]
            members[d.index(min(d))].append(v)
        for c, m in zip(c64, members):
            if m:
                assert c == float(sum(m) / len(m))   # Fraction -> float rounds to nearest


def test_rows_of_L_distinct_values():
    for bits in (2, 3, 4):
        L = 1 << bits
        vals = np.array([0.25 * (j + 1) * (-1) ** j for j in range(L)])
        row = np.repeat(vals, 8)
        np.random.default_rng(bits).shuffle(row)
        idx, cb, upd = oracle.kmeans_row(_bf16(row), bits, 10)
        order = np.sort(vals)
        assert np.array_equal(oracle.f16_bits_to_f64(cb), order)
        assert np.array_equal(order[idx], row)
        assert upd == 1


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_permutation_and_scale_invariance(bits):
    w = datagen.weights_bf16(3000 + bits, datagen.TAG_W_FULL, 0, 1, 256)[0]
    idx, cb, upd = oracle.kmeans_row(w, bits, 40)
    perm = np.random.default_rng(bits).permutation(w.shape[0])
    idx_p, cb_p, upd_p = oracle.kmeans_row(w[perm], bits, 40)
    assert np.array_equal(cb_p, cb) and upd_p == upd and np.array_equal(idx_p, idx[perm])
    w2 = _bf16(oracle.bf16_bits_to_f64(w) * 4.0)   # exact in bf16
    idx_s, cb_s, upd_s = oracle.kmeans_row(w2, bits, 40)
    assert np.array_equal(idx_s, idx) and upd_s == upd
    assert np.array_equal(oracle.f16_bits_to_f64(cb_s), oracle.f16_bits_to_f64(cb) * 4.0)


def test_zero_iterations_give_rank_centroids():
    w = datagen.weights_bf16(4000, datagen.TAG_W_FULL, 0, 1, 64)[0]
    idx, cb, upd = oracle.kmeans_row(w, 2, 0)
    srt = np.sort(oracle.bf16_bits_to_f64(w))
    ranks = [(2 * j + 1) * 64 // 8 for j in range(4)]
    assert upd == 0
    assert np.array_equal(oracle.f16_bits_to_f64(cb), oracle.f16_bits_to_f64(oracle.round_f64_to_f16_bits(srt[ranks])))
