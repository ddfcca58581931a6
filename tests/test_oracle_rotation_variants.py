"""Pins for the oracle's rotation variants (CPU only): per-channel smoothing scales and
random signs applied before the Hadamard blocks (CodeQuant2, Figure 1: per-channel
scales and a rotation folded into the weights smooth the activation outliers; Table 5
caption: the base setting is a fixed random rotation with SmoothQuant scaling).

The smoothed values are tied to an independent rounding of the exact products, a sign
flip to its exact effect on the rotation, one-hot tokens to a closed form, and blocks
beyond the fp64 bound to exact rational sums."""
import math
from fractions import Fraction

import numpy as np

import datagen
import oracle


def _bf16(x):
    return datagen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _nearest_f32(q: Fraction) -> np.float32:
    """fp32 nearest to the rational q (ties to even), by comparing the neighbours of a
    first approximation exactly."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _random_smooth(seed, K):
    g = np.random.default_rng(seed)
    return np.exp2(g.uniform(-3, 3, K)).astype(np.float32)


def _random_signs(seed, K):
    return np.random.default_rng(seed).integers(0, 256, K // 8, dtype=np.uint8)


def test_identity_transforms_change_nothing():
    x = datagen.random_tokens(5, 6, 512)
    a = oracle.rotate_quantize(x, 0, 4)
    b = oracle.rotate_quantize(x, 0, 4, smooth=np.ones(512, np.float32),
                               signs=np.zeros(64, np.uint8))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scale"], b["scale"])


def test_smoothing_rounds_the_exact_product_once():
    x = datagen.random_tokens(6, 4, 256)
    m = _random_smooth(6, 256)
    v, sig = oracle.smooth_and_sign(x, m, None)
    assert sig == 24
    # bf16 x fp32 has at most 32 significant bits: exact in fp64, then one rounding
    exact = oracle.bf16_bits_to_f64(x) * m.astype(np.float64)[None, :]
    assert np.array_equal(v, exact.astype(np.float32).astype(np.float64))


def test_sign_flip_changes_the_rotation_exactly():
    K, b = 128, 128
    x = datagen.random_tokens(7, 1, K)
    signs = np.zeros(K // 8, np.uint8)
    c = 37
    signs[c >> 3] |= 1 << (c & 7)
    v0, _ = oracle.smooth_and_sign(x, None, None)
    v1, _ = oracle.smooth_and_sign(x, None, signs)
    u0 = oracle.rotate_fp64(v0, b)[0]
    u1 = oracle.rotate_fp64(v1, b)[0]
    H = oracle.sylvester_hadamard(b)
    assert np.array_equal(u1, u0 - 2.0 * v0[0, c] * H[:, c])
    # D H H D = b I: rotating twice and undoing the signs returns the token
    back = oracle.rotate_fp64(oracle.rotate_fp64(v1, b), b)[0] / b
    assert np.array_equal(np.where(np.arange(K) == c, -back, back), v0[0])


def test_one_hot_token_closed_form():
    K, c = 256, 77
    x = np.zeros((1, K), np.float32)
    x[0, c] = 3.0
    m = np.ones(K, np.float32)
    m[c] = 0.25
    signs = np.zeros(K // 8, np.uint8)
    signs[c >> 3] |= 1 << (c & 7)
    for act_bits, Q in ((4, 7), (8, 127)):
        r = oracle.rotate_quantize(_bf16(x), 0, act_bits, smooth=m, signs=signs)
        H = oracle.sylvester_hadamard(K)
        assert np.array_equal(r["q"][0], -Q * H[:, c])          # v_c = -0.75 everywhere
        assert r["scale"][0] == np.float32(np.float32(0.75 / Q) * np.float32(1 / 16))


def test_common_power_of_two_smoothing_scales_only_the_scale():
    x = datagen.random_tokens(8, 5, 768)
    a = oracle.rotate_quantize(x, 0, 8)
    b = oracle.rotate_quantize(x, 0, 8, smooth=np.full(768, 0.125, np.float32))
    assert np.array_equal(a["q"], b["q"])
    assert np.array_equal(b["scale"], (a["scale"] * np.float32(0.125)).astype(np.float32))


def test_fp32_blocks_beyond_the_fp64_bound_are_exact():
    b = 64
    # 24-bit significands 40 binades apart: beyond 53 - 24 - 6 = 23
    vals = np.array([(1 + 2.0 ** -23) * 2.0 ** 20, (1 + 3 * 2.0 ** -23) * 2.0 ** -20] * 32)
    v = (vals * np.where(np.arange(64) % 3 == 0, -1.0, 1.0)).astype(np.float32).astype(np.float64)
    ok = oracle.rotation_precondition(v[None, None, :], b, 24)
    assert not ok.all()
    u32, _ = oracle.rotate_values(v[None, :], b, 24)
    H = oracle.sylvester_hadamard(b)
    for j in range(b):
        exact = sum(Fraction(float(vi)) * int(H[j, i]) for i, vi in enumerate(v))
        assert u32[0, j] == _nearest_f32(exact)
    # and within the bound the fp64 path is used and agrees with the exact sums
    w = datagen.random_tokens(9, 1, 64)
    m = _random_smooth(9, 64)
    v2, _ = oracle.smooth_and_sign(w, m, _random_signs(9, 64))
    assert oracle.rotation_precondition(v2.reshape(1, 1, 64), b, 24).all()
    u2, _ = oracle.rotate_values(v2, b, 24)
    for j in range(0, b, 7):
        exact = sum(Fraction(float(vi)) * int(H[j, i]) for i, vi in enumerate(v2[0]))
        assert u2[0, j] == _nearest_f32(exact)
