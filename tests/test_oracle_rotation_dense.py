"""Pins of the oracle's dense rotation (a K x K orthogonal matrix standing for a learned
rotation, CodeQuant2 Figure 1) against results fixed by other means: the block
Walsh-Hadamard path, signed permutations, and exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle


def _bf16(a):
    return datagen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_identity_is_no_rotation():
    x = datagen.random_tokens(11, 9, 128)
    eye = _bf16(np.eye(128))
    for a in (4, 8):
        d = oracle.rotate_quantize_dense(x, eye, a)
        r = oracle.rotate_quantize(x, 1, a)                # had_block 1: no rotation
        assert np.array_equal(d["codes"], r["codes"])
        assert np.array_equal(d["scale"], r["scale"])


@pytest.mark.parametrize("K", [256, 512])
def test_hadamard_blocks_as_a_dense_matrix(K):
    # H_256 / 16 has entries +-1/16 (exact in bf16); block-diagonal for K = 512
    H = oracle.sylvester_hadamard(256).astype(np.float64) / 16.0
    R = np.kron(np.eye(K // 256), H)
    x = datagen.random_tokens(12, 7, K)
    for a in (4, 8):
        d = oracle.rotate_quantize_dense(x, _bf16(R), a)
        r = oracle.rotate_quantize(x, 256, a)
        assert np.array_equal(d["q"], r["q"])
        assert np.array_equal(d["scale"], r["scale"])      # 1/16 = fp32(1/sqrt(256))


def test_signed_permutation():
    K = 96
    rng = np.random.default_rng(5)
    perm = rng.permutation(K)
    sgn = rng.choice([-1.0, 1.0], K)
    R = np.zeros((K, K))
    R[np.arange(K), perm] = sgn                            # u[j] = sgn[j] * x[perm[j]]
    x = datagen.random_tokens(13, 5, K)
    xf = datagen.bf16_bits_to_f32(x)
    moved = _bf16(xf[:, perm] * sgn[None, :])
    d = oracle.rotate_quantize_dense(x, _bf16(R), 4)
    r = oracle.rotate_quantize(moved, 1, 4)
    assert np.array_equal(d["codes"], r["codes"])
    assert np.array_equal(d["scale"], r["scale"])


def _nearest_f32(v: np.float32, exact: Fraction) -> bool:
    f = Fraction(float(v))
    for nb in (np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))):
        g = Fraction(float(nb))
        if abs(g - exact) < abs(f - exact):
            return False
        if abs(g - exact) == abs(f - exact) and (int(v.view(np.uint32)) & 1):
            return False                                   # ties go to the even one
    return True


def test_exact_rounding_outside_and_inside_the_bound():
    K = 32
    rng = np.random.default_rng(8)
    xf = rng.standard_normal((3, K)).astype(np.float32)
    xf[0, 5] = 2.0 ** -60                                  # token 0: huge exponent spread
    xf[0, 6] = 2.0 ** 40
    xb = _bf16(xf)
    Rb = datagen.rotation_bf16(3, K)
    ok = oracle.dense_rotation_precondition(xb, Rb)
    assert not ok[0] and ok[1:].all()
    u32, ok2 = oracle.rotate_dense(xb, Rb)
    assert np.array_equal(ok, ok2)
    x = [[Fraction(float(v)) for v in row] for row in datagen.bf16_bits_to_f32(xb)]
    R = [[Fraction(float(v)) for v in row] for row in datagen.bf16_bits_to_f32(Rb)]
    for t in range(3):
        for j in range(K):
            exact = sum(R[j][k] * x[t][k] for k in range(K))
            assert _nearest_f32(u32[t, j], exact), (t, j)


def test_precondition_boundary():
    K = 64                                                 # bound 37 - 6 = 31
    x = np.zeros((2, K), np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 2.0 ** -20                                   # spread 20 in both tokens
    R = np.eye(K, dtype=np.float32)
    R[3, 4] = 2.0 ** -11                                   # row spread 11: 31, inside
    assert oracle.dense_rotation_precondition(_bf16(x), _bf16(R)).all()
    R[3, 4] = 2.0 ** -12                                   # 32: outside
    assert not oracle.dense_rotation_precondition(_bf16(x), _bf16(R)).any()
    x[1] = 0.0                                             # an all-zero token is always inside
    assert list(oracle.dense_rotation_precondition(_bf16(x), _bf16(R))) == [False, True]


def test_zero_token_and_generator_spread():
    Rb = datagen.rotation_bf16(4, 256)
    er = np.abs(datagen.bf16_bits_to_f32(Rb))
    nz = er[er > 0]
    assert np.log2(nz.max() / nz.min()) < 8                # flushed below 2^-7 of the largest
    q = datagen.bf16_bits_to_f32(Rb).astype(np.float64)
    assert np.abs(q @ q.T - np.eye(256)).max() < 0.05      # close to orthogonal
    x = datagen.random_tokens(14, 3, 256)
    x[1] = 0
    d = oracle.rotate_quantize_dense(x, Rb, 4)
    assert d["scale"][1] == 0 and not d["q"][1].any()
