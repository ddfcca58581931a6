"""Pins for the oracle's rotation and activation quantiser (CPU only).

Each test ties the oracle to something other than its own formula: the closed form
of the Sylvester Hadamard matrix, orthogonality, an independent butterfly transform,
hand-derived worked examples (tests/golden), exactness at the fp64 boundary, and
invariants of absmax quantisation."""
import math
import os

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
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def _bf16(x):
    return datagen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_hadamard_closed_form(b):
    H = oracle.sylvester_hadamard(b)
    i = np.arange(b)[:, None]
    j = np.arange(b)[None, :]
    parity = np.bitwise_count((i & j).astype(np.uint64)) & 1
    assert np.array_equal(H, np.where(parity == 1, -1, 1))


@pytest.mark.parametrize("b", [2, 8, 128, 512, 2048, 4096])
def test_hadamard_orthogonal_symmetric(b):
    H = oracle.sylvester_hadamard(b)
    assert np.array_equal(H, H.T)
    Hf = H.astype(np.float64)          # +-1 sums up to 4096 are exact in fp64
    assert np.array_equal(Hf @ Hf.T, b * np.eye(b))


def _fwht_butterfly(x):
    """Independent in-place fast Walsh-Hadamard transform over the last axis."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        c = y[..., 1, :].copy()
        y[..., 0, :] = a + c
        y[..., 1, :] = a - c
        y = y.reshape(*y.shape[:-3], n)
        h *= 2
    return y


@pytest.mark.parametrize("K,b", [(256, 256), (1408, 128), (2560, 512), (768, 256), (2048, 2048)])
def test_rotation_matches_butterfly_and_round_trips(K, b):
    xb = datagen.random_tokens(K, 6, K)
    x = oracle.bf16_bits_to_f64(xb)
    u = oracle.rotate_fp64(x, b)
    ref = _fwht_butterfly(x.reshape(6, K // b, b)).reshape(6, K)
    assert np.array_equal(u, ref)                     # exact under the bf16 precondition
    assert oracle.rotation_precondition(x.reshape(6, K // b, b), b).all()
    assert np.array_equal(oracle.rotate_fp64(u, b), b * x)   # H H = b I, exact
    u32, ok = oracle.rotate(xb, b)
    assert ok.all() and np.array_equal(u32, ref.astype(np.float32))


def test_rotation_one_hot_and_constant():
    b = 64
    for i in (0, 5, 63):
        x = np.zeros((1, b), dtype=np.float32)
        x[0, i] = 1.0
        u32, _ = oracle.rotate(_bf16(x), b)
        j = np.arange(b)
        expect = np.where(np.bitwise_count((i & j).astype(np.uint64)) & 1, -1.0, 1.0)
        assert np.array_equal(u32[0], expect.astype(np.float32))
    u32, _ = oracle.rotate(_bf16(np.ones((1, b))), b)
    assert u32[0, 0] == b and not u32[0, 1:].any()


def test_rotation_block_diagonal():
    K, b = 384, 128
    xb = datagen.random_tokens(3, 2, K)
    u32, _ = oracle.rotate(xb, b)
    for blk in range(K // b):
        ub, _ = oracle.rotate(xb[:, blk * b:(blk + 1) * b], b)
        assert np.array_equal(u32[:, blk * b:(blk + 1) * b], ub)


def test_rotation_exact_beyond_fp64():
    """1 + 2^-24 + 2^-80 rounds up to 1 + 2^-23 in fp32; an fp64 sum loses 2^-80 and
    lands on the tie, which rounds to 1.0.  The oracle must give the exact answer."""
    b = 4
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -80, 0.0]], dtype=np.float32)
    u32, ok = oracle.rotate(_bf16(x), b)
    assert not ok[0, 0]
    assert u32[0, 0] == np.float32(1.0 + 2.0 ** -23)
    # entries 1..3: 1 - 2^-24 + 2^-80, 1 + 2^-24 - 2^-80, 1 - 2^-24 - 2^-80; below 1 the
    # fp32 spacing is 2^-24, so 1 - 2^-24 is representable
    assert u32[0, 1] == np.float32(1.0 - 2.0 ** -24)
    assert u32[0, 2] == np.float32(1.0)
    assert u32[0, 3] == np.float32(1.0 - 2.0 ** -24)


def test_precondition_boundary():
    b = 128   # log2 b = 7 -> spread allowed 38
    x = np.zeros((1, 1, b))
    x[0, 0, 0] = 1.0
    x[0, 0, 1] = 2.0 ** -38
    assert oracle.rotation_precondition(x, b).all()
    x[0, 0, 1] = 2.0 ** -39
    assert not oracle.rotation_precondition(x, b).any()


def test_round_int_pow2_to_f32():
    assert oracle.round_int_pow2_to_f32(3, -1) == np.float32(1.5)
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2 -> even (2^24)
    assert oracle.round_int_pow2_to_f32(2 ** 24 + 1, 0) == np.float32(2 ** 24)
    assert oracle.round_int_pow2_to_f32(2 ** 24 + 3, 0) == np.float32(2 ** 24 + 4)
    assert oracle.round_int_pow2_to_f32(-(2 ** 24 + 3), 0) == np.float32(-(2 ** 24 + 4))
    # agreement with numpy's own fp64 -> fp32 rounding when the value is exact in fp64
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(-2 ** 52, 2 ** 52))
        s = int(rng.integers(-140, 60))
        assert oracle.round_int_pow2_to_f32(n, s) == np.float32(math.ldexp(n, s))


def test_golden_a4_tie_example():
    g = _golden("a4_tie_k256.txt")
    v = np.array([float(t) for t in g["v"].split()])
    x = np.tile(v / 32.0, 32)[None, :]
    xb = _bf16(x)
    assert np.array_equal(datagen.bf16_bits_to_f32(xb)[0], x[0].astype(np.float32))
    r = oracle.rotate_quantize(xb, 0, 4)
    expect = np.zeros(256, dtype=np.int8)
    expect[:8] = [int(t) for t in g["codes_first8"].split()]
    assert r["b"] == 256
    assert np.array_equal(r["q"][0], expect)
    assert r["scale"][0] == np.float32(g["scale"])


def test_golden_a8_tie_example():
    g = _golden("a8_tie_k8.txt")
    x = np.array([float(t) for t in g["x"].split()])[None, :]
    xb = _bf16(x)
    assert np.array_equal(datagen.bf16_bits_to_f32(xb)[0], x[0].astype(np.float32))
    r = oracle.rotate_quantize(xb, 0, 8)
    assert np.array_equal(r["u32"][0], np.array([float(t) for t in g["u"].split()], dtype=np.float32))
    assert np.array_equal(r["q"][0], np.array([int(t) for t in g["codes"].split()], dtype=np.int8))
    assert r["scale"][0] == np.float32(2.0 * float(np.float32(1 / math.sqrt(8))))


@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("K", [256, 1408, 2560])
def test_quantizer_invariants(act_bits, K):
    Q = 7 if act_bits == 4 else 127
    xb = datagen.random_tokens(K + act_bits, 8, K)
    xb[3] = 0                                         # an all-zero token
    r = oracle.rotate_quantize(xb, 0, act_bits)
    q, s, u = r["q"].astype(np.int64), r["scale"].astype(np.float64), r["u32"].astype(np.float64)
    b = r["b"]
    nz = np.arange(8) != 3
    assert np.all(np.abs(q[nz]).max(axis=1) == Q)
    assert not q[3].any() and s[3] == 0
    # dequantised codes reproduce the rotated value to half a step (step = s*sqrt(b))
    step = s * math.sqrt(b)
    err = np.abs(u - q * step[:, None])
    assert np.all(err[nz] <= 0.5 * step[nz, None] * (1 + 2 ** -20))
    # step is max|u| / Q up to fp32 rounding
    M = np.abs(u).max(axis=1)
    assert np.allclose(step[nz], M[nz] / Q, rtol=1e-6)


def test_quantizer_one_hot_and_scale_invariance():
    K = 512
    x = np.zeros((1, K), dtype=np.float32)
    x[0, 17] = 3.0
    r = oracle.rotate_quantize(_bf16(x), 0, 4)
    assert np.all(np.abs(r["q"][0]) == 7)
    xb = datagen.random_tokens(11, 4, K)
    xf = datagen.bf16_bits_to_f32(xb)
    r1 = oracle.rotate_quantize(xb, 0, 8)
    r2 = oracle.rotate_quantize(_bf16(xf * np.float32(2.0 ** -5)), 0, 8)
    assert np.array_equal(r1["q"], r2["q"])
    assert np.array_equal(r2["scale"], (r1["scale"] * np.float32(2.0 ** -5)).astype(np.float32))


def test_code_packing_literals_and_round_trip():
    g = _golden("index_packing.txt")
    vals, byts = g["a4"].split("->")
    q = np.array([[int(t) for t in vals.split()]], dtype=np.int8)
    assert oracle.pack_codes(q, 4)[0].tolist() == [int(t, 16) for t in byts.split()]
    rng = np.random.default_rng(5)
    q4 = rng.integers(-8, 8, size=(3, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q4, 4), 64, 4), q4)
    q8 = rng.integers(-127, 128, size=(3, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q8, 8), 64, 8), q8)


# The rotation block of every layer width the workloads use: the largest power of two
# dividing K (a width with no Sylvester Hadamard matrix of its own is rotated in
# blocks of that size), and K itself for a power of two.  Values written out by hand.
@pytest.mark.parametrize("K, b", [(2560, 512), (9728, 512), (768, 256), (14336, 2048),
                                  (1408, 128), (256, 256), (2048, 2048), (4096, 4096),
                                  (96, 32), (32, 32)])
def test_block_size_literals(K, b):
    assert oracle.block_size(K) == b
    assert K % b == 0 and (K // b) % 2 == 1       # no larger power of two divides K


def test_block_size_override():
    assert oracle.block_size(2560, 1) == 1          # no rotation
    assert oracle.block_size(2560, 256) == 256
    assert oracle.block_size(2048, 2048) == 2048
    for bad in (3, 1024, 4096, -2):                 # not a power of two dividing K
        with pytest.raises(ValueError):
            oracle.block_size(2560, bad)
