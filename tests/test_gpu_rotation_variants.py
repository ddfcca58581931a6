"""GPU parity of rotate_quantize with smoothing multipliers and random signs
(cbq_rotate_quantize_ex): codes and scales bit-exact with the oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import DEV, bf16_dev, to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _smooth(seed, K):
    return np.exp2(np.random.default_rng(seed).uniform(-3, 3, K)).astype(np.float32)


def _signs(seed, K):
    return np.random.default_rng(seed + 1).integers(0, 256, K // 8, dtype=np.uint8)


@pytest.mark.parametrize("K", [256, 768, 1408, 2048, 4096, 14336])
@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("which", ["smooth", "signs", "both"])
def test_rotation_variants_bit_exact(K, act_bits, which):
    T = 5 if K > 8192 else 11
    xb = datagen.random_tokens(K + 3, T, K)
    xb[1] = 0                                              # an all-zero token
    m = _smooth(K, K) if which in ("smooth", "both") else None
    sg = _signs(K, K) if which in ("signs", "both") else None
    ref = oracle.rotate_quantize(xb, 0, act_bits, smooth=m, signs=sg)
    pre = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes, scales = cbq.rotate_quantize(bf16_dev(xb), act_bits, precond=pre,
                                        smooth=None if m is None else to_dev(m),
                                        signs=None if sg is None else to_dev(sg))
    torch.cuda.synchronize()
    # the counter reports exactly the (token, block) pairs outside the fp64 bound; the
    # codes are guaranteed (and compared) for the tokens inside it
    assert int(pre.item()) == int((~ref["ok"]).sum())
    inside = ref["ok"].all(axis=1)
    assert inside.any()
    assert np.array_equal(codes.cpu().numpy()[inside], ref["codes"][inside])
    assert np.array_equal(scales.cpu().numpy()[inside], ref["scale"][inside])


@pytest.mark.parametrize("had_block", [8, 64, 512])
def test_rotation_variants_explicit_blocks_and_stride(had_block):
    K, T = 1024, 6
    xb = datagen.random_tokens(88, T, K + 64)
    m, sg = _smooth(88, K), _signs(88, K)
    ref = oracle.rotate_quantize(np.ascontiguousarray(xb[:, :K]), had_block, 4, smooth=m, signs=sg)
    codes, scales = cbq.rotate_quantize(bf16_dev(xb)[:, :K], 4, had_block=had_block,
                                        smooth=to_dev(m), signs=to_dev(sg))
    inside = ref["ok"].all(axis=1)
    assert inside.any()
    assert np.array_equal(codes.cpu().numpy()[inside], ref["codes"][inside])
    assert np.array_equal(scales.cpu().numpy()[inside], ref["scale"][inside])


def test_smoothing_within_the_bound_everywhere():
    """Moderate multipliers on tokens without tiny channels: every block is inside the
    fp64 bound, so every code is compared."""
    K, T = 1408, 16
    g = np.random.default_rng(5)
    x = (np.sign(g.standard_normal((T, K))) * g.uniform(0.25, 4.0, (T, K))).astype(np.float32)
    xb = datagen.f32_to_bf16_bits(x)
    m = np.exp2(g.uniform(-1, 1, K)).astype(np.float32)
    ref = oracle.rotate_quantize(xb, 0, 4, smooth=m, signs=_signs(5, K))
    assert ref["ok"].all()
    codes, scales = cbq.rotate_quantize(bf16_dev(xb), 4, smooth=to_dev(m), signs=to_dev(_signs(5, K)))
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scale"])


def test_identity_variants_match_plain_call():
    K, T = 2048, 9
    xb = datagen.random_tokens(99, T, K)
    c0, s0 = cbq.rotate_quantize(bf16_dev(xb), 4)
    c1, s1 = cbq.rotate_quantize(bf16_dev(xb), 4, smooth=to_dev(np.ones(K, np.float32)),
                                 signs=to_dev(np.zeros(K // 8, np.uint8)))
    assert torch.equal(c0, c1) and torch.equal(s0, s1)
