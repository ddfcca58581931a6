"""GPU parity of cbq_rotate_quantize_dense (a dense K x K rotation standing for a learned
one, CodeQuant2 Figure 1) against the oracle: codes and scales bit-exact for every token
inside the exactness bound, the violation counter equal to the oracle's count."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import DEV, bf16_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _run(xb, Rb, K, act_bits):
    x = bf16_dev(xb)[:, :K]
    R = bf16_dev(Rb)
    pre = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes, scales = cbq.rotate_quantize_dense(x, R, act_bits, precond=pre)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), int(pre.item())


@pytest.mark.parametrize("T,K,act_bits,pad", [(1, 64, 4, 0), (37, 256, 8, 64), (100, 1024, 4, 0),
                                              (130, 1408, 8, 0), (17, 2048, 4, 32)])
def test_dense_rotation_parity(T, K, act_bits, pad):
    xb = datagen.random_tokens(K + T, T, K + pad)          # ldx = K + pad
    xb[T // 2] = 0                                         # an all-zero token
    Rb = datagen.rotation_bf16(K, K)
    xs = np.ascontiguousarray(xb[:, :K])
    ref = oracle.rotate_quantize_dense(xs, Rb, act_bits)
    codes, scales, viol = _run(xb, Rb, K, act_bits)
    ok = ref["ok"]
    assert ok.mean() > 0.8
    assert np.array_equal(codes[ok], ref["codes"][ok])
    assert np.array_equal(scales[ok], ref["scale"][ok])
    assert viol == int((~ok).sum())
    assert scales[T // 2] == 0 and not codes[T // 2].any()


def test_dense_rotation_counter_flags_a_wide_token():
    K, T = 128, 6
    xb = datagen.random_tokens(91, T, K)
    xf = datagen.bf16_bits_to_f32(xb)
    xf[2, 9] = 2.0 ** -40                                  # token 2: spread beyond the bound
    xb = datagen.f32_to_bf16_bits(xf)
    Rb = datagen.rotation_bf16(92, K)
    ref = oracle.rotate_quantize_dense(xb, Rb, 4)
    assert list(~ref["ok"]) == [False, False, True, False, False, False]
    codes, scales, viol = _run(xb, Rb, K, 4)
    assert viol == 1
    ok = ref["ok"]
    assert np.array_equal(codes[ok], ref["codes"][ok])


def test_dense_hadamard_matches_block_path():
    # R = H_256 / 16 (entries +-1/16, exact in bf16) gives the block rotation with b = 256
    K, T = 256, 40
    xb = datagen.random_tokens(93, T, K)
    R = oracle.sylvester_hadamard(256).astype(np.float32) / 16.0
    Rb = datagen.f32_to_bf16_bits(R)
    codes, scales, _ = _run(xb, Rb, K, 4)
    c2, s2 = cbq.rotate_quantize(bf16_dev(xb), 4, had_block=256)
    assert np.array_equal(codes, c2.cpu().numpy())
    assert np.array_equal(scales, s2.cpu().numpy())


def test_dense_rotation_full_size_sampled():
    # 4096 tokens x 2048 channels, the layer input of the 64-expert workload; the oracle
    # checks a sample of tokens inside the bound
    K, T = 2048, 4096
    xb = datagen.random_tokens(94, T, K)
    Rb = datagen.rotation_bf16(95, K)
    codes, scales, viol = _run(xb, Rb, K, 4)
    rng = np.random.default_rng(3)
    sample = np.sort(rng.choice(T, 48, replace=False))
    sample = sample[oracle.dense_rotation_precondition(xb[sample], Rb)]
    ref = oracle.rotate_quantize_dense(xb[sample], Rb, 4)
    assert len(sample) > 30
    assert np.array_equal(codes[sample], ref["codes"])
    assert np.array_equal(scales[sample], ref["scale"])
    ok_all = oracle.dense_rotation_precondition(xb, Rb)
    assert viol == int((~ok_all).sum())


def test_dense_rotation_empty_and_workspace():
    K = 256
    R = bf16_dev(datagen.rotation_bf16(96, K))
    x = bf16_dev(datagen.random_tokens(97, 0, K))
    codes, scales = cbq.rotate_quantize_dense(x, R, 4)
    assert codes.shape == (0, K // 2) and scales.shape == (0,)
    assert cbq.rotate_dense_workspace(10, K) == 10 * K * 4 + 256
    x = bf16_dev(datagen.random_tokens(98, 10, K))
    small = torch.empty(100, dtype=torch.uint8, device=DEV)
    with pytest.raises(cbq.CbqError):
        cbq.rotate_quantize_dense(x, R, 4, ws=small)
