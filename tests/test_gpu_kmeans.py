"""GPU parity of offline codebook construction (cbq_kmeans_codebooks) with the oracle:
indices, fp16 codebooks and update counts bit-exact, on seeded synthetic weight rows
(N(0, 0.02) with one entry in 256 scaled by 8)."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import DEV, assert_normwise, to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _run(w_bits, bits, max_iters, ldw=None):
    R, K = w_bits.shape
    if ldw is not None:
        padded = np.zeros((R, ldw), dtype=np.uint16)
        padded[:, :K] = w_bits
        w = to_dev(padded.view(np.int16))[:, :K]
    else:
        w = to_dev(w_bits.view(np.int16))
    it = torch.empty((R,), dtype=torch.int32, device=DEV)
    cw = cbq.kmeans_codebooks(w, bits, max_iters, iters_done=it)
    torch.cuda.synchronize()
    return (cw.idx[0].cpu().numpy(), cw.codebook[0].cpu().numpy().view(np.uint16),
            it.cpu().numpy(), cw)


def _check(w_bits, bits, max_iters, ldw=None):
    idx, cb, it, cw = _run(w_bits, bits, max_iters, ldw)
    ref_idx, ref_cb, ref_it = oracle.kmeans_codebooks(w_bits, bits, max_iters)
    assert np.array_equal(cb, ref_cb), "codebooks"
    assert np.array_equal(it, ref_it), "update counts"
    assert np.array_equal(idx, datagen.pack_lsb_first(ref_idx.astype(np.uint8), bits)), "indices"
    return cw


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("K", [64, 256, 1408, 2048])
def test_kmeans_bit_exact(bits, K):
    R = 24 if K >= 1408 else 40
    w = datagen.weights_bf16(10 + bits, datagen.TAG_W_FULL, K, R, K)
    _check(w, bits, 50)


@pytest.mark.parametrize("max_iters", [0, 1, 3])
def test_kmeans_iteration_cap(max_iters):
    w = datagen.weights_bf16(20, datagen.TAG_W_FULL, max_iters, 16, 512)
    _check(w, 4, max_iters)


def test_kmeans_long_rows_and_stride():
    w = datagen.weights_bf16(21, datagen.TAG_W_FULL, 0, 3, 14336)
    _check(w, 4, 20)
    w = datagen.weights_bf16(22, datagen.TAG_W_FULL, 0, 9, 96)
    _check(w, 3, 30, ldw=160)


def test_kmeans_golden_row_and_degenerate_rows():
    vals = [12, 0, 21, 11, 2, 20, 1, 10] * 4                     # the worked example, K = 32
    rows = [vals, [0.0] * 32, [1.5] * 31 + [-1.5], [-0.0] * 16 + [0.0] * 16, [-0.0] * 32]
    w = datagen.f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    _check(w, 2, 10)
    idx, cb, it, _ = _run(w[:1], 2, 10)
    assert [int(c) for c in cb[0]] == [0x3C00, 0x4940, 0x4A00, 0x4D20]


def test_kmeans_empty():
    w = torch.empty((0, 64), dtype=torch.int16, device=DEV)
    cw = cbq.kmeans_codebooks(w, 2, 10)
    assert cw.idx.shape == (1, 0, 16)


def test_kmeans_output_feeds_the_gemm():
    """Codebooks built on the GPU drive the LUT GEMM; the result matches the oracle's
    dequantise-then-matmul of the oracle's own codebooks."""
    N, K, T = 64, 512, 6
    w = datagen.weights_bf16(23, datagen.TAG_W_FULL, 0, N, K)
    cw = _check(w, 3, 40)
    x = datagen.random_tokens(23, T, K)
    rq = oracle.rotate_quantize(x, 0, 4)
    ref_idx, ref_cb, _ = oracle.kmeans_codebooks(w, 3, 40)
    ref = oracle.dense_gemm(rq["q"].astype(np.int64), rq["scale"],
                            oracle.dequantize(ref_idx, ref_cb))
    codes, scales = cbq.rotate_quantize(to_dev(x.view(np.int16)).view(torch.bfloat16), 4)
    y = cbq.codebook_lut_gemm(codes, scales, 4, [cw])
    torch.cuda.synchronize()
    assert_normwise(y.cpu().numpy(), ref, 1e-3, "gemm on built codebooks")
