"""The host codebook-LUT GEMM (cbq_cpu_lut_gemm) against the oracle, on this machine's
CPU: all index widths and activation widths, token counts across the 8-token register
block, several thread counts (the result must not depend on them), and the
2560 -> 9728 decode linear of the dense workload."""
import numpy as np
import pytest

import datagen
import oracle

cbq = pytest.importorskip("codebook_bit_quantized_amd")


def _have_lib():
    try:
        cbq.load_library()
        return True
    except ImportError:
        return False


pytestmark = pytest.mark.skipif(not _have_lib(), reason="libcbq.so not built")


def _case(seed, T, N, K, bits, act_bits):
    ws = datagen.random_weights(seed, 1, N, K, bits, keep_raw=True)
    x = datagen.random_tokens(seed, T, K)
    rq = oracle.rotate_quantize(x, 0, act_bits)
    ref = oracle.dense_gemm(rq["q"].astype(np.int64), rq["scale"],
                            oracle.dequantize(ws.raw[0].astype(np.int64), ws.codebook[0]))
    return ws, rq, ref


def _normwise(y, ref):
    return float(np.abs(y - ref).max() / np.abs(ref).max())


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("T", [1, 5, 8, 19])
@pytest.mark.parametrize("avx512", [False, True])
def test_cpu_lut_matches_oracle(bits, act_bits, T, avx512):
    ws, rq, ref = _case(100 + bits * 10 + T, T, 80, 288, bits, act_bits)
    y = cbq.cpu_lut_gemm(rq["codes"], rq["scale"], act_bits, ws.idx, ws.codebook, ws.K, bits,
                         avx512=avx512)
    assert _normwise(y, ref) <= 1e-3


def test_cpu_lut_thread_count_does_not_change_the_result():
    ws, rq, _ = _case(7, 6, 192, 512, 3, 4)
    ys = [cbq.cpu_lut_gemm(rq["codes"], rq["scale"], 4, ws.idx, ws.codebook, ws.K, 3, n_threads=n)
          for n in (1, 3, 0)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_cpu_lut_identity_codebook_layout():
    """Codebook {0, 1} per row with idx[n][k] = 1 iff k == n: y = scale * q (checks the
    index unpacking and the lane order of the lookups)."""
    N = K = 64
    for bits in (2, 3, 4):
        raw = np.eye(N, K, dtype=np.uint8)
        idx = datagen.pack_lsb_first(raw, bits)
        cb = np.zeros((N, 1 << bits), dtype=np.uint16)
        cb[:, 1] = 0x3C00                                   # fp16 1.0
        x = datagen.random_tokens(3, 4, K)
        rq = oracle.rotate_quantize(x, 0, 4)
        for avx512 in (False, True):
            y = cbq.cpu_lut_gemm(rq["codes"], rq["scale"], 4, idx, cb, K, bits, avx512=avx512)
            assert np.array_equal(y, (rq["q"].astype(np.float32) * rq["scale"][:, None]).astype(np.float32))


def test_cpu_lut_dense_decode_linear():
    wl = datagen.WORKLOADS["dense2560x9728"]
    ws = datagen.dense_weights(wl, "gate_up")
    x = datagen.dense_tokens(wl, 4)
    rq = oracle.rotate_quantize(x, 0, 4)
    W = oracle.dequantize(oracle.unpack_indices(ws.idx[0], ws.K, ws.bits), ws.codebook[0])
    ref = oracle.dense_gemm(rq["q"].astype(np.int64), rq["scale"], W)
    y = cbq.cpu_lut_gemm(rq["codes"], rq["scale"], 4, ws.idx, ws.codebook, ws.K, ws.bits)
    assert _normwise(y, ref) <= 1e-3


def test_cpu_lut_validation():
    import ctypes
    lib = cbq.load_library()
    w = cbq.cbq_weights(0x1000, 0x2000, 2, 64, 256, 4)       # E = 2: one weight set only
    assert lib.cbq_cpu_lut_gemm(None, None, 4, 4, ctypes.byref(w), None, 64, 0, 0) == cbq.CBQ_EUNSUPPORTED
    w = cbq.cbq_weights(0x1000, 0x2000, 1, 64, 256, 4)
    assert lib.cbq_cpu_lut_gemm(None, None, 4, 0, ctypes.byref(w), None, 64, 0, 0) == cbq.CBQ_OK
    assert lib.cbq_cpu_lut_gemm(None, None, 4, 4, ctypes.byref(w), None, 64, 0, 0) == cbq.CBQ_EINVAL
    assert lib.cbq_cpu_lut_gemm(None, None, 6, 4, ctypes.byref(w), None, 64, 0, 0) == cbq.CBQ_EINVAL
    assert lib.cbq_cpu_lut_gemm(None, None, 4, 0, ctypes.byref(w), None, 64, 0, 2) == cbq.CBQ_EINVAL
