"""GPU parity of the table forms of the codebook GEMM against the CPU oracle:
CBQ_PATH_PAGES_PRODUCTS (per-row tables of |a| * C[c] in LDS, sign applied after the
lookup) and CBQ_PATH_PAGES_BUCKETS (per-row integer buckets of the activation codes in
LDS, then sum_c C[c] * bucket[c]); 4-bit codebooks and A4 activations.

Every product is exact in both forms (|a| * C[c] in fp32; integer bucket sums times
C[c] in fp64), so the tolerances are those of the other paths: normwise 1e-3 for fp32
outputs, one bf16 step for SwiGLU outputs.  The shapes cover a K tail of 32 channels,
ragged column tiles, experts of 0 to 40 rows (the product form takes four tokens a pass,
the bucket form two), both index layouts, every code value -8..7 through an identity
weight matrix (exact), and bucket sums at the largest K with codes of one sign."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import (assert_bf16_close, assert_normwise, bf16_to_bits, to_dev,  # noqa: E402
                      upload_weights)

MODES = [cbq.PATH_PAGES_PRODUCTS, cbq.PATH_PAGES_BUCKETS]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def _device_weights(ws, layout):
    W = upload_weights(ws)
    return cbq.prepack_weights(W) if layout == "blocked" else W


@pytest.mark.parametrize("path", MODES)
@pytest.mark.parametrize("layout", ["rows", "blocked"])
@pytest.mark.parametrize("T,N,K", [(1, 256, 256), (3, 80, 160), (4, 48, 1408), (5, 144, 2048),
                                   (13, 208, 800)])
def test_pages_dense(path, layout, T, N, K):
    ws = datagen.random_weights(500 + T + N, 1, N, K, 4)
    rq = oracle.rotate_quantize(datagen.random_tokens(600 + T + K, T, K), 0, 4)
    ref = oracle.expert_gemm(rq["q"], rq["scale"], None, None, ws.idx, ws.codebook, K, 4)
    y = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), 4,
                              [_device_weights(ws, layout)], path=path)
    assert_normwise(y.cpu().numpy(), ref, 1e-3, f"path {path} {layout} T={T} N={N} K={K}")


@pytest.mark.parametrize("path", MODES)
def test_pages_identity_every_code(path):
    """W = I (index 1 on the diagonal, C[1] = 1, C[0] = 0): y = scale * q exactly, for
    codes that take every value -8..7 in every position class, so each magnitude row of
    the product table, the sign folding and each bucket are checked bit for bit."""
    K = N = 256
    T = 9
    raw = np.eye(N, K, dtype=np.uint8)[None]
    cbv = np.zeros((N, 16), dtype=np.float32)
    cbv[:, 1] = 1.0
    ws = datagen.WeightSet(1, N, K, 4, datagen.pack_lsb_first(raw, 4), datagen.f32_to_f16_bits(cbv)[None])
    q = ((np.arange(T)[:, None] * 7 + np.arange(K)[None, :] * 3) % 16 - 8).astype(np.int64)
    codes = datagen.pack_lsb_first((q & 15).astype(np.uint8), 4)
    assert np.array_equal(oracle.unpack_codes(codes, K, 4), q)
    scale = (0.25 * (np.arange(T) + 1)).astype(np.float32)
    expect = q.astype(np.float32) * scale[:, None]
    for layout in ("rows", "blocked"):
        y = cbq.codebook_lut_gemm(to_dev(codes), to_dev(scale), 4, [_device_weights(ws, layout)], path=path)
        assert np.array_equal(y.cpu().numpy(), expect), layout


@pytest.mark.parametrize("path", MODES)
def test_pages_large_sums_exact(path):
    """K = 16384 with every weight on one centroid and constant codes -8, 7, -8: each
    lane's bucket takes its largest sums of either sign (the packed pair of tokens must
    split exactly, the negative first token borrowing from the second); y is exact."""
    N, K, T = 32, 16384, 3
    raw = np.full((1, N, K), 5, dtype=np.uint8)
    rng = np.random.default_rng(17)
    cbv = rng.standard_normal((N, 16)).astype(np.float32) * 0.02
    cbv[:, 5] = 0.5
    ws = datagen.WeightSet(1, N, K, 4, datagen.pack_lsb_first(raw, 4), datagen.f32_to_f16_bits(cbv)[None])
    q = np.array([-8, 7, -8], dtype=np.int64)[:, None] * np.ones((1, K), dtype=np.int64)
    codes = datagen.pack_lsb_first((q & 15).astype(np.uint8), 4)
    scale = np.array([1.0, 0.5, 0.25], dtype=np.float32)
    expect = (q.sum(axis=1) * 0.5 * scale)[:, None] * np.ones((1, N), dtype=np.float32)
    y = cbq.codebook_lut_gemm(to_dev(codes), to_dev(scale), 4, [_device_weights(ws, "blocked")], path=path)
    assert np.array_equal(y.cpu().numpy(), expect.astype(np.float32))


@pytest.mark.parametrize("path", MODES)
@pytest.mark.parametrize("T,E,k,S", [(6, 8, 2, 0), (40, 8, 2, 1), (96, 16, 4, 0)])
def test_pages_grouped_swiglu_and_down(path, T, E, k, S):
    H, F = 256, 192
    wl = datagen.Workload("t", 2500 + T + E, "moe", 4, H=H, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=4, bits_down=4)
    gate, up, down = datagen.moe_weights(wl)
    x, lg = datagen.moe_tokens(wl, T)
    rq = oracle.rotate_quantize(x, 0, 4)
    rt = oracle.route(lg, k, True, S)
    if T >= 40:
        assert np.diff(rt["offsets"]).max() > 4   # some expert needs several token passes
    G, U, D = upload_weights(gate), upload_weights(up), upload_weights(down)
    offs, toks = to_dev(rt["offsets"]), to_dev(rt["sorted_tokens"])
    h = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), 4, [G, U],
                              expert_offsets=offs, row_token=toks, path=path)
    g = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], gate.idx,
                           gate.codebook, H, 4)
    u = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], up.idx,
                           up.codebook, H, 4)
    assert_bf16_close(bf16_to_bits(h), oracle.silu_mul_bf16(g, u), "swiglu")
    hb = bf16_to_bits(h)
    rqh = oracle.rotate_quantize(hb, 0, 4)
    ch, sh = cbq.rotate_quantize(h, 4)
    out = cbq.codebook_lut_gemm(ch, sh, 4, [D], expert_offsets=offs, path=path)
    ref = oracle.expert_gemm(rqh["q"], rqh["scale"], None, rt["offsets"], down.idx, down.codebook, F, 4)
    assert_normwise(out.cpu().numpy(), ref, 1e-3, "down")


@pytest.mark.parametrize("path", MODES)
def test_pages_match_lut_path(path):
    """The same rows through a table form and the register-table LUT path: equal
    products, another fp32 summation order, so bf16 h is equal or one step apart."""
    T, E, k, S, H, F = 24, 16, 4, 1, 512, 320
    wl = datagen.Workload("t", 2700, "moe", 4, H=H, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=4, bits_down=4)
    gate, up, _ = datagen.moe_weights(wl)
    x, lg = datagen.moe_tokens(wl, T)
    rq = oracle.rotate_quantize(x, 0, 4)
    rt = oracle.route(lg, k, True, S)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), 4, [upload_weights(gate), upload_weights(up)])
    kw = dict(expert_offsets=to_dev(rt["offsets"]), row_token=to_dev(rt["sorted_tokens"]))
    a = bf16_to_bits(cbq.codebook_lut_gemm(*args, path=path, **kw)).astype(np.int32)
    b = bf16_to_bits(cbq.codebook_lut_gemm(*args, path=cbq.PATH_LUT, **kw)).astype(np.int32)
    same_sign = (a ^ b) & 0x8000 == 0
    step = np.where(same_sign, np.abs(a - b), np.abs((a & 0x7FFF) + (b & 0x7FFF)))
    assert step.max() <= 1
