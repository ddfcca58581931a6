"""GPU parity of each library call against the CPU oracle on small seeded inputs.

Sizes are chosen so the oracle finishes in seconds while the kernels still cover
several tiles, ragged tails (rows, columns, a K tail of 32), empty experts and the
degenerate cases (zero tokens, all-zero tokens, one expert)."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import (DEV, assert_bf16_close, assert_normwise, bf16_dev, bf16_to_bits, to_dev,  # noqa: E402
                      upload_weights)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


# ---------------------------------------------------------------------------
# rotate_quantize: codes and scales bit-exact
@pytest.mark.parametrize("K", [256, 768, 1408, 2048, 2560, 4096, 9728, 14336])
@pytest.mark.parametrize("act_bits", [4, 8])
def test_rotate_quantize_bit_exact(K, act_bits):
    T = 5 if K > 8192 else 13
    xb = datagen.random_tokens(K + act_bits, T, K)
    xb[2] = 0                                              # an all-zero token
    ref = oracle.rotate_quantize(xb, 0, act_bits)
    assert ref["ok"].all()
    x = bf16_dev(xb)
    pre = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes, scales = cbq.rotate_quantize(x, act_bits, precond=pre)
    torch.cuda.synchronize()
    assert int(pre.item()) == 0
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scale"])


@pytest.mark.parametrize("had_block", [1, 8, 64, 512])
def test_rotate_quantize_explicit_blocks_and_stride(had_block):
    K, T = 1024, 6
    xb = datagen.random_tokens(77, T, K + 64)              # ldx = K + 64
    ref = oracle.rotate_quantize(np.ascontiguousarray(xb[:, :K]), had_block, 4)
    x = bf16_dev(xb)[:, :K]
    codes, scales = cbq.rotate_quantize(x, 4, had_block=had_block)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scale"])


@pytest.mark.parametrize("K,had_block,act_bits", [(1056, 0, 4), (1088, 0, 8), (1408, 0, 4), (1536, 0, 8),
                                                   (1984, 0, 4), (1408, 8, 8), (1408, 32, 4)])
def test_rotate_quantize_packed_tokens(K, had_block, act_bits):
    # K/32 lanes per token, not a power of two: tokens packed back to back, some of
    # them straddling two waves; 50 tokens fill two workgroups and part of a third
    T = 50
    xb = datagen.random_tokens(K + 3 * act_bits, T, K + 32)  # ldx = K + 32
    xb[7] = 0                                                # an all-zero token
    ref = oracle.rotate_quantize(np.ascontiguousarray(xb[:, :K]), had_block, act_bits)
    x = bf16_dev(xb)[:, :K]
    codes, scales = cbq.rotate_quantize(x, act_bits, had_block=had_block)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scale"])


def test_rotate_quantize_golden_tie_example():
    v = np.array([1.5, 1.625, 1.125, 0, 0.375, 0.25, 1.75, 0.375])
    x = datagen.f32_to_bf16_bits(np.tile(v / 32.0, 32)[None, :].astype(np.float32))
    codes, scales = cbq.rotate_quantize(bf16_dev(x), 4)
    q = oracle.unpack_codes(codes.cpu().numpy(), 256, 4)[0]
    assert q[:8].tolist() == [7, 2, 0, -2, 2, 0, 4, 0] and not q[8:].any()
    assert float(scales.item()) == 0.0625


def test_rotate_quantize_precondition_counter():
    K, b = 256, 256
    x = np.zeros((3, K), dtype=np.float32)
    x[:, 0] = 1.0
    x[1, 1] = 2.0 ** -60          # spread 60 > 45 - 8
    x[2, 5] = 2.0 ** -30          # spread 30: fine
    pre = torch.zeros(1, dtype=torch.int32, device=DEV)
    cbq.rotate_quantize(bf16_dev(datagen.f32_to_bf16_bits(x)), 4, precond=pre)
    torch.cuda.synchronize()
    ok = oracle.rotation_precondition(x.astype(np.float64).reshape(3, 1, b), b)
    assert int(pre.item()) == int((~ok).sum()) == 1


def test_rotate_quantize_empty():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    codes, scales = cbq.rotate_quantize(x, 4)
    assert codes.shape == (0, 128)


# ---------------------------------------------------------------------------
# routing: integer outputs bit-exact, weights within 1e-6
@pytest.mark.parametrize("T,E,k,S,renorm", [(1, 128, 8, 0, True), (64, 128, 8, 0, True),
                                            (512, 8, 2, 0, True), (37, 64, 6, 2, True),
                                            (4096, 64, 6, 2, True), (300, 256, 8, 1, False),
                                            (2500, 16, 1, 0, True), (5, 4, 4, 0, False),
                                            (3000, 1, 1, 0, True), (65536, 64, 6, 2, True)])
def test_route_bit_exact(T, E, k, S, renorm):
    lg = datagen.random_logits(T + E + k, T, E)
    lg[0, :min(E, 6)] = np.float32(1.25)                 # a tie
    ref = oracle.route(lg, k, renorm, S)
    r = cbq.moe_route_gather(to_dev(lg), k, renorm, S)
    torch.cuda.synchronize()
    assert np.array_equal(r["ids"].cpu().numpy(), ref["ids"])
    assert np.array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(r["sorted_tokens"].cpu().numpy(), ref["sorted_tokens"])
    assert np.array_equal(r["slot_of"].cpu().numpy(), ref["slot_of"])
    assert np.abs(r["weights"].cpu().numpy().astype(np.float64) - ref["weights64"]).max() <= 1e-6


@pytest.mark.parametrize("E,k,S", [(8, 2, 1), (256, 8, 2)])
def test_route_zero_tokens(E, k, S):
    r = cbq.moe_route_gather(torch.empty((0, E), dtype=torch.float32, device=DEV), k, True, S)
    assert r["offsets"].cpu().tolist() == [0] * (E + S + 1)


# ---------------------------------------------------------------------------
# GEMM
def _dense_case(seed, T, N, K, bits, act_bits):
    ws = datagen.random_weights(seed, 1, N, K, bits)
    xb = datagen.random_tokens(seed + 1, T, K)
    rq = oracle.rotate_quantize(xb, 0, act_bits)
    ref = oracle.expert_gemm(rq["q"], rq["scale"], None, None, ws.idx, ws.codebook, K, bits)
    return ws, rq, ref


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("path", [cbq.PATH_LUT, cbq.PATH_MFMA])
@pytest.mark.parametrize("T,N,K", [(4, 256, 256), (13, 80, 160), (1, 48, 1408), (40, 144, 800),
                                   (150, 208, 544)])
def test_dense_gemm(bits, act_bits, path, T, N, K):
    ws, rq, ref = _dense_case(100 * bits + act_bits + T, T, N, K, bits, act_bits)
    W = upload_weights(ws)
    y = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [W], path=path)
    assert_normwise(y.cpu().numpy(), ref, 1e-3, f"dense bits={bits} a={act_bits} path={path}")


def test_dense_gemm_identity_codebook():
    """W = I through the kernels: y = scale * q exactly (checks operand layouts)."""
    K = N = 256
    raw = np.eye(N, K, dtype=np.uint8)[None]
    idx = datagen.pack_lsb_first(raw, 4)
    cb = datagen.f32_to_f16_bits(np.tile(np.arange(16, dtype=np.float32), (N, 1)))[None]
    ws = datagen.WeightSet(1, N, K, 4, idx, cb)
    rq = oracle.rotate_quantize(datagen.random_tokens(5, 20, K), 0, 4)
    expect = rq["q"].astype(np.float32) * rq["scale"][:, None]
    for path in (cbq.PATH_LUT, cbq.PATH_MFMA):
        y = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), 4, [upload_weights(ws)], path=path)
        assert np.array_equal(y.cpu().numpy(), expect), path


def _moe_case(seed, T, E, k, S, H, F, bits, act_bits):
    wl = datagen.Workload("t", 2000 + seed, "moe", act_bits, H=H, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=bits, bits_down=bits)
    gate, up, down = datagen.moe_weights(wl)
    x, lg = datagen.moe_tokens(wl, T)
    return wl, gate, up, down, x, lg


@pytest.mark.parametrize("path", [cbq.PATH_AUTO, cbq.PATH_LUT, cbq.PATH_MFMA])
@pytest.mark.parametrize("bits,act_bits", [(4, 4), (3, 4), (2, 8)])
@pytest.mark.parametrize("T,E,k,S", [(6, 8, 2, 0), (96, 8, 2, 1), (300, 4, 2, 0)])
def test_grouped_swiglu_and_down(path, bits, act_bits, T, E, k, S):
    H, F = 256, 192
    wl, gate, up, down, x, lg = _moe_case(T + E + bits, T, E, k, S, H, F, bits, act_bits)
    rq = oracle.rotate_quantize(x, 0, act_bits)
    rt = oracle.route(lg, k, True, S)
    G, U, D = upload_weights(gate), upload_weights(up), upload_weights(down)
    offs, toks = to_dev(rt["offsets"]), to_dev(rt["sorted_tokens"])
    h = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [G, U],
                              expert_offsets=offs, row_token=toks, path=path)
    g = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], gate.idx,
                           gate.codebook, H, bits)
    u = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], up.idx,
                           up.codebook, H, bits)
    assert_bf16_close(bf16_to_bits(h), oracle.silu_mul_bf16(g, u), "swiglu")
    # down projection, teacher-forced on the GPU's own h
    hb = bf16_to_bits(h)
    rqh = oracle.rotate_quantize(hb, 0, act_bits)
    ch, sh = cbq.rotate_quantize(h, act_bits)
    assert np.array_equal(ch.cpu().numpy(), rqh["codes"])
    out = cbq.codebook_lut_gemm(ch, sh, act_bits, [D], expert_offsets=offs, path=path)
    ref = oracle.expert_gemm(rqh["q"], rqh["scale"], None, rt["offsets"], down.idx, down.codebook, F, bits)
    assert_normwise(out.cpu().numpy(), ref, 1e-3, "down")


@pytest.mark.parametrize("bits,act_bits,n_w", [(3, 4, 2), (4, 8, 2), (2, 4, 1), (3, 8, 1), (4, 4, 1)])
@pytest.mark.parametrize("path", [cbq.PATH_AUTO, cbq.PATH_LUT])
def test_many_tile_decode_gemm(bits, act_bits, n_w, path):
    # 64 experts x 2080 rows: enough 16-row tiles that no wave splits K (the decode
    # layout of the large MoE layers); K = 160 leaves a 32-channel chunk tail, N = 2080
    # leaves part of the last two-group wave empty, and the row counts include
    # empty experts, full 32-row blocks and one expert of 40 rows (two row blocks when
    # forced onto the LUT path; AUTO sends it to the MFMA path)
    E, N, K, T = 64, 2080, 160, 50
    rng = np.random.default_rng(bits * 10 + act_bits + n_w)
    counts = rng.integers(0, 6, E)
    counts[[3, 17, 40]] = 0
    counts[5], counts[9], counts[63] = 32, 16, 40
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    row_token = rng.integers(0, T, R).astype(np.int32)
    xb = datagen.random_tokens(300 + bits, T, K)
    rq = oracle.rotate_quantize(xb, 0, act_bits)
    ws = [datagen.random_weights(40 + bits + m, E, N, K, bits, keep_raw=False) for m in range(n_w)]
    Wd = [upload_weights(w) for w in ws]
    out = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, Wd,
                                expert_offsets=to_dev(offsets), row_token=to_dev(row_token), path=path)
    ref = [oracle.expert_gemm(rq["q"], rq["scale"], row_token, offsets, w.idx, w.codebook, K, bits)
           for w in ws]
    if n_w == 2:
        assert_bf16_close(bf16_to_bits(out), oracle.silu_mul_bf16(ref[0], ref[1]), "swiglu")
    else:
        assert_normwise(out.cpu().numpy(), ref[0], 1e-3, "f32")


def test_gemm_deterministic():
    wl, gate, up, down, x, lg = _moe_case(7, 200, 8, 2, 1, 256, 192, 4, 4)
    rq = oracle.rotate_quantize(x, 0, 4)
    rt = oracle.route(lg, 2, True, 1)
    G, U = upload_weights(gate), upload_weights(up)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), 4, [G, U])
    kw = dict(expert_offsets=to_dev(rt["offsets"]), row_token=to_dev(rt["sorted_tokens"]))
    a = cbq.codebook_lut_gemm(*args, **kw).cpu()
    b = cbq.codebook_lut_gemm(*args, **kw).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# combine
@pytest.mark.parametrize("T,k,S,H", [(1, 8, 0, 2048), (37, 6, 2, 2048), (512, 2, 0, 4096), (9, 3, 1, 12)])
def test_combine(T, k, S, H):
    rng = np.random.default_rng(T * k + H)
    R = T * k + S * T
    out = rng.standard_normal((R, H)).astype(np.float32)
    lg = datagen.random_logits(T + 3, T, max(k, 8))
    rt = oracle.route(lg, k, True, 0)
    slot = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    ref = oracle.combine(out, slot, rt["weights"], T, k, S)
    y = cbq.moe_combine(to_dev(out), to_dev(slot), to_dev(rt["weights"]), S)
    assert_normwise(y.cpu().numpy(), ref, 1e-5, "combine")
