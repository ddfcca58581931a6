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
                                                   (1984, 0, 4), (1408, 8, 8), (1408, 32, 4),
                                                   (1280, 0, 8), (1536, 256, 4), (1536, 64, 8)])
def test_rotate_quantize_packed_tokens(K, had_block, act_bits):
    # K/32 lanes per token, not a power of two: tokens packed back to back in 512-lane
    # workgroups (8 to 15 tokens each), some of them straddling two waves; 50 tokens fill
    # several workgroups and part of another
    T = 50
    xb = datagen.random_tokens(K + 3 * act_bits, T, K + 32)  # ldx = K + 32
    xb[7] = 0                                                # an all-zero token
    ref = oracle.rotate_quantize(np.ascontiguousarray(xb[:, :K]), had_block, act_bits)
    x = bf16_dev(xb)[:, :K]
    codes, scales = cbq.rotate_quantize(x, act_bits, had_block=had_block)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scale"])


@pytest.mark.parametrize("K,had_block,act_bits,T", [(1408, 0, 4, 9000), (1280, 0, 8, 9601),
                                                     (1088, 0, 4, 12001), (2048, 0, 4, 6200),
                                                     (2560, 0, 8, 4801), (768, 0, 4, 17000),
                                                     (512, 0, 8, 24700), (2048, 1024, 4, 6199),
                                                     (14336, 0, 8, 1700), (9728, 0, 4, 2500)])
def test_rotate_quantize_packed_tokens_looping(K, had_block, act_bits, T):
    # enough token groups that each workgroup of the packed kernel loops over several
    # (three workgroups per CU), loading the next group while working on the current one
    # and rotating its absmax sets; T leaves the last group ragged.  Blocks of 32 to 2048
    # channels: half-swap stages only (b <= 128) or after one to four DPP stages; K = 14336
    # takes workgroups of 448 lanes (one token each), K = 9728 the general kernel
    xb = datagen.random_tokens(K + T, T, K)
    xb[T // 3] = 0
    xb[-1] = 0
    ref = oracle.rotate_quantize(xb, had_block, act_bits)
    codes, scales = cbq.rotate_quantize(bf16_dev(xb), act_bits, had_block=had_block)
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


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("path", [cbq.PATH_LUT, cbq.PATH_MFMA])
@pytest.mark.parametrize("tables", [cbq.PATH_REG_TABLES, cbq.PATH_LDS_TABLES])
@pytest.mark.parametrize("T,N,K", [(4, 256, 256), (40, 144, 800), (150, 208, 544)])
def test_dense_gemm_table_placements(bits, act_bits, path, tables, T, N, K):
    """2- and 3-bit codebooks through either table placement on either path (register
    tables or LDS pair tables): the same products, another summation order."""
    ws, rq, ref = _dense_case(200 * bits + act_bits + T, T, N, K, bits, act_bits)
    W = upload_weights(ws)
    y = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [W],
                              path=path | tables)
    assert_normwise(y.cpu().numpy(), ref, 1e-3, f"tables {tables} bits={bits} a={act_bits} path={path}")


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


@pytest.mark.parametrize("bits", [2, 3])
def test_pair_table_identity_codebook(bits):
    """W = I with a 2- or 3-bit codebook {0, 1, 0, ...} through the LDS pair tables: every
    output is scale * q exactly, so each table entry, its row and the pair order of the
    lookups line up with the activation fragments (checks layouts bit for bit)."""
    K = N = 256
    raw = np.eye(N, K, dtype=np.uint8)[None]
    idx = datagen.pack_lsb_first(raw, bits)
    cbv = np.zeros((N, 1 << bits), dtype=np.float32)
    cbv[:, 1] = 1.0
    ws = datagen.WeightSet(1, N, K, bits, idx, datagen.f32_to_f16_bits(cbv)[None])
    for act_bits in (4, 8):
        rq = oracle.rotate_quantize(datagen.random_tokens(6 + act_bits, 70, K), 0, act_bits)
        expect = rq["q"].astype(np.float32) * rq["scale"][:, None]
        for path in (cbq.PATH_LUT, cbq.PATH_MFMA):
            y = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits,
                                      [upload_weights(ws)], path=path | cbq.PATH_LDS_TABLES)
            assert np.array_equal(y.cpu().numpy(), expect), (act_bits, path)


def _moe_case(seed, T, E, k, S, H, F, bits, act_bits):
    wl = datagen.Workload("t", 2000 + seed, "moe", act_bits, H=H, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=bits, bits_down=bits)
    gate, up, down = datagen.moe_weights(wl)
    x, lg = datagen.moe_tokens(wl, T)
    return wl, gate, up, down, x, lg


@pytest.mark.parametrize("path", [cbq.PATH_AUTO, cbq.PATH_LUT, cbq.PATH_MFMA,
                                  cbq.PATH_AUTO | cbq.PATH_REG_TABLES,
                                  cbq.PATH_AUTO | cbq.PATH_LDS_TABLES])
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
@pytest.mark.parametrize("path", [cbq.PATH_AUTO, cbq.PATH_LUT, cbq.PATH_LUT | cbq.PATH_REG_TABLES,
                                  cbq.PATH_MFMA | cbq.PATH_LDS_TABLES])
def test_many_tile_decode_gemm(bits, act_bits, n_w, path):
    # 64 experts x 2080 rows: enough 16-row tiles that no wave splits K (the decode
    # layout of the large MoE layers); K = 160 leaves a 32-channel chunk tail, N = 2080
    # leaves part of the last two-group wave empty, and the row counts include
    # empty experts, full 32-row blocks, 16 and 17 rows (one sub-tile, and a second one of
    # one row), and experts of 33 and 40 rows (a second row block, of one and of eight
    # rows, when forced onto the LUT path; AUTO sends them to the MFMA path)
    E, N, K, T = 64, 2080, 160, 50
    rng = np.random.default_rng(bits * 10 + act_bits + n_w)
    counts = rng.integers(0, 6, E)
    counts[[3, 17, 40]] = 0
    counts[5], counts[9], counts[12], counts[20], counts[63] = 32, 16, 17, 33, 40
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


def _prefill_run_length(counts, bm, min_rows):
    """The run length the MFMA kernel picks for these expert row counts: the largest power of
    two <= 4 with 8G <= the call's tile count T, then halved while padding each expert's last
    run to G tiles would leave more than T / 4 slots empty."""
    nt = np.where(counts > min_rows, (counts + bm - 1) // bm, 0)
    t = int(nt.sum())
    g = 1
    while 2 * g <= 4 and 16 * g <= t:
        g *= 2
    while g > 1 and int(((-nt) % g).sum()) > t // 4:
        g //= 2
    return g


# Expert row counts for the MFMA GEMM's placement of M-tiles on the XCDs: 80 experts (the
# tile scan works through experts 64 at a time), experts of several runs on both sides of
# expert 64, empty experts, and one set for each run length the kernel can pick.
_RUN_CASES = {
    # long experts only: runs of 4 (3-bit tiles of 128 rows), of 2 (4-bit tiles of 256)
    "long": {2: 1100, 10: 260, 30: 512, 65: 520, 70: 900, 79: 1024},
    # plus three one-tile experts: padding halves the runs of 4
    "mixed": {2: 1100, 10: 260, 30: 512, 65: 520, 70: 900, 79: 1024, 5: 90, 40: 70, 77: 100},
    # mostly one-tile experts: runs of one
    "short": {1: 1100, 66: 700, **{e: 40 + e for e in range(20, 60, 2)}},
    # two experts of 4096 rows last (as shared experts are): scanned first, they fill the
    # first block of 16 runs, whose groups of 8 runs stay on four XCDs; then a ragged tail
    "shared": {3: 300, 12: 500, 40: 380, 66: 200, 78: 4096, 79: 4096},
}


@pytest.mark.parametrize("case", sorted(_RUN_CASES))
@pytest.mark.parametrize("bits,act_bits,n_w", [(3, 4, 2), (4, 8, 2), (3, 4, 1), (4, 4, 1)])
@pytest.mark.parametrize("path", [cbq.PATH_MFMA, cbq.PATH_AUTO])
def test_prefill_run_placement(case, bits, act_bits, n_w, path):
    E, N, K, T = 80, 272, 96, 600
    counts = np.zeros(E, dtype=np.int64)
    for e, c in _RUN_CASES[case].items():
        counts[e] = c
    if path == cbq.PATH_AUTO:
        counts[[7, 50, 71]] = [1, 32, 17]       # experts AUTO sends to the LUT path
    bm = 256 if bits == 4 else 128
    min_rows = cbq.AUTO_MAX_LUT_ROWS if path == cbq.PATH_AUTO else 0
    want_g = {("long", 128): 4, ("long", 256): 2, ("mixed", 128): 2, ("mixed", 256): 2,
              ("short", 128): 1, ("short", 256): 1, ("shared", 128): 4, ("shared", 256): 4}[(case, bm)]
    assert _prefill_run_length(counts, bm, min_rows) == want_g
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    rng = np.random.default_rng(bits * 100 + act_bits * 10 + n_w + len(case))
    row_token = rng.integers(0, T, R).astype(np.int32)
    rq = oracle.rotate_quantize(datagen.random_tokens(700 + bits, T, K), 0, act_bits)
    ws = [datagen.random_weights(80 + bits + m, E, N, K, bits, keep_raw=False) for m in range(n_w)]
    out = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits,
                                [upload_weights(w) for w in ws], expert_offsets=to_dev(offsets),
                                row_token=to_dev(row_token), path=path)
    ref = [oracle.expert_gemm(rq["q"], rq["scale"], row_token, offsets, w.idx, w.codebook, K, bits)
           for w in ws]
    if n_w == 2:
        assert_bf16_close(bf16_to_bits(out), oracle.silu_mul_bf16(ref[0], ref[1]), f"swiglu {case}")
    else:
        assert_normwise(out.cpu().numpy(), ref[0], 1e-3, f"f32 {case}")


@pytest.mark.parametrize("bits,act_bits", [(3, 4), (4, 8)])
def test_swiglu_paths_agree(bits, act_bits):
    """Both GEMM paths end in the same SwiGLU formula; only the fp32 summation order of g
    and u differs.  So on the same rows the bf16 h of the LUT and MFMA paths is equal or
    one bf16 step apart (where g or u moved across a rounding midpoint), and AUTO gives,
    bit for bit, the LUT result for experts of at most 32 rows and the MFMA result for
    the others."""
    T, E, k, S, H, F = 120, 8, 2, 1, 512, 320
    wl, gate, up, down, x, lg = _moe_case(90 + bits, T, E, k, S, H, F, bits, act_bits)
    rq = oracle.rotate_quantize(x, 0, act_bits)
    rt = oracle.route(lg, k, True, S)
    G, U = upload_weights(gate), upload_weights(up)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [G, U])
    kw = dict(expert_offsets=to_dev(rt["offsets"]), row_token=to_dev(rt["sorted_tokens"]))
    h = {p: bf16_to_bits(cbq.codebook_lut_gemm(*args, path=p, **kw))
         for p in (cbq.PATH_LUT, cbq.PATH_MFMA, cbq.PATH_AUTO)}
    a = h[cbq.PATH_LUT].astype(np.int32)
    b = h[cbq.PATH_MFMA].astype(np.int32)
    same_sign = (a ^ b) & 0x8000 == 0
    step = np.where(same_sign, np.abs(a - b), np.abs((a & 0x7FFF) + (b & 0x7FFF)))
    assert step.max() <= 1, f"LUT and MFMA h differ by {step.max()} bf16 steps"
    print(f"bits={bits} A{act_bits}: h equal on both paths for {np.mean(step == 0):.5f} of values")
    counts = np.diff(rt["offsets"])
    assert counts.min() <= cbq.AUTO_MAX_LUT_ROWS < counts.max()      # both paths taken
    for e in range(E + S):
        r0, r1 = rt["offsets"][e], rt["offsets"][e + 1]
        want = h[cbq.PATH_LUT] if r1 - r0 <= cbq.AUTO_MAX_LUT_ROWS else h[cbq.PATH_MFMA]
        assert np.array_equal(h[cbq.PATH_AUTO][r0:r1], want[r0:r1]), e


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


@pytest.mark.parametrize("act_bits,K,path,dense", [(8, 4096, cbq.PATH_MFMA, False),
                                                   (4, 4160, cbq.PATH_AUTO, False),
                                                   (8, 4160, cbq.PATH_MFMA, True)])
def test_mfma_split_k_workspace(act_bits, K, path, dense):
    """A single 4-bit matrix with K >= 4096 whose 256-row tiles would leave CUs idle splits
    K in two when given the workspace cbq_gemm_workspace asks for: the second half's partial
    sums go to the workspace and are added to out in a second, ordered pass.  The result
    equals the unsplit call up to the fp32 summation order and the oracle within 1e-3;
    rows of experts AUTO sends to the LUT path (at most 32 rows) are not touched by the
    pass (bit-identical to the unsplit call).  K = 4160 leaves the second half a ragged
    last step; the dense case has no expert offsets."""
    E, N, T = (1, 384, 300) if dense else (8, 384, 500)
    rng = np.random.default_rng(act_bits * 1000 + K + dense)
    if dense:
        counts = np.array([T])
    else:
        counts = np.array([140, 0, 17, 300, 129, 32, 260, 90])   # empty, LUT-sized and MFMA experts
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    row_token = None if dense else rng.integers(0, T, R).astype(np.int32)
    rq = oracle.rotate_quantize(datagen.random_tokens(900 + act_bits, T, K), 0, act_bits)
    ws_np = datagen.random_weights(910 + act_bits, E, N, K, 4, keep_raw=False)
    W = upload_weights(ws_np)
    need = cbq.gemm_workspace([W], R, act_bits, path)
    assert need == R * N * 4
    assert cbq.gemm_workspace([W], R, act_bits, cbq.PATH_LUT) == 0
    kw = dict(expert_offsets=None if dense else to_dev(offsets),
              row_token=None if dense else to_dev(row_token), path=path, n_rows=R)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [W])
    plain = cbq.codebook_lut_gemm(*args, **kw)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)      # stale contents
    split = cbq.codebook_lut_gemm(*args, ws=ws, **kw)
    split2 = cbq.codebook_lut_gemm(*args, ws=ws, **kw)                  # the workspace reused
    torch.cuda.synchronize()
    p, s, s2 = plain.cpu().numpy(), split.cpu().numpy(), split2.cpu().numpy()
    assert np.array_equal(s, s2), "the split call is deterministic"
    ref = oracle.expert_gemm(rq["q"], rq["scale"], row_token, None if dense else offsets,
                             ws_np.idx, ws_np.codebook, K, 4)
    assert_normwise(s, ref, 1e-3, "split")
    assert_normwise(s, p, 1e-6, "split vs unsplit")
    if path == cbq.PATH_AUTO:
        lut_rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in range(E)
                                   if 0 < counts[e] <= cbq.AUTO_MAX_LUT_ROWS])
        assert np.array_equal(s[lut_rows], p[lut_rows])
    assert not np.array_equal(s, p), "the split path ran (its sums differ in order)"


def _bf16_steps(a, b):
    a, b = a.astype(np.int32), b.astype(np.int32)
    same_sign = (a ^ b) & 0x8000 == 0
    return np.where(same_sign, np.abs(a - b), np.abs((a & 0x7FFF) + (b & 0x7FFF)))


@pytest.mark.parametrize("case", ["auto_ragged", "mfma_many_tiles", "dense"])
def test_mfma_gate_up_tail_split(case):
    """The gate/up pair with 4-bit codebooks (256-row tiles, one workgroup per CU), given
    the workspace cbq_gemm_workspace asks for: in a call of at most 8 row tiles each XCD
    works through one tile's column tiles in rounds of its CUs, and the column tiles of a
    last round at most half full split K in two; both halves' sums of g and u go to the
    workspace and a second pass forms h.  h equals the oracle's, and the unsplit call's,
    within the SwiGLU tolerance (bit for bit left of the split columns); the split call is
    deterministic
    (stale workspace contents, two calls); rows AUTO sends to the LUT path are untouched.
    With more than 8 row tiles the call does not split (bit-identical to the unsplit call).
    N = 4672 leaves a ragged last column tile inside the split ones."""
    K, act_bits = 2048, 8
    if case == "dense":
        E, N, T, path = 1, 4224, 600, cbq.PATH_MFMA
        counts = np.array([T])
    else:
        E, N, T = 10, 4672, 700
        path = cbq.PATH_AUTO if case == "auto_ragged" else cbq.PATH_MFMA
        counts = np.array([140, 0, 17, 250, 129, 32, 200, 90, 160, 256])
    rng = np.random.default_rng(len(case))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    dense = case == "dense"
    row_token = None if dense else rng.integers(0, T, R).astype(np.int32)
    rq = oracle.rotate_quantize(datagen.random_tokens(950 + len(case), T, K), 0, act_bits)
    wn = [datagen.random_weights(960 + m, E, N, K, 4, keep_raw=False) for m in range(2)]
    G, U = upload_weights(wn[0]), upload_weights(wn[1])
    need = cbq.gemm_workspace([G, U], R, act_bits, path)
    assert need == 4 * R * 2048 * 4
    min_rows = cbq.AUTO_MAX_LUT_ROWS if path == cbq.PATH_AUTO else 0
    tiles = int(np.sum(np.where(counts > min_rows, (counts + 255) // 256, 0)))
    per = torch.cuda.get_device_properties(0).multi_processor_count // 8
    ntc = (N + 127) // 128
    splits = tiles <= 8 and 0 < ntc % per <= per // 2
    print(f"{case}: {tiles} row tiles, {ntc} column tiles, {per} CUs per XCD, split {splits}")
    kw = dict(expert_offsets=None if dense else to_dev(offsets),
              row_token=None if dense else to_dev(row_token), path=path, n_rows=R)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [G, U])
    plain = bf16_to_bits(cbq.codebook_lut_gemm(*args, **kw))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)      # stale contents
    split = bf16_to_bits(cbq.codebook_lut_gemm(*args, ws=ws, **kw))
    split2 = bf16_to_bits(cbq.codebook_lut_gemm(*args, ws=ws, **kw))
    assert np.array_equal(split, split2), "the split call is deterministic"
    ref = [oracle.expert_gemm(rq["q"], rq["scale"], row_token, None if dense else offsets,
                              w.idx, w.codebook, K, 4) for w in wn]
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in range(E)
                           if counts[e] > min_rows])
    want = oracle.silu_mul_bf16(ref[0], ref[1])
    assert_bf16_close(split[rows], want[rows], f"swiglu {case}")
    if path == cbq.PATH_AUTO:
        lut_rows = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in range(E)
                                   if 0 < counts[e] <= min_rows])
        assert np.array_equal(split[lut_rows], plain[lut_rows])
    # the split halves' sums land in the workspace; h left of the split column tiles is
    # computed exactly as without it
    used = bool((ws != 0x7F).any().item())
    assert used == splits
    c0 = (ntc - ntc % per) * 128 if splits else N
    assert np.array_equal(split[:, :c0], plain[:, :c0])
    # right of it only the fp32 order of the two halves' sums differs: an absolute change
    # of a few units in the last place of the partial sums, which moves h by more than one
    # bf16 step only where g or u nearly cancels (h small against the tile's values)
    assert_bf16_close(split[rows], plain[rows], f"split vs unsplit {case}")
    steps = _bf16_steps(split[rows], plain[rows])
    print(f"{case}: split h equal to unsplit for {np.mean(steps == 0):.6f} of values, "
          f"within one bf16 step for {np.mean(steps <= 1):.7f}")


def test_moe_ffn_with_workspaces():
    """moe_ffn hands its GEMMs the workspaces gemm_workspace asks for.  At 300 tokens, top-2
    of 4 routed experts (600 rows of 137-161 each, 4-bit codebooks, H 2048, F 4224, A8) both
    K splits run: the gate/up pair's last column tile on each XCD, and the down projection
    (K = 4224).  Every stage against the oracle, teacher forced on the GPU's own
    intermediates."""
    T, E, k, S, H, F, a = 300, 4, 2, 0, 2048, 4224, 8
    wl, gate, up, down, x, lg = _moe_case(77, T, E, k, S, H, F, 4, a)
    G, U, D = upload_weights(gate), upload_weights(up), upload_weights(down)
    R = T * k
    assert cbq.gemm_workspace([G, U], R, a) > 0 and cbq.gemm_workspace([D], R, a) > 0
    y, mid = cbq.moe_ffn(bf16_dev(x), to_dev(lg), G, U, D, k, S, a, keep=True)
    torch.cuda.synchronize()
    rq = oracle.rotate_quantize(x, 0, a)
    assert rq["ok"].all()
    assert np.array_equal(mid["codes"].cpu().numpy(), rq["codes"])
    rt = oracle.route(lg, k, True, S)
    for key in ("offsets", "sorted_tokens", "slot_of"):
        assert np.array_equal(mid["route"][key].cpu().numpy(), rt[key]), key
    g = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], gate.idx,
                           gate.codebook, H, 4)
    u = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], up.idx,
                           up.codebook, H, 4)
    h = bf16_to_bits(mid["h"])
    assert_bf16_close(h, oracle.silu_mul_bf16(g, u), "h")
    rqh = oracle.rotate_quantize(h, 0, a)
    assert np.array_equal(mid["codes_h"].cpu().numpy(), rqh["codes"])
    d = oracle.expert_gemm(rqh["q"], rqh["scale"], None, rt["offsets"], down.idx, down.codebook, F, 4)
    out = mid["out"].cpu().numpy()
    assert_normwise(out, d, 1e-3, "down")
    y_ref = oracle.combine(out, rt["slot_of"], rt["weights"], T, k, S)
    assert_normwise(y.cpu().numpy(), y_ref, 1e-3, "y")
