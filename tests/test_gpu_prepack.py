"""The blocked index layout (cbq_prepack_weights): its bytes against the layout written
out on the host from its definition, and the GEMM on blocked weights against the oracle
on the row-layout weights it came from, on every path, bit width and activation width,
with K tails that are not a multiple of 128 and every split mode.  The kernels load the
same indices into the same lanes in the same order from either layout (3-bit units
re-encoded so their byte selectors are cheaper, decoding to the same indices), so outputs
must also be bit-identical to the row layout's."""
import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import (assert_bf16_close, assert_normwise, bf16_to_bits, to_dev,  # noqa: E402
                      upload_weights)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


def reencode3(unit):
    """A 3-bit unit (12 bytes, 32 LSB-first indices) in the blocked layout's encoding:
    dword g < 3 holds indices 8g+2b (bits 0-2) and 8g+2b+1 (bits 3-5) in byte b; the
    six-bit pair b of indices 24+2b, 25+2b is spread over bits 6-7 of byte b of dwords
    0, 1, 2, two bits each, lowest first."""
    v = int.from_bytes(bytes(unit), "little")
    i = [(v >> (3 * k)) & 7 for k in range(32)]
    d = [0, 0, 0]
    for g in range(3):
        for b in range(4):
            d[g] |= (i[8 * g + 2 * b] | (i[8 * g + 2 * b + 1] << 3)) << (8 * b)
    for b in range(4):
        pr = i[24 + 2 * b] | (i[25 + 2 * b] << 3)
        for w in range(3):
            d[w] |= ((pr >> (2 * w)) & 3) << (8 * b + 6)
    return np.frombuffer(b"".join(x.to_bytes(4, "little") for x in d), dtype=np.uint8)


def blocked_host(idx, N, K, bits):
    """The blocked layout from its definition: the 4*bits bytes of 32 consecutive indices
    of row 16G + r at channel 128c + 32j go to ((e*N/16 + G)*Kp/128 + c)*256*bits +
    (16j + r)*4*bits (3-bit units re-encoded by reencode3); zeros past K."""
    E = idx.shape[0]
    kc = (K + 127) // 128
    u = 4 * bits
    out = np.zeros(E * (N // 16) * kc * 64 * u, dtype=np.uint8)
    rb = K * bits // 8
    for e in range(E):
        for n in range(N):
            G, r = divmod(n, 16)
            for c in range(kc):
                for j in range(4):
                    k0 = 128 * c + 32 * j
                    if k0 >= K:
                        continue
                    src = idx[e, n, k0 * bits // 8:k0 * bits // 8 + u]
                    dst = (((e * (N // 16) + G) * kc + c) * 64 + 16 * j + r) * u
                    out[dst:dst + u] = reencode3(src) if bits == 3 else src
    assert rb * 8 == K * bits
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("E,N,K", [(1, 48, 160), (3, 32, 256), (2, 16, 1408)])
def test_prepack_bytes(bits, E, N, K):
    ws = datagen.random_weights(60 + bits, E, N, K, bits, keep_raw=False)
    got = cbq.prepack_weights(upload_weights(ws))
    assert got.layout == cbq.LAYOUT_BLOCKED
    assert np.array_equal(got.idx.cpu().numpy().reshape(-1), blocked_host(ws.idx, N, K, bits))


def _dense(seed, T, N, K, bits, act_bits):
    ws = datagen.random_weights(seed, 1, N, K, bits)
    rq = oracle.rotate_quantize(datagen.random_tokens(seed + 1, T, K), 0, act_bits)
    ref = oracle.expert_gemm(rq["q"], rq["scale"], None, None, ws.idx, ws.codebook, K, bits)
    return ws, rq, ref


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("act_bits", [4, 8])
@pytest.mark.parametrize("path", [cbq.PATH_LUT, cbq.PATH_MFMA, cbq.PATH_LUT | cbq.PATH_REG_TABLES,
                                  cbq.PATH_LUT | cbq.PATH_LDS_TABLES, cbq.PATH_MFMA | cbq.PATH_LDS_TABLES])
@pytest.mark.parametrize("T,N,K", [(4, 256, 256), (13, 80, 160), (1, 48, 1408), (150, 208, 544),
                                   (16, 1024, 2560)])
def test_dense_gemm_blocked(bits, act_bits, path, T, N, K):
    ws, rq, ref = _dense(300 * bits + act_bits + T, T, N, K, bits, act_bits)
    rows = upload_weights(ws)
    blk = cbq.prepack_weights(rows)
    args = (to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits)
    y = cbq.codebook_lut_gemm(*args, [blk], path=path)
    assert_normwise(y.cpu().numpy(), ref, 1e-3, f"blocked bits={bits} a={act_bits} path={path}")
    # with the same table placement on both layouts the kernels see the same indices in
    # the same order, so the outputs are bit-identical (the default placement of 3-bit
    # codebooks differs between the layouts, so each placement is compared explicitly)
    placements = [path] if path & (cbq.PATH_REG_TABLES | cbq.PATH_LDS_TABLES) else \
        [path | cbq.PATH_REG_TABLES, path | cbq.PATH_LDS_TABLES]
    for p in placements:
        y_blk = cbq.codebook_lut_gemm(*args, [blk], path=p)
        y_rows = cbq.codebook_lut_gemm(*args, [rows], path=p)
        assert torch.equal(y_blk.view(torch.int32), y_rows.view(torch.int32)), p


@pytest.mark.parametrize("bits,act_bits", [(3, 4), (2, 8), (4, 4)])
@pytest.mark.parametrize("path", [cbq.PATH_AUTO, cbq.PATH_LUT, cbq.PATH_MFMA])
def test_moe_blocked(bits, act_bits, path):
    T, E, k, S, H, F = 96, 8, 2, 1, 384, 160
    wl = datagen.Workload("t", 2500 + bits, "moe", act_bits, H=H, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=bits, bits_down=bits)
    gate, up, down = datagen.moe_weights(wl)
    x, lg = datagen.moe_tokens(wl, T)
    rq = oracle.rotate_quantize(x, 0, act_bits)
    rt = oracle.route(lg, k, True, S)
    G, U, D = (cbq.prepack_weights(upload_weights(w)) for w in (gate, up, down))
    offs, toks = to_dev(rt["offsets"]), to_dev(rt["sorted_tokens"])
    h = cbq.codebook_lut_gemm(to_dev(rq["codes"]), to_dev(rq["scale"]), act_bits, [G, U],
                              expert_offsets=offs, row_token=toks, path=path)
    g = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], gate.idx,
                           gate.codebook, H, bits)
    u = oracle.expert_gemm(rq["q"], rq["scale"], rt["sorted_tokens"], rt["offsets"], up.idx,
                           up.codebook, H, bits)
    assert_bf16_close(bf16_to_bits(h), oracle.silu_mul_bf16(g, u), "swiglu")
    hb = bf16_to_bits(h)
    rqh = oracle.rotate_quantize(hb, 0, act_bits)
    ch, sh = cbq.rotate_quantize(h, act_bits)
    out = cbq.codebook_lut_gemm(ch, sh, act_bits, [D], expert_offsets=offs, path=path)
    ref = oracle.expert_gemm(rqh["q"], rqh["scale"], None, rt["offsets"], down.idx, down.codebook,
                             F, bits)
    assert_normwise(out.cpu().numpy(), ref, 1e-3, "down")
