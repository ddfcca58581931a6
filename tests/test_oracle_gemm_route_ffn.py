"""Pins for the oracle's codebook GEMM, routing, SwiGLU and combine (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _packing_cases():
    out = {}
    with open(os.path.join(GOLDEN, "index_packing.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals, byts = v.split("->")
                out[k] = ([int(t) for t in vals.split()], [int(t, 16) for t in byts.split()])
    return out


# ---------------------------------------------------------------------------
# index format
@pytest.mark.parametrize("key,bits", [("bits3", 3), ("bits2", 2), ("bits4", 4)])
def test_index_packing_literals(key, bits):
    vals, byts = _packing_cases()[key]
    packed = np.array([byts], dtype=np.uint8)
    assert oracle.unpack_indices(packed, len(vals), bits)[0].tolist() == vals
    assert datagen.pack_lsb_first(np.array([vals]), bits)[0].tolist() == byts


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_index_unpack_round_trip(bits):
    w = datagen.random_weights(bits, 2, 5, 96, bits, keep_raw=True)
    assert np.array_equal(oracle.unpack_indices(w.idx, 96, bits), w.raw)
    # the generator's distribution: last index rare, the rest used
    L = (1 << bits) - 1
    assert set(np.unique(w.raw)) <= set(range(L + 1))


# ---------------------------------------------------------------------------
# GEMM
def _brute_gemm(q, s, idx, C):
    R, K = q.shape
    N = idx.shape[0]
    y = np.zeros((R, N))
    for r in range(R):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(q[r, k]) * float(C[n, idx[n, k]])
            y[r, n] = acc * float(s[r])
    return y


@pytest.mark.parametrize("bits,act_bits", [(4, 4), (3, 4), (2, 8), (4, 8)])
def test_gemm_brute_force(bits, act_bits):
    K, N, R = 64, 7, 3
    w = datagen.random_weights(10 + bits, 1, N, K, bits, keep_raw=True)
    rq = oracle.rotate_quantize(datagen.random_tokens(20 + bits, R, K), 0, act_bits)
    C = oracle.f16_bits_to_f64(w.codebook[0])
    ref = _brute_gemm(rq["q"], rq["scale"], w.raw[0], C)
    y = oracle.expert_gemm(rq["q"], rq["scale"], None, None, w.idx, w.codebook, K, bits)
    assert np.array_equal(y, ref)      # sums exact in fp64, single rounding at the scale


def test_gemm_identity_codebook():
    """codebook {0, 1, ...} with idx[n][k] = 1 iff n == k gives W = I: y = scale * q."""
    K = N = 32
    raw = np.eye(N, K, dtype=np.uint8)
    idx = datagen.pack_lsb_first(raw[None], 4)
    cb = datagen.f32_to_f16_bits(np.tile(np.arange(16, dtype=np.float32), (N, 1)))[None]
    rq = oracle.rotate_quantize(datagen.random_tokens(31, 4, K), 0, 4)
    y = oracle.expert_gemm(rq["q"], rq["scale"], None, None, idx, cb, K, 4)
    assert np.array_equal(y, rq["q"].astype(np.float64) * rq["scale"][:, None].astype(np.float64))


def test_gemm_constant_index():
    K, N, c = 64, 5, 6
    raw = np.full((1, N, K), c, dtype=np.uint8)
    w = datagen.random_weights(40, 1, N, K, 4)
    idx = datagen.pack_lsb_first(raw, 4)
    rq = oracle.rotate_quantize(datagen.random_tokens(41, 3, K), 0, 4)
    y = oracle.expert_gemm(rq["q"], rq["scale"], None, None, idx, w.codebook, K, 4)
    C = oracle.f16_bits_to_f64(w.codebook[0])
    expect = rq["scale"][:, None].astype(np.float64) * C[None, :, c] * rq["q"].sum(axis=1)[:, None]
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


@pytest.mark.parametrize("bits,act_bits", [(4, 4), (3, 4), (2, 4), (4, 8)])
def test_lut_equals_dequantised_product_exactly(bits, act_bits):
    """The pages' level x centroid table, the bucketed sums and the dense dequantised
    product are the same number: checked in exact integer arithmetic (fp16 centroids
    are multiples of 2^-24)."""
    K, N, R = 96, 6, 4
    w = datagen.random_weights(50 + bits, 1, N, K, bits, keep_raw=True)
    rq = oracle.rotate_quantize(datagen.random_tokens(51, R, K), 0, act_bits)
    q = rq["q"].astype(np.int64)
    C = oracle.f16_bits_to_f64(w.codebook[0])
    Ci = np.rint(C * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(Ci.astype(np.float64) * 2.0 ** -24, C)
    idx = w.raw[0].astype(np.int64)
    dense = np.array([[int(np.dot(q[r], Ci[n, idx[n]])) for n in range(N)] for r in range(R)])
    Q, lo, hi = oracle.ACT_LEVELS[act_bits]
    table = np.arange(lo, hi + 1)[None, :, None] * Ci[:, None, :]
    lut = np.array([[int(table[n][q[r] - lo, idx[n]].sum()) for n in range(N)] for r in range(R)])
    onehot = idx[:, None, :] == np.arange(1 << bits)[None, :, None]
    buckets = np.array([[int((onehot[n] @ q[r]) @ Ci[n]) for n in range(N)] for r in range(R)])
    assert np.array_equal(dense, lut) and np.array_equal(dense, buckets)
    one = np.ones(R, dtype=np.float32)
    ref = dense.astype(np.float64) * 2.0 ** -24
    assert np.array_equal(oracle.lut_gemm_table(q, one, idx, w.codebook[0], act_bits), ref)
    assert np.array_equal(oracle.lut_gemm_buckets(q, one, idx, w.codebook[0]), ref)
    assert np.array_equal(oracle.expert_gemm(q, one, None, None, w.idx, w.codebook, K, bits), ref)


def test_grouped_gemm_rows_and_experts():
    E, N, K, T = 3, 5, 64, 6
    w = datagen.random_weights(60, E, N, K, 4, keep_raw=True)
    rq = oracle.rotate_quantize(datagen.random_tokens(61, T, K), 0, 4)
    row_token = np.array([4, 0, 2, 5, 1, 3, 3], dtype=np.int32)
    offsets = np.array([0, 2, 2, 7])       # expert 1 empty
    y = oracle.expert_gemm(rq["q"], rq["scale"], row_token, offsets, w.idx, w.codebook, K, 4)
    for r, t in enumerate(row_token):
        e = 0 if r < 2 else 2
        C = oracle.f16_bits_to_f64(w.codebook[e])
        ref = _brute_gemm(rq["q"][t:t + 1], rq["scale"][t:t + 1], w.raw[e], C)[0]
        assert np.array_equal(y[r], ref)
        for n in (0, N - 1):
            assert oracle.gemm_entry(rq["q"][t], rq["scale"][t], w.idx[e, n], w.codebook[e, n], K, 4) == ref[n]


# ---------------------------------------------------------------------------
# routing
def _brute_topk(row, k):
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("T,E,k,S", [(1, 8, 2, 0), (37, 64, 6, 2), (20, 128, 8, 0), (5, 4, 4, 1)])
def test_route_brute_force_and_invariants(T, E, k, S):
    lg = datagen.random_logits(T * E + k, T, E)
    lg[0, 1] = lg[0, 2] = lg[0, 5 % E] = np.float32(3.5)     # ties -> lower id first
    if T > 1:
        lg[1, :] = 0.0
        lg[1, 3 % E] = -0.0
    r = oracle.route(lg, k, True, S)
    for t in range(T):
        assert r["ids"][t].tolist() == _brute_topk(lg[t].tolist(), k)
        sel = lg[t, r["ids"][t]].astype(np.float64)
        ex = [math.exp(v - max(sel)) for v in sel]
        assert np.allclose(r["weights64"][t], np.array(ex) / sum(ex), rtol=1e-14)
    if T > 1:
        assert r["ids"][1].tolist() == list(range(k))
    offs, st, so = r["offsets"], r["sorted_tokens"], r["slot_of"]
    assert offs[0] == 0 and offs[-1] == T * k + S * T and np.all(np.diff(offs) >= 0)
    for e in range(E + S):
        seg = st[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) > 0)
    for t in range(T):
        assert len(set(r["ids"][t].tolist())) == k
        for j in range(k):
            row = so[t, j]
            assert st[row] == t
            e = np.searchsorted(offs, row, side="right") - 1
            assert e == r["ids"][t, j]


def test_route_weights_closed_forms():
    lg = np.array([[0.0, 1.0, -1.0, 0.5]], dtype=np.float32)
    r = oracle.route(lg, 2, True)
    assert r["ids"][0].tolist() == [1, 3]
    assert math.isclose(r["weights64"][0, 0], 1 / (1 + math.exp(-0.5)), rel_tol=1e-15)
    r2 = oracle.route(lg, 2, False)
    z = sum(math.exp(v) for v in (0.0, 1.0, -1.0, 0.5))
    assert math.isclose(r2["weights64"][0, 0], math.exp(1.0) / z, rel_tol=1e-14)
    assert math.isclose(r2["weights64"][0, 1], math.exp(0.5) / z, rel_tol=1e-14)


# ---------------------------------------------------------------------------
# SwiGLU and bf16 rounding
def test_bf16_rounding_literals_and_torch():
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -9: 0x3F81, 1.0 + 2 ** -7: 0x3F81,
             1.0 + 3 * 2 ** -8: 0x3F82, -2.0: 0xC000, 0.0: 0x0000, 2.0 ** -130: 0x0008, 3 * 2.0 ** -134: 0x0002}
    for v, bits in cases.items():
        assert int(oracle.round_f64_to_bf16_bits(np.array([v]))[0]) == bits, v
    # fp32-representable inputs: torch's CPU fp32 -> bf16 conversion (round to nearest even)
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_f64_to_bf16_bits(f.astype(np.float64)), tb)
    # a value just above a tie that fp32 cannot hold still rounds up
    assert int(oracle.round_f64_to_bf16_bits(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0]) == 0x3F81


def test_silu_mul_closed_forms():
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0])
    u = np.array([5.0, 2.0, 2.0, 0.5])
    h = datagen.bf16_bits_to_f32(oracle.silu_mul_bf16(g, u)).astype(np.float64)
    expect = np.array([0.0, 0.75 * math.log(3.0) * 2.0, -0.25 * math.log(3.0) * 2.0, 20.0])
    assert np.allclose(h, expect, rtol=2 ** -8)
    assert h[0] == 0.0 and h[3] == 20.0


# ---------------------------------------------------------------------------
# combine
def test_combine_one_hot_identical_and_shared():
    T, k, S, Hd = 4, 3, 1, 16
    rng = np.random.default_rng(8)
    out = rng.standard_normal((T * k + S * T, Hd))
    slot = np.arange(T * k).reshape(T, k)
    w = np.zeros((T, k), dtype=np.float32)
    w[:, 1] = 1
    y = oracle.combine(out, slot, w, T, k, 0)
    assert np.array_equal(y, out[slot[:, 1]])
    y2 = oracle.combine(out, slot, w, T, k, S)
    assert np.array_equal(y2, out[slot[:, 1]] + out[T * k:])
    same = np.tile(out[:1], (T * k, 1))
    wr = oracle.route(rng.standard_normal((T, 8)).astype(np.float32), k)["weights"]
    y3 = oracle.combine(same, slot, wr, T, k, 0)
    assert np.allclose(y3, np.tile(out[:1], (T, 1)), rtol=1e-6)


# ---------------------------------------------------------------------------
# whole layer, token by token
def test_moe_layer_matches_per_token_brute_force():
    T, Hd, F, E, k, S = 5, 64, 32, 4, 2, 1
    wl = datagen.Workload("tiny", 900, "moe", 4, H=Hd, F=F, E=E, topk=k, n_shared=S,
                          bits_gate_up=3, bits_down=2)
    gate, up, down = datagen.moe_weights(wl, keep_raw=True)
    x, lg = datagen.moe_tokens(wl, T)
    res = oracle.moe_layer(x, lg, gate, up, down, k, S, 4)
    rq = oracle.rotate_quantize(x, 0, 4)
    rt = oracle.route(lg, k, True, S)

    def dense(ws, e):
        return oracle.f16_bits_to_f64(ws.codebook[e])[np.arange(ws.N)[:, None], ws.raw[e]]

    for t in range(T):
        experts = [(int(e), float(w)) for e, w in zip(rt["ids"][t], rt["weights"][t])]
        experts += [(E + s, 1.0) for s in range(S)]
        acc = np.zeros(Hd)
        for e, w in experts:
            qx = rq["q"][t].astype(np.float64)
            g = (dense(gate, e) @ qx) * float(rq["scale"][t])
            u = (dense(up, e) @ qx) * float(rq["scale"][t])
            h = oracle.silu_mul_bf16(g, u)[None, :]
            rh = oracle.rotate_quantize(h, 0, 4)
            o = (dense(down, e) @ rh["q"][0].astype(np.float64)) * float(rh["scale"][0])
            acc += w * o
        assert np.allclose(res["y"][t], acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())
