"""GPU parity at the full sizes of the five synthetic workloads.

MoE layers run through the benchmark's own call sequence and path choice (its MoEPhase
class and choose_path rule), so what is checked here is what the benchmark times.

* Integer outputs are compared in full and bit-exactly: the token codes and scales of
  both rotate_quantize calls, the routing ids, offsets, row lists and slot map.
* GEMM outputs are checked on a seeded sample of (row, column) entries that the
  oracle computes one by one (every expert's first and last row, the first and last
  column, plus uniform draws).  Each stage is teacher forced: its oracle input is the
  GPU's own input to that stage (the h codes come from the GPU's bf16 h, the down
  GEMM reads the GPU's h codes, combine reads the GPU's expert outputs).
* Dense linears are small enough to compare every output.
* The weights are regrouped into the blocked index layout, as the benchmark runs them;
  the oracle reads the row layout they were generated in.
* The free-running comparison (oracle end to end from x) is run where the oracle
  finishes in seconds; it reports the h-code flips that near-ties cause.

Tolerances are those of the small-shape tests: normwise 1e-3 for fp32 outputs, one
bf16 step plus 1e-3 of the sampled max for the SwiGLU outputs, 1e-6 for routing
weights.
"""
import os
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

cbq = pytest.importorskip("codebook_bit_quantized_amd")
from gpu_util import (DEV, assert_bf16_close, assert_normwise, bf16_dev, bf16_to_bits,  # noqa: E402
                      to_dev, upload_weights)

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

N_SAMPLES = 1500


def bench_weights(ws):
    """The device weights the benchmark times: the blocked index layout."""
    return bench.upload_weights(cbq, torch, ws)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cbq.load_library()


_CACHE = {}


def moe_setup(name):
    """Host and device weights of one MoE workload, generated once per module."""
    if name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        wl = datagen.WORKLOADS[name]
        g, u, d = datagen.moe_weights(wl)
        W = dict(gate=bench_weights(g), up=bench_weights(u), down=bench_weights(d))
        _CACHE[name] = (wl, dict(gate=g, up=u, down=d), W)
    return _CACHE[name]


def sample_entries(rng, offsets, R, N, n=N_SAMPLES):
    """(row, column) pairs: uniform draws plus each expert's first and last row at
    the first and last column."""
    rows = list(rng.integers(0, R, n))
    cols = list(rng.integers(0, N, n))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            rows += [r0, r1 - 1]
            cols += [0, N - 1]
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def expert_of(offsets, rows):
    return np.searchsorted(np.asarray(offsets, dtype=np.int64), rows, side="right") - 1


def oracle_entries(q, scale, rows, cols, row_tok, experts, ws):
    """y[r][n] for the sampled pairs; q [T][K] int codes, scale [T]."""
    ref = np.empty(len(rows), dtype=np.float64)
    for i, (r, n, e) in enumerate(zip(rows, cols, experts)):
        t = int(row_tok[r]) if row_tok is not None else int(r)
        ref[i] = oracle.gemm_entry(q[t], float(scale[t]), ws.idx[e][n], ws.codebook[e][n],
                                   ws.K, ws.bits)
    return ref


def run_bench_phase(wl, W, x, lg, decode):
    """Route once to pick the paths exactly as the benchmark does, then run its
    MoEPhase and return it (all buffers filled)."""
    counts = np.diff(cbq.moe_route_gather(to_dev(lg), wl.topk, True, wl.n_shared)["offsets"]
                     .cpu().numpy()[: wl.E + 1])
    path = bench.choose_path(cbq, counts, wl.E)
    ph = bench.MoEPhase(cbq, torch, wl, W, x, lg, path, path)
    ph.run()
    torch.cuda.synchronize()
    return ph, path


def check_moe_phase(wl, host, ph, x, lg, seed, extra_paths=()):
    """Every stage of one MoE layer against the oracle (teacher forced)."""
    T, a = x.shape[0], wl.act_bits
    # stage 1: rotate + quantise of the layer input, all tokens, bit-exact
    rq = oracle.rotate_quantize(x, 0, a)
    assert rq["ok"].all()
    assert np.array_equal(ph.codes.cpu().numpy(), rq["codes"]), "x codes"
    assert np.array_equal(ph.scales.cpu().numpy(), rq["scale"]), "x scales"
    # stage 2: routing, bit-exact ids / lists, weights within 1e-6
    rt = oracle.route(lg, wl.topk, True, wl.n_shared)
    for key in ("ids", "offsets", "sorted_tokens", "slot_of"):
        assert np.array_equal(ph.rt[key].cpu().numpy(), rt[key]), key
    assert np.abs(ph.rt["weights"].cpu().numpy().astype(np.float64) - rt["weights64"]).max() <= 1e-6
    offs, toks = rt["offsets"], rt["sorted_tokens"]
    R = len(toks)
    rng = np.random.default_rng(seed)
    # stage 3: gate/up GEMM with SwiGLU on sampled entries
    q_x = rq["q"].astype(np.int64)
    rows, cols = sample_entries(rng, offs, R, wl.F)
    ex = expert_of(offs, rows)
    g = oracle_entries(q_x, rq["scale"], rows, cols, toks, ex, host["gate"])
    u = oracle_entries(q_x, rq["scale"], rows, cols, toks, ex, host["up"])
    h_ref = oracle.silu_mul_bf16(g, u)
    h_gpu = bf16_to_bits(ph.h)
    assert_bf16_close(h_gpu[rows, cols], h_ref, "gate/up SwiGLU")
    # stage 4: rotate + quantise of the GPU's h, all rows, bit-exact
    rqh = oracle.rotate_quantize(h_gpu, 0, a)
    assert np.array_equal(ph.codes_h.cpu().numpy(), rqh["codes"]), "h codes"
    assert np.array_equal(ph.scales_h.cpu().numpy(), rqh["scale"]), "h scales"
    # stage 5: down GEMM on the GPU's h codes, sampled
    q_h = oracle.unpack_codes(ph.codes_h.cpu().numpy(), wl.F, a)
    s_h = ph.scales_h.cpu().numpy()
    rows_d, cols_d = sample_entries(rng, offs, R, wl.H)
    ex_d = expert_of(offs, rows_d)
    d_ref = oracle_entries(q_h, s_h, rows_d, cols_d, None, ex_d, host["down"])
    out_gpu = ph.out.cpu().numpy()
    assert_normwise(out_gpu[rows_d, cols_d], d_ref, 1e-3, "down")
    # stage 6: combine of the GPU's expert outputs, all tokens
    y_ref = oracle.combine(out_gpu, rt["slot_of"], rt["weights"], T, wl.topk, wl.n_shared)
    assert_normwise(ph.y.cpu().numpy(), y_ref, 1e-3, "combine")
    # the other GEMM paths on the same inputs and samples
    for p in extra_paths:
        h2 = cbq.codebook_lut_gemm(ph.codes, ph.scales, a, [ph.W["gate"], ph.W["up"]],
                                   expert_offsets=ph.rt["offsets"],
                                   row_token=ph.rt["sorted_tokens"], path=p)
        o2 = cbq.codebook_lut_gemm(ph.codes_h, ph.scales_h, a, [ph.W["down"]],
                                   expert_offsets=ph.rt["offsets"], path=p)
        torch.cuda.synchronize()
        assert_bf16_close(bf16_to_bits(h2)[rows, cols], h_ref, f"gate/up path {p}")
        assert_normwise(o2.cpu().numpy()[rows_d, cols_d], d_ref, 1e-3, f"down path {p}")
    return rq, rt


# ---------------------------------------------------------------------------
# 4-token 256x256 linear, A4, 4-bit codebooks: every output
def test_dense256_full():
    wl = datagen.WORKLOADS["dense256"]
    ws = datagen.dense_weights(wl)
    T = wl.T_list[0]
    x = datagen.dense_tokens(wl, T)
    codes, scales = cbq.rotate_quantize(bf16_dev(x), wl.act_bits)
    y = cbq.codebook_lut_gemm(codes, scales, wl.act_bits, [bench_weights(ws)])
    torch.cuda.synchronize()
    rq = oracle.rotate_quantize(x, 0, wl.act_bits)
    assert np.array_equal(codes.cpu().numpy(), rq["codes"])
    assert np.array_equal(scales.cpu().numpy(), rq["scale"])
    ref = oracle.expert_gemm(rq["q"], rq["scale"], None, None, ws.idx, ws.codebook, ws.K, ws.bits)
    assert_normwise(y.cpu().numpy(), ref, 1e-3, "dense256")


# ---------------------------------------------------------------------------
# 2560 -> 9728 and 9728 -> 2560 decode linears, T in {1, 4, 16}, A4 and A8
_DENSE = {}


def dense_setup(which):
    if which not in _DENSE:
        wl = datagen.WORKLOADS["dense2560x9728"]
        ws = datagen.dense_weights(wl, which)
        Wd = oracle.dequantize(oracle.unpack_indices(ws.idx[0], ws.K, ws.bits), ws.codebook[0])
        _DENSE[which] = (wl, ws, bench_weights(ws), Wd)
    return _DENSE[which]


@pytest.mark.parametrize("which", ["gate_up", "down"])
@pytest.mark.parametrize("T", [1, 4, 16])
@pytest.mark.parametrize("act_bits", [4, 8])
def test_dense_decode_linear_full(which, T, act_bits):
    wl, ws, Wg, Wd = dense_setup(which)
    x = datagen.dense_tokens(wl, T, which)
    codes, scales = cbq.rotate_quantize(bf16_dev(x), act_bits)
    for path in (cbq.PATH_AUTO, cbq.PATH_MFMA):
        y = cbq.codebook_lut_gemm(codes, scales, act_bits, [Wg], path=path)
        torch.cuda.synchronize()
        if path == cbq.PATH_AUTO:
            rq = oracle.rotate_quantize(x, 0, act_bits)
            assert np.array_equal(codes.cpu().numpy(), rq["codes"])
            assert np.array_equal(scales.cpu().numpy(), rq["scale"])
            ref = oracle.dense_gemm(rq["q"].astype(np.int64), rq["scale"], Wd)
        assert_normwise(y.cpu().numpy(), ref, 1e-3, f"{which} T={T} A{act_bits} path {path}")


# ---------------------------------------------------------------------------
# 128-expert top-8 MoE, decode batches 1 / 8 / 64
@pytest.mark.parametrize("T", [1, 8, 64])
def test_moe128_decode_layer(T):
    wl, host, W = moe_setup("moe128_h2048_f768")
    x, lg = datagen.moe_tokens(wl, T)
    ph, path = run_bench_phase(wl, W, x, lg, decode=True)
    assert path == cbq.PATH_LUT
    check_moe_phase(wl, host, ph, x, lg, seed=100 + T,
                    extra_paths=(cbq.PATH_MFMA, cbq.PATH_PAGES_PRODUCTS, cbq.PATH_PAGES_BUCKETS))


def _flips(ph, ref):
    """h-code bytes that differ from the free-running oracle, and the bound they are held
    to.  A GPU h value differs from the exactly rounded one only when its fp32 value
    (fp32 sums, hardware exp2 and reciprocal: a relative error of about 1e-6) lands on
    the other side of a bf16 rounding midpoint, for about 5e-4 of the values.  Such a
    one-step change moves the codes of its 128-channel block by under 1e-3 of a
    quantisation step, so it flips a code with probability about 2e-3: roughly 1e-4 of
    the codes flip.  The bound is 1e-4 of the codes (two per byte for A4), at least 4."""
    got = ph.codes_h.cpu().numpy()
    flips = int((got != ref["rqh"]["codes"]).sum())
    n_codes = got.size * (8 // 4 if ph.wl.act_bits == 4 else 1)
    return flips, max(4, int(1e-4 * n_codes))


@pytest.mark.parametrize("T", [1, 8])
def test_moe128_free_running(T):
    """Oracle end to end from x (no teacher forcing) on the small decode batches."""
    wl, host, W = moe_setup("moe128_h2048_f768")
    x, lg = datagen.moe_tokens(wl, T)
    ph, _ = run_bench_phase(wl, W, x, lg, decode=True)
    ref = oracle.moe_layer(x, lg, host["gate"], host["up"], host["down"], wl.topk, wl.n_shared,
                           wl.act_bits)
    flips, bound = _flips(ph, ref)
    err = assert_normwise(ph.y.cpu().numpy(), ref["y"], 2e-2, "free-running y")
    print(f"moe128 T={T}: free-running normwise {err:.2e}, h-code byte flips {flips} "
          f"(bound {bound})")
    assert flips <= bound
    if flips == 0:
        assert err <= 1e-3


# ---------------------------------------------------------------------------
# 8-expert top-2 MoE, 512-token prefill, A8: MFMA path, and the forced LUT path
def test_moe8_prefill_layer():
    wl, host, W = moe_setup("moe8_h4096_f14336")
    x, lg = datagen.moe_tokens(wl, 512)
    ph, path = run_bench_phase(wl, W, x, lg, decode=False)
    assert path == cbq.PATH_MFMA
    # the benchmark's gate/up call carries the workspace of its tail K split, and the down
    # call that of its K split
    assert ph.ws_gu is not None and ph.ws_dn is not None
    check_moe_phase(wl, host, ph, x, lg, seed=300, extra_paths=(cbq.PATH_LUT,))


# ---------------------------------------------------------------------------
# 64 + 2 expert top-6 MoE, 3-bit gate/up and 2-bit down: 4096-token prefill, then a
# 32-token decode batch (the benchmark's workload)
def test_moe64s2_prefill_layer():
    wl, host, W = moe_setup("moe64s2_h2048_f1408")
    x, lg = datagen.moe_tokens(wl, 4096)
    ph, path = run_bench_phase(wl, W, x, lg, decode=False)
    assert path == cbq.PATH_MFMA
    check_moe_phase(wl, host, ph, x, lg, seed=400)


def test_moe64s2_decode_layer():
    wl, host, W = moe_setup("moe64s2_h2048_f1408")
    x, lg = datagen.moe_tokens(wl, 32, decode=True)
    ph, path = run_bench_phase(wl, W, x, lg, decode=True)
    # the shared experts hold 32 rows each: every expert takes the LUT path
    assert path == cbq.PATH_LUT
    check_moe_phase(wl, host, ph, x, lg, seed=401, extra_paths=(cbq.PATH_MFMA, cbq.PATH_AUTO))


def test_moe64s2_decode_free_running():
    wl, host, W = moe_setup("moe64s2_h2048_f1408")
    x, lg = datagen.moe_tokens(wl, 32, decode=True)
    ph, _ = run_bench_phase(wl, W, x, lg, decode=True)
    ref = oracle.moe_layer(x, lg, host["gate"], host["up"], host["down"], wl.topk, wl.n_shared,
                           wl.act_bits)
    flips, bound = _flips(ph, ref)
    err = assert_normwise(ph.y.cpu().numpy(), ref["y"], 2e-2, "free-running y")
    print(f"moe64s2 decode: free-running normwise {err:.2e}, h-code byte flips {flips} "
          f"(bound {bound})")
    assert flips <= bound
    if flips == 0:
        assert err <= 1e-3


def test_moe64s2_two_streams_match_one_stream():
    """The benchmark's step runs the decode batch on a second stream beside the prefill
    batch.  The calls keep no global state and every kernel is deterministic, so each
    output of both batches must be bit-identical to the one-stream step, on every
    repetition."""
    wl, host, W = moe_setup("moe64s2_h2048_f1408")
    phases = []
    for T, decode in ((4096, False), (32, True)):
        x, lg = datagen.moe_tokens(wl, T, decode=decode)
        ph, _ = run_bench_phase(wl, W, x, lg, decode=decode)
        phases.append(ph)

    def outputs(ph):
        d = dict(codes=ph.codes, scales=ph.scales, h=ph.h, codes_h=ph.codes_h,
                 scales_h=ph.scales_h, out=ph.out, y=ph.y)
        d.update({"rt_" + k: v for k, v in ph.rt.items() if k != "ws"})
        return d

    bench.run_mixed_step(torch, phases)
    torch.cuda.synchronize()
    ref = [{k: v.clone() for k, v in outputs(ph).items()} for ph in phases]
    side = torch.cuda.Stream()
    for rep in range(3):
        for ph in phases:
            for v in outputs(ph).values():
                v.view(torch.uint8).fill_(0xA5)     # stale values must not survive
        torch.cuda.synchronize()
        bench.run_mixed_step(torch, phases, side)
        torch.cuda.synchronize()
        for i, ph in enumerate(phases):
            for k, v in outputs(ph).items():
                assert torch.equal(v.view(torch.uint8), ref[i][k].view(torch.uint8)), \
                    f"phase {i} output {k} differs on repetition {rep}"
