"""Throughput of the codebook-LUT MoE path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole path over one batch of seeded synthetic input,
with inputs resident in HBM before the timed region (bracketed by device
synchronisation).  For an MoE workload the pass is rotate+quantise, route, gate/up
GEMM with SwiGLU, rotate+quantise of h, down GEMM and combine for every token batch
of the workload; for a dense workload it is rotate+quantise and the GEMM of each of
its two linears for every batch size.

The default workload is the 64-routed + 2-shared expert layer (hidden 2048, FFN 1408,
top-6, 3-bit gate/up and 2-bit down codebooks, A4): a 4096-token prefill batch and a
32-token decode batch, the one workload that exercises every step of the path
including both GEMM inner paths.  The decode batch runs on a second stream once the
prefill gate/up GEMM is issued, and both finish inside the step
(--decode-overlap serial runs them one after the other on one stream).

Prints one JSON line: tokens/s over the timed steps; the roofline of the dominant
kernel (the gate/up GEMM of the largest batch: against the fp16 MFMA peak when it
runs on the MFMA path, with its duration measured by HIP events on its stream inside
the timed loop; against HBM bandwidth when it runs on the LUT path, measured with the
caches flushed); the decode gate/up GEMM against HBM for a workload that has both;
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402

METRIC = "MoE LUT-GEMM tokens/s + % HBM roofline (decode) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
F64_MFMA_PEAK_TFLOPS = 78.6
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "mfma_prefill": ["codebook_bit_quantized_amd/csrc/lut_gemm_prefill.hip",
                     "codebook_bit_quantized_amd/csrc/cbq_device.hpp"],
    "lut_decode": ["codebook_bit_quantized_amd/csrc/lut_gemm_decode.hip",
                   "codebook_bit_quantized_amd/csrc/cbq_device.hpp"],
}


class CacheFlush:
    """Evicts L2 and the MALL (256 MB) before a cold measurement.

    mode "read" sums a 1 GiB buffer, leaving the caches full of clean lines.  Mode
    "write" fills it instead: that also evicts everything, but leaves up to the MALL's
    size of dirty lines whose write-back then lands inside the measured kernel and
    roughly halves the read bandwidth it sees.
    """

    def __init__(self, torch, dev, mode="read"):
        self.mode = mode
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.buf.sum()

    def __call__(self):
        if self.mode == "write":
            self.buf.fill_(1.0)
        else:
            self.buf.sum()


def cold_us(torch, flush, fn, reps):
    """Median time in us of fn() over reps launches, each after flush() (caches cold)."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) * 1000.0)
    return float(np.median(ts))


def upload_weights(cbq, torch, ws, layout="blocked", dev="cuda:0"):
    """A host weight set on the device, regrouped into the blocked index layout
    (cbq_prepack_weights) unless layout == "rows"."""
    w = cbq.CodebookWeights(idx=torch.from_numpy(ws.idx).to(dev),
                            codebook=torch.from_numpy(ws.codebook.view(np.int16)).to(dev),
                            K=ws.K, bits=ws.bits)
    if layout == "rows":
        return w
    blk = cbq.prepack_weights(w)
    torch.cuda.synchronize()
    return blk


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_hash(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
class MoEPhase:
    """Device buffers and the call sequence for one MoE layer over T tokens."""

    def __init__(self, cbq, torch, wl, W, x_bits, logits, path_gu, path_dn):
        self.cbq, self.torch, self.wl, self.W = cbq, torch, wl, W
        dev = "cuda:0"
        T, H, F, E, k, S, a = (x_bits.shape[0], wl.H, wl.F, wl.E, wl.topk, wl.n_shared, wl.act_bits)
        self.T, self.R = T, T * k + S * T
        self.x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        self.logits = torch.from_numpy(logits).to(dev)
        self.codes = torch.empty((T, H * a // 8), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((T,), dtype=torch.float32, device=dev)
        self.rt = dict(ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                       weights=torch.empty((T, k), dtype=torch.float32, device=dev),
                       offsets=torch.empty((E + S + 1,), dtype=torch.int32, device=dev),
                       sorted_tokens=torch.empty((self.R,), dtype=torch.int32, device=dev),
                       slot_of=torch.empty((T, k), dtype=torch.int32, device=dev),
                       ws=torch.empty((max(int(cbq.route_workspace(T, E, k, S)), 1),),
                                      dtype=torch.uint8, device=dev))
        self.h = torch.empty((self.R, F), dtype=torch.bfloat16, device=dev)
        self.codes_h = torch.empty((self.R, F * a // 8), dtype=torch.uint8, device=dev)
        self.scales_h = torch.empty((self.R,), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.R, H), dtype=torch.float32, device=dev)
        self.y = torch.empty((T, H), dtype=torch.float32, device=dev)
        # the GEMMs' optional workspaces (K splits where their tiles would leave CUs idle)
        nws = cbq.gemm_workspace([W["down"]], self.R, a, cbq.PATH_AUTO)
        self.ws_dn = torch.empty((nws,), dtype=torch.uint8, device=dev) if nws > 0 else None
        nws = cbq.gemm_workspace([W["gate"], W["up"]], self.R, a, cbq.PATH_AUTO)
        self.ws_gu = torch.empty((nws,), dtype=torch.uint8, device=dev) if nws > 0 else None
        self.path_gu, self.path_dn = path_gu, path_dn
        self.ev = None   # (start, end) events around the gate/up GEMM when timing it

    def run(self, stream=None, after_gate_up=None):
        cbq, wl, W = self.cbq, self.wl, self.W
        a = wl.act_bits
        cbq.rotate_quantize(self.x, a, codes=self.codes, scales=self.scales, stream=stream)
        cbq.moe_route_gather(self.logits, wl.topk, True, wl.n_shared, out=self.rt, stream=stream)
        if self.ev is not None:
            self.ev[0].record()
        cbq.codebook_lut_gemm(self.codes, self.scales, a, [W["gate"], W["up"]],
                              n_rows=self.R, expert_offsets=self.rt["offsets"],
                              row_token=self.rt["sorted_tokens"], path=self.path_gu, out=self.h,
                              ws=self.ws_gu, stream=stream)
        if self.ev is not None:
            self.ev[1].record()
        if after_gate_up is not None:
            after_gate_up()
        cbq.rotate_quantize(self.h, a, codes=self.codes_h, scales=self.scales_h, stream=stream)
        cbq.codebook_lut_gemm(self.codes_h, self.scales_h, a, [W["down"]], n_rows=self.R,
                              expert_offsets=self.rt["offsets"], path=self.path_dn, out=self.out,
                              ws=self.ws_dn, stream=stream)
        cbq.moe_combine(self.out, self.rt["slot_of"], self.rt["weights"], wl.n_shared, y=self.y,
                        stream=stream)

    def gemm_gu_only(self):
        self.cbq.codebook_lut_gemm(self.codes, self.scales, self.wl.act_bits,
                                   [self.W["gate"], self.W["up"]], n_rows=self.R,
                                   expert_offsets=self.rt["offsets"],
                                   row_token=self.rt["sorted_tokens"], path=self.path_gu,
                                   out=self.h, ws=self.ws_gu)


    def gemm_dn_only(self):
        self.cbq.codebook_lut_gemm(self.codes_h, self.scales_h, self.wl.act_bits, [self.W["down"]],
                                   n_rows=self.R, expert_offsets=self.rt["offsets"],
                                   path=self.path_dn, out=self.out, ws=self.ws_dn)


def run_mixed_step(torch, phases, side=None):
    """One step over the phases.  Without `side`, one phase after the other on the
    current stream.  With it (a prefill phase then a decode phase), the decode phase
    runs on `side`, released once the prefill gate/up GEMM is issued, and the current
    stream waits for it at the end."""
    if side is None:
        for ph in phases:
            ph.run()
        return
    main_s = torch.cuda.current_stream()

    def launch_decode():
        side.wait_stream(main_s)
        with torch.cuda.stream(side):
            phases[1].run()

    phases[0].run(after_gate_up=launch_decode)
    main_s.wait_stream(side)


class DensePhase:
    """Device buffers and the call sequence for the two decode linears of a dense
    workload over T tokens: rotate+quantise then GEMM, for 2560 -> 9728 and for
    9728 -> 2560 (each linear with its own synthetic input)."""

    def __init__(self, cbq, torch, wl, W, xs):
        self.cbq, self.torch, self.wl, self.W = cbq, torch, wl, W
        dev = "cuda:0"
        a = wl.act_bits
        self.T = xs["gate_up"].shape[0]
        self.R = self.T
        self.io = {}
        for which, x_bits in xs.items():
            K = x_bits.shape[1]
            N = W[which].N
            self.io[which] = dict(
                x=torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16),
                codes=torch.empty((self.T, K * a // 8), dtype=torch.uint8, device=dev),
                scales=torch.empty((self.T,), dtype=torch.float32, device=dev),
                out=torch.empty((self.T, N), dtype=torch.float32, device=dev))
        self.path_gu = self.path_dn = cbq.PATH_AUTO
        self.ev = None
        self.decode = True
        self.counts = np.array([self.T])

    def run(self, stream=None):
        cbq, a = self.cbq, self.wl.act_bits
        for which in ("gate_up", "down"):
            b = self.io[which]
            cbq.rotate_quantize(b["x"], a, codes=b["codes"], scales=b["scales"], stream=stream)
            if which == "gate_up" and self.ev is not None:
                self.ev[0].record()
            cbq.codebook_lut_gemm(b["codes"], b["scales"], a, [self.W[which]], path=self.path_gu,
                                  out=b["out"], stream=stream)
            if which == "gate_up" and self.ev is not None:
                self.ev[1].record()

    def gemm_gu_only(self):
        b = self.io["gate_up"]
        self.cbq.codebook_lut_gemm(b["codes"], b["scales"], self.wl.act_bits,
                                   [self.W["gate_up"]], path=self.path_gu, out=b["out"])


def choose_path(cbq, counts, routed_E):
    """The path AUTO would give every expert with rows, made explicit so each GEMM is
    one kernel launch (AUTO also launches the other path's grid, which then exits)."""
    active = counts[counts > 0]
    if active.size == 0 or active.max() <= cbq.AUTO_MAX_LUT_ROWS:
        return cbq.PATH_LUT
    if active.min() > cbq.AUTO_MAX_LUT_ROWS:
        return cbq.PATH_MFMA
    return cbq.PATH_AUTO


def gate_up_bytes(wl, counts, T):
    """Algorithmic HBM bytes of one gate/up launch: each active expert's gate and up
    indices + codebooks once, the token codes and scales once, h written once."""
    per_matrix = wl.F * wl.H * wl.bits_gate_up // 8 + wl.F * (1 << wl.bits_gate_up) * 2
    n_active = int((counts > 0).sum())
    R = int(counts.sum())
    return (2 * per_matrix * n_active + T * (wl.H * wl.act_bits // 8 + 4) + R * 4 + R * wl.F * 2)


def dense_gemm_bytes(wl, T):
    """Algorithmic HBM bytes of the 2560 -> 9728 linear: indices + codebooks once, the
    token codes and scales once, the fp32 output once."""
    return (wl.N * wl.K * wl.bits // 8 + wl.N * (1 << wl.bits) * 2 + T * (wl.K * wl.act_bits // 8 + 4)
            + T * wl.N * 4)


def gate_up_flops(wl, counts):
    return 2.0 * 2.0 * float(counts.sum()) * wl.F * wl.H


# ---------------------------------------------------------------------------
def cpu_baseline(wl, weights_np, prefill_sample: int, decode_T: int):
    """Time the oracle (as it stands) on a bounded sample of the workload on this host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    gate, up, down = weights_np
    t0 = time.perf_counter()
    ntok = 0
    for T, dec in ((prefill_sample, False), (decode_T, True)):
        x, lg = datagen.moe_tokens(wl, T if not dec else decode_T, decode=dec)
        if not dec:
            x, lg = x[:prefill_sample], lg[:prefill_sample]
        oracle.moe_layer(x, lg, gate, up, down, wl.topk, wl.n_shared, wl.act_bits)
        ntok += x.shape[0]
    dt = time.perf_counter() - t0
    return dict(value=ntok / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"oracle MoE layer on the first {prefill_sample} prefill tokens plus the "
                       f"{decode_T}-token decode batch ({ntok} tokens, {dt:.1f} s, numpy fp64, "
                       f"BLAS threads {threads})")


def cpu_baseline_dense(wl, weights_np):
    """Time the oracle on the dense workload's own inputs: rotate+quantise and the
    dequantise-then-matmul of both linears for every batch size."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    ntok = 0
    for T in wl.T_list:
        for which, ws in zip(("gate_up", "down"), weights_np):
            x = datagen.dense_tokens(wl, T, which)
            rq = oracle.rotate_quantize(x, 0, wl.act_bits)
            oracle.expert_gemm(rq["q"].astype(np.int64), rq["scale"], None, None, ws.idx,
                               ws.codebook, ws.K, ws.bits)
        ntok += T
    dt = time.perf_counter() - t0
    return dict(value=ntok / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"oracle rotate+quantise and both linears for T in {list(wl.T_list)} "
                       f"({ntok} tokens, {dt:.1f} s, numpy fp64, BLAS threads {threads})")


def bench_cpu_lut(args, cbq, torch):
    """The host LUT GEMM on the 2560 -> 9728 decode linear (4-bit, A4), T = 1/4/16, all
    host threads: tokens/s and weight GB/s against this host's measured streaming read
    rate; beside it a bf16 GEMM of the dequantised weights (torch on the CPU: the dense
    model the method replaces) and the oracle."""
    import oracle
    from codebook_bit_quantized_amd import allocation
    wl = datagen.WORKLOADS["dense2560x9728"]
    ws = datagen.dense_weights(wl, "gate_up")
    nbytes_w = ws.idx.nbytes + ws.codebook.nbytes
    big = torch.ones(1 << 28, dtype=torch.float32)            # 1 GiB, summed by all host threads
    big.sum()
    t0 = time.perf_counter()
    for _ in range(5):
        big.sum()
    stream_gbs = 5 * big.numel() * 4 / (time.perf_counter() - t0) / 1e9
    del big
    W = torch.from_numpy(allocation.dequantize_rows(ws.idx[0], ws.codebook[0], ws.K, ws.bits)
                         .astype(np.float32)).to(torch.bfloat16)
    rows = {}
    for T in wl.T_list:
        x = datagen.dense_tokens(wl, T)
        # the activation codes come from the library's rotate_quantize on the GPU
        codes_d, scales_d = cbq.rotate_quantize(
            torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16), wl.act_bits)
        rq = dict(codes=codes_d.cpu().numpy(), scale=scales_d.cpu().numpy())
        out = np.empty((T, wl.N), dtype=np.float32)
        reps = max(5, args.steps)
        t_var = {}
        for name, wide in (("avx2", False), ("avx512", True)):
            cbq.cpu_lut_gemm(rq["codes"], rq["scale"], 4, ws.idx, ws.codebook, ws.K, ws.bits,
                             out=out, avx512=wide)
            t0 = time.perf_counter()
            for _ in range(reps):
                cbq.cpu_lut_gemm(rq["codes"], rq["scale"], 4, ws.idx, ws.codebook, ws.K, ws.bits,
                                 out=out, avx512=wide)
            t_var[name] = (time.perf_counter() - t0) / reps
        t_lut = t_var["avx512"]
        xb = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
        torch.matmul(xb, W.t())
        t0 = time.perf_counter()
        for _ in range(reps):
            torch.matmul(xb, W.t())
        t_bf16 = (time.perf_counter() - t0) / reps
        rows[T] = dict(lut_us=round(t_lut * 1e6, 1), lut_avx2_us=round(t_var["avx2"] * 1e6, 1),
                       bf16_us=round(t_bf16 * 1e6, 1),
                       speedup_vs_bf16=round(t_bf16 / t_lut, 2),
                       weight_gbs=round(nbytes_w / t_lut / 1e9, 1))
    T = max(wl.T_list)
    cpu = None
    if not args.no_cpu_baseline:
        x = datagen.dense_tokens(wl, T)
        t0 = time.perf_counter()
        rq = oracle.rotate_quantize(x, 0, wl.act_bits)
        oracle.expert_gemm(rq["q"].astype(np.int64), rq["scale"], None, None, ws.idx, ws.codebook,
                           ws.K, ws.bits)
        dt = time.perf_counter() - t0
        cpu = dict(value=round(T / dt, 2), unit="tokens/s", cores=1, kind="oracle",
                   sample=f"oracle rotate+quantise and dequantise-then-matmul of the 2560->9728 "
                          f"linear for {T} tokens ({dt:.2f} s, numpy fp64)")
    # tokens/s over one pass of every batch size; roofline of the single-token GEMV
    t_all = sum(r["lut_us"] for r in rows.values()) / 1e6
    tokens = sum(wl.T_list)
    t_lut = rows[min(wl.T_list)]["lut_us"] / 1e6
    gbs = nbytes_w / t_lut / 1e9
    line = dict(metric="CPU LUT GEMM tokens/s", value=round(tokens / t_all, 1), unit="tokens/s",
                n_gpus=0, steps=max(5, args.steps), warmup=1, ms_per_step=round(t_all * 1e3, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
                config=dict(workload="cpu_lut_dense2560x9728", K=wl.K, N=wl.N, bits=wl.bits,
                            act_bits=wl.act_bits, host_threads=os.cpu_count(), per_batch=rows),
                roofline=dict(bound="dram", achieved=round(gbs, 1), peak=round(stream_gbs, 1),
                              unit="GB/s", frac=round(gbs / stream_gbs, 4), traffic=None,
                              kernel="cpu_lut_gemm, 1 token (weights once per call)",
                              peak_note="host streaming read rate (all threads) measured in this run"),
                cpu_baseline=cpu, host=platform.node())
    print(json.dumps(line))


def bench_latency_table(args, cbq, torch):
    """Adaptive cluster allocation on the 64 + 2 expert layer: the decode GEMMs timed
    (caches flushed) with every matrix at 2, 3 and 4 bits give the latency per matrix
    and width; a synthetic importance (the expert's share of the routed prefill tokens,
    times the K-means clustering error of synthetic bf16 weights at that width, built on
    the GPU) gives the error; the allocation minimises the summed error within the
    latency of a uniform 3-bit layer."""
    from codebook_bit_quantized_amd.allocation import allocate_bits, clustering_errors, route_share
    wl = datagen.WORKLOADS[args.workload]
    dev = "cuda:0"
    E = wl.E + wl.n_shared
    choices = (2, 3, 4)
    flush = CacheFlush(torch, dev, args.flush)

    def cold(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e) * 1000.0)
        return float(np.median(ts))

    xd, lgd = datagen.moe_tokens(wl, 32, decode=True)
    xdt = torch.from_numpy(xd.view(np.int16)).to(dev).view(torch.bfloat16)
    codes, scales = cbq.rotate_quantize(xdt, wl.act_bits)
    rt = cbq.moe_route_gather(torch.from_numpy(lgd).to(dev), wl.topk, True, wl.n_shared)
    R = rt["sorted_tokens"].shape[0]
    h = torch.empty((R, wl.F), dtype=torch.bfloat16, device=dev)
    out = torch.empty((R, wl.H), dtype=torch.float32, device=dev)

    def upw(ws):
        return upload_weights(cbq, torch, ws, args.layout, dev)

    table = {}
    for bits in choices:
        G = upw(datagen.weight_set(wl.wid, datagen.TAG_GATE_IDX, datagen.TAG_GATE_CB, E, wl.F, wl.H, bits))
        U = upw(datagen.weight_set(wl.wid, datagen.TAG_UP_IDX, datagen.TAG_UP_CB, E, wl.F, wl.H, bits))
        D = upw(datagen.weight_set(wl.wid, datagen.TAG_DOWN_IDX, datagen.TAG_DOWN_CB, E, wl.H, wl.F, bits))
        gu = cold(lambda: cbq.codebook_lut_gemm(codes, scales, wl.act_bits, [G, U],
                                                expert_offsets=rt["offsets"],
                                                row_token=rt["sorted_tokens"], path=cbq.PATH_LUT, out=h))
        ch, sh = cbq.rotate_quantize(h, wl.act_bits)
        dn = cold(lambda: cbq.codebook_lut_gemm(ch, sh, wl.act_bits, [D], expert_offsets=rt["offsets"],
                                                path=cbq.PATH_LUT, out=out))
        table[bits] = dict(decode_gate_up_us=round(gu, 2), decode_down_us=round(dn, 2))
        del G, U, D
    del flush

    # importance: share of the routed prefill tokens per expert (shared experts: all),
    # from the library's own routing of the prefill batch
    xp, lgp = datagen.moe_tokens(wl, wl.T_list[0])
    share = route_share(cbq, torch.from_numpy(lgp).to(dev), wl.topk, wl.n_shared)
    # clustering error per matrix and width on a sample of synthetic bf16 weight rows,
    # clustered on the GPU and decoded by the allocation module
    rows = 64
    kinds = (("gate", wl.F, wl.H), ("up", wl.F, wl.H), ("down", wl.H, wl.F))
    err = np.zeros((E * 3, len(choices)))
    lat = np.zeros((E * 3, len(choices)))
    for m, (name, N, K) in enumerate(kinds):
        w_np = np.concatenate([datagen.weights_bf16(wl.wid, datagen.TAG_W_FULL, 3 * e + m, rows, K)
                               for e in range(E)])
        sq = clustering_errors(cbq, torch, w_np, E, choices, 30, dev)
        err[3 * np.arange(E) + m, :] = share[:, None] * sq * (N / rows)
        key = "decode_down_us" if name == "down" else "decode_gate_up_us"
        for c, bits in enumerate(choices):
            lat[3 * np.arange(E) + m, c] = table[bits][key] / E / (1 if name == "down" else 2)
    budget = float(lat[:, 1].sum()) * 1.01      # a uniform 3-bit layer (+1 %: latency grid slack)
    bits = allocate_bits(lat, err, budget)
    pick = bits - 2
    res = dict(uniform3_error=float(err[:, 1].sum()),
               allocated_error=float(err[np.arange(len(bits)), pick].sum()),
               budget_us=round(budget, 2),
               allocated_latency_us=round(float(lat[np.arange(len(bits)), pick].sum()), 2),
               bits_histogram={str(b): int((bits == b).sum()) for b in choices},
               shared_expert_bits=[int(b) for b in bits[3 * wl.E:]])
    line = dict(metric="cluster allocation at equal decode latency", value=round(
                    res["uniform3_error"] / max(res["allocated_error"], 1e-30), 4),
                unit="error reduction vs uniform 3-bit (x)", n_gpus=1, steps=10, warmup=1,
                ms_per_step=None, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="f16", data="synthetic",
                config=dict(workload=f"allocation_{wl.name}", latency_table_us=table,
                            matrices=E * 3, sample_rows=rows),
                roofline=None, cpu_baseline=None, allocation=res, host=platform.node())
    print(json.dumps(line))


def bench_kmeans(args, cbq, torch):
    """Codebook construction for every gate matrix of the workload (E + S experts x F rows
    of H bf16 weights, 2^bits_gate_up clusters): rows/s, against the time to stream the
    rows in and the codebooks out at HBM bandwidth (the kernel is bound by its
    sort and its dependent search steps, well short of that)."""
    import oracle
    from codebook_bit_quantized_amd import allocation
    wl = datagen.WORKLOADS[args.workload]
    dev = "cuda:0"
    R, K, bits = (wl.E + wl.n_shared) * wl.F, wl.H, wl.bits_gate_up
    max_iters = 50
    w_np = datagen.weights_bf16(wl.wid, datagen.TAG_W_FULL, 0, R, K)
    w = torch.from_numpy(w_np.view(np.int16)).to(dev)
    it = torch.empty((R,), dtype=torch.int32, device=dev)
    cw = cbq.kmeans_codebooks(w, bits, max_iters, iters_done=it)
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, args.steps // 4)):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        cbq.kmeans_codebooks(w, bits, max_iters, idx=cw.idx, codebook=cw.codebook, iters_done=it)
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) / 1000.0)
    t = float(np.median(times))
    rounds = it.cpu().numpy().astype(np.int64) + 1          # the last round finds no change
    # streaming bound: the bf16 rows in, the packed indices and fp16 codebooks out
    nbytes = R * K * 2 + R * K * bits // 8 + R * (1 << bits) * 2
    gbs = nbytes / t / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        n = 64
        t0 = time.perf_counter()
        oracle.kmeans_codebooks(w_np[:n], bits, max_iters)
        dt = time.perf_counter() - t0
        cpu = dict(value=n / dt, unit="rows/s", cores=1, kind="oracle",
                   sample=f"oracle per-row K-means on the first {n} rows ({dt:.1f} s, numpy fp64)")
    # output-aware refit on 128 calibration tokens of the layer input; its effect on the
    # output error is measured on held-out tokens for a sample of rows
    n_cal = 128
    xc_np = datagen.activations_bf16(wl.wid, datagen.TAG_X_DECODE, n_cal, K)
    xt_np = datagen.activations_bf16(wl.wid + 1, datagen.TAG_X_DECODE, n_cal, K)
    xc = torch.from_numpy(xc_np.view(np.int16)).to(dev)
    cb0 = cw.codebook.clone()
    rtimes = []
    for _ in range(max(1, args.steps // 4)):
        cw.codebook.copy_(cb0)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        cbq.refit_codebooks(w, cw, xc)
        e.record()
        torch.cuda.synchronize()
        rtimes.append(s.elapsed_time(e) / 1000.0)
    tr = float(np.median(rtimes))
    rows = np.arange(0, R, max(1, R // 256))[:256]
    idx_np = cw.idx.cpu().numpy().reshape(R, -1)[rows]
    cb_before = cb0.cpu().numpy().reshape(R, -1)[rows].view(np.uint16)
    cb_after = cw.codebook.cpu().numpy().reshape(R, -1)[rows].view(np.uint16)
    err0 = allocation.output_error(w_np[rows], idx_np, cb_before, xt_np, K, bits)
    err1 = allocation.output_error(w_np[rows], idx_np, cb_after, xt_np, K, bits)
    refit = dict(rows_per_s=round(R / tr, 1), ms=round(tr * 1000.0, 3), calibration_tokens=n_cal,
                 held_out_output_error_kmeans=round(err0, 5), held_out_output_error_refit=round(err1, 5),
                 sample_rows=int(len(rows)))
    line = dict(metric="codebook construction rows/s", value=round(R / t, 1), unit="rows/s",
                n_gpus=1, steps=len(times), warmup=1, ms_per_step=round(t * 1000.0, 3),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f64",
                data="synthetic",
                config=dict(workload=f"kmeans_gate_{wl.name}", rows=R, K=K, bits=bits,
                            max_iters=max_iters, mean_rounds=round(float(rounds.mean()), 2)),
                refit=refit,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None,
                              kernel="kmeans_rows", algorithmic_bytes=nbytes),
                cpu_baseline=cpu, host=platform.node())
    print(json.dumps(line))


def bench_peaks(args, torch):
    """Measured ceilings beside the vendor figures used as roofline peaks: HBM with a
    plain 1 GiB device copy and a 1 GiB read (a sum), cold launch and read floors at the
    decode GEMMs' sizes, and the fp16/bf16 matrix cores
    with library GEMMs (torch.matmul, which calls hipBLASLt), at a large square shape
    and at the 8-expert layer's per-expert shapes (about 128 rows per expert)."""
    dev = "cuda:0"

    def time_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = time_ms(lambda: dst.copy_(src), 10)
    read_ms = time_ms(lambda: src.sum(), 10)
    del src, dst
    hbm = dict(copy_GBs=round(2 * n / (copy_ms / 1000) / 1e9, 1),
               read_GBs=round(n / (read_ms / 1000) / 1e9, 1))

    # cold floors, each launch after the decode measurements' read flush: a trivial kernel
    # (launch and cold fetch of the kernel itself), and plain reads (sums) of the bytes of
    # the dense 2560 -> 9728 decode at T = 16 and of the headline decode gate/up
    flush = CacheFlush(torch, dev, "read")
    tiny = torch.zeros(1, device=dev)
    cold = dict(trivial_kernel_us=round(cold_us(torch, flush, lambda: tiny.add_(1), 30), 2))
    for name, nbytes in (("read_13MB", 13_406_272), ("read_144MB", 144_258_176)):
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        out = torch.zeros(1, dtype=torch.float32, device=dev)
        us = cold_us(torch, flush, lambda: torch.sum(buf, dim=0, out=out[0]), 30)
        cold[name] = dict(bytes=nbytes, us=round(us, 2), GBs=round(nbytes / us / 1e3, 1))
        del buf
    # the same decode GEMMs on uncompressed bf16 weights (the model the method replaces),
    # cold, through the library GEMM: the headline decode gate/up's 65 active experts (gate
    # and up side by side, 8 rows each, one batched GEMM) and the dense 2560 -> 9728 linear
    # at T = 16; both operands contiguous
    torch.manual_seed(0)
    bf16_decode = {}
    for name, E_, M, K, N in (("moe64s2_gate_up_65_experts", 65, 8, 2048, 2 * 1408),
                              ("dense_2560x9728_T16", 1, 16, 2560, 9728)):
        x = torch.randn(E_, M, K, device=dev).to(torch.bfloat16)
        w = (torch.randn(E_, K, N, device=dev) * 0.02).to(torch.bfloat16)
        o = torch.empty(E_, M, N, device=dev, dtype=torch.bfloat16)
        us = cold_us(torch, flush, lambda: torch.bmm(x, w, out=o), 20)
        wbytes = E_ * K * N * 2
        bf16_decode[name] = dict(experts=E_, rows=M, K=K, N=N, weight_bytes=wbytes, us=round(us, 2),
                                 GBs=round(wbytes / us / 1e3, 1))
        del x, w, o
    del flush

    gemms = {}
    shapes = [("square_8192", 8192, 8192, 8192),
              ("moe8_gate_up_M128", 128, 4096, 2 * 14336),
              ("moe8_down_M128", 128, 14336, 4096),
              ("moe8_gate_up_M1024", 1024, 4096, 2 * 14336)]
    torch.manual_seed(0)
    for dt_name, dt in (("fp16", torch.float16), ("bf16", torch.bfloat16)):
        for name, M, K, N in shapes:
            a = torch.randn(M, K, device=dev).to(dt)
            b = torch.randn(K, N, device=dev).to(dt)     # contiguous, no transposed view
            ms = time_ms(lambda: torch.matmul(a, b), 20)
            gemms[f"{dt_name}_{name}"] = dict(M=M, K=K, N=N, us=round(ms * 1000, 1),
                                               TFLOPs=round(2 * M * K * N / (ms / 1000) / 1e12, 1))
            del a, b
    line = dict(mode="peaks", hbm=hbm, cold=cold, bf16_decode_cold=bf16_decode,
                hbm_vendor_GBs=HBM_PEAK_GBS,
                hbm_copy_frac_of_vendor=round(hbm["copy_GBs"] / HBM_PEAK_GBS, 3),
                hbm_read_frac_of_vendor=round(hbm["read_GBs"] / HBM_PEAK_GBS, 3),
                gemm=gemms, mfma_vendor_TFLOPs=F16_MFMA_PEAK_TFLOPS,
                note="torch.matmul on ROCm dispatches fp16/bf16 GEMMs to hipBLASLt")
    print(json.dumps(line))


def bench_crossover(args, cbq, torch):
    """LUT path against MFMA path with the caches flushed, for 16 experts of exactly M
    rows each, on three matrix shapes of the workloads: where AUTO's row threshold
    should sit."""
    dev = "cuda:0"
    flush = CacheFlush(torch, dev, args.flush)

    def cold_us(fn, reps=8):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e) * 1000.0)
        ts.sort()
        return round(sum(ts[1:-1]) / (len(ts) - 2), 1)

    def upw(ws):
        return upload_weights(cbq, torch, ws, args.layout, dev)

    E = 16
    rows = []
    for (N, K, bits, n_w, label) in ((1408, 2048, 3, 2, "gate/up 3-bit, 64+2-expert layer"),
                                     (2048, 1408, 2, 1, "down 2-bit, 64+2-expert layer"),
                                     (768, 2048, 4, 2, "gate/up 4-bit, 128-expert layer")):
        Ws = [upw(datagen.random_weights(100 + i, E, N, K, bits, keep_raw=False))
              for i in range(n_w)]
        for M in (8, 16, 24, 32, 48, 64, 96, 128):
            T = E * M
            x = datagen.random_tokens(7, T, K)
            xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            codes, scales = cbq.rotate_quantize(xt, 4)
            offs = torch.arange(0, T + 1, M, dtype=torch.int32, device=dev)
            out = torch.empty((T, N), dtype=torch.bfloat16 if n_w == 2 else torch.float32,
                              device=dev)
            t = {name: cold_us(lambda: cbq.codebook_lut_gemm(codes, scales, 4, Ws,
                                                             expert_offsets=offs, path=p,
                                                             out=out))
                 for name, p in (("lut_us", cbq.PATH_LUT), ("mfma_us", cbq.PATH_MFMA))}
            rows.append(dict(shape=label, N=N, K=K, bits=bits, experts=E, rows_per_expert=M, **t))
    print(json.dumps(dict(mode="crossover", auto_max_lut_rows=cbq.AUTO_MAX_LUT_ROWS,
                          cache_flush=args.flush, results=rows)))


def bench_decode_table(args, cbq, torch):
    """Cold (caches flushed) rooflines of the decode GEMMs at every batch size the decode
    workloads name: both linears of the 4B-like dense layer at T = 1 / 4 / 16 with A4 and
    A8 activations, the gate/up GEMM of the 128-expert layer at T = 1 / 8 / 64 and of the
    64 + 2 expert layer at T = 32, against 8 TB/s.  Each GEMM runs on the LUT path with
    both codebook table placements where they differ (2- and 3-bit codebooks)."""
    dev = "cuda:0"
    flush = CacheFlush(torch, dev, args.flush)

    def entry(label, T, nbytes, us, **kw):
        gbs = nbytes / (us * 1e-6) / 1e9
        return dict(gemm=label, tokens=T, algorithmic_bytes=int(nbytes), median_us=round(us, 2),
                    achieved_GBs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4), **kw)

    reps = max(5, args.decode_reps)
    layouts = ("blocked", "rows")
    rows = []
    wl = datagen.WORKLOADS["dense2560x9728"]
    for which, (K, N) in (("gate_up", (wl.K, wl.N)), ("down", (wl.N, wl.K))):
        ws = datagen.dense_weights(wl, which)
        wbytes = N * K * wl.bits // 8 + N * (1 << wl.bits) * 2
        for layout in layouts:
            Wd = upload_weights(cbq, torch, ws, layout, dev)
            for a in (4, 8):
                for T in wl.T_list:
                    xt = torch.from_numpy(datagen.dense_tokens(wl, T, which).view(np.int16)).to(dev)
                    codes, scales = cbq.rotate_quantize(xt.view(torch.bfloat16), a)
                    out = torch.empty((T, N), dtype=torch.float32, device=dev)
                    us = cold_us(torch, flush, lambda: cbq.codebook_lut_gemm(codes, scales, a, [Wd],
                                                                             path=cbq.PATH_LUT, out=out), reps)
                    nbytes = wbytes + T * (K * a // 8 + 4) + T * N * 4
                    rows.append(entry(f"dense {K}->{N}", T, nbytes, us, act_bits=a, bits=wl.bits,
                                      layout=layout))
            del Wd
    for name, Ts in (("moe128_h2048_f768", (1, 8, 64)), ("moe64s2_h2048_f1408", (32,))):
        wl = datagen.WORKLOADS[name]
        host = datagen.moe_weights(wl)
        placements = (("lds", cbq.PATH_LDS_TABLES), ("reg", cbq.PATH_REG_TABLES)) \
            if wl.bits_gate_up <= 3 else (("reg", 0),)
        for layout in layouts:
            W = dict(zip(("gate", "up", "down"), (upload_weights(cbq, torch, w, layout, dev) for w in host)))
            for T in Ts:
                x, lg = datagen.moe_tokens(wl, T, decode=(name == "moe64s2_h2048_f1408"))
                for tname, flag in placements:
                    ph = MoEPhase(cbq, torch, wl, W, x, lg, cbq.PATH_LUT | flag, cbq.PATH_LUT | flag)
                    ph.run()
                    torch.cuda.synchronize()
                    counts = np.diff(ph.rt["offsets"].cpu().numpy().astype(np.int64))
                    us = cold_us(torch, flush, ph.gemm_gu_only, reps)
                    rows.append(entry(f"{name} gate/up+SwiGLU", T, gate_up_bytes(wl, counts, T), us,
                                      act_bits=wl.act_bits, bits=wl.bits_gate_up, tables=tname,
                                      layout=layout,
                                      active_experts=int((counts[:wl.E] > 0).sum()) + wl.n_shared))
            del W
    del flush
    print(json.dumps(dict(mode="decode_table", cache_flush=args.flush, peak_GBs=HBM_PEAK_GBS,
                          reps=reps, results=rows)))


def down_bytes(wl, counts, R):
    """Algorithmic HBM bytes of one down launch: each active expert's indices + codebooks
    once, the h codes and scales of every row once, the fp32 output once."""
    per_matrix = wl.H * wl.F * wl.bits_down // 8 + wl.H * (1 << wl.bits_down) * 2
    return per_matrix * int((counts > 0).sum()) + R * (wl.F * wl.act_bits // 8 + 4) + R * wl.H * 4


def bench_lut_forms(args, cbq, torch):
    """The 128-expert layer's decode GEMMs (gate/up with SwiGLU, and down) on the
    register-table LUT path and on the pages' two table forms (per-row product tables
    with sign folding; per-row integer buckets of the activation codes), cold (caches
    flushed) and warm, at the decode batches given by --forms-tokens."""
    dev = "cuda:0"
    flush = CacheFlush(torch, dev, args.flush)
    wl = datagen.WORKLOADS["moe128_h2048_f768"]
    host = datagen.moe_weights(wl)
    W = dict(zip(("gate", "up", "down"), (upload_weights(cbq, torch, w, args.layout, dev) for w in host)))
    forms = (("lut_reg_tables", cbq.PATH_LUT), ("pages_products", cbq.PATH_PAGES_PRODUCTS),
             ("pages_buckets", cbq.PATH_PAGES_BUCKETS))
    reps = max(5, args.decode_reps)
    rows = []
    for T in (int(t) for t in args.forms_tokens.split(",")):
        x, lg = datagen.moe_tokens(wl, T)
        for name, path in forms:
            ph = MoEPhase(cbq, torch, wl, W, x, lg, path, path)
            ph.run()
            torch.cuda.synchronize()
            counts = np.diff(ph.rt["offsets"].cpu().numpy().astype(np.int64))
            for gemm, fn, nbytes in (("gate/up+SwiGLU", ph.gemm_gu_only, gate_up_bytes(wl, counts, T)),
                                     ("down", ph.gemm_dn_only, down_bytes(wl, counts, ph.R))):
                cold = cold_us(torch, flush, fn, reps)
                warm = cold_us(torch, None, fn, reps)
                gbs = nbytes / (cold * 1e-6) / 1e9
                rows.append(dict(gemm=f"moe128_h2048_f768 {gemm}", form=name, tokens=T,
                                 max_rows_per_expert=int(counts.max()),
                                 algorithmic_bytes=int(nbytes), cold_us=round(cold, 2),
                                 warm_us=round(warm, 2), cold_frac=round(gbs / HBM_PEAK_GBS, 4)))
    del flush
    print(json.dumps(dict(mode="lut_forms", cache_flush=args.flush, layout=args.layout,
                          peak_GBs=HBM_PEAK_GBS, reps=reps, results=rows)))


def bench_dense_rotation(args, cbq, torch):
    """The dense-rotation variant of rotate_quantize on the workload's layer input
    (T prefill tokens x H channels, R a seeded H x H stand-in for a learned rotation):
    tokens/s, and the fp64 matrix-core rate of the whole call against the fp64 MFMA peak
    (the quantise pass is a few percent of it)."""
    import oracle
    wl = datagen.WORKLOADS[args.workload]
    dev = "cuda:0"
    T, K = wl.T_list[0], wl.H
    xb = datagen.activations_bf16(wl.wid, datagen.TAG_X, T, K)
    Rb = datagen.rotation_bf16(wl.wid, K)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    R = torch.from_numpy(Rb.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = torch.empty((cbq.rotate_dense_workspace(T, K),), dtype=torch.uint8, device=dev)
    codes, scales = cbq.rotate_quantize_dense(x, R, wl.act_bits, ws=ws)
    torch.cuda.synchronize()
    times = []
    for _ in range(max(3, args.steps)):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        cbq.rotate_quantize_dense(x, R, wl.act_bits, codes=codes, scales=scales, ws=ws)
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) / 1000.0)
    t = float(np.mean(times))
    flops = 2.0 * T * K * K
    tf = flops / t / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        n = 128
        t0 = time.perf_counter()
        oracle.rotate_quantize_dense(xb[:n], Rb, wl.act_bits)
        dt = time.perf_counter() - t0
        cpu = dict(value=n / dt, unit="tokens/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                   sample=f"oracle dense rotation + quantisation of the first {n} tokens "
                          f"({dt:.1f} s; numpy fp64, exact-integer fallback outside the bound)")
    line = dict(metric="dense-rotation rotate_quantize tokens/s", value=round(T / t, 1),
                unit="tokens/s", n_gpus=1, steps=len(times), warmup=1,
                ms_per_step=round(t * 1000.0, 3), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="f64", data="synthetic",
                config=dict(workload=f"dense_rotation_{wl.name}", tokens=T, K=K,
                            act_bits=wl.act_bits),
                roofline=dict(bound="mfma", achieved=round(tf, 2), peak=F64_MFMA_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(tf / F64_MFMA_PEAK_TFLOPS, 4), traffic=None,
                              kernel="dense_rot_gemm + dense_quant (whole call)",
                              avg_launch_us=round(t * 1e6, 1), algorithmic_flops=flops),
                cpu_baseline=cpu, host=platform.node())
    print(json.dumps(line))


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 untimed steps (about 0.1 s) bring the GPU clocks to their steady state; with 3,
    # the first timed steps still ran about 10 % slower
    ap.add_argument("--warmup", type=int, default=100)
    # untimed steps run for at least this long before the W warm-up steps, whatever W is:
    # with 5 warm-up steps alone the dominant kernel measured 384 us against 361 us settled
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="minimum wall time of untimed steps before the warm-up steps")
    ap.add_argument("--workload", default="moe64s2_h2048_f1408")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prefill-sample", type=int, default=4096)
    ap.add_argument("--decode-reps", type=int, default=20)
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="how caches are emptied before cold GEMM timings (see CacheFlush)")
    ap.add_argument("--cpu-lut", action="store_true",
                    help="measure the host (CPU) LUT GEMM on the dense decode linear instead")
    ap.add_argument("--latency-table", action="store_true",
                    help="measure GEMM latency per codebook width and run the cluster allocation")
    ap.add_argument("--kmeans", action="store_true",
                    help="measure offline codebook construction (per-row K-means) instead")
    ap.add_argument("--path", choices=("choose", "lut", "mfma"), default="choose",
                    help="GEMM path of every MoE phase: as AUTO would choose (default), or forced")
    ap.add_argument("--layout", choices=("blocked", "rows"), default="blocked",
                    help="index layout the GEMMs read: regrouped by cbq_prepack_weights "
                         "(default) or the row bitstreams as generated")
    ap.add_argument("--tables", choices=("default", "lds", "reg"), default="default",
                    help="where 2- and 3-bit codebooks are looked up: the library's default (LUT "
                         "path: LDS pair tables, except register tables for 3-bit blocked "
                         "weights; MFMA path: register tables), or forced for every GEMM")
    ap.add_argument("--dense-rotation", action="store_true",
                    help="measure the dense K x K rotation variant of rotate_quantize instead")
    ap.add_argument("--decode-overlap", choices=("down", "serial"), default="down",
                    help="down: the decode batch runs on a second stream, beside the prefill "
                         "batch's down projection; serial: after the prefill batch, on one stream")
    ap.add_argument("--decode-table", action="store_true",
                    help="cold HBM rooflines of every decode GEMM (dense T 1/4/16 with A4 and A8, "
                         "128-expert T 1/8/64, 64 + 2 expert T 32) instead")
    ap.add_argument("--lut-forms", action="store_true",
                    help="time the 128-expert decode GEMMs on the register-table LUT path and "
                         "the two table forms (product tables, activation buckets) instead")
    ap.add_argument("--forms-tokens", default="1,8,64",
                    help="decode batches for --lut-forms (comma separated)")
    ap.add_argument("--crossover", action="store_true",
                    help="time the LUT and MFMA paths against rows per expert instead")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the HBM and fp16/bf16 GEMM ceilings with a device copy and "
                         "library GEMMs instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for calibrating HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported (a layer "
              "would shard its experts across GPUs, which is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    import codebook_bit_quantized_amd as cbq

    if args.cpu_lut:
        bench_cpu_lut(args, cbq, torch)
        return
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    cbq.load_library()
    dev = "cuda:0"

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))
        return

    if args.kmeans:
        bench_kmeans(args, cbq, torch)
        return
    if args.latency_table:
        bench_latency_table(args, cbq, torch)
        return
    if args.peaks:
        bench_peaks(args, torch)
        return
    if args.crossover:
        bench_crossover(args, cbq, torch)
        return
    if args.decode_table:
        bench_decode_table(args, cbq, torch)
        return
    if args.lut_forms:
        bench_lut_forms(args, cbq, torch)
        return
    if args.dense_rotation:
        bench_dense_rotation(args, cbq, torch)
        return

    wl = datagen.WORKLOADS[args.workload]
    t_setup = time.perf_counter()

    def upw(ws):
        return upload_weights(cbq, torch, ws, args.layout, dev)

    tflag = {"default": 0, "reg": cbq.PATH_REG_TABLES, "lds": cbq.PATH_LDS_TABLES}[args.tables]
    phases = []
    if wl.kind == "moe":
        weights_np = datagen.moe_weights(wl)
        W = dict(gate=upw(weights_np[0]), up=upw(weights_np[1]), down=upw(weights_np[2]))
        phases_T = list(wl.T_list)
        for i, T in enumerate(phases_T):
            decode = (len(phases_T) == 2 and i == 1)
            x, lg = datagen.moe_tokens(wl, T, decode=decode)
            ph = MoEPhase(cbq, torch, wl, W, x, lg, cbq.PATH_AUTO, cbq.PATH_AUTO)
            ph.run()
            torch.cuda.synchronize()
            offs = ph.rt["offsets"].cpu().numpy().astype(np.int64)
            counts = np.diff(offs)
            ph.counts = counts
            ph.path_gu = ph.path_dn = (choose_path(cbq, counts, wl.E) if args.path == "choose" else
                                       cbq.PATH_LUT if args.path == "lut" else cbq.PATH_MFMA) | tflag
            ph.decode = decode or T <= 64
            phases.append(ph)
    else:
        weights_np = (datagen.dense_weights(wl, "gate_up"), datagen.dense_weights(wl, "down"))
        W = {"gate_up": upw(weights_np[0]), "down": upw(weights_np[1])}
        for T in wl.T_list:
            xs = {w: datagen.dense_tokens(wl, T, w) for w in ("gate_up", "down")}
            ph = DensePhase(cbq, torch, wl, W, xs)
            ph.path_gu = ph.path_dn = cbq.PATH_AUTO | tflag
            ph.run()
            phases.append(ph)
        torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # dominant kernel: the gate/up GEMM of the largest phase
    dom = max(phases, key=lambda p: p.R)
    start_evs, end_evs = [], []

    # A prefill batch and a decode batch are independent.  The decode batch runs on a
    # second stream (default priority), released once the prefill gate/up GEMM has been
    # issued, so its latency-bound kernels share the GPU with the prefill batch's
    # rotate_quantize of h and down GEMM, not with the dominant kernel.  The two streams
    # join at the end of every step, as one serving iteration would.
    side = None
    if (wl.kind == "moe" and len(phases) == 2 and phases[1].decode and not phases[0].decode
            and args.decode_overlap != "serial"):
        side = torch.cuda.Stream()

    def run_step():
        run_mixed_step(torch, phases, side)

    # clock settling: untimed steps for at least --settle-ms, checked once per 10 steps
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1000.0 < args.settle_ms:
        for _ in range(10):
            run_step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dom.ev = (s, e)
        run_step()
        start_evs.append(s)
        end_evs.append(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom.ev = None
    ms_per_step = (t1 - t0) * 1000.0 / args.steps

    # The same step with every GEMM on PATH_AUTO, as a layer that cannot read the routing
    # counts on the host runs it: each call launches both paths' grids and every expert
    # goes to the LUT path (at most 32 rows) or the MFMA path on the device.  Timed after
    # the main loop, outside it.
    # The comparison takes the host-chosen paths again right after, with no events in the
    # loop, so both sides run under the same clocks.
    auto_info = None
    if wl.kind == "moe":
        def timed_loop():
            for _ in range(args.warmup):
                run_step()
            torch.cuda.synchronize()
            ta = time.perf_counter()
            for _ in range(args.steps):
                run_step()
            torch.cuda.synchronize()
            return (time.perf_counter() - ta) * 1000.0 / args.steps

        saved = [(p.path_gu, p.path_dn) for p in phases]
        for p in phases:
            p.path_gu = p.path_dn = cbq.PATH_AUTO | tflag
        auto_ms = timed_loop()
        for p, (gu, dn) in zip(phases, saved):
            p.path_gu, p.path_dn = gu, dn
        host_ms = timed_loop()
        auto_info = dict(ms_per_step=round(auto_ms, 4),
                         tokens_per_s=round(sum(p.T for p in phases) / (auto_ms / 1000.0), 1),
                         host_choice_ms_per_step=round(host_ms, 4),
                         extra_ms_vs_host_choice=round(auto_ms - host_ms, 4))
    tokens = sum(p.T for p in phases)
    value = tokens / (ms_per_step / 1000.0)
    dom_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(start_evs, end_evs)]))

    def cold_gemm_ms(p):
        """Median duration of p's gate/up GEMM with L2 and the MALL flushed before every
        repetition (by default by reading 1 GiB)."""
        flush = CacheFlush(torch, dev, args.flush)
        times = []
        for _ in range(args.decode_reps):
            flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            p.gemm_gu_only()
            e.record()
            torch.cuda.synchronize()
            times.append(s.elapsed_time(e))
        del flush
        return float(np.median(times))

    def hbm_roofline(p, label):
        d_ms = cold_gemm_ms(p)
        if wl.kind == "moe":
            d_bytes = gate_up_bytes(wl, p.counts, p.T)
            extra = dict(active_experts=int((p.counts > 0).sum()))
        else:
            d_bytes = dense_gemm_bytes(wl, p.T)
            extra = {}
        gbs = d_bytes / (d_ms / 1000.0) / 1e9
        return dict(tokens=p.T, bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                    traffic=read_traffic("lut_decode", wl.name), kernel=label,
                    avg_launch_us=round(d_ms * 1000.0, 2), algorithmic_bytes=d_bytes,
                    cache_flush=args.flush, **extra)

    decode_info = None
    if wl.kind == "moe" and (dom.path_gu & 0xF) == cbq.PATH_MFMA:
        dom_flops = gate_up_flops(wl, dom.counts)
        achieved = dom_flops / (dom_ms / 1000.0) / 1e12
        roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=F16_MFMA_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=round(achieved / F16_MFMA_PEAK_TFLOPS, 4),
                        traffic=read_traffic("mfma_prefill", wl.name),
                        kernel="mfma_prefill gate/up+SwiGLU", avg_launch_us=round(dom_ms * 1000.0, 2),
                        algorithmic_flops=dom_flops)
        # the decode gate/up GEMM, cold caches
        dec = [p for p in phases if p.decode and p is not dom]
        if dec:
            decode_info = hbm_roofline(dec[0], "lut_decode gate/up+SwiGLU (caches flushed)")
            decode_info["median_launch_us"] = decode_info.pop("avg_launch_us")
    else:
        # every phase is decode-sized: the dominant GEMM is HBM-bound; its roofline is
        # taken with cold caches (the in-loop launches may hit the MALL)
        label = ("lut_decode gate/up+SwiGLU" if wl.kind == "moe" else
                 f"lut_decode {wl.K}->{wl.N} linear") + " (caches flushed)"
        roofline = hbm_roofline(dom, label)
        roofline["in_loop_avg_launch_us"] = round(dom_ms * 1000.0, 2)

    cpu = None
    if not args.no_cpu_baseline:
        if wl.kind == "moe":
            cpu = cpu_baseline(wl, weights_np, args.cpu_prefill_sample,
                               wl.T_list[1] if len(wl.T_list) > 1 else 32)
        else:
            cpu = cpu_baseline_dense(wl, weights_np)

    if wl.kind == "moe":
        cfg = dict(workload=wl.name, tokens_per_step=tokens, phases=[p.T for p in phases],
                   hidden=wl.H, ffn=wl.F, experts=wl.E, shared_experts=wl.n_shared, topk=wl.topk,
                   bits_gate_up=wl.bits_gate_up, bits_down=wl.bits_down, act_bits=wl.act_bits,
                   paths={str(p.T): int(p.path_gu) for p in phases},
                   decode_overlap=args.decode_overlap if side is not None else "serial")
    else:
        cfg = dict(workload=wl.name, tokens_per_step=tokens, phases=[p.T for p in phases],
                   linears=[f"{wl.K}->{wl.N}", f"{wl.N}->{wl.K}"], bits=wl.bits,
                   act_bits=wl.act_bits, paths={str(p.T): int(p.path_gu) for p in phases})
    cfg["tables"] = args.tables
    cfg["index_layout"] = args.layout
    line = dict(metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, settle_steps=settle_steps,
                ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f16", data="synthetic", config=cfg,
                roofline=roofline, decode_roofline=decode_info, auto_path_step=auto_info,
                cpu_baseline=cpu,
                setup_s=round(setup_s, 1), host=platform.node())
    print(json.dumps(line))


if __name__ == "__main__":
    main()
