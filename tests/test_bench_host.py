"""Host-side logic of bench.py, without a GPU.

* More than one GPU is refused with a message.
* The algorithmic work behind the roofline figures matches closed forms: the gate/up
  flops of the 4096-token prefill batch, and the byte counts whose weight terms equal the
  per-matrix figures derived independently for these shapes (3-bit 1408 x 2048 gate/up:
  1,081,344 index bytes and 22,528 codebook bytes per matrix; 4-bit 9728 x 2560 linear:
  12,451,840 + 311,296 bytes).
* Every committed HBM-traffic summary still matches the kernel sources it was taken
  from, so the benchmark reports its figure rather than null.
"""
import glob
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import datagen  # noqa: E402
import oracle  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counts(wl, T, decode):
    _, lg = datagen.moe_tokens(wl, T, decode=decode)
    rt = oracle.route(lg, wl.topk, True, wl.n_shared)
    return np.diff(np.asarray(rt["offsets"], dtype=np.int64))


def test_prefill_gate_up_flops():
    wl = datagen.WORKLOADS["moe64s2_h2048_f1408"]
    counts = _counts(wl, 4096, False)
    # every token has top-6 routed rows and one row per shared expert
    assert int(counts.sum()) == 4096 * (6 + 2)
    assert bench.gate_up_flops(wl, counts) == 4.0 * 4096 * 8 * 1408 * 2048


def test_decode_gate_up_bytes():
    wl = datagen.WORKLOADS["moe64s2_h2048_f1408"]
    counts = _counts(wl, 32, True)
    n_active = int((counts > 0).sum())
    R = int(counts.sum())
    assert R == 32 * 8
    per_matrix = 1_081_344 + 22_528
    codes = 32 * (2048 // 2 + 4)          # A4 codes and one fp32 scale per token
    rows = R * 4 + R * 1408 * 2           # row list, bf16 h written once
    assert bench.gate_up_bytes(wl, counts, 32) == 2 * per_matrix * n_active + codes + rows


def test_dense_linear_bytes():
    wl = datagen.WORKLOADS["dense2560x9728"]
    for T in wl.T_list:
        act = T * (2560 * wl.act_bits // 8 + 4)
        out = T * 9728 * 4
        assert bench.dense_gemm_bytes(wl, T) == 12_451_840 + 311_296 + act + out


def test_committed_traffic_follows_kernel_sources():
    # a traffic summary counts for the bench line only while its kernel's sources are the
    # ones it was measured on (their hash is stored with it); otherwise traffic is null
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt")))
    assert files
    for path in files:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        got = bench.read_traffic(kv["kernel"], kv["workload"])
        if kv["kernel_source_sha256"] == bench.source_hash(kv["kernel"]):
            assert got == float(kv["hbm_bytes_per_launch"]), os.path.basename(path)
        else:
            assert got is None, os.path.basename(path)
