"""Helpers for the GPU parity tests: uploads and the tolerance checks.

Tolerances (derived from the arithmetic):
* integer outputs (codes, ids, offsets, row lists) and fp32 scales: bit-exact;
* routing weights: |gpu - oracle| <= 1e-6 (fp32 exp/sum vs fp64);
* fp32 GEMM / combine outputs: normwise max|gpu - ref| / max|ref| <= 1e-3; the
  products are exact in every path and only the fp32 summation order differs;
* bf16 SwiGLU outputs: |gpu - ref| <= 2^-8 |ref| + 1e-3 max|ref| elementwise (one
  bf16 rounding step may land on the other side of a tie after fp32 rounding).
"""
import numpy as np
import torch

import codebook_bit_quantized_amd as cbq

DEV = "cuda:0"


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def upload_weights(ws):
    """datagen.WeightSet -> CodebookWeights on the GPU."""
    return cbq.CodebookWeights(idx=to_dev(ws.idx), codebook=to_dev(ws.codebook.view(np.int16)),
                               K=ws.K, bits=ws.bits)


def bf16_dev(bits_u16):
    return to_dev(bits_u16.view(np.int16)).view(torch.bfloat16)


def bf16_to_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def normwise(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / (m if m > 0 else 1.0))


def assert_normwise(gpu, ref, tol=1e-3, what=""):
    err = normwise(gpu, ref)
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol:.1e}"
    return err


def assert_bf16_close(gpu_bits, ref_bits, what=""):
    g = (np.asarray(gpu_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (np.asarray(ref_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = np.abs(r).max()
    bound = 2.0 ** -8 * np.abs(r) + 1e-3 * m
    bad = np.abs(g - r) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} bf16 outputs outside tolerance; worst " \
                          f"{float(np.abs(g - r).max()):.3e} (max|ref| {m:.3e})"
    return float(np.mean(g != r))
