"""Seeded synthetic inputs for the codebook-LUT MoE path.

This module only draws random numbers and encodes them in the storage formats the
path consumes (bf16 / fp16 bit patterns, LSB-first packed index bitstreams).  It
holds none of the method's arithmetic: no rotation, quantisation, lookup, routing
or combine.  Both the CPU oracle's tests and the GPU tests/benchmark draw their
inputs from here, so the two sides always see the same bytes.

Distributions (shapes of the models the CodeQuant / CodeQuant2 pages evaluate:
Qwen3-4B-like dense linears, Qwen3-30B-A3B-like and Mixtral-8x7B-like MoE layers,
and a 64-routed + 2-shared expert layer with mixed 2/3-bit codebooks):

* activations: fp32 N(0,1), channels 3 and 77 multiplied by 40, rounded once to
  bf16 (round-to-nearest-even);
* codebook row: 2^bits fp32 draws from N(0, 0.02) (0.02 read as the standard
  deviation), sorted ascending, the last entry replaced by +8 sigma = 0.16, rounded
  to fp16;
* indices: uniform over 0 .. 2^bits-2 with probability 255/256, and 2^bits-1 with
  probability 1/256; packed per row as an LSB-first bitstream (index k occupies
  bits [k*bits, (k+1)*bits) of the row);
* router logits: fp32 N(0,1).

Every tensor is drawn from ``Generator(PCG64(SeedSequence([workload_id, tag,
expert])))`` so any single expert can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# tensor tags used in the seed sequence
TAG_X = 1
TAG_LOGITS = 2
TAG_X_DECODE = 3
TAG_LOGITS_DECODE = 4
TAG_X_DOWN = 5
TAG_GATE_IDX = 10
TAG_GATE_CB = 11
TAG_UP_IDX = 12
TAG_UP_CB = 13
TAG_DOWN_IDX = 14
TAG_DOWN_CB = 15
TAG_W_FULL = 16        # full-precision weights (input of codebook construction)
TAG_ROT = 17           # dense rotation matrices
TAG_MISC = 99

OUTLIER_CHANNELS = (3, 77)
OUTLIER_GAIN = 40.0
CODEBOOK_SIGMA = 0.02
CODEBOOK_TOP = 8.0 * CODEBOOK_SIGMA  # 0.16


def rng_for(workload_id: int, tag: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tag, expert])))


# ---------------------------------------------------------------------------
# storage encodings (bit patterns); no method arithmetic
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def pack_lsb_first(idx: np.ndarray, bits: int) -> np.ndarray:
    """Pack an integer array [..., K] (values < 2^bits) into an LSB-first bitstream
    per leading row: index k occupies bits [k*bits, (k+1)*bits).  K*bits must be a
    multiple of 8.  Returns uint8 [..., K*bits/8]."""
    idx = np.asarray(idx)
    K = idx.shape[-1]
    if (K * bits) % 8:
        raise ValueError("K*bits must be a multiple of 8")
    lead = idx.shape[:-1]
    flat = idx.reshape(-1, K).astype(np.uint8)
    if bits == 8:
        return flat.reshape(*lead, K).copy()
    if bits in (2, 4):
        per = 8 // bits
        g = flat.reshape(flat.shape[0], K // per, per).astype(np.uint32)
        out = np.zeros(g.shape[:2], dtype=np.uint32)
        for j in range(per):
            out |= g[:, :, j] << (j * bits)
        return out.astype(np.uint8).reshape(*lead, K * bits // 8)
    # generic path (3-bit and anything else): expand to bits, pack little-endian
    bitplanes = ((flat[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    packed = np.packbits(bitplanes.reshape(flat.shape[0], K * bits), axis=1, bitorder="little")
    return packed.reshape(*lead, K * bits // 8)


# ---------------------------------------------------------------------------
# primitive generators
def activations_bf16(workload_id: int, tag: int, T: int, K: int) -> np.ndarray:
    """bf16 bit patterns [T][K]: N(0,1) with the outlier channels scaled by 40."""
    g = rng_for(workload_id, tag)
    x = g.standard_normal((T, K), dtype=np.float32)
    for c in OUTLIER_CHANNELS:
        if c < K:
            x[:, c] *= np.float32(OUTLIER_GAIN)
    return f32_to_bf16_bits(x)


def logits_f32(workload_id: int, tag: int, T: int, E: int) -> np.ndarray:
    g = rng_for(workload_id, tag)
    return g.standard_normal((T, E), dtype=np.float32)


def codebook_f16(workload_id: int, tag: int, expert: int, N: int, bits: int) -> np.ndarray:
    """fp16 bit patterns [N][2^bits]: sorted N(0,0.02) draws, top entry = 0.16."""
    g = rng_for(workload_id, tag, expert)
    c = g.standard_normal((N, 1 << bits), dtype=np.float32) * np.float32(CODEBOOK_SIGMA)
    c.sort(axis=1)
    c[:, -1] = np.float32(CODEBOOK_TOP)
    return f32_to_f16_bits(c)


def indices_u8(workload_id: int, tag: int, expert: int, N: int, K: int, bits: int) -> np.ndarray:
    """Unpacked indices [N][K]: the top index with probability 1/256, the others uniform."""
    g = rng_for(workload_id, tag, expert)
    L = (1 << bits) - 1
    v = g.integers(0, 256 * L, size=(N, K), dtype=np.uint32)
    out = (v % L).astype(np.uint8)
    out[v < L] = L
    return out


def weights_bf16(workload_id: int, tag: int, expert: int, N: int, K: int) -> np.ndarray:
    """bf16 bit patterns [N][K] of full-precision weights: N(0, 0.02) draws with one
    entry in 256 scaled by 8 (weight outliers)."""
    g = rng_for(workload_id, tag, expert)
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(CODEBOOK_SIGMA)
    w[g.random((N, K)) < 1.0 / 256.0] *= np.float32(8.0)
    return f32_to_bf16_bits(w)


# ---------------------------------------------------------------------------
@dataclass
class WeightSet:
    """One weight matrix type for E experts: packed indices + fp16 codebooks."""
    E: int
    N: int
    K: int
    bits: int
    idx: np.ndarray       # uint8 [E][N][K*bits/8]
    codebook: np.ndarray  # uint16 [E][N][2^bits] (fp16 patterns)
    raw: Optional[np.ndarray] = None  # uint8 [E][N][K] unpacked indices (kept on request)


def weight_set(workload_id: int, idx_tag: int, cb_tag: int, E: int, N: int, K: int, bits: int,
               keep_raw: bool = False) -> WeightSet:
    idx = np.empty((E, N, K * bits // 8), dtype=np.uint8)
    cb = np.empty((E, N, 1 << bits), dtype=np.uint16)
    raw = np.empty((E, N, K), dtype=np.uint8) if keep_raw else None
    for e in range(E):
        r = indices_u8(workload_id, idx_tag, e, N, K, bits)
        idx[e] = pack_lsb_first(r, bits)
        cb[e] = codebook_f16(workload_id, cb_tag, e, N, bits)
        if keep_raw:
            raw[e] = r
    return WeightSet(E, N, K, bits, idx, cb, raw)


# ---------------------------------------------------------------------------
# workloads
@dataclass
class Workload:
    name: str
    wid: int                      # seed namespace
    kind: str                     # "dense" or "moe"
    act_bits: int
    # dense
    K: int = 0
    N: int = 0
    bits: int = 4
    # moe
    H: int = 0
    F: int = 0
    E: int = 0
    topk: int = 0
    n_shared: int = 0
    bits_gate_up: int = 4
    bits_down: int = 4
    T_list: Tuple[int, ...] = ()
    note: str = ""


WORKLOADS: Dict[str, Workload] = {
    # one linear, 1 expert: 4 tokens, K = N = 256, A4, 4-bit codebooks
    "dense256": Workload("dense256", 0, "dense", 4, K=256, N=256, bits=4, T_list=(4,),
                         note="single 256x256 linear, 4 tokens, A4, 4-bit codebooks"),
    # Qwen3-4B-like decode linears (hidden 2560, intermediate 9728), batches 1/4/16, A4 and A8
    "dense2560x9728": Workload("dense2560x9728", 1, "dense", 4, K=2560, N=9728, bits=4,
                               T_list=(1, 4, 16),
                               note="gate/up 2560->9728 and down 9728->2560 decode linears"),
    # Qwen3-30B-A3B-like MoE decode: H 2048, 128 experts, top-8, FFN 768, A4
    "moe128_h2048_f768": Workload("moe128_h2048_f768", 2, "moe", 4, H=2048, F=768, E=128,
                                  topk=8, bits_gate_up=4, bits_down=4, T_list=(1, 8, 64),
                                  note="128-expert top-8 MoE decode batches 1/8/64"),
    # Mixtral-8x7B-like MoE prefill chunk: H 4096, 8 experts, top-2, FFN 14336, A8
    "moe8_h4096_f14336": Workload("moe8_h4096_f14336", 3, "moe", 8, H=4096, F=14336, E=8,
                                  topk=2, bits_gate_up=4, bits_down=4, T_list=(512,),
                                  note="8-expert top-2 MoE, 512-token prefill chunk, A8"),
    # 64 routed + 2 shared experts, top-6, FFN 1408, 3-bit gate/up and 2-bit down, A4;
    # a 4096-token prefill followed by a 32-token decode batch
    "moe64s2_h2048_f1408": Workload("moe64s2_h2048_f1408", 4, "moe", 4, H=2048, F=1408, E=64,
                                    topk=6, n_shared=2, bits_gate_up=3, bits_down=2,
                                    T_list=(4096, 32),
                                    note="64+2-expert top-6 MoE, 3/2-bit codebooks, "
                                         "prefill 4096 then decode 32"),
}


@dataclass
class MoEInputs:
    x: np.ndarray          # bf16 bits [T][H]
    logits: np.ndarray     # fp32 [T][E]
    gate: WeightSet        # [E+S][F][H]
    up: WeightSet
    down: WeightSet        # [E+S][H][F]


def moe_weights(w: Workload, keep_raw: bool = False, n_experts: Optional[int] = None):
    """Gate/up/down weight sets for all routed + shared experts (or the first
    ``n_experts`` of them)."""
    ne = (w.E + w.n_shared) if n_experts is None else n_experts
    gate = weight_set(w.wid, TAG_GATE_IDX, TAG_GATE_CB, ne, w.F, w.H, w.bits_gate_up, keep_raw)
    up = weight_set(w.wid, TAG_UP_IDX, TAG_UP_CB, ne, w.F, w.H, w.bits_gate_up, keep_raw)
    down = weight_set(w.wid, TAG_DOWN_IDX, TAG_DOWN_CB, ne, w.H, w.F, w.bits_down, keep_raw)
    return gate, up, down


def moe_tokens(w: Workload, T: int, decode: bool = False):
    tx, tl = (TAG_X_DECODE, TAG_LOGITS_DECODE) if decode else (TAG_X, TAG_LOGITS)
    return activations_bf16(w.wid, tx, T, w.H), logits_f32(w.wid, tl, T, w.E)


def dense_weights(w: Workload, which: str = "gate_up", keep_raw: bool = False) -> WeightSet:
    if which == "gate_up":
        return weight_set(w.wid, TAG_GATE_IDX, TAG_GATE_CB, 1, w.N, w.K, w.bits, keep_raw)
    if which == "down":
        return weight_set(w.wid, TAG_DOWN_IDX, TAG_DOWN_CB, 1, w.K, w.N, w.bits, keep_raw)
    raise ValueError(which)


def dense_tokens(w: Workload, T: int, which: str = "gate_up") -> np.ndarray:
    if which == "gate_up":
        return activations_bf16(w.wid, TAG_X, T, w.K)
    return activations_bf16(w.wid, TAG_X_DOWN, T, w.N)


# ---------------------------------------------------------------------------
# small random shapes for property tests (same distributions, any sizes)
def random_weights(seed: int, E: int, N: int, K: int, bits: int, keep_raw: bool = True) -> WeightSet:
    return weight_set(1000 + seed, TAG_GATE_IDX, TAG_GATE_CB, E, N, K, bits, keep_raw)


def rotation_bf16(seed: int, K: int, flush_binades: int = 7) -> np.ndarray:
    """A seeded stand-in for a learned K x K rotation, as bf16 bits [K][K].

    The matrix is Haar-random orthogonal (QR of a Gaussian matrix, column signs fixed
    by the diagonal of R); entries smaller than 2^-flush_binades of the largest are set
    to zero, so every row's nonzero exponents span at most flush_binades binades; then
    each entry is rounded once to bf16."""
    g = rng_for(seed, TAG_ROT).standard_normal((K, K))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    m = np.abs(q).max()
    q = np.where(np.abs(q) < m * 2.0 ** -flush_binades, 0.0, q)
    return f32_to_bf16_bits(q.astype(np.float32))


def random_tokens(seed: int, T: int, K: int) -> np.ndarray:
    return activations_bf16(1000 + seed, TAG_X, T, K)


def random_logits(seed: int, T: int, E: int) -> np.ndarray:
    return logits_f32(1000 + seed, TAG_LOGITS, T, E)
