"""Plain CPU definitions of the codebook-LUT MoE path (test infrastructure).

Sources (cited by page title and the section / figure on it):

* CodeQuant2 - "Enhanced Outlier Mitigation and Adaptive Clustering for Low-Precision
  LRMs" (abstract; Figure 1: the outlier-smoothing rotation and per-channel scales are
  folded into the weights, and inference runs a table-lookup kernel; Figure 3 right: a
  centroid matrix plus per-row binary assignment matrices, i.e. one codebook per weight
  row; Figure 4: the kernel builds its table once and then reads products from it
  instead of multiplying, the table sitting in on-chip shared memory; Tables 1 and 9:
  the A4W4 and A8W4 settings; Table 5 caption: the base configuration pairs a fixed
  rotation with SmoothQuant scaling).
* CodeQuant - "Unified Clustering and Quantization for Enhanced Outlier Smoothing in
  Low-Precision Mixture-of-Experts" (abstract: rotation smooths activation outliers,
  weight outliers are absorbed into cluster centroids, MoE models, dedicated LUT
  kernels); the AI Radio episode on the same paper (introduction: a router sends each
  input to an expert; "Improvements": the kernel precomputes products and looks them
  up instead of recomputing them; shared-memory bank conflicts).

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):

* rotation: the Sylvester-ordered Walsh-Hadamard matrix, H[i,j] = (-1)^popcount(i&j),
  applied block-diagonally with block b = K & -K (the largest power of two dividing
  K); codes are taken from the unnormalised rotation, the factor 1/sqrt(b) goes into
  the per-token scale;
* the rotation is computed exactly; the pinned fp32 sequence is then
  fp32(u), M = max|u|, s = fp32(M/Q), r = fp32(u/s), q = clamp(rint_half_even(r)),
  scale = fp32(s * fp32(1/sqrt(b))), with Q = 7 / clamp [-8, 7] for A4 and
  Q = 127 / clamp [-127, 127] for A8; an all-zero token gives codes 0 and scale 0;
* A4 codes are two's-complement nibbles, even k in the low nibble; A8 codes are int8;
* weight indices are an LSB-first bitstream per row (index k at bits [k*b, (k+1)*b));
* GEMM output y = scale[token] * sum_k q[token][k] * C[n][idx[n][k]];
* routing: top-k on the logits, ties to the lower expert id, softmax weights over the
  k selected (optionally over all experts), rows sorted by (expert, token);
  shared experts take every token with weight 1 after the routed rows;
* expert FFN: h = silu(g) * u rounded once to bf16, re-rotated and re-quantised;
* combine: y[t] = sum_j w[t][j] * out[slot(t, j)] (j ascending), then the shared
  experts' rows.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "sylvester_hadamard", "block_size", "bf16_bits_to_f64", "f16_bits_to_f64",
    "rotation_precondition", "rotate", "rotate_values", "smooth_and_sign", "rotate_fp64",
    "round_int_pow2_to_f32",
    "quantize", "rotate_quantize", "pack_codes", "unpack_codes", "unpack_indices",
    "dequantize", "expert_gemm", "dense_gemm", "gemm_entry", "lut_gemm_table",
    "lut_gemm_buckets", "route", "silu_mul_bf16", "round_f64_to_bf16_bits", "combine",
    "moe_layer", "ACT_LEVELS", "bf16_order_keys", "round_f64_to_f16_bits",
    "kmeans_precondition", "kmeans_row", "kmeans_codebooks",
    "dense_rotation_precondition", "rotate_dense", "rotate_quantize_dense",
    "refit_row", "refit_codebooks", "output_error",
]

# quantiser parameters per activation width: (Q, lower clamp, upper clamp)
ACT_LEVELS = {4: (7, -8, 7), 8: (127, -127, 127)}


# ---------------------------------------------------------------------------
# rotation (CodeQuant2 Figure 1; CodeQuant abstract; CodeQuant2 Table 5 caption)
def sylvester_hadamard(b: int) -> np.ndarray:
    """Sylvester construction H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]] (int64)."""
    if b < 1 or b & (b - 1):
        raise ValueError("Hadamard order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < b:
        H = np.block([[H, H], [H, -H]])
    return H


def block_size(K: int, had_block: int = 0) -> int:
    """Rotation block: K & -K when had_block == 0, else had_block (a power of two
    dividing K; 1 means no rotation)."""
    if had_block == 0:
        return K & -K
    if had_block < 1 or had_block & (had_block - 1) or K % had_block:
        raise ValueError("had_block must be a power of two dividing K")
    return had_block


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def rotation_precondition(xb: np.ndarray, b: int, sig_bits: int = 8) -> np.ndarray:
    """True where fp64 summation of a block of values is exact in any order.

    Every value with exponent e (|x| in [2^e, 2^(e+1))) and sig_bits significant bits
    (8 for bf16, 24 for fp32) is a multiple of 2^(e-sig_bits+1); the block's partial
    sums are then integers in units of 2^(e_min-sig_bits+1) whose size is below
    2^(log2 b + e_max - e_min + sig_bits).  They stay below 2^53 when
    e_max - e_min <= 53 - sig_bits - log2 b (45 - log2 b for bf16).  xb: [..., b] fp64."""
    a = np.abs(xb)
    nz = a > 0
    _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1
    big = np.int64(1 << 40)
    emax = np.where(nz, e, -big).max(axis=-1)
    emin = np.where(nz, e, big).min(axis=-1)
    spread_ok = (emax - emin) <= (53 - sig_bits - int(round(math.log2(b))))
    return spread_ok | ~nz.any(axis=-1)


def round_int_pow2_to_f32(n: int, s: int) -> np.float32:
    """Round the exact value n * 2^s (Python int n) to fp32, nearest-even."""
    if n == 0:
        return np.float32(0.0)
    sign = -1 if n < 0 else 1
    a = -n if n < 0 else n
    E = a.bit_length() - 1 + s             # a*2^s in [2^E, 2^(E+1))
    q = max(E, -126) - 23                  # spacing of fp32 numbers there
    if q <= s:
        return np.float32(sign * math.ldexp(a, s))
    sh = q - s
    m = a >> sh
    rem = a - (m << sh)
    half = 1 << (sh - 1)
    if rem > half or (rem == half and (m & 1)):
        m += 1
    with np.errstate(over="ignore"):
        return np.float32(sign * math.ldexp(m, q)) if q < 200 else np.float32(sign * np.inf)


def _exact_block_f32(xblock: np.ndarray, H: np.ndarray, sig_bits: int = 8) -> np.ndarray:
    """Exact H @ x for one block of fp64 inputs with sig_bits significant bits (bf16: 8,
    fp32: 24), rounded once to fp32."""
    vals = [float(v) for v in xblock]
    nz = [v for v in vals if v != 0.0]
    out = np.zeros(len(vals), dtype=np.float32)
    if not nz:
        return out
    s = min(math.frexp(abs(v))[1] - 1 for v in nz) - (sig_bits - 1)
    ints = [int(math.ldexp(v, -s)) for v in vals]   # exact: each v is a multiple of 2^s
    for j in range(len(vals)):
        acc = 0
        row = H[j]
        for i, n in enumerate(ints):
            if n:
                acc += n if row[i] > 0 else -n
        out[j] = round_int_pow2_to_f32(acc, s)
    return out


def rotate_fp64(x: np.ndarray, b: int) -> np.ndarray:
    """u = (I_{K/b} kron H_b) x per token, in fp64 ([T][K] -> [T][K])."""
    T, K = x.shape
    H = sylvester_hadamard(b).astype(np.float64)
    return (x.reshape(T, K // b, b) @ H).reshape(T, K)   # H is symmetric


def rotate_values(x: np.ndarray, b: int, sig_bits: int = 8) -> Tuple[np.ndarray, np.ndarray]:
    """Exact block rotation of tokens whose values (fp64 [T][K]) have sig_bits
    significant bits, rounded once to fp32.

    Returns (u32 [T][K] float32, precondition_ok [T][K/b] bool).  Blocks whose exponent
    spread breaks the fp64 exactness bound are recomputed in exact integer arithmetic,
    so u32 is always the correctly rounded exact rotation."""
    T, K = x.shape
    if K % b:
        raise ValueError("block must divide K")
    xb = x.reshape(T, K // b, b)
    ok = rotation_precondition(xb, b, sig_bits)
    u32 = rotate_fp64(x, b).astype(np.float32).reshape(T, K // b, b)
    if not ok.all():
        H = sylvester_hadamard(b)
        for t, j in zip(*np.nonzero(~ok)):
            u32[t, j] = _exact_block_f32(xb[t, j], H, sig_bits)
    return u32.reshape(T, K), ok


def rotate(x_bits: np.ndarray, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Exact block rotation of bf16 tokens, rounded once to fp32 (see rotate_values)."""
    return rotate_values(bf16_bits_to_f64(x_bits), b, 8)


def smooth_and_sign(x_bits: np.ndarray, smooth: Optional[np.ndarray] = None,
                    signs: Optional[np.ndarray] = None) -> Tuple[np.ndarray, int]:
    """The per-channel transforms applied before the Hadamard blocks (CodeQuant2,
    Figure 1: per-channel scales and a rotation, both folded into the weights, smooth the
    activation outliers; Table 5 caption: the base setting is a fixed random rotation
    with SmoothQuant scaling).

    v_c = fp32(x_c * m_c) with fp32 multipliers m (one rounding; skipped when smooth is
    None), negated where bit c of the LSB-first bitmask signs is set.  Returns (v as
    fp64 [T][K], significant bits of v: 24 after smoothing, else 8)."""
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)
    K = x32.shape[1]
    if smooth is not None:
        x32 = (x32 * np.asarray(smooth, dtype=np.float32)[None, :K]).astype(np.float32)
    v = x32.astype(np.float64)
    if signs is not None:
        bits = np.unpackbits(np.asarray(signs, dtype=np.uint8), bitorder="little")[:K].astype(bool)
        v = np.where(bits[None, :], -v, v)
    return v, (24 if smooth is not None else 8)


# ---------------------------------------------------------------------------
# activation quantisation (CodeQuant2 Tables 1 and 9: A4W4 / A8W4)
def quantize(u32: np.ndarray, b: int, act_bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token symmetric absmax quantisation of the rotated fp32 values.

    Returns (q int8 [T][K], scale float32 [T]); scale = fp32(s * fp32(1/sqrt(b)))."""
    Q, lo, hi = ACT_LEVELS[act_bits]
    u32 = np.asarray(u32, dtype=np.float32)
    M = np.max(np.abs(u32), axis=1).astype(np.float32)
    zero = M == 0
    s = (M / np.float32(Q)).astype(np.float32)
    s_safe = np.where(zero, np.float32(1), s).astype(np.float32)
    r = (u32 / s_safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(r), lo, hi).astype(np.int8)
    q[zero] = 0
    c_b = np.float32(1.0 / math.sqrt(float(b)))
    scale = (s * c_b).astype(np.float32)
    scale[zero] = 0
    return q, scale


def pack_codes(q: np.ndarray, act_bits: int) -> np.ndarray:
    """A4: byte j = (q[2j] & 15) | (q[2j+1] & 15) << 4; A8: the int8 bytes."""
    q = np.asarray(q, dtype=np.int8)
    if act_bits == 8:
        return q.view(np.uint8).copy()
    u = q.view(np.uint8) & 0x0F
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, K: int, act_bits: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    if act_bits == 8:
        return p[:, :K].view(np.int8).astype(np.int64)
    lo = (p & 0x0F).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out = np.where(out >= 8, out - 16, out)          # two's complement nibble
    return out[:, :K]


def rotate_quantize(x_bits: np.ndarray, had_block: int, act_bits: int,
                    smooth: Optional[np.ndarray] = None, signs: Optional[np.ndarray] = None):
    """(Optional smoothing and random signs,) rotation, quantisation and packing.

    Returns dict(codes=packed uint8, q=int8 [T][K], scale=float32 [T], u32, b, ok)."""
    T, K = x_bits.shape
    b = block_size(K, had_block)
    if smooth is None and signs is None:
        u32, ok = rotate(x_bits, b)
    else:
        v, sig = smooth_and_sign(x_bits, smooth, signs)
        u32, ok = rotate_values(v, b, sig)
    q, scale = quantize(u32, b, act_bits)
    return dict(codes=pack_codes(q, act_bits), q=q, scale=scale, u32=u32, b=b, ok=ok)


# ---------------------------------------------------------------------------
# dense rotation (CodeQuant2 Figure 1: a rotation fused into the model smooths the
# activation outliers; CodeQuant abstract: the rotation may be learned).  A dense
# orthogonal K x K matrix R in bf16 stands for a learned rotation: u = R x per token.
def _exponents(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """floor(log2|a|) and the nonzero mask."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, ex = np.frexp(a)
    return ex.astype(np.int64) - 1, a > 0


def dense_rotation_precondition(x_bits: np.ndarray, R_bits: np.ndarray) -> np.ndarray:
    """True for tokens whose u = R x is summed exactly by fp64 in any order.

    bf16 x with exponent e is a multiple of 2^(e-7), so every product x_k R[j][k] is a
    multiple of 2^(emin_x + emin_Rj - 14) and below 2^(emax_x + emax_Rj + 2) in size;
    the K-term partial sums stay below 2^53 units when
    (emax_x - emin_x) + (emax_Rj - emin_Rj) <= 37 - ceil(log2 K).  The check takes the
    largest row spread of R (over rows with a nonzero entry) for every j."""
    x = bf16_bits_to_f64(x_bits)
    R = bf16_bits_to_f64(R_bits)
    K = x.shape[1]
    bound = 37 - int(math.ceil(math.log2(K)))
    big = np.int64(1 << 40)
    ex, nzx = _exponents(x)
    dx = np.where(nzx, ex, -big).max(axis=1) - np.where(nzx, ex, big).min(axis=1)
    er, nzr = _exponents(R)
    rows = nzr.any(axis=1)
    if not rows.any():
        return np.ones(x.shape[0], dtype=bool)
    dr = (np.where(nzr, er, -big).max(axis=1) - np.where(nzr, er, big).min(axis=1))[rows].max()
    return (dx + dr <= bound) | ~nzx.any(axis=1)


def _exact_dense_token(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """R @ x for one token in exact integer arithmetic, each output rounded once to fp32."""
    K = x.shape[0]
    out = np.zeros(K, dtype=np.float32)
    xs = [float(v) for v in x]
    nzx = [v for v in xs if v != 0.0]
    nzr = R[R != 0]
    if not nzx or nzr.size == 0:
        return out
    sx = min(math.frexp(abs(v))[1] - 1 for v in nzx) - 7
    sr = int(min(math.frexp(abs(float(v)))[1] - 1 for v in nzr)) - 7
    nx = [int(math.ldexp(v, -sx)) for v in xs]
    for j in range(K):
        acc = 0
        for k, r in enumerate(R[j]):
            if r != 0.0 and nx[k]:
                acc += nx[k] * int(math.ldexp(float(r), -sr))
        out[j] = round_int_pow2_to_f32(acc, sx + sr)
    return out


def rotate_dense(x_bits: np.ndarray, R_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """u32 = fp32(exact R @ x) per token ([T][K] bf16 bits, R [K][K] bf16 bits).

    Returns (u32 [T][K] float32, ok [T] bool).  Tokens inside the precondition are
    summed in fp64 (exact, so any order gives the same value); the others in exact
    integer arithmetic."""
    x = bf16_bits_to_f64(x_bits)
    R = bf16_bits_to_f64(R_bits)
    ok = dense_rotation_precondition(x_bits, R_bits)
    u32 = (x @ R.T).astype(np.float32)
    for t in np.nonzero(~ok)[0]:
        u32[t] = _exact_dense_token(x[t], R)
    return u32, ok


def rotate_quantize_dense(x_bits: np.ndarray, R_bits: np.ndarray, act_bits: int):
    """Dense rotation, then the same quantiser with the factor 1 in the scale (R is
    orthonormal, so no 1/sqrt(b) normalisation is left to apply).

    Returns dict(codes=packed uint8, q=int8 [T][K], scale=float32 [T], u32, ok)."""
    u32, ok = rotate_dense(x_bits, R_bits)
    q, scale = quantize(u32, 1, act_bits)
    return dict(codes=pack_codes(q, act_bits), q=q, scale=scale, u32=u32, ok=ok)


# ---------------------------------------------------------------------------
# codebook weights (CodeQuant2 Figure 3 right: per-row centroid codebooks)
def unpack_indices(packed: np.ndarray, K: int, bits: int) -> np.ndarray:
    """LSB-first bitstream per row -> indices [..., K] (int64)."""
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    p2 = p.reshape(-1, p.shape[-1])
    bitarr = np.unpackbits(p2, axis=1, bitorder="little")[:, :K * bits]
    bitarr = bitarr.reshape(p2.shape[0], K, bits).astype(np.int64)
    idx = np.zeros((p2.shape[0], K), dtype=np.int64)
    for j in range(bits):
        idx |= bitarr[:, :, j] << j
    return idx.reshape(*lead, K)


def dequantize(idx: np.ndarray, codebook_bits: np.ndarray) -> np.ndarray:
    """W[n][k] = C[n][idx[n][k]] in fp64."""
    C = f16_bits_to_f64(codebook_bits)
    return np.take_along_axis(C, np.asarray(idx, dtype=np.int64), axis=1)


def dense_gemm(q_rows: np.ndarray, scale_rows: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y[r][n] = scale[r] * sum_k q[r][k] W[n][k] (fp64).

    The integer-by-fp16 products and their sums are exact in fp64 for every shape
    used here (multiples of 2^-24 below 2^29), so only the final scaling rounds."""
    acc = np.asarray(q_rows, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    return acc * np.asarray(scale_rows, dtype=np.float64)[:, None]


def expert_gemm(q_tokens: np.ndarray, scale_tokens: np.ndarray, row_token: Optional[np.ndarray],
                offsets: Optional[np.ndarray], idx_packed: np.ndarray, codebooks: np.ndarray,
                K: int, bits: int, experts: Optional[Sequence[int]] = None) -> np.ndarray:
    """Grouped expert GEMM over sorted rows.

    q_tokens [T][K] int codes, scale_tokens [T]; row r reads token row_token[r]
    (identity when None); rows [offsets[e], offsets[e+1]) use expert e (all rows use
    expert 0 when offsets is None).  idx_packed [E][N][K*bits/8], codebooks
    [E][N][2^bits].  Returns fp64 [R][N] (rows of experts not listed stay 0)."""
    q_tokens = np.asarray(q_tokens)
    R = len(row_token) if row_token is not None else q_tokens.shape[0]
    if offsets is None:
        offsets = np.array([0, R])
    E = len(offsets) - 1
    N = idx_packed.shape[1]
    y = np.zeros((R, N), dtype=np.float64)
    for e in (range(E) if experts is None else experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        toks = np.arange(r0, r1) if row_token is None else np.asarray(row_token[r0:r1])
        W = dequantize(unpack_indices(idx_packed[e], K, bits), codebooks[e])
        y[r0:r1] = dense_gemm(q_tokens[toks], np.asarray(scale_tokens)[toks], W)
    return y


def gemm_entry(q_row: np.ndarray, scale: float, idx_row_packed: np.ndarray,
               codebook_row: np.ndarray, K: int, bits: int) -> float:
    """One output y = scale * sum_k q[k] * C[idx[k]] (fp64), for sampled checks."""
    idx = unpack_indices(idx_row_packed[None, :], K, bits)[0]
    C = f16_bits_to_f64(codebook_row)
    return float(np.dot(np.asarray(q_row, dtype=np.float64), C[idx]) * float(scale))


def lut_gemm_table(q_rows: np.ndarray, scale_rows: np.ndarray, idx: np.ndarray,
                   codebook_bits: np.ndarray, act_bits: int) -> np.ndarray:
    """The pages' formulation (CodeQuant2 Figure 4; AI Radio 'Improvements'): for each
    weight row a table T_n[a][c] = a * C[n][c] over every activation level a is built
    once, and each product is a lookup T_n[q[k]][idx[n][k]].  Slow; tiny inputs."""
    Q, lo, hi = ACT_LEVELS[act_bits]
    C = f16_bits_to_f64(codebook_bits)                      # [N][L]
    levels = np.arange(lo, hi + 1, dtype=np.float64)        # [A]
    tables = levels[None, :, None] * C[:, None, :]          # [N][A][L]
    q = np.asarray(q_rows, dtype=np.int64)
    R, K = q.shape
    N = C.shape[0]
    y = np.zeros((R, N), dtype=np.float64)
    for n in range(N):
        Tn = tables[n]
        for r in range(R):
            y[r, n] = Tn[q[r] - lo, idx[n]].sum()
    return y * np.asarray(scale_rows, dtype=np.float64)[:, None]


def lut_gemm_buckets(q_rows: np.ndarray, scale_rows: np.ndarray, idx: np.ndarray,
                     codebook_bits: np.ndarray) -> np.ndarray:
    """Bucketed form: S[r][n][c] = sum of q[r][k] over k with idx[n][k] == c (integers),
    then y[r][n] = sum_c C[n][c] * S[r][n][c]."""
    C = f16_bits_to_f64(codebook_bits)
    q = np.asarray(q_rows, dtype=np.int64)
    R, K = q.shape
    N, L = C.shape
    y = np.zeros((R, N), dtype=np.float64)
    for n in range(N):
        onehot = (idx[n][None, :] == np.arange(L)[:, None]).astype(np.int64)   # [L][K]
        S = q @ onehot.T                                                        # [R][L]
        y[:, n] = S.astype(np.float64) @ C[n]
    return y * np.asarray(scale_rows, dtype=np.float64)[:, None]


# ---------------------------------------------------------------------------
# MoE routing (AI Radio episode introduction: a router picks the experts)
def route(logits: np.ndarray, topk: int, renormalize: bool = True, n_shared: int = 0) -> Dict:
    """Top-k routing and the per-expert row lists.

    ids[t] = the k experts with the largest logits (ties to the lower id), weights a
    softmax over the k selected logits (or over all experts when renormalize is
    False), computed in fp64 and stored fp32.  Rows are numbered expert by expert,
    tokens ascending inside an expert; shared expert s owns rows
    T*k + s*T + t.  slot_of[t][j] is the row of token t's j-th choice."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :topk].astype(np.int32)
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
    if renormalize:
        m = sel.max(axis=1, keepdims=True) if topk else np.zeros((T, 1))
        ex = np.exp(sel - m)
        w = ex / ex.sum(axis=1, keepdims=True)
    else:
        m = lg.max(axis=1, keepdims=True)
        w = np.exp(sel - m) / np.exp(lg - m).sum(axis=1, keepdims=True)
    counts = np.bincount(ids.ravel().astype(np.int64), minlength=E)[:E]
    offsets = np.zeros(E + n_shared + 1, dtype=np.int64)
    offsets[1:E + 1] = np.cumsum(counts)
    for s in range(n_shared):
        offsets[E + s + 1] = offsets[E + s] + T
    R = T * topk + n_shared * T
    sorted_tokens = np.empty(R, dtype=np.int32)
    slot_of = np.empty((T, topk), dtype=np.int32)
    for e in range(E):
        t_e, j_e = np.nonzero(ids == e)          # row-major: tokens ascending
        rows = offsets[e] + np.arange(len(t_e))
        sorted_tokens[rows] = t_e
        slot_of[t_e, j_e] = rows
    for s in range(n_shared):
        sorted_tokens[T * topk + s * T: T * topk + (s + 1) * T] = np.arange(T)
    return dict(ids=ids, weights=w.astype(np.float32), weights64=w, offsets=offsets.astype(np.int32),
                sorted_tokens=sorted_tokens, slot_of=slot_of, counts=counts)


# ---------------------------------------------------------------------------
# expert FFN activation
def round_f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 directly to bf16 (nearest, ties to even); uint16 patterns."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    q = np.maximum(ex.astype(np.int64) - 1, -126) - 7        # bf16 spacing at |x|
    r = np.rint(np.ldexp(x, -q))
    y = np.ldexp(r, q)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def silu_mul_bf16(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u = g * u / (1 + exp(-g)) in fp64, rounded once to bf16."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = g * np.asarray(u, dtype=np.float64) / (1.0 + np.exp(-g))
    return round_f64_to_bf16_bits(h)


def combine(expert_out: np.ndarray, slot_of: np.ndarray, weights: np.ndarray, T: int, topk: int,
            n_shared: int = 0) -> np.ndarray:
    """y[t] = sum_j w[t][j] * out[slot_of[t][j]] (j ascending) + sum_s out[T*k + s*T + t]."""
    out = np.asarray(expert_out, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    y = np.zeros((T, out.shape[1]), dtype=np.float64)
    for j in range(topk):
        y += w[:, j:j + 1] * out[slot_of[:, j]]
    for s in range(n_shared):
        y += out[T * topk + s * T: T * topk + (s + 1) * T]
    return y


# ---------------------------------------------------------------------------
def moe_layer(x_bits: np.ndarray, logits: np.ndarray, gate, up, down, topk: int, n_shared: int,
              act_bits: int, renormalize: bool = True, h_override: Optional[np.ndarray] = None,
              codes_h_override: Optional[Tuple[np.ndarray, np.ndarray]] = None,
              down_override: Optional[np.ndarray] = None, route_override: Optional[Dict] = None) -> Dict:
    """One MoE FFN layer, every stage kept.

    gate/up/down: objects with .idx [E+S][N][K*bits/8], .codebook, .K, .bits.  The
    *_override arguments replace a stage's input with a given tensor (teacher forcing:
    checking each stage against the oracle applied to the other side's own input)."""
    T, H = x_bits.shape
    rq = rotate_quantize(x_bits, 0, act_bits)
    rt = route(logits, topk, renormalize, n_shared) if route_override is None else route_override
    offs, toks = rt["offsets"], rt["sorted_tokens"]
    q_x = rq["q"].astype(np.int64)
    g = expert_gemm(q_x, rq["scale"], toks, offs, gate.idx, gate.codebook, gate.K, gate.bits)
    u = expert_gemm(q_x, rq["scale"], toks, offs, up.idx, up.codebook, up.K, up.bits)
    h_bits = silu_mul_bf16(g, u) if h_override is None else h_override
    if codes_h_override is None:
        rqh = rotate_quantize(h_bits, 0, act_bits)
        q_h, s_h = rqh["q"].astype(np.int64), rqh["scale"]
    else:
        rqh = None
        q_h, s_h = codes_h_override
    out = expert_gemm(q_h, s_h, None, offs, down.idx, down.codebook, down.K, down.bits)
    out_in = out if down_override is None else down_override
    y = combine(out_in, rt["slot_of"], rt["weights"], T, topk, n_shared)
    return dict(rq=rq, route=rt, gate=g, up=u, h=h_bits, rqh=rqh, out=out, y=y)


# ---------------------------------------------------------------------------
# Offline codebook construction (CodeQuant2 Figure 3 right: K-means initialises the
# centroid matrix and the per-row assignments; CodeQuant abstract: weight outliers are
# absorbed into cluster centroids).  One 1-D K-means per weight row.
def bf16_order_keys(bits: np.ndarray) -> np.ndarray:
    """uint16 keys that sort bf16 patterns in numeric order (-0 just before +0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000).astype(np.uint16)


def round_f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 once to fp16 (nearest, ties to even, subnormals kept, overflow to
    inf); uint16 patterns.  Written out on the fp16 grid so that no intermediate
    format rounds first."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    q = np.maximum(ex.astype(np.int64) - 1, -14) - 10        # fp16 spacing at |x|
    m = np.rint(np.ldexp(a, -q))                              # exact scaling, RNE
    y = np.ldexp(m, q)
    with np.errstate(over="ignore"):
        h = np.where(y >= 65520.0, np.inf, y).astype(np.float16)   # exact or inf
    h = np.where(np.signbit(x), -h, h).astype(np.float16)
    return h.view(np.uint16)


def kmeans_precondition(w_bits: np.ndarray) -> bool:
    """True when fp64 sums of any subset of the row are exact (same bound as the
    rotation: nonzero exponents spread at most 45 - ceil(log2 K) binades)."""
    w = bf16_bits_to_f64(w_bits)
    K = w.shape[-1]
    return bool(rotation_precondition(w[None, :], 1 << max(0, (K - 1).bit_length()))[0])


def kmeans_row(w_bits: np.ndarray, bits: int, max_iters: int, return_f64: bool = False):
    """Lloyd's K-means of one bf16 row into L = 2^bits clusters.

    * init: sort the row (by value; -0 before +0) and take the values at ranks
      floor((2j + 1) K / (2L)), j = 0..L-1;
    * each round: assign every weight to the centroid at the smallest |w - c| (fp64,
      ties to the lower index); stop if no assignment changed since the last round;
      otherwise every non-empty cluster's centroid becomes the mean of its weights
      (exact fp64 sum / count, one IEEE division); at most max_iters updates;
    * output: centroids rounded once to fp16, then a final assignment against the
      fp16 values (same rule).
    Returns (indices [K] int64, codebook fp16 bits [L], number of updates), plus the
    fp64 centroids before rounding when return_f64."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    w = bf16_bits_to_f64(w_bits)
    K, L = w.shape[0], 1 << bits
    order = np.argsort(bf16_order_keys(w_bits), kind="stable")
    ranks = ((2 * np.arange(L) + 1) * K) // (2 * L)
    c = w[order][ranks].copy()
    prev = None
    updates = 0
    for _ in range(max_iters):
        a = np.argmin(np.abs(w[:, None] - c[None, :]), axis=1)   # first minimum: lower index
        if prev is not None and np.array_equal(a, prev):
            break
        for j in range(L):
            m = a == j
            n = int(m.sum())
            if n:
                c[j] = math.fsum(w[m]) / n
        prev = a
        updates += 1
    cb = round_f64_to_f16_bits(c)
    a = np.argmin(np.abs(w[:, None] - f16_bits_to_f64(cb)[None, :]), axis=1)
    if return_f64:
        return a.astype(np.int64), cb, updates, c
    return a.astype(np.int64), cb, updates


def kmeans_codebooks(w_bits: np.ndarray, bits: int, max_iters: int):
    """kmeans_row over every row of w_bits [R][K]: (indices [R][K], codebooks [R][L],
    updates [R])."""
    R = w_bits.shape[0]
    idx = np.empty(w_bits.shape, dtype=np.int64)
    cb = np.empty((R, 1 << bits), dtype=np.uint16)
    it = np.empty(R, dtype=np.int64)
    for r in range(R):
        idx[r], cb[r], it[r] = kmeans_row(w_bits[r], bits, max_iters)
    return idx, cb, it


# ---------------------------------------------------------------------------
# output-aware centroid refit (the AI Radio episode on CodeQuant: the centroids are
# fine-tuned to minimise the error of the layer's output, not of the weights alone;
# CodeQuant2, Figure 1 right: centroids and assignments are tuned after clustering)
REFIT_PIVOT_REL = 1e-12


def refit_row(w_bits: np.ndarray, a: np.ndarray, cb_bits: np.ndarray, x_bits: np.ndarray):
    """New centroids for one row with its assignments a fixed.

    Minimises sum_i (sum_k X[i][k] (w_k - c[a_k]))^2 over c, with X the bf16 calibration
    activations [n][K]: with P[i][j] = sum_{k: a_k = j} X[i][k] and y = X w, the normal
    equations (P^T P) c = P^T y over the non-empty clusters, solved by Cholesky in
    cluster order.  A cluster whose pivot is at most 1e-12 of the largest diagonal
    entry (it adds nothing independent to the output) is left out and the
    factorisation restarts without it; a cluster left out keeps its old centroid and
    its share P c moves to the right-hand side.  Empty clusters keep theirs too.  The sums P and y are exact (math.fsum); P^T P and P^T y are fp64 dot
    products; the solution is rounded once to fp16.  Returns fp16 bits [L]."""
    w = bf16_bits_to_f64(np.asarray(w_bits, dtype=np.uint16))
    X = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    a = np.asarray(a, dtype=np.int64)
    L = np.asarray(cb_bits).shape[0]
    n = X.shape[0]
    P = np.zeros((n, L))
    for j in range(L):
        m = a == j
        if m.any():
            for i in range(n):
                P[i, j] = math.fsum(X[i, m])
    y = np.array([math.fsum(X[i] * w) for i in range(n)])   # bf16 x bf16 products are exact
    M = P.T @ P
    b = P.T @ y
    nonempty = [j for j in range(L) if (a == j).any()]
    active = list(nonempty)
    c = f16_bits_to_f64(np.asarray(cb_bits, dtype=np.uint16)).copy()
    while active:
        sub = M[np.ix_(active, active)]
        thr = REFIT_PIVOT_REL * max(sub.diagonal().max(), 0.0)
        Lc = np.zeros_like(sub)
        bad = None
        for p_ in range(len(active)):
            d = sub[p_, p_] - float(np.dot(Lc[p_, :p_], Lc[p_, :p_]))
            if not d > thr:
                bad = p_
                break
            Lc[p_, p_] = math.sqrt(d)
            for q in range(p_ + 1, len(active)):
                Lc[q, p_] = (sub[q, p_] - float(np.dot(Lc[q, :p_], Lc[p_, :p_]))) / Lc[p_, p_]
        if bad is not None:
            del active[bad]
            continue
        # clusters left out keep their centroid: their share of the output moves to the
        # right-hand side
        fixed = [j for j in nonempty if j not in active]
        rhs = P[:, active].T @ (y - P[:, fixed] @ c[fixed]) if fixed else b[active]
        z = np.zeros(len(active))
        for p_ in range(len(active)):
            z[p_] = (rhs[p_] - float(np.dot(Lc[p_, :p_], z[:p_]))) / Lc[p_, p_]
        sol = np.zeros(len(active))
        for p_ in reversed(range(len(active))):
            sol[p_] = (z[p_] - float(np.dot(Lc[p_ + 1:, p_], sol[p_ + 1:]))) / Lc[p_, p_]
        c[active] = sol
        break
    out = np.asarray(cb_bits, dtype=np.uint16).copy()
    new = round_f64_to_f16_bits(c)
    keep = np.zeros(L, dtype=bool)
    keep[active] = True
    out[keep] = new[keep]
    return out


def refit_codebooks(w_bits: np.ndarray, idx: np.ndarray, cb_bits: np.ndarray, x_bits: np.ndarray):
    """refit_row over every row (w_bits [R][K], idx [R][K] unpacked, cb_bits [R][L])."""
    return np.stack([refit_row(w_bits[r], idx[r], cb_bits[r], x_bits) for r in range(w_bits.shape[0])])


def output_error(w_bits: np.ndarray, idx: np.ndarray, cb_bits: np.ndarray, x_bits: np.ndarray) -> float:
    """Relative output error ||X (W - W_hat)^T||_F / ||X W^T||_F of a clustered matrix."""
    W = bf16_bits_to_f64(np.asarray(w_bits, dtype=np.uint16))
    C = f16_bits_to_f64(np.asarray(cb_bits, dtype=np.uint16))
    Wh = np.take_along_axis(C, np.asarray(idx, dtype=np.int64), axis=1)
    X = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    return float(np.linalg.norm(X @ (W - Wh).T) / np.linalg.norm(X @ W.T))

