"""ctypes binding of libcbq.so.

Argument marshalling only: every step of the path runs in the library's HIP kernels.
torch supplies device memory (output tensors are allocated here with torch) and the
current HIP stream.  There is no CPU or Python fallback: if the library is missing or
the GPU is absent, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libcbq.so")

CBQ_OK, CBQ_EINVAL, CBQ_EUNSUPPORTED, CBQ_EWORKSPACE, CBQ_EHIP = 0, -1, -2, -3, -4
EPI_F32, EPI_SWIGLU_BF16 = 0, 1
PATH_AUTO, PATH_LUT, PATH_MFMA = 0, 1, 2
PATH_PAGES_PRODUCTS, PATH_PAGES_BUCKETS = 3, 4   # the table forms (4-bit, A4; never chosen by AUTO)
PATH_REG_TABLES = 0x10   # flags: where 2-/3-bit codebooks are looked up (default: per path)
PATH_LDS_TABLES = 0x20
AUTO_MAX_LUT_ROWS = 32

# every symbol include/cbq.h declares
EXPORTED = ("cbq_rotate_quantize", "cbq_rotate_quantize_ex", "cbq_rotate_dense_workspace",
            "cbq_rotate_quantize_dense", "cbq_route_workspace", "cbq_moe_route_gather",
            "cbq_moe_route_gather_noalloc", "cbq_prepack_bytes", "cbq_prepack_weights",
            "cbq_gemm_workspace", "cbq_codebook_lut_gemm", "cbq_moe_combine",
            "cbq_kmeans_codebooks", "cbq_refit_codebooks", "cbq_cpu_lut_gemm", "cbq_status_string", "cbq_last_error",
            "cbq_version")


class CbqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


LAYOUT_ROWS, LAYOUT_BLOCKED = 0, 1


class cbq_weights(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("codebook", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcbq.so (built in-tree by codebook_bit_quantized_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libcbq.so not found at {path}; build it with "
                          "`python -m codebook_bit_quantized_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    W = ctypes.POINTER(cbq_weights)
    sig = {
        "cbq_rotate_quantize": (ctypes.c_int, [vp, i64, i32, i64, i32, i32, vp, vp, vp, vp]),
        "cbq_rotate_quantize_ex": (ctypes.c_int, [vp, i64, i32, i64, i32, i32, vp, vp, vp, vp, vp,
                                                  vp]),
        "cbq_rotate_dense_workspace": (sz, [i64, i32]),
        "cbq_rotate_quantize_dense": (ctypes.c_int, [vp, i64, i32, i64, vp, i32, vp, vp, vp, vp, sz,
                                                     vp]),
        "cbq_route_workspace": (sz, [i64, i32, i32, i32]),
        "cbq_moe_route_gather": (ctypes.c_int, [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                vp, sz, vp]),
        "cbq_moe_route_gather_noalloc": (ctypes.c_int, [vp, i64, i32, i32, i32, i32, vp, vp, vp,
                                                        vp, vp, vp]),
        "cbq_prepack_bytes": (sz, [W]),
        "cbq_prepack_weights": (ctypes.c_int, [W, vp, vp]),
        "cbq_gemm_workspace": (sz, [W, i32, i64, i32, i32]),
        "cbq_codebook_lut_gemm": (ctypes.c_int, [vp, vp, i32, i64, vp, vp, W, i32, i32, i32, vp,
                                                 i64, vp, sz, vp]),
        "cbq_moe_combine": (ctypes.c_int, [vp, vp, vp, i64, i32, i32, i32, vp, vp]),
        "cbq_kmeans_codebooks": (ctypes.c_int, [vp, i64, i32, i64, i32, i32, vp, vp, vp, vp]),
        "cbq_refit_codebooks": (ctypes.c_int, [vp, i64, i32, i64, i32, vp, vp, i32, i64, vp, vp]),
        "cbq_cpu_lut_gemm": (ctypes.c_int, [vp, vp, i32, i64, W, vp, i64, i32, i32]),
        "cbq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "cbq_last_error": (ctypes.c_char_p, []),
        "cbq_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != CBQ_OK:
        lib = load_library()
        raise CbqError(status, f"{lib.cbq_status_string(status).decode()}: "
                               f"{lib.cbq_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _require_gpu(*ts: Optional[torch.Tensor]):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("cbq operates on device tensors only")


@dataclass
class CodebookWeights:
    """One weight matrix type for E experts: packed indices and fp16 codebooks (device).
    idx is [E][N][K*bits/8] in the row layout, or the blocked layout's bytes as
    [E][N][Kp*bits/8] (Kp = K rounded up to 128) after prepack_weights."""
    idx: torch.Tensor        # uint8 [E][N][row bytes]
    codebook: torch.Tensor   # int16/uint16/float16 [E][N][2^bits]
    K: int
    bits: int
    layout: int = LAYOUT_ROWS

    @property
    def E(self) -> int:
        return self.idx.shape[0]

    @property
    def N(self) -> int:
        return self.idx.shape[1]

    def c_struct(self) -> cbq_weights:
        return cbq_weights(self.idx.data_ptr(), self.codebook.data_ptr(), self.E, self.N, self.K,
                           self.bits, self.layout)


# ---------------------------------------------------------------------------
def rotate_quantize(x: torch.Tensor, act_bits: int = 4, had_block: int = 0,
                    codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                    precond: Optional[torch.Tensor] = None, smooth: Optional[torch.Tensor] = None,
                    signs: Optional[torch.Tensor] = None, stream=None):
    """x: bf16 (or int16 bit patterns) [T][K] on the GPU -> (codes uint8, scales fp32).

    smooth (fp32 [K]) and signs (uint8 [K/8] bitmask) select cbq_rotate_quantize_ex."""
    lib = load_library()
    _require_gpu(x, smooth, signs)
    T, K = x.shape
    ldx = x.stride(0)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along channels")
    if codes is None:
        codes = torch.empty((T, K * act_bits // 8), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T,), dtype=torch.float32, device=x.device)
    if smooth is None and signs is None:
        _check(lib.cbq_rotate_quantize(_ptr(x), T, K, ldx, had_block, act_bits, _ptr(codes),
                                       _ptr(scales), _ptr(precond), _stream(stream)))
    else:
        _check(lib.cbq_rotate_quantize_ex(_ptr(x), T, K, ldx, had_block, act_bits, _ptr(smooth),
                                          _ptr(signs), _ptr(codes), _ptr(scales), _ptr(precond),
                                          _stream(stream)))
    return codes, scales


def rotate_dense_workspace(T: int, K: int) -> int:
    """Bytes of device workspace rotate_quantize_dense needs (cbq_rotate_dense_workspace)."""
    return int(load_library().cbq_rotate_dense_workspace(T, K))


def rotate_quantize_dense(x: torch.Tensor, R: torch.Tensor, act_bits: int = 4,
                          codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                          precond: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          stream=None):
    """x: bf16 [T][K], R: bf16 [K][K] (u = R x per token) on the GPU -> (codes, scales).

    ws: optional uint8 device workspace of rotate_dense_workspace(T, K) bytes."""
    lib = load_library()
    _require_gpu(x, R, ws)
    T, K = x.shape
    if (T > 0 and x.stride(1) != 1) or not R.is_contiguous() or tuple(R.shape) != (K, K):
        raise ValueError("x needs unit channel stride and R must be a contiguous [K][K] tensor")
    if codes is None:
        codes = torch.empty((T, K * act_bits // 8), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T,), dtype=torch.float32, device=x.device)
    need = int(lib.cbq_rotate_dense_workspace(T, K))
    if ws is None and T > 0:
        ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.cbq_rotate_quantize_dense(_ptr(x), T, K, max(x.stride(0), K), _ptr(R), act_bits, _ptr(codes),
                                         _ptr(scales), _ptr(precond), _ptr(ws), nbytes,
                                         _stream(stream)))
    return codes, scales


def route_workspace(T: int, E: int, topk: int, n_shared: int = 0) -> int:
    """Bytes of device workspace moe_route_gather needs (cbq_route_workspace)."""
    return int(load_library().cbq_route_workspace(T, E, topk, n_shared))


def moe_route_gather(logits: torch.Tensor, topk: int, renormalize: bool = True, n_shared: int = 0,
                     out: Optional[dict] = None, stream=None) -> dict:
    """logits fp32 [T][E] -> dict(ids, weights, offsets, sorted_tokens, slot_of).

    ``out`` may hold preallocated outputs under those names and a workspace under "ws"."""
    lib = load_library()
    _require_gpu(logits)
    T, E = logits.shape
    dev = logits.device
    o = out or {}
    ids = o.get("ids") if o.get("ids") is not None else torch.empty((T, topk), dtype=torch.int32, device=dev)
    w = o.get("weights") if o.get("weights") is not None else torch.empty((T, topk), dtype=torch.float32, device=dev)
    offs = o.get("offsets") if o.get("offsets") is not None else torch.empty((E + n_shared + 1,), dtype=torch.int32, device=dev)
    R = T * topk + n_shared * T
    st = o.get("sorted_tokens") if o.get("sorted_tokens") is not None else torch.empty((max(R, 1),), dtype=torch.int32, device=dev)
    so = o.get("slot_of") if o.get("slot_of") is not None else torch.empty((T, topk), dtype=torch.int32, device=dev)
    need = int(lib.cbq_route_workspace(T, E, topk, n_shared))
    ws = o.get("ws")
    if need > 0 and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    _check(lib.cbq_moe_route_gather(_ptr(logits), T, E, topk, int(bool(renormalize)), n_shared,
                                    _ptr(ids), _ptr(w), _ptr(offs), _ptr(st), _ptr(so),
                                    _ptr(ws) if need > 0 else None, need, _stream(stream)))
    return dict(ids=ids, weights=w, offsets=offs, sorted_tokens=st[:R], slot_of=so)


def moe_route_gather_noalloc(logits: torch.Tensor, topk: int, renormalize: bool = True,
                             n_shared: int = 0, out: Optional[dict] = None, stream=None) -> dict:
    """moe_route_gather through cbq_moe_route_gather_noalloc: the library's own scratch
    replaces the workspace.  ``out`` may hold preallocated outputs as for
    moe_route_gather (its "ws" entry is ignored)."""
    lib = load_library()
    _require_gpu(logits)
    T, E = logits.shape
    dev = logits.device
    o = out or {}

    def get(name, shape, dtype):
        t = o.get(name)
        return t if t is not None else torch.empty(shape, dtype=dtype, device=dev)

    R = T * topk + n_shared * T
    ids = get("ids", (T, topk), torch.int32)
    w = get("weights", (T, topk), torch.float32)
    offs = get("offsets", (E + n_shared + 1,), torch.int32)
    st = get("sorted_tokens", (max(R, 1),), torch.int32)
    so = get("slot_of", (T, topk), torch.int32)
    _check(lib.cbq_moe_route_gather_noalloc(_ptr(logits), T, E, topk, int(bool(renormalize)),
                                            n_shared, _ptr(ids), _ptr(w), _ptr(offs), _ptr(st),
                                            _ptr(so), _stream(stream)))
    return dict(ids=ids, weights=w, offsets=offs, sorted_tokens=st[:R], slot_of=so)


def prepack_weights(w: CodebookWeights, stream=None) -> CodebookWeights:
    """The blocked-layout copy of a row-layout weight set (cbq_prepack_weights); the
    codebooks are shared, not copied."""
    lib = load_library()
    _require_gpu(w.idx, w.codebook)
    if w.layout != LAYOUT_ROWS:
        raise ValueError("prepack_weights takes a row-layout weight set")
    s = w.c_struct()
    n = int(lib.cbq_prepack_bytes(ctypes.byref(s)))
    kp = (w.K + 127) // 128 * 128
    dst = torch.empty((w.E, w.N, kp * w.bits // 8), dtype=torch.uint8, device=w.idx.device)
    assert dst.numel() == n
    _check(lib.cbq_prepack_weights(ctypes.byref(s), _ptr(dst), _stream(stream)))
    return CodebookWeights(idx=dst, codebook=w.codebook, K=w.K, bits=w.bits, layout=LAYOUT_BLOCKED)


def gemm_workspace(weights: Sequence[CodebookWeights], n_rows: int, act_bits: int,
                   path: int = PATH_AUTO) -> int:
    """Bytes of optional GEMM workspace (cbq_gemm_workspace): with it, a single-matrix MFMA
    call whose tiles would leave CUs idle splits K in two, and a 4-bit gate/up call the
    column tiles of a half-empty last round; 0 when no call of these sizes can."""
    arr = (cbq_weights * len(weights))(*[w.c_struct() for w in weights])
    return int(load_library().cbq_gemm_workspace(arr, len(weights), n_rows, act_bits, path))


def codebook_lut_gemm(codes: torch.Tensor, scales: torch.Tensor, act_bits: int,
                      weights: Sequence[CodebookWeights], n_rows: Optional[int] = None,
                      expert_offsets: Optional[torch.Tensor] = None,
                      row_token: Optional[torch.Tensor] = None, epilogue: Optional[int] = None,
                      path: int = PATH_AUTO, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """Grouped codebook GEMM.  One weight set -> fp32 [R][N]; {gate, up} -> bf16 SwiGLU [R][N].

    ws: optional device workspace (a tensor of gemm_workspace(...) bytes or more)."""
    lib = load_library()
    _require_gpu(codes, scales, expert_offsets, row_token, ws)
    n_w = len(weights)
    if epilogue is None:
        epilogue = EPI_SWIGLU_BF16 if n_w == 2 else EPI_F32
    if n_rows is None:
        n_rows = row_token.shape[0] if row_token is not None else codes.shape[0]
    N = weights[0].N
    if out is None:
        dt = torch.bfloat16 if epilogue == EPI_SWIGLU_BF16 else torch.float32
        out = torch.empty((n_rows, N), dtype=dt, device=codes.device)
    arr = (cbq_weights * n_w)(*[w.c_struct() for w in weights])
    _check(lib.cbq_codebook_lut_gemm(_ptr(codes), _ptr(scales), act_bits, n_rows,
                                     _ptr(expert_offsets), _ptr(row_token), arr, n_w, epilogue,
                                     path, _ptr(out), out.stride(0), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return out


def moe_combine(expert_out: torch.Tensor, slot_of: torch.Tensor, topk_w: torch.Tensor,
                n_shared: int = 0, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    lib = load_library()
    _require_gpu(expert_out, slot_of, topk_w)
    T, topk = slot_of.shape
    H = expert_out.shape[1]
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=expert_out.device)
    _check(lib.cbq_moe_combine(_ptr(expert_out), _ptr(slot_of), _ptr(topk_w), T, topk, H, n_shared,
                               _ptr(y), _stream(stream)))
    return y


def kmeans_codebooks(w: torch.Tensor, bits: int, max_iters: int = 50, idx: Optional[torch.Tensor] = None,
                     codebook: Optional[torch.Tensor] = None, iters_done: Optional[torch.Tensor] = None,
                     stream=None) -> CodebookWeights:
    """bf16 weight rows [R][K] (last dim contiguous) -> CodebookWeights (E = 1, N = R): one
    K-means per row (cbq_kmeans_codebooks)."""
    lib = load_library()
    _require_gpu(w)
    R, K = w.shape
    if w.stride(1) != 1:
        raise ValueError("w rows must be contiguous")
    dev = w.device
    if idx is None:
        idx = torch.empty((1, R, K * bits // 8), dtype=torch.uint8, device=dev)
    if codebook is None:
        codebook = torch.empty((1, R, 1 << bits), dtype=torch.int16, device=dev)
    _check(lib.cbq_kmeans_codebooks(_ptr(w), R, K, w.stride(0), bits, max_iters, _ptr(idx),
                                    _ptr(codebook), _ptr(iters_done), _stream(stream)))
    return CodebookWeights(idx=idx, codebook=codebook, K=K, bits=bits)


def refit_codebooks(w: torch.Tensor, cw: "CodebookWeights", x: torch.Tensor, stream=None) -> "CodebookWeights":
    """Output-aware refit of cw's centroids (in place) on bf16 calibration activations
    x [n][K] (cbq_refit_codebooks); w: the bf16 rows [R][K] that cw clusters."""
    lib = load_library()
    _require_gpu(w, x, cw.idx, cw.codebook)
    R, K = w.shape
    n = x.shape[0]
    if w.stride(1) != 1 or x.stride(1) != 1 or x.shape[1] != K or K != cw.K:
        raise ValueError("w and x need contiguous rows of the weights' K channels")
    if not cw.codebook.is_contiguous() or not cw.idx.is_contiguous():
        raise ValueError("the codebook and index tensors must be contiguous")
    _check(lib.cbq_refit_codebooks(_ptr(w), R, K, w.stride(0), cw.bits, _ptr(cw.idx), _ptr(x), n,
                                   x.stride(0), _ptr(cw.codebook), _stream(stream)))
    return cw


CPU_NO_AVX512 = 1


def cpu_lut_gemm(codes, scales, act_bits: int, idx, codebook, K: int, bits: int,
                 n_threads: int = 0, out=None, avx512: bool = True):
    """The LUT GEMM on host cores (cbq_cpu_lut_gemm).  numpy arrays: codes uint8
    [T][K*act_bits/8], scales float32 [T], idx uint8 [N][K*bits/8] (or [1][N][...]),
    codebook uint16 [N][2^bits]; returns float32 [T][N]."""
    import numpy as np
    lib = load_library()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.uint8).reshape(-1, K * bits // 8)
    codebook = np.ascontiguousarray(codebook).view(np.uint16).reshape(-1, 1 << bits)
    T, N = codes.shape[0], idx.shape[0]
    if out is None:
        out = np.empty((T, N), dtype=np.float32)
    w = cbq_weights(idx.ctypes.data, codebook.ctypes.data, 1, N, K, bits, LAYOUT_ROWS)
    _check(lib.cbq_cpu_lut_gemm(ctypes.c_void_p(codes.ctypes.data), ctypes.c_void_p(scales.ctypes.data),
                                act_bits, T, ctypes.byref(w), ctypes.c_void_p(out.ctypes.data),
                                out.strides[0] // 4, n_threads, 0 if avx512 else CPU_NO_AVX512))
    return out


def moe_ffn(x: torch.Tensor, logits: torch.Tensor, gate: CodebookWeights, up: CodebookWeights,
            down: CodebookWeights, topk: int, n_shared: int = 0, act_bits: int = 4,
            renormalize: bool = True, path: int = PATH_AUTO, keep: bool = False, stream=None):
    """One MoE FFN layer as a sequence of the four library calls (no compute here).

    gate/up/down hold E routed + n_shared shared experts.  Returns y fp32 [T][H], or
    (y, intermediates) when keep is True.  The GEMMs get the optional workspaces
    gemm_workspace asks for."""
    codes, scales = rotate_quantize(x, act_bits, stream=stream)
    rt = moe_route_gather(logits, topk, renormalize, n_shared, stream=stream)
    R = int(rt["sorted_tokens"].shape[0])

    def workspace(ws):
        n = gemm_workspace(ws, R, act_bits, path)
        return torch.empty((n,), dtype=torch.uint8, device=x.device) if n > 0 else None

    h = codebook_lut_gemm(codes, scales, act_bits, [gate, up], expert_offsets=rt["offsets"],
                          row_token=rt["sorted_tokens"], path=path, ws=workspace([gate, up]),
                          stream=stream)
    codes_h, scales_h = rotate_quantize(h, act_bits, stream=stream)
    out = codebook_lut_gemm(codes_h, scales_h, act_bits, [down], expert_offsets=rt["offsets"],
                            path=path, ws=workspace([down]), stream=stream)
    y = moe_combine(out, rt["slot_of"], rt["weights"], n_shared, stream=stream)
    if keep:
        return y, dict(codes=codes, scales=scales, route=rt, h=h, codes_h=codes_h,
                       scales_h=scales_h, out=out)
    return y
