"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/cbq.h declares, and reject
invalid arguments with the documented status before touching HIP, so each error
path can be exercised on a machine without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cbq.h")

cbq = pytest.importorskip("codebook_bit_quantized_amd")


def _lib():
    if not os.path.exists(cbq.LIB_PATH):
        pytest.skip("libcbq.so not built")
    return cbq.load_library()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cbq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_symbols():
    assert _declared() == sorted(cbq.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.cbq_version() >= 100
    assert lib.cbq_status_string(cbq.CBQ_EINVAL) == b"CBQ_EINVAL"
    assert lib.cbq_status_string(123) == b"CBQ_UNKNOWN"


class _Fake:
    """A pointer value that is never dereferenced (validation fails before use)."""
    P = ctypes.c_void_p(0x1000)
    UNALIGNED = ctypes.c_void_p(0x1004)


def test_rotate_quantize_validation():
    lib = _lib()
    P, U = _Fake.P, _Fake.UNALIGNED
    rq = lib.cbq_rotate_quantize
    assert rq(P, -1, 256, 256, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL
    assert rq(P, 4, 250, 256, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL      # K % 32
    assert b"K" in lib.cbq_last_error()
    assert rq(P, 4, 32768, 32768, 0, 4, P, P, None, None) == cbq.CBQ_EUNSUPPORTED
    assert rq(P, 4, 256, 200, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL      # ldx < K
    assert rq(P, 4, 256, 260, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL      # ldx % 8
    assert rq(P, 4, 256, 256, 0, 5, P, P, None, None) == cbq.CBQ_EINVAL      # act_bits
    assert rq(P, 4, 256, 256, 3, 4, P, P, None, None) == cbq.CBQ_EINVAL      # had_block
    assert rq(P, 4, 384, 384, 256, 4, P, P, None, None) == cbq.CBQ_EINVAL    # 256 does not divide 384
    assert rq(None, 4, 256, 256, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL   # null x
    assert rq(U, 4, 256, 256, 0, 4, P, P, None, None) == cbq.CBQ_EINVAL      # misaligned
    assert rq(None, 0, 256, 256, 0, 4, None, None, None, None) == cbq.CBQ_OK  # T = 0 no-op


def test_rotate_quantize_ex_validation():
    lib = _lib()
    P, U = _Fake.P, _Fake.UNALIGNED
    ex = lib.cbq_rotate_quantize_ex
    assert ex(P, 4, 256, 256, 0, 4, U, None, P, P, None, None) == cbq.CBQ_EINVAL    # smooth alignment
    assert ex(P, 4, 256, 256, 0, 4, None, ctypes.c_void_p(0x1002), P, P, None, None) == cbq.CBQ_EINVAL
    assert ex(P, 4, 250, 256, 0, 4, P, P, P, P, None, None) == cbq.CBQ_EINVAL      # K % 32
    assert ex(P, 0, 256, 256, 0, 4, P, P, P, P, None, None) == cbq.CBQ_OK          # empty


def test_rotate_quantize_dense_validation():
    lib = _lib()
    P, U = _Fake.P, _Fake.UNALIGNED
    rd = lib.cbq_rotate_quantize_dense
    assert lib.cbq_rotate_dense_workspace(4, 256) == 4 * 256 * 4 + 256
    assert lib.cbq_rotate_dense_workspace(4, 96) == 0                               # K % 64
    need = lib.cbq_rotate_dense_workspace(4, 256)
    assert rd(P, 4, 96, 96, P, 4, P, P, None, P, need, None) == cbq.CBQ_EINVAL      # K % 64
    assert rd(P, 4, 256, 250, P, 4, P, P, None, P, need, None) == cbq.CBQ_EINVAL    # ldx
    assert rd(P, 4, 256, 256, P, 5, P, P, None, P, need, None) == cbq.CBQ_EINVAL    # act_bits
    assert rd(P, 4, 256, 256, U, 4, P, P, None, P, need, None) == cbq.CBQ_EINVAL    # R alignment
    assert rd(P, 4, 256, 256, P, 4, P, P, None, P, need - 1, None) == cbq.CBQ_EWORKSPACE
    assert rd(P, 4, 256, 256, P, 4, P, P, None, None, 0, None) == cbq.CBQ_EWORKSPACE
    assert rd(P, 4, 32768, 32768, P, 4, P, P, None, P, need, None) == cbq.CBQ_EUNSUPPORTED
    assert rd(None, 0, 256, 256, None, 4, None, None, None, None, 0, None) == cbq.CBQ_OK  # T = 0


def test_refit_validation():
    lib = _lib()
    P = _Fake.P
    rf = lib.cbq_refit_codebooks
    assert rf(P, 4, 96, 96, 3, P, P, 0, 96, P, None) == cbq.CBQ_EINVAL        # n = 0
    assert rf(P, 4, 96, 96, 3, P, P, 257, 96, P, None) == cbq.CBQ_EINVAL      # n > 256
    assert rf(P, 4, 100, 100, 3, P, P, 8, 100, P, None) == cbq.CBQ_EINVAL     # K % 32
    assert rf(P, 4, 96, 96, 5, P, P, 8, 96, P, None) == cbq.CBQ_EUNSUPPORTED  # bits
    assert rf(P, 4, 96, 64, 3, P, P, 8, 96, P, None) == cbq.CBQ_EINVAL        # ldw < K
    assert rf(None, 0, 96, 96, 3, None, None, 8, 96, None, None) == cbq.CBQ_OK  # R = 0


def test_route_validation():
    lib = _lib()
    P = _Fake.P
    rg = lib.cbq_moe_route_gather
    # one int32 count per (chunk of >= 16 tokens, expert), at most 256 chunks
    assert lib.cbq_route_workspace(64, 128, 8, 0) == 4 * 128 * 4
    assert lib.cbq_route_workspace(4096, 64, 6, 2) == 256 * 64 * 4
    assert lib.cbq_route_workspace(1 << 20, 256, 8, 0) == 256 * 256 * 4
    assert lib.cbq_route_workspace(0, 64, 6, 2) == 0
    W = ctypes.c_void_p(0x7000)
    assert rg(P, 64, 128, 8, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EWORKSPACE   # no ws
    assert rg(P, 64, 128, 8, 1, 0, P, P, P, P, P, W, 100, None) == cbq.CBQ_EWORKSPACE    # too small
    assert rg(P, 64, 128, 8, 1, 0, P, P, P, P, P, ctypes.c_void_p(0x7002), 4096, None) == \
        cbq.CBQ_EINVAL                                                                 # misaligned
    assert rg(P, 4, 0, 1, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EUNSUPPORTED   # E = 0
    assert rg(P, 4, 300, 1, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EUNSUPPORTED
    assert rg(P, 4, 8, 9, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL          # topk > 8
    assert rg(P, 4, 4, 5, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL          # topk > E
    assert rg(P, 4, 8, 2, 2, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL          # renormalize
    assert rg(P, 4, 8, 2, 1, 9, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL          # n_shared
    assert rg(P, -1, 8, 2, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL
    assert rg(None, 4, 8, 2, 1, 0, P, P, P, P, P, None, 0, None) == cbq.CBQ_EINVAL       # null logits
    assert rg(P, 4, 8, 2, 1, 0, P, P, None, P, P, None, 0, None) == cbq.CBQ_EINVAL       # null offsets
    # the no-allocation variant validates the same way, without a workspace argument
    rn = lib.cbq_moe_route_gather_noalloc
    assert rn(P, 4, 300, 1, 1, 0, P, P, P, P, P, None) == cbq.CBQ_EUNSUPPORTED         # E > 256
    assert rn(P, 4, 8, 9, 1, 0, P, P, P, P, P, None) == cbq.CBQ_EINVAL                # topk > 8
    assert rn(P, (1 << 24) + 1, 8, 2, 1, 0, P, P, P, P, P, None) == cbq.CBQ_EUNSUPPORTED
    assert rn(P, 4, 8, 2, 1, 0, P, P, None, P, P, None) == cbq.CBQ_EINVAL              # null offsets


def _w(E=1, N=64, K=256, bits=4, idx=0x1000, cb=0x2000, layout=0):
    return cbq.cbq_weights(idx, cb, E, N, K, bits, layout)


def _gemm(lib, W, n_w=1, act_bits=4, n_rows=4, epi=0, path=0, out=0x3000, ldo=64, codes=0x4000):
    arr = (cbq.cbq_weights * len(W))(*W)
    return lib.cbq_codebook_lut_gemm(ctypes.c_void_p(codes), ctypes.c_void_p(0x5000), act_bits,
                                     n_rows, None, None, arr, n_w, epi, path,
                                     ctypes.c_void_p(out), ldo, None, 0, None)


def test_gemm_validation():
    lib = _lib()
    E = cbq.CBQ_EINVAL
    assert _gemm(lib, [_w(bits=5)]) == cbq.CBQ_EUNSUPPORTED
    assert _gemm(lib, [_w(bits=1)]) == cbq.CBQ_EUNSUPPORTED
    assert _gemm(lib, [_w(K=100)]) == E
    assert _gemm(lib, [_w(N=40)]) == E
    assert _gemm(lib, [_w(E=0)]) == E
    assert _gemm(lib, [_w(idx=0)]) == E
    assert _gemm(lib, [_w(idx=0x1004)]) == E                      # misaligned idx
    assert _gemm(lib, [_w()], act_bits=6) == E
    assert _gemm(lib, [_w(), _w()], n_w=2, epi=0) == E            # F32 needs one set
    assert _gemm(lib, [_w()], n_w=1, epi=1) == E                  # SwiGLU needs two
    assert _gemm(lib, [_w(), _w(N=128)], n_w=2, epi=1) == E       # mismatched gate/up
    assert _gemm(lib, [_w()], epi=7) == E
    assert _gemm(lib, [_w()], path=5) == E
    # the table forms take 4-bit codebooks and A4 only, and no table flags
    assert _gemm(lib, [_w(bits=3)], path=cbq.PATH_PAGES_PRODUCTS) == cbq.CBQ_EUNSUPPORTED
    assert _gemm(lib, [_w()], act_bits=8, path=cbq.PATH_PAGES_BUCKETS) == cbq.CBQ_EUNSUPPORTED
    assert _gemm(lib, [_w()], path=cbq.PATH_PAGES_PRODUCTS | cbq.PATH_REG_TABLES) == E
    assert _gemm(lib, [_w()], path=cbq.PATH_PAGES_BUCKETS | cbq.PATH_LDS_TABLES) == E
    assert _gemm(lib, [_w()], path=cbq.PATH_PAGES_BUCKETS, n_rows=0) == cbq.CBQ_OK
    assert _gemm(lib, [_w()], path=cbq.PATH_LUT | 0x40) == E     # unknown flag
    assert _gemm(lib, [_w()], path=cbq.PATH_LUT | cbq.PATH_REG_TABLES | cbq.PATH_LDS_TABLES) == E
    assert _gemm(lib, [_w()], path=cbq.PATH_MFMA | cbq.PATH_LDS_TABLES, n_rows=0) == cbq.CBQ_OK
    assert _gemm(lib, [_w()], ldo=32) == E                        # ldo < N
    assert _gemm(lib, [_w()], ldo=66) == E                        # ldo % 4
    assert _gemm(lib, [_w()], n_rows=-1) == E
    assert _gemm(lib, [_w()], out=0) == E                         # null out
    assert _gemm(lib, [_w()], codes=0x4004) == E                  # misaligned codes
    assert _gemm(lib, [_w()], n_rows=0) == cbq.CBQ_OK             # empty: no-op
    assert lib.cbq_gemm_workspace(ctypes.pointer(_w()), 1, 16, 4, 0) == 0
    # the K-split workspace: one 4-bit matrix with K >= 4096 on the AUTO or MFMA path only
    w4k = _w(K=4096)
    assert lib.cbq_gemm_workspace(ctypes.pointer(w4k), 1, 16, 4, cbq.PATH_AUTO) == 16 * 64 * 4
    assert lib.cbq_gemm_workspace(ctypes.pointer(w4k), 1, 16, 8, cbq.PATH_MFMA | cbq.PATH_REG_TABLES) == 16 * 64 * 4
    assert lib.cbq_gemm_workspace(ctypes.pointer(w4k), 1, 16, 4, cbq.PATH_LUT) == 0
    assert lib.cbq_gemm_workspace(ctypes.pointer(w4k), 1, 16, 4, cbq.PATH_PAGES_PRODUCTS) == 0
    assert lib.cbq_gemm_workspace(ctypes.pointer(_w(K=4096, bits=3)), 1, 16, 4, cbq.PATH_AUTO) == 0
    # the gate/up pair with 4-bit codebooks, K >= 2048 and 512 to 4096 rows: four fp32
    # planes of the at most 16 split column tiles (2048 columns)
    pair = (cbq.cbq_weights * 2)(w4k, w4k)
    assert lib.cbq_gemm_workspace(pair, 2, 512, 4, cbq.PATH_AUTO) == 4 * 512 * 64 * 4
    assert lib.cbq_gemm_workspace(pair, 2, 4096, 4, cbq.PATH_MFMA) == 4 * 4096 * 64 * 4
    assert lib.cbq_gemm_workspace(pair, 2, 511, 4, cbq.PATH_AUTO) == 0
    assert lib.cbq_gemm_workspace(pair, 2, 600, 8, cbq.PATH_LUT) == 0
    assert lib.cbq_gemm_workspace(pair, 2, 4097, 8, cbq.PATH_MFMA) == 0
    wide = _w(K=2048, N=6144)
    assert lib.cbq_gemm_workspace((cbq.cbq_weights * 2)(wide, wide), 2, 1000, 8, cbq.PATH_MFMA) == 4 * 1000 * 2048 * 4
    short = _w(K=1984)
    assert lib.cbq_gemm_workspace((cbq.cbq_weights * 2)(short, short), 2, 600, 4, cbq.PATH_AUTO) == 0
    three = _w(K=4096, bits=3)
    assert lib.cbq_gemm_workspace((cbq.cbq_weights * 2)(three, three), 2, 600, 4, cbq.PATH_AUTO) == 0
    arr = (cbq.cbq_weights * 1)(w4k)
    assert lib.cbq_codebook_lut_gemm(ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000), 4, 16, None, None,
                                     arr, 1, 0, 0, ctypes.c_void_p(0x3000), 64, ctypes.c_void_p(0x6004),
                                     4096, None) == E               # misaligned workspace
    assert _gemm(lib, [_w(layout=2)]) == E                        # unknown layout
    assert _gemm(lib, [_w(), _w(layout=1)], n_w=2, epi=1) == E    # gate/up layouts differ
    assert _gemm(lib, [_w(layout=1)], n_rows=0) == cbq.CBQ_OK


def test_prepack_validation():
    lib = _lib()
    E = cbq.CBQ_EINVAL
    # blocked bytes: K rounded up to 128 channels
    assert lib.cbq_prepack_bytes(ctypes.pointer(_w(E=2, N=64, K=256, bits=4))) == 2 * 64 * 256 // 2
    assert lib.cbq_prepack_bytes(ctypes.pointer(_w(E=1, N=16, K=160, bits=3))) == 16 * 256 * 3 // 8
    assert lib.cbq_prepack_bytes(ctypes.pointer(_w(E=3, N=2048, K=1408, bits=2))) == 3 * 2048 * 1408 // 4
    assert lib.cbq_prepack_bytes(ctypes.pointer(_w(K=100))) == 0
    pp = lib.cbq_prepack_weights
    dst = ctypes.c_void_p(0x100000)
    assert pp(ctypes.pointer(_w()), None, None) == E                       # null dst
    assert pp(ctypes.pointer(_w()), ctypes.c_void_p(0x100004), None) == E  # misaligned dst
    assert pp(ctypes.pointer(_w(layout=1)), dst, None) == E               # already blocked
    assert pp(ctypes.pointer(_w(idx=0x1000)), ctypes.c_void_p(0x1000), None) == E  # overlap
    assert pp(ctypes.pointer(_w(bits=5)), dst, None) == cbq.CBQ_EUNSUPPORTED


def test_combine_validation():
    lib = _lib()
    P, U = _Fake.P, _Fake.UNALIGNED
    cb = lib.cbq_moe_combine
    assert cb(P, P, P, -1, 2, 64, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(P, P, P, 4, 0, 64, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(P, P, P, 4, 9, 64, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(P, P, P, 4, 2, 62, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(P, P, P, 4, 2, 64, 9, P, None) == cbq.CBQ_EINVAL
    assert cb(None, P, P, 4, 2, 64, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(U, P, P, 4, 2, 64, 0, P, None) == cbq.CBQ_EINVAL
    assert cb(None, None, None, 0, 2, 64, 0, None, None) == cbq.CBQ_OK


def test_error_message_is_per_call():
    lib = _lib()
    P = _Fake.P
    lib.cbq_rotate_quantize(P, 4, 250, 256, 0, 4, P, P, None, None)
    assert lib.cbq_last_error() != b""
    lib.cbq_rotate_quantize(None, 0, 256, 256, 0, 4, None, None, None, None)
    assert lib.cbq_last_error() == b""
