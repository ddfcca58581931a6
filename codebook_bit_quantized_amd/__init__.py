"""codebook_bit_quantized_amd - the codebook-LUT MoE expert path on MI355X (gfx950).

The work runs in libcbq.so (hand-written HIP kernels behind a C ABI, declared in
include/cbq.h).  This package is its thin Python binding: torch provides device
memory and streams; nothing is computed in Python.

Calls (same names as the C ABI without the ``cbq_`` prefix):
  rotate_quantize, route_workspace, moe_route_gather, codebook_lut_gemm, moe_combine
and ``moe_ffn``, which sequences them into one MoE FFN layer, and
``kmeans_codebooks``, the offline construction of codebooks from bf16 weights (with
``refit_codebooks``, the output-aware centroid refit on calibration activations), and
``cpu_lut_gemm``, the LUT GEMM on host cores, and ``rotate_quantize_dense`` (with
``rotate_dense_workspace``), a dense K x K rotation in place of the Hadamard blocks.
"""
from ._binding import (AUTO_MAX_LUT_ROWS, CBQ_EHIP, CBQ_EINVAL, CBQ_EUNSUPPORTED, CBQ_EWORKSPACE,
                       CBQ_OK, EPI_F32, EPI_SWIGLU_BF16, EXPORTED, LIB_PATH, PATH_AUTO, PATH_LUT,
                       PATH_MFMA, PATH_PAGES_PRODUCTS, PATH_PAGES_BUCKETS, PATH_REG_TABLES, PATH_LDS_TABLES, CbqError, CodebookWeights, cbq_weights, codebook_lut_gemm,
                       cpu_lut_gemm, kmeans_codebooks, load_library, moe_combine, moe_ffn, moe_route_gather,
                       moe_route_gather_noalloc, prepack_weights, LAYOUT_ROWS, LAYOUT_BLOCKED,
                       refit_codebooks,
                       rotate_dense_workspace, rotate_quantize, rotate_quantize_dense,
                       route_workspace, gemm_workspace)

__all__ = [
    "rotate_quantize", "moe_route_gather", "moe_route_gather_noalloc", "prepack_weights", "LAYOUT_ROWS", "LAYOUT_BLOCKED",
    "codebook_lut_gemm", "moe_combine", "moe_ffn",
    "route_workspace", "gemm_workspace", "kmeans_codebooks", "refit_codebooks", "cpu_lut_gemm", "rotate_quantize_dense",
    "rotate_dense_workspace",
    "CodebookWeights", "CbqError", "load_library", "LIB_PATH", "EXPORTED", "cbq_weights",
    "EPI_F32", "EPI_SWIGLU_BF16", "PATH_AUTO", "PATH_LUT", "PATH_MFMA", "PATH_PAGES_PRODUCTS", "PATH_PAGES_BUCKETS", "PATH_REG_TABLES", "PATH_LDS_TABLES", "AUTO_MAX_LUT_ROWS",
    "CBQ_OK", "CBQ_EINVAL", "CBQ_EUNSUPPORTED", "CBQ_EWORKSPACE", "CBQ_EHIP",
]
