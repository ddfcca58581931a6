// C ABI of libcbq: argument validation (host only, before any HIP call), dispatch to
// the kernels, status codes and the per-thread error message.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/cbq.h"
#include "cpu_lut.hpp"
#include "cbq_internal.hpp"

#define CBQ_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CBQ_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_weights(const cbq_weights* W, int i) {
  if (!W->idx || !W->codebook) return fail(CBQ_EINVAL, "W[%d]: idx and codebook must be non-null", i);
  if (!aligned16(W->idx) || !aligned16(W->codebook))
    return fail(CBQ_EINVAL, "W[%d]: idx and codebook must be 16-byte aligned", i);
  if (W->E < 1) return fail(CBQ_EINVAL, "W[%d]: E must be >= 1 (got %d)", i, W->E);
  if (W->N < 16 || W->N % 16) return fail(CBQ_EINVAL, "W[%d]: N must be a positive multiple of 16 (got %d)", i, W->N);
  if (W->K < 32 || W->K % 32) return fail(CBQ_EINVAL, "W[%d]: K must be a positive multiple of 32 (got %d)", i, W->K);
  if (W->bits < 2 || W->bits > 4) return fail(CBQ_EUNSUPPORTED, "W[%d]: bits must be 2, 3 or 4 (got %d)", i, W->bits);
  if (W->layout != CBQ_LAYOUT_ROWS && W->layout != CBQ_LAYOUT_BLOCKED)
    return fail(CBQ_EINVAL, "W[%d]: unknown index layout %d", i, W->layout);
  return CBQ_OK;
}

}  // namespace

CBQ_EXPORT const char* cbq_status_string(int status) {
  switch (status) {
    case CBQ_OK: return "CBQ_OK";
    case CBQ_EINVAL: return "CBQ_EINVAL";
    case CBQ_EUNSUPPORTED: return "CBQ_EUNSUPPORTED";
    case CBQ_EWORKSPACE: return "CBQ_EWORKSPACE";
    case CBQ_EHIP: return "CBQ_EHIP";
  }
  return "CBQ_UNKNOWN";
}

CBQ_EXPORT const char* cbq_last_error(void) { return g_err; }

CBQ_EXPORT int cbq_version(void) { return 100; }

CBQ_EXPORT int cbq_rotate_quantize_ex(const uint16_t* x, int64_t T, int32_t K, int64_t ldx,
                                      int32_t had_block, int32_t act_bits, const float* smooth,
                                      const uint8_t* signs, uint8_t* codes, float* scales,
                                      uint32_t* precond_violations, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
  if (T > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "T must be < 2^31");
  if (K < 32 || K % 32) return fail(CBQ_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (K > 16384) return fail(CBQ_EUNSUPPORTED, "K must be <= 16384 (got %d)", K);
  if (ldx < K || ldx % 8) return fail(CBQ_EINVAL, "ldx must be >= K and a multiple of 8 (got %lld)", (long long)ldx);
  if (act_bits != 4 && act_bits != 8) return fail(CBQ_EINVAL, "act_bits must be 4 or 8 (got %d)", act_bits);
  int b = had_block;
  if (b == 0) b = K & -K;
  if (!pow2(b) || K % b) return fail(CBQ_EINVAL, "had_block must be 0 or a power of two dividing K (got %d)", had_block);
  if ((smooth && !aligned16(smooth)) || (signs && (reinterpret_cast<uintptr_t>(signs) & 3u)))
    return fail(CBQ_EINVAL, "smooth must be 16-byte and signs 4-byte aligned");
  if (T == 0) return CBQ_OK;
  if (!x || !codes || !scales) return fail(CBQ_EINVAL, "x, codes and scales must be non-null");
  if (!aligned16(x) || !aligned16(codes)) return fail(CBQ_EINVAL, "x and codes must be 16-byte aligned");
  hipError_t e = cbq::launch_rotate_quantize(x, T, K, ldx, b, act_bits, smooth, signs, codes,
                                             scales, precond_violations, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rotate_quantize launch");
  return CBQ_OK;
}

CBQ_EXPORT int cbq_rotate_quantize(const uint16_t* x, int64_t T, int32_t K, int64_t ldx,
                                   int32_t had_block, int32_t act_bits, uint8_t* codes,
                                   float* scales, uint32_t* precond_violations, void* stream) {
  return cbq_rotate_quantize_ex(x, T, K, ldx, had_block, act_bits, nullptr, nullptr, codes,
                                scales, precond_violations, stream);
}

CBQ_EXPORT size_t cbq_rotate_dense_workspace(int64_t T, int32_t K) {
  if (T < 0 || T > 0x7FFFFFFF || K < 64 || K % 64 || K > 16384) return 0;
  return cbq::dense_rotation_workspace_bytes(T, K);
}

CBQ_EXPORT int cbq_rotate_quantize_dense(const uint16_t* x, int64_t T, int32_t K, int64_t ldx,
                                         const uint16_t* R, int32_t act_bits, uint8_t* codes,
                                         float* scales, uint32_t* precond_violations, void* ws,
                                         size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
  if (T > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "T must be < 2^31");
  if (K < 64 || K % 64) return fail(CBQ_EINVAL, "K must be a positive multiple of 64 (got %d)", K);
  if (K > 16384) return fail(CBQ_EUNSUPPORTED, "K must be <= 16384 (got %d)", K);
  if (ldx < K || ldx % 8) return fail(CBQ_EINVAL, "ldx must be >= K and a multiple of 8 (got %lld)", (long long)ldx);
  if (act_bits != 4 && act_bits != 8) return fail(CBQ_EINVAL, "act_bits must be 4 or 8 (got %d)", act_bits);
  if (T == 0) return CBQ_OK;
  if (!x || !R || !codes || !scales) return fail(CBQ_EINVAL, "x, R, codes and scales must be non-null");
  if (!aligned16(x) || !aligned16(R)) return fail(CBQ_EINVAL, "x and R must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(codes) & 7u) return fail(CBQ_EINVAL, "codes must be 8-byte aligned");
  const size_t need = cbq::dense_rotation_workspace_bytes(T, K);
  if (!ws || ws_bytes < need)
    return fail(CBQ_EWORKSPACE, "dense rotation workspace of %zu bytes required (got %zu)", need, ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(CBQ_EINVAL, "ws must be 16-byte aligned");
  hipError_t e = cbq::launch_rotate_dense(x, T, K, ldx, R, act_bits, codes, scales,
                                          precond_violations, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rotate_quantize_dense launch");
  return CBQ_OK;
}

CBQ_EXPORT size_t cbq_route_workspace(int64_t T, int32_t E, int32_t topk, int32_t n_shared) {
  (void)topk; (void)n_shared;
  if (T <= 0 || E < 1 || E > 256 || T > (1 << 24)) return 0;
  return cbq::route_workspace_bytes(T, E);
}

CBQ_EXPORT int cbq_moe_route_gather(const float* logits, int64_t T, int32_t E, int32_t topk,
                                    int32_t renormalize, int32_t n_shared, int32_t* topk_ids,
                                    float* topk_w, int32_t* expert_offsets,
                                    int32_t* sorted_tokens, int32_t* slot_of, void* ws,
                                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
  if (T > (1 << 24)) return fail(CBQ_EUNSUPPORTED, "T must be <= 2^24");
  if (E < 1 || E > 256) return fail(CBQ_EUNSUPPORTED, "E must be in [1, 256] (got %d)", E);
  if (topk < 1 || topk > 8 || topk > E) return fail(CBQ_EINVAL, "topk must be in [1, min(E, 8)] (got %d)", topk);
  if (n_shared < 0 || n_shared > 8) return fail(CBQ_EINVAL, "n_shared must be in [0, 8] (got %d)", n_shared);
  if (renormalize != 0 && renormalize != 1) return fail(CBQ_EINVAL, "renormalize must be 0 or 1");
  if (!expert_offsets) return fail(CBQ_EINVAL, "expert_offsets must be non-null");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_tokens || !slot_of))
    return fail(CBQ_EINVAL, "logits, topk_ids, topk_w, sorted_tokens and slot_of must be non-null");
  const size_t need = cbq::route_workspace_bytes(T, E);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CBQ_EWORKSPACE, "route workspace of %zu bytes required (got %zu)", need, ws ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return fail(CBQ_EINVAL, "ws must be 4-byte aligned");
  hipError_t e = cbq::launch_route(logits, T, E, topk, renormalize, n_shared, topk_ids, topk_w,
                                   expert_offsets, sorted_tokens, slot_of,
                                   static_cast<int32_t*>(ws), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route_gather launch");
  return CBQ_OK;
}

CBQ_EXPORT int cbq_moe_route_gather_noalloc(const float* logits, int64_t T, int32_t E, int32_t topk,
                                            int32_t renormalize, int32_t n_shared,
                                            int32_t* topk_ids, float* topk_w,
                                            int32_t* expert_offsets, int32_t* sorted_tokens,
                                            int32_t* slot_of, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
  if (T > (1 << 24)) return fail(CBQ_EUNSUPPORTED, "T must be <= 2^24");
  if (E < 1 || E > 256) return fail(CBQ_EUNSUPPORTED, "E must be in [1, 256] (got %d)", E);
  if (topk < 1 || topk > 8 || topk > E) return fail(CBQ_EINVAL, "topk must be in [1, min(E, 8)] (got %d)", topk);
  if (n_shared < 0 || n_shared > 8) return fail(CBQ_EINVAL, "n_shared must be in [0, 8] (got %d)", n_shared);
  if (renormalize != 0 && renormalize != 1) return fail(CBQ_EINVAL, "renormalize must be 0 or 1");
  if (!expert_offsets) return fail(CBQ_EINVAL, "expert_offsets must be non-null");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_tokens || !slot_of))
    return fail(CBQ_EINVAL, "logits, topk_ids, topk_w, sorted_tokens and slot_of must be non-null");
  const size_t need = cbq::route_workspace_bytes(T, E);
  if (need > cbq::route_scratch_bytes())
    return fail(CBQ_EUNSUPPORTED, "routing needs %zu bytes of scratch, above the library's %zu",
                need, cbq::route_scratch_bytes());
  int32_t* scratch = nullptr;
  hipError_t e = cbq::route_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "moe_route_gather_noalloc scratch lookup");
  e = cbq::launch_route(logits, T, E, topk, renormalize, n_shared, topk_ids, topk_w, expert_offsets,
                        sorted_tokens, slot_of, scratch, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route_gather_noalloc launch");
  return CBQ_OK;
}

CBQ_EXPORT size_t cbq_prepack_bytes(const cbq_weights* src) {
  if (!src || src->E < 1 || src->N < 16 || src->N % 16 || src->K < 32 || src->K % 32 ||
      src->bits < 2 || src->bits > 4)
    return 0;
  return (size_t)src->E * src->N * cbq::index_row_bytes(src->K, src->bits, true);
}

CBQ_EXPORT int cbq_prepack_weights(const cbq_weights* src, uint8_t* dst, void* stream) {
  g_err[0] = 0;
  if (!src) return fail(CBQ_EINVAL, "src must be non-null");
  if (int rc = check_weights(src, 0)) return rc;
  if (src->layout != CBQ_LAYOUT_ROWS) return fail(CBQ_EINVAL, "src must be in the row layout");
  if (!dst || !aligned16(dst)) return fail(CBQ_EINVAL, "dst must be non-null and 16-byte aligned");
  const size_t n_src = (size_t)src->E * src->N * ((size_t)src->K * src->bits / 8);
  const size_t n_dst = cbq_prepack_bytes(src);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src->idx), d0 = reinterpret_cast<uintptr_t>(dst);
  if (d0 < s0 + n_src && s0 < d0 + n_dst) return fail(CBQ_EINVAL, "dst must not overlap src->idx");
  hipError_t e = cbq::launch_prepack(src->idx, dst, src->E, src->N, src->K, src->bits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prepack_weights launch");
  return CBQ_OK;
}

CBQ_EXPORT size_t cbq_gemm_workspace(const cbq_weights* W, int32_t n_w, int64_t n_rows,
                                     int32_t act_bits, int32_t path) {
  (void)act_bits;
  if (!W || (n_w != 1 && n_w != 2)) return 0;
  const int p = path & ~(CBQ_PATH_REG_TABLES | CBQ_PATH_LDS_TABLES);
  if (p != CBQ_PATH_AUTO && p != CBQ_PATH_MFMA) return 0;   // only the MFMA path uses it
  return cbq::mfma_split_workspace_bytes(n_w, W[0].bits, n_rows, W[0].N, W[0].K);
}

CBQ_EXPORT int cbq_codebook_lut_gemm(const uint8_t* codes, const float* scales, int32_t act_bits,
                                     int64_t n_rows, const int32_t* expert_offsets,
                                     const int32_t* row_token, const cbq_weights* W, int32_t n_w,
                                     int32_t epilogue, int32_t path, void* out, int64_t ldo,
                                     void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!W) return fail(CBQ_EINVAL, "W must be non-null");
  if (n_w != 1 && n_w != 2) return fail(CBQ_EINVAL, "n_w must be 1 or 2 (got %d)", n_w);
  for (int i = 0; i < n_w; ++i) {
    int st = check_weights(&W[i], i);
    if (st != CBQ_OK) return st;
  }
  if (n_w == 2 && (W[1].E != W[0].E || W[1].N != W[0].N || W[1].K != W[0].K || W[1].bits != W[0].bits ||
                   W[1].layout != W[0].layout))
    return fail(CBQ_EINVAL, "gate and up weights must have equal E, N, K, bits and layout");
  if (act_bits != 4 && act_bits != 8) return fail(CBQ_EINVAL, "act_bits must be 4 or 8 (got %d)", act_bits);
  if (epilogue == CBQ_EPI_F32) {
    if (n_w != 1) return fail(CBQ_EINVAL, "CBQ_EPI_F32 takes exactly one weight set");
  } else if (epilogue == CBQ_EPI_SWIGLU_BF16) {
    if (n_w != 2) return fail(CBQ_EINVAL, "CBQ_EPI_SWIGLU_BF16 takes the gate and up weight sets (n_w = 2)");
  } else {
    return fail(CBQ_EINVAL, "unknown epilogue %d", epilogue);
  }
  const int tflags = path & (CBQ_PATH_REG_TABLES | CBQ_PATH_LDS_TABLES);
  if (tflags == (CBQ_PATH_REG_TABLES | CBQ_PATH_LDS_TABLES))
    return fail(CBQ_EINVAL, "CBQ_PATH_REG_TABLES and CBQ_PATH_LDS_TABLES exclude each other");
  path &= ~(CBQ_PATH_REG_TABLES | CBQ_PATH_LDS_TABLES);
  if (path < CBQ_PATH_AUTO || path > CBQ_PATH_PAGES_BUCKETS) return fail(CBQ_EINVAL, "unknown path %d", path);
  const bool pages = path == CBQ_PATH_PAGES_PRODUCTS || path == CBQ_PATH_PAGES_BUCKETS;
  if (pages && tflags) return fail(CBQ_EINVAL, "table flags apply to CBQ_PATH_AUTO, CBQ_PATH_LUT and CBQ_PATH_MFMA only");
  if (pages && (W[0].bits != 4 || act_bits != 4))
    return fail(CBQ_EUNSUPPORTED, "the table paths take 4-bit codebooks and act_bits == 4 (got bits %d, act_bits %d)",
                W[0].bits, act_bits);
  if (pages && W[0].K > 16384) return fail(CBQ_EUNSUPPORTED, "the table paths take K <= 16384 (got %d)", W[0].K);
  if (n_rows < 0) return fail(CBQ_EINVAL, "n_rows must be >= 0");
  if (n_rows > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "n_rows must be < 2^31");
  if (ldo < W[0].N || ldo % 4) return fail(CBQ_EINVAL, "ldo must be >= N and a multiple of 4 (got %lld)", (long long)ldo);
  if (n_rows == 0) return CBQ_OK;
  {
    const int64_t esz = epilogue == CBQ_EPI_SWIGLU_BF16 ? 2 : 4;
    if (n_rows * ldo * esz >= (int64_t(1) << 30))
      return fail(CBQ_EUNSUPPORTED, "output must be smaller than 1 GiB per call (n_rows * ldo * %lld bytes)", (long long)esz);
    if ((int64_t)W[0].N * cbq::index_row_bytes(W[0].K, W[0].bits, W[0].layout == CBQ_LAYOUT_BLOCKED) >=
        (int64_t(1) << 31))
      return fail(CBQ_EUNSUPPORTED, "one expert's index block must be smaller than 2 GiB");
    if (!row_token && n_rows * ((int64_t)W[0].K * act_bits / 8) >= (int64_t(1) << 31))
      return fail(CBQ_EUNSUPPORTED, "codes must be smaller than 2 GiB");
  }
  if (!codes || !scales || !out) return fail(CBQ_EINVAL, "codes, scales and out must be non-null");
  if (!aligned16(codes) || !aligned16(out)) return fail(CBQ_EINVAL, "codes and out must be 16-byte aligned");
  if (ws && ws_bytes > 0 && !aligned16(ws)) return fail(CBQ_EINVAL, "ws must be 16-byte aligned");

  cbq::GemmArgs a{};
  a.ws = ws_bytes > 0 ? ws : nullptr;
  a.ws_bytes = a.ws ? ws_bytes : 0;
  a.codes = codes; a.scales = scales; a.act_bits = act_bits; a.n_rows = n_rows;
  a.offsets = expert_offsets; a.row_token = row_token;
  a.w[0] = cbq::GemmW{W[0].idx, W[0].codebook};
  a.w[1] = n_w == 2 ? cbq::GemmW{W[1].idx, W[1].codebook} : a.w[0];
  a.n_w = n_w; a.E = W[0].E; a.N = W[0].N; a.K = W[0].K; a.bits = W[0].bits;
  a.swiglu = epilogue == CBQ_EPI_SWIGLU_BF16;
  a.blocked = W[0].layout == CBQ_LAYOUT_BLOCKED;
  a.tables = tflags == CBQ_PATH_REG_TABLES ? cbq::kTablesReg
             : tflags == CBQ_PATH_LDS_TABLES ? cbq::kTablesLds : cbq::kTablesDefault;
  a.out = out; a.ldo = ldo;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (path == CBQ_PATH_LUT) {
    e = cbq::launch_lut_decode(a, -1, s);
  } else if (path == CBQ_PATH_MFMA) {
    e = cbq::launch_mfma_prefill(a, 0, s);
  } else if (pages) {
    e = cbq::launch_lut_pages(a, path == CBQ_PATH_PAGES_PRODUCTS ? 0 : 1, s);
  } else {
    e = cbq::launch_lut_decode(a, CBQ_AUTO_MAX_LUT_ROWS, s);
    if (e == hipSuccess && n_rows > CBQ_AUTO_MAX_LUT_ROWS)
      e = cbq::launch_mfma_prefill(a, CBQ_AUTO_MAX_LUT_ROWS, s);
  }
  if (e != hipSuccess) return hip_fail(e, "codebook_lut_gemm launch");
  return CBQ_OK;
}

CBQ_EXPORT int cbq_kmeans_codebooks(const uint16_t* w, int64_t R, int32_t K, int64_t ldw,
                                    int32_t bits, int32_t max_iters, uint8_t* idx,
                                    uint16_t* codebook, int32_t* iters_done, void* stream) {
  g_err[0] = 0;
  if (R < 0) return fail(CBQ_EINVAL, "R must be >= 0 (got %lld)", (long long)R);
  if (R > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "R must be < 2^31");
  if (K < 32 || K % 32) return fail(CBQ_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (K > 16384) return fail(CBQ_EUNSUPPORTED, "K must be <= 16384 (got %d)", K);
  if (ldw < K) return fail(CBQ_EINVAL, "ldw must be >= K (got %lld)", (long long)ldw);
  if (bits < 2 || bits > 4) return fail(CBQ_EUNSUPPORTED, "bits must be 2, 3 or 4 (got %d)", bits);
  if (max_iters < 0 || max_iters > 1000) return fail(CBQ_EINVAL, "max_iters must be in [0, 1000]");
  if (R == 0) return CBQ_OK;
  if (!w || !idx || !codebook) return fail(CBQ_EINVAL, "w, idx and codebook must be non-null");
  if ((reinterpret_cast<uintptr_t>(idx) & 3u) || (reinterpret_cast<uintptr_t>(w) & 1u) ||
      (reinterpret_cast<uintptr_t>(codebook) & 1u))
    return fail(CBQ_EINVAL, "idx must be 4-byte aligned, w and codebook 2-byte aligned");
  hipError_t e = cbq::launch_kmeans(w, R, K, ldw, bits, max_iters, idx, codebook, iters_done,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kmeans_codebooks launch");
  return CBQ_OK;
}

CBQ_EXPORT int cbq_refit_codebooks(const uint16_t* w, int64_t R, int32_t K, int64_t ldw, int32_t bits,
                                   const uint8_t* idx, const uint16_t* x, int32_t n, int64_t ldx,
                                   uint16_t* codebook, void* stream) {
  g_err[0] = 0;
  if (R < 0) return fail(CBQ_EINVAL, "R must be >= 0 (got %lld)", (long long)R);
  if (R > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "R must be < 2^31");
  if (K < 32 || K % 32) return fail(CBQ_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (K > 16384) return fail(CBQ_EUNSUPPORTED, "K must be <= 16384 (got %d)", K);
  if (ldw < K || ldx < K) return fail(CBQ_EINVAL, "ldw and ldx must be >= K");
  if (bits < 2 || bits > 4) return fail(CBQ_EUNSUPPORTED, "bits must be 2, 3 or 4 (got %d)", bits);
  if (n < 1 || n > 256) return fail(CBQ_EINVAL, "n must be in [1, 256] (got %d)", n);
  if (R == 0) return CBQ_OK;
  if (!w || !idx || !x || !codebook) return fail(CBQ_EINVAL, "w, idx, x and codebook must be non-null");
  if ((reinterpret_cast<uintptr_t>(w) & 1u) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(codebook) & 1u))
    return fail(CBQ_EINVAL, "w, x and codebook must be 2-byte aligned");
  hipError_t e = cbq::launch_refit(w, R, K, ldw, bits, idx, x, n, ldx, codebook, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "refit_codebooks launch");
  return CBQ_OK;
}

CBQ_EXPORT int cbq_cpu_lut_gemm(const uint8_t* codes, const float* scales, int32_t act_bits,
                                int64_t T, const cbq_weights* W, float* out, int64_t ldo,
                                int32_t n_threads, int32_t flags) {
  g_err[0] = 0;
  if (!W) return fail(CBQ_EINVAL, "W must be non-null");
  if (int rc = check_weights(W, 0)) return rc;
  if (W->E != 1) return fail(CBQ_EUNSUPPORTED, "the CPU kernel takes one weight set (E = 1, got %d)", W->E);
  if (W->layout != CBQ_LAYOUT_ROWS) return fail(CBQ_EUNSUPPORTED, "the CPU kernel reads the row layout only");
  if (act_bits != 4 && act_bits != 8) return fail(CBQ_EINVAL, "act_bits must be 4 or 8 (got %d)", act_bits);
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0");
  if (ldo < W->N) return fail(CBQ_EINVAL, "ldo must be >= N");
  if (n_threads < 0) return fail(CBQ_EINVAL, "n_threads must be >= 0");
  if (flags & ~CBQ_CPU_NO_AVX512) return fail(CBQ_EINVAL, "unknown flags 0x%x", flags);
  if (T == 0) return CBQ_OK;
  if (!codes || !scales || !out) return fail(CBQ_EINVAL, "codes, scales and out must be non-null");
  if (!cbq::cpu_lut_supported()) return fail(CBQ_EUNSUPPORTED, "the CPU kernel needs AVX2, FMA, F16C and BMI2");
  cbq::cpu_lut_gemm_impl(codes, scales, act_bits, T, W->N, W->K, W->bits, W->idx, W->codebook, out,
                         ldo, n_threads, (flags & CBQ_CPU_NO_AVX512) == 0);
  return CBQ_OK;
}

CBQ_EXPORT int cbq_moe_combine(const float* expert_out, const int32_t* slot_of, const float* topk_w,
                               int64_t T, int32_t topk, int32_t H, int32_t n_shared, float* y,
                               void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(CBQ_EINVAL, "T must be >= 0");
  if (T > 0x7FFFFFFF) return fail(CBQ_EUNSUPPORTED, "T must be < 2^31");
  if (topk < 1 || topk > 8) return fail(CBQ_EINVAL, "topk must be in [1, 8] (got %d)", topk);
  if (n_shared < 0 || n_shared > 8) return fail(CBQ_EINVAL, "n_shared must be in [0, 8]");
  if (H < 4 || H % 4) return fail(CBQ_EINVAL, "H must be a positive multiple of 4 (got %d)", H);
  if (T == 0) return CBQ_OK;
  if (!expert_out || !slot_of || !topk_w || !y) return fail(CBQ_EINVAL, "pointers must be non-null");
  if (!aligned16(expert_out) || !aligned16(y)) return fail(CBQ_EINVAL, "expert_out and y must be 16-byte aligned");
  hipError_t e = cbq::launch_combine(expert_out, slot_of, topk_w, T, topk, H, n_shared, y,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_combine launch");
  return CBQ_OK;
}
