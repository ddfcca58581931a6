// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "cbq_device.hpp"

namespace cbq {

// Device view of one weight set (see cbq_weights in cbq.h).
struct GemmW {
  const uint8_t* idx;
  const uint16_t* codebook;
};

struct GemmArgs {
  const uint8_t* codes;
  const float* scales;
  int act_bits;
  int64_t n_rows;
  const int32_t* offsets;   // nullptr: dense
  const int32_t* row_token; // nullptr: identity
  GemmW w[2];
  int n_w;
  int E, N, K, bits;
  bool swiglu;
  void* out;
  int64_t ldo;
};

hipError_t launch_rotate_quantize(const uint16_t* x, int64_t T, int K, int64_t ldx, int b,
                                  int act_bits, const float* smooth, const uint8_t* signs,
                                  uint8_t* codes, float* scales, uint32_t* precond,
                                  hipStream_t stream);

size_t route_workspace_bytes(int64_t T, int E);
hipError_t launch_route(const float* logits, int64_t T, int E, int topk, int renormalize,
                        int n_shared, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_tokens, int32_t* slot_of, int32_t* ws, hipStream_t stream);

// LUT (decode) path.  max_rows >= 0: experts with more rows are skipped (AUTO split).
hipError_t launch_lut_decode(const GemmArgs& a, int max_rows, hipStream_t stream);

// MFMA (prefill) path.  Experts with at most min_rows rows are skipped (AUTO split).
hipError_t launch_mfma_prefill(const GemmArgs& a, int min_rows, hipStream_t stream);

hipError_t launch_kmeans(const uint16_t* w, int64_t R, int K, int64_t ldw, int bits, int max_iters,
                         uint8_t* idx, uint16_t* codebook, int32_t* iters_done,
                         hipStream_t stream);

hipError_t launch_refit(const uint16_t* w, int64_t R, int K, int64_t ldw, int bits, const uint8_t* idx,
                        const uint16_t* x, int n, int64_t ldx, uint16_t* codebook, hipStream_t stream);

size_t dense_rotation_workspace_bytes(int64_t T, int K);
hipError_t launch_rotate_dense(const uint16_t* x, int64_t T, int K, int64_t ldx, const uint16_t* R,
                               int act_bits, uint8_t* codes, float* scales, uint32_t* precond,
                               void* ws, hipStream_t stream);

hipError_t launch_combine(const float* expert_out, const int32_t* slot_of, const float* w,
                          int64_t T, int topk, int H, int n_shared, float* y, hipStream_t stream);

}  // namespace cbq
