// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "cbq_device.hpp"

namespace cbq {

// Where 2- and 3-bit codebooks are looked up: each path's default, register tables or
// LDS pair tables.
enum { kTablesDefault = 0, kTablesReg = 1, kTablesLds = 2 };

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
  int tables;               // kTables*: placement of 2- and 3-bit codebook tables
  int blocked;              // 1: indices in the blocked layout (cbq_prepack_weights)
  void* out;
  int64_t ldo;
  void* ws;                 // optional workspace (K-split partial sums of the MFMA path)
  size_t ws_bytes;
};

hipError_t launch_rotate_quantize(const uint16_t* x, int64_t T, int K, int64_t ldx, int b,
                                  int act_bits, const float* smooth, const uint8_t* signs,
                                  uint8_t* codes, float* scales, uint32_t* precond,
                                  hipStream_t stream);

// Compute units of the current device (cached per device after the first query).
hipError_t device_cu_count(int* out);

size_t route_workspace_bytes(int64_t T, int E);
// The library's own route scratch (no allocation): its size, and its device address on
// the current device (looked up on that device's first call).
size_t route_scratch_bytes();
hipError_t route_scratch(int32_t** out);
hipError_t launch_route(const float* logits, int64_t T, int E, int topk, int renormalize,
                        int n_shared, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_tokens, int32_t* slot_of, int32_t* ws, hipStream_t stream);

// LUT (decode) path.  max_rows >= 0: experts with more rows are skipped (AUTO split).
hipError_t launch_lut_decode(const GemmArgs& a, int max_rows, hipStream_t stream);

// MFMA (prefill) path.  Experts with at most min_rows rows are skipped (AUTO split).
hipError_t launch_mfma_prefill(const GemmArgs& a, int min_rows, hipStream_t stream);

// Workspace bytes with which a single-matrix MFMA call of these sizes may split K in two
// (0: it never splits).  The launcher splits when the workspace holds that many bytes and
// the call's 256-row tiles would leave CUs idle.
size_t mfma_split_workspace_bytes(int n_w, int bits, int64_t n_rows, int N, int K);

// The pages' table forms (4-bit codebooks, A4): mode 0 per-row product tables with sign
// folding, mode 1 per-row integer buckets of the activation codes.
hipError_t launch_lut_pages(const GemmArgs& a, int mode, hipStream_t stream);

// Regroups a row-layout index block [E][N][K*bits/8] into the blocked layout.
hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int E, int N, int K, int bits,
                          hipStream_t stream);

// Bytes per row of one expert's index block: K (rows layout) or K rounded up to a
// multiple of 128 (blocked layout), times bits / 8.
__host__ __device__ inline int64_t index_row_bytes(int K, int bits, bool blocked) {
  const int64_t kp = blocked ? (int64_t)(K + 127) / 128 * 128 : K;
  return kp * bits / 8;
}

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
