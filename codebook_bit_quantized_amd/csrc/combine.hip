// Weighted combine of expert outputs per token (routing weights from the router's
// softmax; shared experts added with weight 1).  One workgroup per token, float4
// accesses; HBM-bound.
#include "cbq_internal.hpp"

namespace cbq {

__global__ void __launch_bounds__(256)
combine_kernel(const f32x4* __restrict__ out, const int32_t* __restrict__ slot_of,
               const float* __restrict__ w, int64_t T, int topk, int H4, int n_shared,
               f32x4* __restrict__ y) {
  const int64_t t = blockIdx.x;
  int32_t rows[8];
  float ws[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < topk ? slot_of[t * topk + j] : 0;
    ws[j] = j < topk ? w[t * topk + j] : 0.0f;
  }
  for (int h = threadIdx.x; h < H4; h += blockDim.x) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < topk) acc += ws[j] * out[(int64_t)rows[j] * H4 + h];
    for (int s = 0; s < n_shared; ++s) acc += out[(T * topk + s * T + t) * H4 + h];
    y[t * H4 + h] = acc;
  }
}

hipError_t launch_combine(const float* expert_out, const int32_t* slot_of, const float* w,
                          int64_t T, int topk, int H, int n_shared, float* y, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(expert_out), slot_of, w, T, topk, H / 4,
                     n_shared, reinterpret_cast<f32x4*>(y));
  return hipGetLastError();
}

}  // namespace cbq
