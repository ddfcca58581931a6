// MoE top-k routing and per-expert row lists.
//
// The AI Radio episode on CodeQuant (introduction): a router sends every input to
// the experts that should handle it.  Readings: top-k on the logits with ties to
// the lower expert id; softmax weights over the k selected logits (or over all E);
// rows grouped expert by expert with tokens ascending; shared experts after.
//
// Kernel 1: one wave per token; the k winners are found by k rounds of a wave-wide
// max over 64-bit keys (order-preserving logit bits, then inverted expert id).
// Kernel 2: one workgroup does a counting sort by (expert, token).  Ranks come from
// per-expert token bitmaps, never from the order of atomics, so every integer output
// is deterministic.
#include "cbq_internal.hpp"

namespace cbq {

__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);   // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int topk, int renormalize,
                  int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  constexpr int PER = 4;   // E <= 256
  uint64_t key[PER];
  float val[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    val[i] = e < E ? row[e] : 0.0f;
    key[i] = e < E ? (((uint64_t)order_bits(val[i]) << 32) | (0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  int sel_id[8];
  float sel_v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= topk) break;
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) best = key[i] > best ? key[i] : best;
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    sel_id[j] = e;
    sel_v[j] = from_order_bits((uint32_t)(best >> 32));
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
  }
  const float vmax = sel_v[0];
  float denom;
  if (renormalize) {
    denom = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < topk) denom += expf(sel_v[j] - vmax);
  } else {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < E) part += expf(val[i] - vmax);
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    denom = part;
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < topk) {
        ids[t * topk + j] = sel_id[j];
        wts[t * topk + j] = expf(sel_v[j] - vmax) / denom;
      }
    }
  }
}

constexpr int SCATTER_CHUNK = 1024;           // tokens per bitmap pass
constexpr int SCATTER_WORDS = SCATTER_CHUNK / 32;

__global__ void __launch_bounds__(1024)
route_scatter_kernel(const int32_t* __restrict__ ids, int64_t T, int E, int topk, int n_shared,
                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_tokens,
                     int32_t* __restrict__ slot_of) {
  __shared__ int cnt[256];
  __shared__ int base[256];
  __shared__ int chunk_cnt[256];
  __shared__ uint32_t mask[256 * SCATTER_WORDS];
  __shared__ int pre[256 * SCATTER_WORDS];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int64_t nslots = T * topk;

  for (int e = tid; e < E; e += nthr) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = tid; i < nslots; i += nthr) atomicAdd(&cnt[ids[i]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      offsets[e] = run;
      run += cnt[e];
    }
    for (int s = 0; s < n_shared; ++s) {
      offsets[E + s] = run;
      run += (int)T;
    }
    offsets[E + n_shared] = run;
  }
  __syncthreads();

  for (int64_t c0 = 0; c0 < T; c0 += SCATTER_CHUNK) {
    const int ct = (int)((T - c0) < SCATTER_CHUNK ? (T - c0) : SCATTER_CHUNK);
    for (int i = tid; i < E * SCATTER_WORDS; i += nthr) mask[i] = 0u;
    __syncthreads();
    for (int i = tid; i < ct * topk; i += nthr) {
      const int lt = i / topk;
      const int e = ids[(c0 + lt) * topk + (i - lt * topk)];
      atomicOr(&mask[e * SCATTER_WORDS + (lt >> 5)], 1u << (lt & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {
      int run = 0;
      for (int w = 0; w < SCATTER_WORDS; ++w) {
        pre[e * SCATTER_WORDS + w] = run;
        run += __popc(mask[e * SCATTER_WORDS + w]);
      }
      chunk_cnt[e] = run;
    }
    __syncthreads();
    for (int i = tid; i < ct * topk; i += nthr) {
      const int lt = i / topk;
      const int j = i - lt * topk;
      const int64_t t = c0 + lt;
      const int e = ids[t * topk + j];
      const int w = lt >> 5;
      const uint32_t below = mask[e * SCATTER_WORDS + w] & ((1u << (lt & 31)) - 1u);
      const int row = base[e] + pre[e * SCATTER_WORDS + w] + __popc(below);
      sorted_tokens[row] = (int32_t)t;
      slot_of[t * topk + j] = row;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) base[e] += chunk_cnt[e];
    __syncthreads();
  }
  const int64_t nsh = (int64_t)n_shared * T;
  for (int64_t i = tid; i < nsh; i += nthr) sorted_tokens[nslots + i] = (int32_t)(i % T);
}

hipError_t launch_route(const float* logits, int64_t T, int E, int topk, int renormalize,
                        int n_shared, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_tokens, int32_t* slot_of, hipStream_t stream) {
  if (T > 0) {
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                       logits, T, E, topk, renormalize, ids, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(route_scatter_kernel, dim3(1), dim3(1024), 0, stream, ids, T, E, topk,
                     n_shared, offsets, sorted_tokens, slot_of);
  return hipGetLastError();
}

}  // namespace cbq
