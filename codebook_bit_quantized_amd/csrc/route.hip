// MoE top-k routing and per-expert row lists.
//
// The AI Radio episode on CodeQuant (introduction): a router sends every input to
// the experts that should handle it.  Readings: top-k on the logits with ties to
// the lower expert id; softmax weights over the k selected logits (or over all E);
// rows grouped expert by expert with tokens ascending; shared experts after.
//
// Kernel 1: one wave per token; the k winners are found by k rounds of a wave-wide
// max over 64-bit keys (order-preserving logit bits, then inverted expert id), with
// DPP row rotations and scalar lane reads rather than LDS permutes.
// Kernel 2: one workgroup does a counting sort by (expert, token).  Ranks come from
// per-expert token bitmaps, never from the order of atomics, so every integer output
// is deterministic.
#include <atomic>
#include <mutex>

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

// value of the lane n places down the same row of 16 (DPP row rotate)
template <int N>
__device__ __forceinline__ uint64_t row_ror_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, 0x120 + N, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), 0x120 + N, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// maximum over the wave, in every lane: rotations by 1, 2, 4 and 8 inside each row of
// 16 lanes (DPP, a few cycles each), then the four row maxima read as scalars
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o = row_ror_u64<1>(v); v = o > v ? o : v;
  o = row_ror_u64<2>(v); v = o > v ? o : v;
  o = row_ror_u64<4>(v); v = o > v ? o : v;
  o = row_ror_u64<8>(v); v = o > v ? o : v;
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  const uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// The k winners of token t, ids sel_id[0..k) and their softmax weights, in every lane.
// Called by whole waves only: the DPP rotations read every lane of a row.
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int64_t t, int E,
                                           int topk, int renormalize, int lane, int* sel_id,
                                           float* sel_w) {
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
  float sel_v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= topk) break;
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
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
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < topk) sel_w[j] = expf(sel_v[j] - vmax) / denom;
}

// One wave per token; workgroup c (16 waves) takes the tokens of chunk c and also
// writes the chunk's per-expert slot counts to ws[c][e] (LDS atomics: the counts do
// not depend on their order).
__global__ void __launch_bounds__(1024)
route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int topk, int renormalize,
                  int chunk, int32_t* __restrict__ ids, float* __restrict__ wts,
                  int32_t* __restrict__ ws) {
  __shared__ int s_cnt[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk < T ? c0 + chunk : T;
  for (int64_t t = c0 + wave; t < c1; t += 16) {
    int sel_id[8];
    float sel_w[8];
    topk_token(logits, t, E, topk, renormalize, lane, sel_id, sel_w);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < topk) {
          ids[t * topk + j] = sel_id[j];
          wts[t * topk + j] = sel_w[j];
          atomicAdd(&s_cnt[sel_id[j]], 1);
        }
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) ws[(int64_t)blockIdx.x * E + e] = s_cnt[e];
}

constexpr int SCATTER_SUB = 1024;             // tokens per bitmap pass
constexpr int SCATTER_WORDS = SCATTER_SUB / 32;

// Workgroup c places the slots of chunk c.  An expert's rows start at the rows of all
// earlier experts plus that expert's slots in earlier chunks (from the counts in
// ws); inside the chunk a slot's rank is the number of earlier tokens in the
// expert's token bitmap, so every output is deterministic.
__global__ void __launch_bounds__(1024)
route_scatter_kernel(const int32_t* __restrict__ ids, int64_t T, int E, int topk, int n_shared,
                     int chunk, int nchunks, const int32_t* __restrict__ ws,
                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_tokens,
                     int32_t* __restrict__ slot_of) {
  __shared__ int total[256];
  __shared__ int base[256];
  __shared__ int sub_cnt[256];
  __shared__ uint32_t mask[256 * SCATTER_WORDS];
  __shared__ int pre[256 * SCATTER_WORDS];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int c = blockIdx.x;
  const int64_t nslots = T * topk;

  for (int e = tid; e < E; e += nthr) {
    total[e] = 0;
    base[e] = 0;
  }
  __syncthreads();
  {
    // thread (part p, expert e) sums chunks p, p + parts, ... of expert e in registers,
    // then adds its two partial sums in LDS (integer sums: the order does not matter)
    const int parts = nthr / E;   // >= 4 with 1024 threads (E <= 256); the zero-token
                                  // launch (64 threads) may get 0 but has no chunks
    if (tid < parts * E) {
      const int e = tid % E, p = tid / E;
      int tot = 0, bs = 0;
      for (int cc = p; cc < nchunks; cc += parts) {
        const int v = ws[(int64_t)cc * E + e];
        tot += v;
        if (cc < c) bs += v;
      }
      if (tot) atomicAdd(&total[e], tot);
      if (bs) atomicAdd(&base[e], bs);
    }
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of the expert totals by the first wave: lane l holds experts
    // 4l .. 4l+3 (E <= 256)
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      v[i] = e < E ? total[e] : 0;
      sum += v[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      if (e < E) {
        base[e] += run;
        if (c == 0) offsets[e] = run;
      }
      run += v[i];
    }
    const int routed = __shfl(incl, 63);   // every routed slot (read by the whole wave)
    if (c == 0 && tid == 0) {
      int r = routed;
      for (int s2 = 0; s2 < n_shared; ++s2) {
        offsets[E + s2] = r;
        r += (int)T;
      }
      offsets[E + n_shared] = r;
    }
  }
  __syncthreads();

  const int64_t t0 = (int64_t)c * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
  for (int64_t s0 = t0; s0 < t1; s0 += SCATTER_SUB) {
    const int ct = (int)((t1 - s0) < SCATTER_SUB ? (t1 - s0) : SCATTER_SUB);
    const int nw = (ct + 31) >> 5;
    for (int i = tid; i < E * nw; i += nthr) mask[(i / nw) * SCATTER_WORDS + i % nw] = 0u;
    __syncthreads();
    for (int i = tid; i < ct * topk; i += nthr) {
      const int lt = i / topk;
      const int e = ids[(s0 + lt) * topk + (i - lt * topk)];
      atomicOr(&mask[e * SCATTER_WORDS + (lt >> 5)], 1u << (lt & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {
      int run = 0;
      for (int w = 0; w < nw; ++w) {
        pre[e * SCATTER_WORDS + w] = run;
        run += __popc(mask[e * SCATTER_WORDS + w]);
      }
      sub_cnt[e] = run;
    }
    __syncthreads();
    for (int i = tid; i < ct * topk; i += nthr) {
      const int lt = i / topk;
      const int j = i - lt * topk;
      const int64_t t = s0 + lt;
      const int e = ids[t * topk + j];
      const int w = lt >> 5;
      const uint32_t below = mask[e * SCATTER_WORDS + w] & ((1u << (lt & 31)) - 1u);
      const int row = base[e] + pre[e * SCATTER_WORDS + w] + __popc(below);
      sorted_tokens[row] = (int32_t)t;
      slot_of[t * topk + j] = row;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) base[e] += sub_cnt[e];
    __syncthreads();
  }
  // shared experts: row T*k + s*T + t holds token t
  for (int s = 0; s < n_shared; ++s)
    for (int64_t t = t0 + tid; t < t1; t += nthr) sorted_tokens[nslots + (int64_t)s * T + t] = (int32_t)t;
}

// tokens per chunk: at least 16, and at most 256 chunks
int64_t route_chunk(int64_t T) {
  int64_t ch = (T + 255) / 256;
  ch = (ch + 15) / 16 * 16;
  return ch < 16 ? 16 : ch;
}

size_t route_workspace_bytes(int64_t T, int E) {
  if (T <= 0) return 0;
  const int64_t ch = route_chunk(T);
  return (size_t)((T + ch - 1) / ch) * (size_t)E * sizeof(int32_t);
}

// Scratch for callers that cannot allocate: the per-chunk expert counts of the largest
// call (256 chunks x 256 experts), in a module-scope device array.  Every GPU that runs
// the library holds its own copy until the process ends.  Host code never uses the
// array's name as an address (on the host it only stands for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device on that device's
// first call and kept per device.
constexpr size_t kRouteScratchBytes = 256 * 256 * sizeof(int32_t);
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

size_t route_scratch_bytes() { return kRouteScratchBytes; }

hipError_t route_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<int32_t*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_route(const float* logits, int64_t T, int E, int topk, int renormalize,
                        int n_shared, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_tokens, int32_t* slot_of, int32_t* ws, hipStream_t stream) {
  if (T == 0) {
    // no tokens: every expert range is empty
    hipLaunchKernelGGL(route_scatter_kernel, dim3(1), dim3(64), 0, stream, ids, T, E, topk,
                       n_shared, 16, 0, ws, offsets, sorted_tokens, slot_of);
    return hipGetLastError();
  }
  const int64_t ch = route_chunk(T);
  const int nch = (int)((T + ch - 1) / ch);
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)nch), dim3(1024), 0, stream, logits, T, E,
                     topk, renormalize, (int)ch, ids, w, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)nch), dim3(1024), 0, stream, ids, T, E,
                     topk, n_shared, (int)ch, nch, ws, offsets, sorted_tokens, slot_of);
  return hipGetLastError();
}

}  // namespace cbq
