// Offline codebook construction: one 1-D K-means per weight row.
//
// CodeQuant2, Figure 3 (right): K-means initialises the centroid matrix and the
// per-row assignments; CodeQuant abstract: weight outliers are absorbed into the
// cluster centroids.  The output is exactly the format the LUT GEMM consumes: per
// row a 2^bits-entry fp16 codebook and an LSB-first bitstream of indices.
//
// One wave per row.  The row's bf16 patterns are sorted in LDS (bitonic network on
// order-preserving 16-bit keys, padded to a power of two with keys that sort last);
// the initial centroids are the values at ranks floor((2j + 1) K / (2L)).  Each
// Lloyd round assigns every weight to the nearest centroid (fp64 |w - c|, ties to
// the lower index), sums the clusters in fp64 (exact for a row whose nonzero
// exponents spread at most 45 - ceil(log2 K) binades, so the order of the sums does
// not matter) and divides once.  In one dimension the clusters of the sorted row
// are contiguous ranges, so the assignment is unchanged exactly when every cluster
// count is; the rounds stop then, or after max_iters updates.  The centroids are
// rounded once to fp16 and the weights, in their original order, are assigned
// against the fp16 values.
#include "cbq_internal.hpp"

namespace cbq {

namespace {

__device__ __forceinline__ uint32_t order_key16(uint32_t b) {
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ uint32_t key16_to_bits(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
}

__device__ __forceinline__ double bf16_bits_to_f64(uint32_t b) {
  return (double)__builtin_bit_cast(float, b << 16);
}

// fp64 -> fp16, one rounding (nearest, ties to even); subnormals kept, overflow to inf.
__device__ uint32_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return sign | 0x7C00u | (a > 0x7FF0000000000000ull ? 0x200u : 0u);
  const int e = (int)(a >> 52) - 1023;
  if (e < -25) return sign;                        // below half the smallest subnormal
  if (e > 15) return sign | 0x7C00u;
  const uint64_t m = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int shift = e >= -14 ? 42 : 28 - e;        // keep 10 fraction bits / subnormal units
  uint64_t r = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  uint32_t h = e >= -14 ? (uint32_t)(((e + 15) << 10) + (int)(r - 1024)) : (uint32_t)r;
  if (h > 0x7C00u) h = 0x7C00u;
  return sign | h;
}

template <int L>
__device__ __forceinline__ int nearest(double w, const double* c) {
  int best = 0;
  double bd = fabs(w - c[0]);
#pragma unroll
  for (int j = 1; j < L; ++j) {
    const double d = fabs(w - c[j]);
    if (d < bd) { bd = d; best = j; }
  }
  return best;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace

template <int BITS>
__global__ void __launch_bounds__(64)
kmeans_rows_kernel(const uint16_t* __restrict__ w, int64_t ldw, int K, int Kp, int max_iters,
                   uint8_t* __restrict__ idx, uint16_t* __restrict__ codebook,
                   int32_t* __restrict__ iters_done) {
  constexpr int L = 1 << BITS;
  extern __shared__ uint16_t keys[];               // [Kp]
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* src = w + row * ldw;

  // ---- sort the row's keys ----
  for (int i = lane; i < Kp; i += 64) keys[i] = i < K ? (uint16_t)order_key16(src[i]) : (uint16_t)0xFFFFu;
  __syncthreads();
  for (int k = 2; k <= Kp; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < Kp; i += 64) {
        const int l = i ^ j;
        if (l > i) {
          const uint16_t a = keys[i], b = keys[l];
          const bool up = (i & k) == 0;
          if (up ? (a > b) : (a < b)) { keys[i] = b; keys[l] = a; }
        }
      }
      __syncthreads();
    }
  }

  // ---- initial centroids: values at ranks floor((2j + 1) K / (2L)) ----
  double c[L];
#pragma unroll
  for (int j = 0; j < L; ++j) c[j] = bf16_bits_to_f64(key16_to_bits(keys[((2 * j + 1) * K) / (2 * L)]));

  // ---- Lloyd rounds over the sorted row ----
  int prev[L];
#pragma unroll
  for (int j = 0; j < L; ++j) prev[j] = -1;
  int updates = 0;
  for (int it = 0; it < max_iters; ++it) {
    double s[L];
    int n[L];
#pragma unroll
    for (int j = 0; j < L; ++j) { s[j] = 0.0; n[j] = 0; }
    for (int i = lane; i < K; i += 64) {
      const double v = bf16_bits_to_f64(key16_to_bits(keys[i]));
      const int a = nearest<L>(v, c);
#pragma unroll
      for (int j = 0; j < L; ++j) {
        if (a == j) { s[j] += v; n[j] += 1; }
      }
    }
    bool same = true;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      n[j] = wave_sum_i32(n[j]);
      same = same && (n[j] == prev[j]);
    }
    if (same) break;                               // counts fix the contiguous clusters
#pragma unroll
    for (int j = 0; j < L; ++j) {
      s[j] = wave_sum_f64(s[j]);
      if (n[j] > 0) c[j] = s[j] / (double)n[j];
      prev[j] = n[j];
    }
    ++updates;
  }

  // ---- fp16 codebook, then the final assignment in the original order ----
  double c16[L];
  uint32_t cb[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    cb[j] = f64_to_f16_rne(c[j]);
    c16[j] = (double)__builtin_bit_cast(_Float16, (uint16_t)cb[j]);
  }
  if (lane < L) {
    uint32_t mine = cb[0];
#pragma unroll
    for (int j = 1; j < L; ++j) mine = lane == j ? cb[j] : mine;
    codebook[row * L + lane] = (uint16_t)mine;
  }
  if (lane == 0 && iters_done) iters_done[row] = updates;

  uint8_t* dst = idx + row * ((int64_t)K * BITS / 8);
  for (int g = lane; g < K / 32; g += 64) {        // 32 indices -> 4*BITS bytes
    uint32_t out[BITS];
#pragma unroll
    for (int q = 0; q < BITS; ++q) out[q] = 0u;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const uint32_t a = (uint32_t)nearest<L>(bf16_bits_to_f64(src[g * 32 + t]), c16);
      const int bit = t * BITS;
      out[bit >> 5] |= a << (bit & 31);
      if ((bit & 31) + BITS > 32) out[(bit >> 5) + 1] |= a >> (32 - (bit & 31));
    }
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + (int64_t)g * 4 * BITS);
#pragma unroll
    for (int q = 0; q < BITS; ++q) d[q] = out[q];
  }
}

hipError_t launch_kmeans(const uint16_t* w, int64_t R, int K, int64_t ldw, int bits, int max_iters,
                         uint8_t* idx, uint16_t* codebook, int32_t* iters_done,
                         hipStream_t stream) {
  int Kp = 1;
  while (Kp < K) Kp <<= 1;
  const size_t lds = (size_t)Kp * sizeof(uint16_t);
  const dim3 grid((unsigned)R), block(64);
  switch (bits) {
    case 2: hipLaunchKernelGGL(kmeans_rows_kernel<2>, grid, block, lds, stream, w, ldw, K, Kp,
                               max_iters, idx, codebook, iters_done); break;
    case 3: hipLaunchKernelGGL(kmeans_rows_kernel<3>, grid, block, lds, stream, w, ldw, K, Kp,
                               max_iters, idx, codebook, iters_done); break;
    case 4: hipLaunchKernelGGL(kmeans_rows_kernel<4>, grid, block, lds, stream, w, ldw, K, Kp,
                               max_iters, idx, codebook, iters_done); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cbq
