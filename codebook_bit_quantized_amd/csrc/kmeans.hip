// Offline codebook construction: one 1-D K-means per weight row.
//
// CodeQuant2, Figure 3 (right): K-means initialises the centroid matrix and the
// per-row assignments; CodeQuant abstract: weight outliers are absorbed into the
// cluster centroids.  The output is exactly the format the LUT GEMM consumes: per
// row a 2^bits-entry fp16 codebook and an LSB-first bitstream of indices.
//
// One wave per row.  The row's bf16 patterns are sorted (bitonic network on
// order-preserving 16-bit keys, padded to a power of two with keys that sort last; in
// registers for rows up to 2048 channels, in LDS beyond);
// the initial centroids are the values at ranks floor((2j + 1) K / (2L)).  Each
// Lloyd round assigns every weight to the nearest centroid (fp64 |w - c|, ties to
// the lower index), sums the clusters in fp64 (exact for a row whose nonzero
// exponents spread at most 45 - ceil(log2 K) binades, so the order of the sums does
// not matter) and divides once.  In one dimension the clusters of the sorted row
// are contiguous ranges: each round finds the range boundaries by binary search and
// takes the cluster sums from exact prefix sums of the sorted row, and the
// assignment is unchanged exactly when every cluster count is; the rounds stop
// then, or after max_iters updates.  The centroids are
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

// Bitonic sort of Kp = 64 * KPL keys held KPL per lane (element i = lane * KPL + r):
// exchanges closer than KPL stay in a lane's registers, wider ones pair lanes.
template <int KPL>
__device__ __forceinline__ void sort_in_registers(uint32_t (&v)[KPL], int lane) {
#pragma unroll
  for (int k = 2; k <= 64 * KPL; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < KPL) {
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const int rp = r ^ j;
          if (rp > r) {
            const bool up = (((lane * KPL + r) & k) == 0);
            const uint32_t a = v[r], b = v[rp];
            const uint32_t lo = a < b ? a : b, hi = a < b ? b : a;
            v[r] = up ? lo : hi;
            v[rp] = up ? hi : lo;
          }
        }
      } else {
        const int m = j / KPL;                     // partner lane = lane ^ m
        const bool lower = (lane & m) == 0;
#pragma unroll
        for (int r = 0; r < KPL; ++r) {
          const bool up = (((lane * KPL + r) & k) == 0);
          const uint32_t p = (uint32_t)__shfl_xor((int)v[r], m);
          const uint32_t lo = v[r] < p ? v[r] : p, hi = v[r] < p ? p : v[r];
          v[r] = (lower == up) ? lo : hi;
        }
      }
    }
  }
}

template <int BITS, int KPL>
__global__ void __launch_bounds__(64)
kmeans_rows_kernel(const uint16_t* __restrict__ w, int64_t ldw, int K, int Kp, int use_prefix,
                   int max_iters, uint8_t* __restrict__ idx, uint16_t* __restrict__ codebook,
                   int32_t* __restrict__ iters_done) {
  constexpr int L = 1 << BITS;
  extern __shared__ __attribute__((aligned(16))) uint16_t keys[];   // [Kp], then fp64 P[K + 1]
  double* P = reinterpret_cast<double*>(keys + ((Kp + 3) & ~3));
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* src = w + row * ldw;

  // ---- sort the row's keys ----
  if constexpr (KPL > 0) {                         // Kp == 64 * KPL: in registers
    uint32_t v[KPL];
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
      const int i = lane * KPL + r;
      v[r] = i < K ? order_key16(src[i]) : 0xFFFFu;
    }
    sort_in_registers<KPL>(v, lane);
#pragma unroll
    for (int r = 0; r < KPL; ++r) keys[lane * KPL + r] = (uint16_t)v[r];
    __syncthreads();
  } else {                                         // longer rows: the network in LDS
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
  }
  auto value = [&](int i) { return bf16_bits_to_f64(key16_to_bits(keys[i])); };

  // ---- prefix sums of the sorted row (exact): P[i] = sum of the i smallest ----
  if (use_prefix) {
    const int seg = (K + 63) / 64;
    const int i0 = min(lane * seg, K), i1 = min(i0 + seg, K);
    double run = 0.0;
    for (int i = i0; i < i1; ++i) run += value(i);
    double incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    double acc = incl - run;                       // exact: a representable partial sum
    if (lane == 0) P[0] = 0.0;
    for (int i = i0; i < i1; ++i) {
      acc += value(i);
      P[i + 1] = acc;
    }
    __syncthreads();
  }

  // ---- initial centroids: values at ranks floor((2j + 1) K / (2L)) ----
  double c[L];
#pragma unroll
  for (int j = 0; j < L; ++j) c[j] = value(((2 * j + 1) * K) / (2 * L));

  // ---- Lloyd rounds over the sorted row ----
  // The nearest-centroid index is non-decreasing along the sorted row (for ordered
  // centroids and monotone rounding), so cluster j is the range [b_j, b_{j+1}) with
  // b_j the first position whose nearest centroid is >= j: one binary search per
  // boundary instead of a pass over the row.
  int prev[L];
#pragma unroll
  for (int j = 0; j < L; ++j) prev[j] = -1;
  int updates = 0;
  for (int it = 0; it < max_iters; ++it) {
    int bnd = K;                                   // lane j: boundary b_{j+1}
    if (lane < L - 1) {
      int lo = 0, hi = K;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (nearest<L>(value(mid), c) >= lane + 1) hi = mid; else lo = mid + 1;
      }
      bnd = lo;
    }
    int b[L + 1];
    b[0] = 0;
    b[L] = K;
#pragma unroll
    for (int j = 1; j < L; ++j) b[j] = __shfl(bnd, j - 1);
    int n[L];
    bool same = true;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      n[j] = b[j + 1] - b[j];
      same = same && (n[j] == prev[j]);
    }
    if (same) break;                               // counts fix the contiguous clusters
    double s[L];
    if (use_prefix) {
#pragma unroll
      for (int j = 0; j < L; ++j) s[j] = P[b[j + 1]] - P[b[j]];   // exact difference
    } else {
#pragma unroll
      for (int j = 0; j < L; ++j) s[j] = 0.0;
      for (int i = lane; i < K; i += 64) {
        const double v = value(i);
#pragma unroll
        for (int j = 0; j < L; ++j)
          if (i >= b[j] && i < b[j + 1]) s[j] += v;
      }
#pragma unroll
      for (int j = 0; j < L; ++j) s[j] = wave_sum_f64(s[j]);
    }
#pragma unroll
    for (int j = 0; j < L; ++j) {
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

template <int B, int KPL>
static void launch_one(dim3 grid, size_t lds, hipStream_t stream, const uint16_t* w, int64_t ldw,
                       int K, int Kp, int use_prefix, int max_iters, uint8_t* idx,
                       uint16_t* codebook, int32_t* iters_done) {
  hipLaunchKernelGGL((kmeans_rows_kernel<B, KPL>), grid, dim3(64), lds, stream, w, ldw, K, Kp,
                     use_prefix, max_iters, idx, codebook, iters_done);
}

template <int B>
static void launch_bits(int kpl, dim3 grid, size_t lds, hipStream_t stream, const uint16_t* w,
                        int64_t ldw, int K, int Kp, int use_prefix, int max_iters, uint8_t* idx,
                        uint16_t* codebook, int32_t* iters_done) {
  switch (kpl) {
    case 1: launch_one<B, 1>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 2: launch_one<B, 2>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 4: launch_one<B, 4>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 8: launch_one<B, 8>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 16: launch_one<B, 16>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 32: launch_one<B, 32>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    default: launch_one<B, 0>(grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
  }
}

// Output-aware refit of a row's centroids with its assignments fixed (the AI Radio
// episode on CodeQuant: centroids fine-tuned to minimise the layer's output error;
// CodeQuant2, Figure 1 right: centroids tuned after clustering).  One wave per row:
//  1. the row's assignments into LDS, and the mask of non-empty clusters;
//  2. for each calibration row i: P[i][j] = sum over k in cluster j of X[i][k] and
//     y[i] = sum_k X[i][k] w_k (lane partial sums, then a butterfly), into LDS;
//  3. M = P^T P and b = P^T y, one entry per lane and pass;
//  4. on lane 0: Cholesky over the non-empty clusters in index order; a pivot at most
//     1e-12 of the largest diagonal entry drops that cluster (it keeps its centroid,
//     its share P c moves to the right-hand side) and the factorisation restarts;
//     then the two triangular solves and one rounding to fp16.
template <int BITS>
__global__ void __launch_bounds__(64)
refit_rows_kernel(const uint16_t* __restrict__ w, int64_t ldw, int K, const uint8_t* __restrict__ idx,
                  const uint16_t* __restrict__ x, int n, int64_t ldx, uint16_t* __restrict__ codebook) {
  constexpr int L = 1 << BITS;
  extern __shared__ __attribute__((aligned(16))) double rsm[];
  double* sP = rsm;                  // [n][L]
  double* sy = sP + n * L;           // [n]
  double* sM = sy + n;               // [L][L]
  double* sb = sM + L * L;           // [L]
  double* sC = sb + L;               // [L][L] Cholesky factor
  uint8_t* sa = reinterpret_cast<uint8_t*>(sC + L * L);   // [K]
  const int lane = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int rb = K * BITS / 8;
  const uint8_t* ir = idx + r * (int64_t)rb;
  const uint16_t* wr = w + r * ldw;

  uint32_t used = 0;
  for (int k = lane; k < K; k += 64) {
    const int bit = k * BITS, byte = bit >> 3;
    const uint32_t v = ir[byte] | (byte + 1 < rb ? (uint32_t)ir[byte + 1] << 8 : 0u);
    const uint32_t a = (v >> (bit & 7)) & (L - 1);
    sa[k] = (uint8_t)a;
    used |= 1u << a;
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) used |= (uint32_t)__shfl_xor((int)used, d);
  __syncthreads();

  for (int i = 0; i < n; ++i) {
    double p[L];
#pragma unroll
    for (int j = 0; j < L; ++j) p[j] = 0.0;
    double yy = 0.0;
    const uint16_t* xi = x + (int64_t)i * ldx;
    for (int k = lane; k < K; k += 64) {
      const double xv = bf16_bits_to_f64(xi[k]);
      const int a = sa[k];
#pragma unroll
      for (int j = 0; j < L; ++j) p[j] += a == j ? xv : 0.0;
      yy = __builtin_fma(xv, bf16_bits_to_f64(wr[k]), yy);   // the product is exact
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
      for (int j = 0; j < L; ++j) p[j] += __shfl_xor(p[j], d);
      yy += __shfl_xor(yy, d);
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < L; ++j) sP[i * L + j] = p[j];
      sy[i] = yy;
    }
  }
  __syncthreads();
  for (int e = lane; e < L * L + L; e += 64) {
    double acc = 0.0;
    if (e < L * L) {
      const int j1 = e / L, j2 = e % L;
      for (int i = 0; i < n; ++i) acc = __builtin_fma(sP[i * L + j1], sP[i * L + j2], acc);
      sM[e] = acc;
    } else {
      const int j = e - L * L;
      for (int i = 0; i < n; ++i) acc = __builtin_fma(sP[i * L + j], sy[i], acc);
      sb[j] = acc;
    }
  }
  __syncthreads();
  if (lane != 0) return;

  uint16_t* cr = codebook + r * L;
  double c[L];
#pragma unroll
  for (int j = 0; j < L; ++j) c[j] = (double)__builtin_bit_cast(_Float16, cr[j]);
  uint32_t act = used;
  for (;;) {
    if (act == 0) return;
    int ix[L], na = 0;
    for (int j = 0; j < L; ++j)
      if (act >> j & 1u) ix[na++] = j;
    double dmax = 0.0;
    for (int q = 0; q < na; ++q) dmax = fmax(dmax, sM[ix[q] * L + ix[q]]);
    const double thr = 1e-12 * dmax;
    int bad = -1;
    for (int p_ = 0; p_ < na && bad < 0; ++p_) {
      double d = sM[ix[p_] * L + ix[p_]];
      for (int t = 0; t < p_; ++t) d -= sC[p_ * L + t] * sC[p_ * L + t];
      if (!(d > thr)) { bad = p_; break; }
      const double lpp = sqrt(d);
      sC[p_ * L + p_] = lpp;
      for (int q = p_ + 1; q < na; ++q) {
        double s = sM[ix[q] * L + ix[p_]];
        for (int t = 0; t < p_; ++t) s -= sC[q * L + t] * sC[p_ * L + t];
        sC[q * L + p_] = s / lpp;
      }
    }
    if (bad >= 0) { act &= ~(1u << ix[bad]); continue; }
    // right-hand side: clusters left out keep their centroid and their output share
    double rhs[L];
    const uint32_t fixed = used & ~act;
    for (int q = 0; q < na; ++q) {
      if (fixed == 0) { rhs[q] = sb[ix[q]]; continue; }
      double s = 0.0;
      for (int i = 0; i < n; ++i) {
        double yi = sy[i];
        for (int j = 0; j < L; ++j)
          if (fixed >> j & 1u) yi -= sP[i * L + j] * c[j];
        s += sP[i * L + ix[q]] * yi;
      }
      rhs[q] = s;
    }
    double z[L], sol[L];
    for (int p_ = 0; p_ < na; ++p_) {
      double s = rhs[p_];
      for (int t = 0; t < p_; ++t) s -= sC[p_ * L + t] * z[t];
      z[p_] = s / sC[p_ * L + p_];
    }
    for (int p_ = na - 1; p_ >= 0; --p_) {
      double s = z[p_];
      for (int t = p_ + 1; t < na; ++t) s -= sC[t * L + p_] * sol[t];
      sol[p_] = s / sC[p_ * L + p_];
    }
    for (int q = 0; q < na; ++q) cr[ix[q]] = (uint16_t)f64_to_f16_rne(sol[q]);
    return;
  }
}

size_t refit_lds_bytes(int K, int bits, int n) {
  const int L = 1 << bits;
  return (size_t)(n * L + n + 2 * L * L + L) * sizeof(double) + (size_t)((K + 15) & ~15);
}

hipError_t launch_refit(const uint16_t* w, int64_t R, int K, int64_t ldw, int bits, const uint8_t* idx,
                        const uint16_t* x, int n, int64_t ldx, uint16_t* codebook, hipStream_t stream) {
  const size_t lds = refit_lds_bytes(K, bits, n);
  const dim3 grid((unsigned)R);
  switch (bits) {
    case 2: hipLaunchKernelGGL(refit_rows_kernel<2>, grid, dim3(64), lds, stream, w, ldw, K, idx, x, n, ldx, codebook); break;
    case 3: hipLaunchKernelGGL(refit_rows_kernel<3>, grid, dim3(64), lds, stream, w, ldw, K, idx, x, n, ldx, codebook); break;
    case 4: hipLaunchKernelGGL(refit_rows_kernel<4>, grid, dim3(64), lds, stream, w, ldw, K, idx, x, n, ldx, codebook); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kmeans(const uint16_t* w, int64_t R, int K, int64_t ldw, int bits, int max_iters,
                         uint8_t* idx, uint16_t* codebook, int32_t* iters_done,
                         hipStream_t stream) {
  int Kp = 1;
  while (Kp < K) Kp <<= 1;
  // prefix sums of the sorted row in LDS up to 8192 channels (80 KB); longer rows sum
  // each cluster range in a pass over the row
  const int use_prefix = K <= 8192;
  const size_t lds = (size_t)((Kp + 3) & ~3) * sizeof(uint16_t) +
                     (use_prefix ? (size_t)(K + 1) * sizeof(double) : 0);
  const dim3 grid((unsigned)R);
  const int kpl = (Kp >= 64 && Kp <= 2048) ? Kp / 64 : 0;   // keys per lane; 0: sort in LDS
  switch (bits) {
    case 2: launch_bits<2>(kpl, grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 3: launch_bits<3>(kpl, grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    case 4: launch_bits<4>(kpl, grid, lds, stream, w, ldw, K, Kp, use_prefix, max_iters, idx, codebook, iters_done); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cbq
