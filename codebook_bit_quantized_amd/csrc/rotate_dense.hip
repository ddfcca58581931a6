// Dense rotation + per-token absmax quantisation: u = R x with R a K x K bf16 matrix
// standing for a learned rotation (CodeQuant2, Figure 1: a rotation fused into the
// model smooths activation outliers; CodeQuant abstract: the rotation may be learned).
//
// u must be the exact sum, rounded once to fp32, for the codes to be those of the
// plain definition.  bf16 x bf16 products are exact in fp64, and the K-term sums stay
// exact in any order while the token's exponent spread plus the widest row spread of
// R is at most 37 - ceil(log2 K) binades (counted, when asked, per token).  So the
// contraction runs on the fp64 matrix cores (v_mfma_f64_16x16x4_f64), which makes the
// summation order irrelevant inside that bound.
//
// Pass 1 (GEMM): a 64-token x 64-output tile per workgroup, 32 channels per step,
// both operands converted to fp64 into LDS (channel-major, padded so a wave's two
// halves fall in opposite bank halves); four waves of 32 x 32, each a 2 x 2 set of
// 16 x 16 fp64 accumulators.  fp32(u) goes to the workspace.
// Pass 2: one wave per token: absmax over K, then the same quantiser as the Hadamard
// path (the quotient as fp64(v) * fp64(1/s) rounded to fp32 equals the IEEE division),
// scale = s (R is orthonormal: no 1/sqrt(b) factor).
#include "cbq_internal.hpp"

namespace cbq {

namespace {
constexpr int DTM = 64, DTN = 64, DTK = 32;
constexpr int DLP = 80;          // LDS pitch in doubles: 160 dwords, half the banks apart
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_f64(uint32_t h) {
  return (double)__builtin_bit_cast(float, h << 16);
}
}  // namespace

__global__ void __launch_bounds__(256)
dense_rot_gemm_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t T, int K,
                      const uint16_t* __restrict__ R, float* __restrict__ u) {
  __shared__ double Xs[DTK][DLP];   // [channel][token]
  __shared__ double Rs[DTK][DLP];   // [channel][output]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.x * DTM;
  const int j0 = blockIdx.y * DTN;
  // loader: thread -> tile row lr (token or output), channels lk .. lk+7 of the step
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const bool xok = t0 + lr < T;
  const uint16_t* xp = x + (xok ? (t0 + lr) * ldx : 0) + lk;
  const uint16_t* rp = R + (int64_t)(j0 + lr) * K + lk;
  f64x4 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f64x4{0.0, 0.0, 0.0, 0.0};

  for (int k0 = 0; k0 < K; k0 += DTK) {
    const u32x4 xv = xok ? *reinterpret_cast<const u32x4*>(xp + k0) : u32x4{0, 0, 0, 0};
    const u32x4 rv = *reinterpret_cast<const u32x4*>(rp + k0);
    __syncthreads();                         // the previous step's tiles are consumed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Xs[lk + 2 * i][lr] = bf16_to_f64(xv[i] & 0xFFFFu);
      Xs[lk + 2 * i + 1][lr] = bf16_to_f64(xv[i] >> 16);
      Rs[lk + 2 * i][lr] = bf16_to_f64(rv[i] & 0xFFFFu);
      Rs[lk + 2 * i + 1][lr] = bf16_to_f64(rv[i] >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < DTK; kk += 4) {
      // A (16 x 4): lane holds A[lane & 15][lane >> 4]; B (4 x 16): B[lane >> 4][lane & 15]
      double a[2], b[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) a[m] = Xs[kk + (lane >> 4)][wr * 32 + m * 16 + (lane & 15)];
#pragma unroll
      for (int n = 0; n < 2; ++n) b[n] = Rs[kk + (lane >> 4)][wc * 32 + n * 16 + (lane & 15)];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[n], acc[m][n], 0, 0, 0);
    }
  }
  // D (16 x 16): lane holds D[(lane >> 4) + 4 * r][lane & 15], r = 0..3 (measured: the
  // fp64 16x16 layout interleaves rows by 4, unlike the fp32 one)
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wr * 32 + m * 16 + (lane >> 4) + 4 * r;
        const int col = j0 + wc * 32 + n * 16 + (lane & 15);
        if (t < T) u[t * K + col] = (float)acc[m][n][r];
      }
}

// widest exponent spread of a row of R over its nonzero entries (-1: R is all zero)
__global__ void __launch_bounds__(1024)
dense_row_spread_kernel(const uint16_t* __restrict__ R, int K, int* __restrict__ out) {
  __shared__ int red[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int best = -1;
  for (int j = wave; j < K; j += 16) {
    int emin = 1 << 20, emax = -(1 << 20);
    for (int k = lane; k < K; k += 64) {
      const float f = __builtin_bit_cast(float, (uint32_t)R[(int64_t)j * K + k] << 16);
      if (f != 0.0f) {
        const int e = __builtin_amdgcn_frexp_expf(f) - 1;
        emin = min(emin, e);
        emax = max(emax, e);
      }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      emin = min(emin, __shfl_xor(emin, d));
      emax = max(emax, __shfl_xor(emax, d));
    }
    if (emax >= emin) best = max(best, emax - emin);
  }
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    int m = red[0];
    for (int w = 1; w < 16; ++w) m = max(m, red[w]);
    out[0] = m;
  }
}

__global__ void __launch_bounds__(256)
dense_quant_kernel(const float* __restrict__ u, int64_t T, int K, int act_bits,
                   uint8_t* __restrict__ codes, float* __restrict__ scales,
                   const uint16_t* __restrict__ x, int64_t ldx, const int* __restrict__ rspread,
                   int bound, uint32_t* __restrict__ precond) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                        // no barriers below
  const float* ur = u + t * K;
  float amax = 0.0f;
  for (int c = lane * 4; c < K; c += 256) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ur + c);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float Q = act_bits == 4 ? 7.0f : 127.0f;
  const float lo = act_bits == 4 ? -8.0f : -127.0f;
  const float s = amax / Q;
  const double rs = amax > 0.0f ? 1.0 / (double)s : 0.0;
  for (int c = lane * 8; c < K; c += 512) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(ur + c);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(ur + c + 4);
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = rintf((float)((double)(i < 4 ? v0[i] : v1[i - 4]) * rs));
      q[i] = (int)__builtin_amdgcn_fmed3f(r, lo, Q);
    }
    if (act_bits == 4) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= ((uint32_t)q[i] & 0xFu) << (4 * i);
      *reinterpret_cast<uint32_t*>(codes + t * (K / 2) + c / 2) = w;
    } else {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= ((uint32_t)q[i] & 0xFFu) << (8 * i);
        w1 |= ((uint32_t)q[i + 4] & 0xFFu) << (8 * i);
      }
      *reinterpret_cast<u32x2*>(codes + t * K + c) = u32x2{w0, w1};
    }
  }
  if (lane == 0) scales[t] = amax > 0.0f ? s : 0.0f;

  if (precond != nullptr) {
    int emin = 1 << 20, emax = -(1 << 20);
    for (int k = lane; k < K; k += 64) {
      const float f = __builtin_bit_cast(float, (uint32_t)x[t * ldx + k] << 16);
      if (f != 0.0f) {
        const int e = __builtin_amdgcn_frexp_expf(f) - 1;
        emin = min(emin, e);
        emax = max(emax, e);
      }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      emin = min(emin, __shfl_xor(emin, d));
      emax = max(emax, __shfl_xor(emax, d));
    }
    const int dr = rspread[0];
    if (lane == 0 && emax >= emin && dr >= 0 && (emax - emin) + dr > bound) atomicAdd(precond, 1u);
  }
}

size_t dense_rotation_workspace_bytes(int64_t T, int K) {
  return (size_t)T * (size_t)K * sizeof(float) + 256;
}

hipError_t launch_rotate_dense(const uint16_t* x, int64_t T, int K, int64_t ldx, const uint16_t* R,
                               int act_bits, uint8_t* codes, float* scales, uint32_t* precond,
                               void* ws, hipStream_t stream) {
  float* u = static_cast<float*>(ws);
  int* rspread = reinterpret_cast<int*>(static_cast<char*>(ws) + (size_t)T * K * sizeof(float));
  int logk = 0;
  while ((1 << logk) < K) ++logk;
  const int bound = 37 - logk;
  hipLaunchKernelGGL(dense_rot_gemm_kernel, dim3((unsigned)((T + DTM - 1) / DTM), (unsigned)(K / DTN)),
                     dim3(256), 0, stream, x, ldx, T, K, R, u);
  if (precond != nullptr)
    hipLaunchKernelGGL(dense_row_spread_kernel, dim3(1), dim3(1024), 0, stream, R, K, rspread);
  hipLaunchKernelGGL(dense_quant_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, u, T,
                     K, act_bits, codes, scales, x, ldx, rspread, bound, precond);
  return hipGetLastError();
}

}  // namespace cbq
