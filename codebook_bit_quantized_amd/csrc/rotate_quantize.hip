// Fused block Walsh-Hadamard rotation + per-token absmax quantisation.
//
// CodeQuant2, Figure 1: the rotation that smooths activation outliers is fused into
// the model; Tables 1 and 9: activations are quantised to 4 or 8 bits (A4W4, A8W4).
//
// One workgroup per token row.  Each thread owns R consecutive channels (one 16- or
// 32-byte load).  The transform runs in fp64, which is exact for bf16 inputs whose
// nonzero exponents in a block spread at most 45 - log2(b) binades: in-thread
// butterflies for strides < R, lane shuffles for strides up to 64*R, and LDS
// exchanges across waves beyond that.  The quantiser then follows one fixed IEEE
// fp32 sequence (round v = fp32(u), s = M / Q, q = rint_even(v / s)), so the codes
// are reproducible bit for bit.
#include "cbq_internal.hpp"

namespace cbq {

template <int R>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ src, bool active, double* v) {
  if constexpr (R == 8) {
    u32x4 p = active ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)__builtin_bit_cast(float, p[i] << 16);
      v[2 * i + 1] = (double)__builtin_bit_cast(float, p[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 p = active ? s4[h] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * h + 2 * i] = (double)__builtin_bit_cast(float, p[i] << 16);
        v[8 * h + 2 * i + 1] = (double)__builtin_bit_cast(float, p[i] & 0xFFFF0000u);
      }
    }
  }
}

// floor(log2|x|) of the nonzero channels -> running (min, max)
__device__ __forceinline__ void exp_range(double x, int& emin, int& emax) {
  float f = (float)x;   // exact: x came from bf16
  if (f != 0.0f) {
    int e = __builtin_amdgcn_frexp_expf(f) - 1;
    emin = min(emin, e);
    emax = max(emax, e);
  }
}

template <int R>
__global__ void __launch_bounds__(1024)
rotate_quantize_kernel(const uint16_t* __restrict__ x, int64_t ldx, int K, int logb, int act_bits,
                       float c_b, uint8_t* __restrict__ codes, float* __restrict__ scales,
                       uint32_t* __restrict__ precond) {
  extern __shared__ double xchg[];          // cross-wave butterflies: [R][nthr_pad]
  __shared__ float red_max[16];
  __shared__ int red_emin[16], red_emax[16];

  const int tid = threadIdx.x;
  const int nthr = K / R;
  const int npad = blockDim.x;
  const bool active = tid < nthr;
  const int64_t t = blockIdx.x;
  const int b = 1 << logb;
  const int lane = tid & 63, wave = tid >> 6;

  double v[R];
  load_row<R>(x + t * ldx + (int64_t)tid * R, active, v);

  // ---- optional exactness check: exponent spread inside each block ----
  if (precond != nullptr) {
    const int limit = 45 - logb;
    if (b <= R) {
      // whole blocks inside this thread
      for (int s = 0; s < R; s += b) {
        int emin = 1 << 20, emax = -(1 << 20);
        for (int i = 0; i < b; ++i) exp_range(v[s + i], emin, emax);
        if (active && emax >= emin && emax - emin > limit) atomicAdd(precond, 1u);
      }
    } else {
      int emin = 1 << 20, emax = -(1 << 20);
#pragma unroll
      for (int i = 0; i < R; ++i) exp_range(v[i], emin, emax);
      const int gth = b / R;                        // threads per block
      for (int m = 1; m < gth && m < 64; m <<= 1) {
        emin = min(emin, __shfl_xor(emin, m));
        emax = max(emax, __shfl_xor(emax, m));
      }
      if (gth > 64) {
        if (lane == 0) { red_emin[wave] = emin; red_emax[wave] = emax; }
        __syncthreads();
        const int wpb = gth / 64;                   // waves per block
        const int w0 = (wave / wpb) * wpb;
        for (int w = w0; w < w0 + wpb; ++w) {
          emin = min(emin, red_emin[w]);
          emax = max(emax, red_emax[w]);
        }
      }
      if (active && (tid % gth) == 0 && emax >= emin && emax - emin > limit) atomicAdd(precond, 1u);
    }
  }

  // ---- fast Walsh-Hadamard transform over blocks of b channels (fp64, exact) ----
#pragma unroll
  for (int h = 1; h < R; h <<= 1) {
    if (h < b) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if (!(i & h)) {
          const double a = v[i], c = v[i + h];
          v[i] = a + c;
          v[i + h] = a - c;
        }
      }
    }
  }
  for (int m = 1; m < 64 && m * R < b; m <<= 1) {
    const bool upper = (tid & m) != 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const double p = __shfl_xor(v[i], m);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
  for (int m = 64; m * R < b; m <<= 1) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) xchg[i * npad + tid] = v[i];
    __syncthreads();
    const bool upper = (tid & m) != 0;
    const int partner = tid ^ m;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const double p = xchg[i * npad + partner];
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }

  // ---- per-token absmax ----
  float u[R];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    u[i] = (float)v[i];                      // round to nearest even
    amax = fmaxf(amax, fabsf(u[i]));
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if (lane == 0) red_max[wave] = amax;
  __syncthreads();
  const int nw = npad >> 6;
  amax = red_max[0];
  for (int w = 1; w < nw; ++w) amax = fmaxf(amax, red_max[w]);

  // ---- quantise: s = M / Q, q = clamp(rint(v / s)) ----
  const float Q = act_bits == 4 ? 7.0f : 127.0f;
  const float lo = act_bits == 4 ? -8.0f : -127.0f;
  const float s = amax / Q;
  int q[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float r = (amax > 0.0f) ? rintf(u[i] / s) : 0.0f;
    r = fminf(fmaxf(r, lo), Q);
    q[i] = (int)r;
  }
  if (active) {
    if (act_bits == 4) {
      uint8_t* dst = codes + t * (K / 2) + (int64_t)tid * (R / 2);
      uint32_t wds[R / 8];
#pragma unroll
      for (int j = 0; j < R / 8; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= ((uint32_t)q[8 * j + i] & 0xFu) << (4 * i);
        wds[j] = w;
      }
      if constexpr (R == 8) *reinterpret_cast<uint32_t*>(dst) = wds[0];
      else *reinterpret_cast<u32x2*>(dst) = u32x2{wds[0], wds[1]};
    } else {
      uint8_t* dst = codes + t * K + (int64_t)tid * R;
      uint32_t wds[R / 4];
#pragma unroll
      for (int j = 0; j < R / 4; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= ((uint32_t)q[4 * j + i] & 0xFFu) << (8 * i);
        wds[j] = w;
      }
      if constexpr (R == 8) *reinterpret_cast<u32x2*>(dst) = u32x2{wds[0], wds[1]};
      else *reinterpret_cast<u32x4*>(dst) = u32x4{wds[0], wds[1], wds[2], wds[3]};
    }
  }
  if (tid == 0) scales[t] = (amax > 0.0f) ? s * c_b : 0.0f;
}

hipError_t launch_rotate_quantize(const uint16_t* x, int64_t T, int K, int64_t ldx, int b,
                                  int act_bits, uint8_t* codes, float* scales, uint32_t* precond,
                                  hipStream_t stream) {
  const int R = K <= 8192 ? 8 : 16;
  const int nthr = K / R;
  const int npad = (nthr + 63) / 64 * 64;
  int logb = 0;
  while ((1 << logb) < b) ++logb;
  const size_t lds = (b > 64 * R) ? (size_t)npad * R * sizeof(double) : 0;
  const float c_b = (float)(1.0 / std::sqrt((double)b));
  if (R == 8)
    hipLaunchKernelGGL(rotate_quantize_kernel<8>, dim3((unsigned)T), dim3(npad), lds, stream, x,
                       ldx, K, logb, act_bits, c_b, codes, scales, precond);
  else
    hipLaunchKernelGGL(rotate_quantize_kernel<16>, dim3((unsigned)T), dim3(npad), lds, stream, x,
                       ldx, K, logb, act_bits, c_b, codes, scales, precond);
  return hipGetLastError();
}

}  // namespace cbq
