// Fused block Walsh-Hadamard rotation + per-token absmax quantisation.
//
// CodeQuant2, Figure 1: the rotation that smooths activation outliers is fused into
// the model; Tables 1 and 9: activations are quantised to 4 or 8 bits (A4W4, A8W4).
//
// Each thread owns 32 consecutive channels of one token (four 16-byte loads).  A
// token takes G lanes, G the power of two >= K/32 when K <= 1024 (then 64/G tokens
// share a wave), else a whole workgroup of ceil(K/2048) waves.  Between 1024 and
// 2048 channels with K/32 not a power of two, tokens of K/32 lanes are packed back to
// back in 1024-lane workgroups (a token may straddle two waves; its absmax then
// meets in LDS), which keeps all but K/32 - 1 lanes of a workgroup busy.  The transform runs
// in fp64, which is exact for bf16 inputs whose nonzero exponents in a block spread
// at most 45 - log2(b) binades: five butterfly stages inside the thread, then one
// lane exchange per further stage (DPP for lane distances 1, 2 and 8, ds_swizzle for
// 4 and 16, a permute for 32) and LDS exchanges across waves beyond 64 lanes.
//
// Optionally, before the rotation, each channel is multiplied by an fp32 smoothing
// factor (one fp32 rounding; the exactness bound then becomes 29 - log2(b) binades)
// and/or negated by a random sign bit (CodeQuant2, Figure 1: rotation and scaling
// fused for outlier smoothing; Table 5 caption: a fixed random rotation with
// SmoothQuant scaling).
//
// The quantiser follows one fixed IEEE fp32 sequence: v = fp32(u), M = max|v|,
// s = M / Q, r = fp32(v / s), q = clamp(rint_even(r)).  The quotient is formed as
// fp64(v) * fp64(1 / s) and then rounded to fp32: for fp32 v and s the exact quotient
// is never an fp32 rounding midpoint and lies at least 2^-49 (relative) away from
// one, while the fp64 product is within 2^-52 of it, so the fp32 rounding, and hence
// q, is that of the correctly rounded division.
#include "cbq_internal.hpp"

namespace cbq {

namespace {

// value of lane (lane ^ M), M a power of two below 64
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
  else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  else if constexpr (M == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101F);              // xor 4 in 32 lanes
  else if constexpr (M == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); // row_ror 8
  else if constexpr (M == 16) return __builtin_amdgcn_ds_swizzle(v, 0x401F);             // xor 16 in 32 lanes
  else return __shfl_xor(v, 32);
}

template <int M>
__device__ __forceinline__ double xor_lane_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)xor_lane<M>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)xor_lane<M>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int M>
__device__ __forceinline__ float xor_lane_f32(float v) {
  return __builtin_bit_cast(float, xor_lane<M>(__builtin_bit_cast(int, v)));
}

// one butterfly stage between lanes j and j ^ M (M lanes = 32 * M channels apart):
// the lower lane keeps p + v, the upper one p + (-v), the sign flipped by one xor on
// the high word instead of a select between two sums
template <int M>
__device__ __forceinline__ void lane_stage(double* v, bool upper) {
  const uint64_t smask = upper ? 0x8000000000000000ull : 0ull;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double p = xor_lane_f64<M>(v[i]);
    v[i] = p + __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, v[i]) ^ smask);
  }
}

template <int M>
__device__ __forceinline__ void minmax_lanes(int& emin, int& emax) {
  emin = min(emin, xor_lane<M>(emin));
  emax = max(emax, xor_lane<M>(emax));
}

// floor(log2|x|) of a nonzero channel -> running (min, max)
__device__ __forceinline__ void exp_range(double x, int& emin, int& emax) {
  const float f = (float)x;   // exact: x came from bf16
  if (f != 0.0f) {
    const int e = __builtin_amdgcn_frexp_expf(f) - 1;
    emin = min(emin, e);
    emax = max(emax, e);
  }
}

}  // namespace

// G: lanes per token (a power of two <= 64, or a multiple of 64 = the workgroup), or
// 0 for K/32 lanes per token packed back to back in the workgroup.
__global__ void __launch_bounds__(1024)
rotate_quantize_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t T, int K, int logb,
                       int G, int act_bits, float c_b, const float* __restrict__ smooth,
                       const uint8_t* __restrict__ signs, uint8_t* __restrict__ codes,
                       float* __restrict__ scales, uint32_t* __restrict__ precond) {
  extern __shared__ double xchg[];          // cross-wave butterflies: [8][blockDim]
  __shared__ float red_max[8];
  __shared__ int red_emin[8], red_emax[8];
  __shared__ uint32_t s_amax[32];            // packed mode: per-token absmax (float bits)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nthr = K >> 5;
  int64_t t;
  int j;                                     // thread index within the token
  int lt = 0;                                // packed mode: token within the workgroup
  const int tpb = G == 0 ? (int)blockDim.x / nthr : 0;
  if (G == 0) {
    lt = tid / nthr;
    j = tid - lt * nthr;
    t = (int64_t)blockIdx.x * tpb + lt;
    if (tid < 32) s_amax[tid] = 0u;
  } else if (G <= 64) {
    const int tpw = 64 / G;                  // tokens per wave
    t = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * tpw + lane / G;
    j = lane & (G - 1);
  } else {
    t = blockIdx.x;
    j = tid;
  }
  const bool active = t < T && j < nthr && lt < (G == 0 ? tpb : 1);
  const int b = 1 << logb;

  double v[32];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (active ? t * ldx + (int64_t)j * 32 : 0));
    float f[32];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 p = active ? src[h] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * h + 2 * i] = __builtin_bit_cast(float, p[i] << 16);
        f[8 * h + 2 * i + 1] = __builtin_bit_cast(float, p[i] & 0xFFFF0000u);
      }
    }
    // optional per-channel transforms before the rotation: v = fp32(x * m), negated
    // where the channel's sign bit is set
    if (smooth != nullptr && active) {
      const f32x4* ms = reinterpret_cast<const f32x4*>(smooth + j * 32);
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const f32x4 m = ms[h];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[4 * h + i] = __fmul_rn(f[4 * h + i], m[i]);
      }
    }
    uint32_t sg = 0;
    if (signs != nullptr && active) sg = reinterpret_cast<const uint32_t*>(signs)[j];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (double)((sg >> i) & 1u ? -f[i] : f[i]);
  }

  // ---- optional exactness check: exponent spread inside each block ----
  if (precond != nullptr) {
    const int limit = (smooth != nullptr ? 29 : 45) - logb;   // 53 - significant bits - log2 b
    if (b <= 32) {                           // whole blocks inside this thread
      int emin = 1 << 20, emax = -(1 << 20);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        exp_range(v[i], emin, emax);
        if (((i + 1) & (b - 1)) == 0) {      // last channel of a block
          if (active && emax >= emin && emax - emin > limit) atomicAdd(precond, 1u);
          emin = 1 << 20;
          emax = -(1 << 20);
        }
      }
    } else {
      int emin = 1 << 20, emax = -(1 << 20);
#pragma unroll
      for (int i = 0; i < 32; ++i) exp_range(v[i], emin, emax);
      const int gth = b >> 5;                // threads per block
      if (gth > 1) minmax_lanes<1>(emin, emax);
      if (gth > 2) minmax_lanes<2>(emin, emax);
      if (gth > 4) minmax_lanes<4>(emin, emax);
      if (gth > 8) minmax_lanes<8>(emin, emax);
      if (gth > 16) minmax_lanes<16>(emin, emax);
      if (gth > 32) minmax_lanes<32>(emin, emax);
      if (gth > 64) {                        // blocks span waves (G > 64 here)
        if (lane == 0) { red_emin[wave] = emin; red_emax[wave] = emax; }
        __syncthreads();
        const int wpb = gth >> 6;            // waves per block
        const int w0 = (wave / wpb) * wpb;
        for (int w = w0; w < w0 + wpb; ++w) {
          emin = min(emin, red_emin[w]);
          emax = max(emax, red_emax[w]);
        }
      }
      if (active && (j & (gth - 1)) == 0 && emax >= emin && emax - emin > limit)
        atomicAdd(precond, 1u);
    }
  }

  // ---- fast Walsh-Hadamard transform over blocks of b channels (fp64, exact) ----
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
    if (h < b) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (!(i & h)) {
          const double a = v[i], c = v[i + h];
          v[i] = a + c;
          v[i + h] = a - c;
        }
      }
    }
  }
  if (b > 32) lane_stage<1>(v, (j & 1) != 0);
  if (b > 64) lane_stage<2>(v, (j & 2) != 0);
  if (b > 128) lane_stage<4>(v, (j & 4) != 0);
  if (b > 256) lane_stage<8>(v, (j & 8) != 0);
  if (b > 512) lane_stage<16>(v, (j & 16) != 0);
  if (b > 1024) lane_stage<32>(v, (j & 32) != 0);
  for (int m = 64; 32 * m < b; m <<= 1) {    // across waves (G > 64 here), 8 values a pass
    const int npad = blockDim.x;
    const bool upper = (j & m) != 0;
#pragma unroll
    for (int c = 0; c < 32; c += 8) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) xchg[i * npad + tid] = v[c + i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double p = xchg[i * npad + (tid ^ m)];
        v[c + i] = upper ? (p - v[c + i]) : (v[c + i] + p);
      }
    }
  }

  // ---- per-token absmax ----
  float u[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    u[i] = (float)v[i];                      // round to nearest even
    amax = fmaxf(amax, fabsf(u[i]));
  }
  if (G == 0) {
    // reduce inside each Hadamard block (its lanes never straddle a wave or a
    // token), then one LDS max per block; absmax >= 0, so the bits order as floats
    const int gth = b >> 5;
    if (gth > 1) amax = fmaxf(amax, xor_lane_f32<1>(amax));
    if (gth > 2) amax = fmaxf(amax, xor_lane_f32<2>(amax));
    if (gth > 4) amax = fmaxf(amax, xor_lane_f32<4>(amax));
    if (gth > 8) amax = fmaxf(amax, xor_lane_f32<8>(amax));
    if (gth > 16) amax = fmaxf(amax, xor_lane_f32<16>(amax));
    if (gth > 32) amax = fmaxf(amax, xor_lane_f32<32>(amax));
    __syncthreads();
    if (active && (gth <= 1 || (j & (gth - 1)) == 0)) atomicMax(&s_amax[lt], __builtin_bit_cast(uint32_t, amax));
    __syncthreads();
    amax = lt < tpb ? __builtin_bit_cast(float, s_amax[lt]) : 0.0f;
  }
  if (G > 1) amax = fmaxf(amax, xor_lane_f32<1>(amax));
  if (G > 2) amax = fmaxf(amax, xor_lane_f32<2>(amax));
  if (G > 4) amax = fmaxf(amax, xor_lane_f32<4>(amax));
  if (G > 8) amax = fmaxf(amax, xor_lane_f32<8>(amax));
  if (G > 16) amax = fmaxf(amax, xor_lane_f32<16>(amax));
  if (G > 32) amax = fmaxf(amax, xor_lane_f32<32>(amax));
  if (G > 64) {
    if (lane == 0) red_max[wave] = amax;
    __syncthreads();
    amax = red_max[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red_max[w]);
  }

  // ---- quantise: s = M / Q, q = clamp(rint(fp32(v / s))) ----
  const float Q = act_bits == 4 ? 7.0f : 127.0f;
  const float lo = act_bits == 4 ? -8.0f : -127.0f;
  const float s = amax / Q;
  const double rs = amax > 0.0f ? 1.0 / (double)s : 0.0;
  int q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = rintf((float)((double)u[i] * rs));
    q[i] = (int)__builtin_amdgcn_fmed3f(r, lo, Q);
  }
  if (active) {
    if (act_bits == 4) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t d = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) d |= ((uint32_t)q[8 * k + i] & 0xFu) << (4 * i);
        w[k] = d;
      }
      *reinterpret_cast<u32x4*>(codes + t * (K / 2) + (int64_t)j * 16) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) d |= ((uint32_t)q[4 * k + i] & 0xFFu) << (8 * i);
        w[k] = d;
      }
      u32x4* dst = reinterpret_cast<u32x4*>(codes + t * K + (int64_t)j * 32);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
    if (j == 0) scales[t] = amax > 0.0f ? s * c_b : 0.0f;
  }
}

hipError_t launch_rotate_quantize(const uint16_t* x, int64_t T, int K, int64_t ldx, int b,
                                  int act_bits, const float* smooth, const uint8_t* signs,
                                  uint8_t* codes, float* scales, uint32_t* precond,
                                  hipStream_t stream) {
  const int nthr = K / 32;
  int logb = 0;
  while ((1 << logb) < b) ++logb;
  const float c_b = (float)(1.0 / std::sqrt((double)b));
  int G, threads;
  int64_t blocks;
  size_t lds = 0;
  if (nthr > 32 && nthr < 64) {
    G = 0;                                   // packed: K/32 lanes per token
    threads = 1024;
    const int64_t per_block = threads / nthr;
    blocks = (T + per_block - 1) / per_block;
  } else if (nthr <= 64) {
    G = 1;
    while (G < nthr) G <<= 1;
    threads = 256;
    const int64_t per_block = 4 * (64 / G);  // tokens per workgroup
    blocks = (T + per_block - 1) / per_block;
  } else {
    G = (nthr + 63) / 64 * 64;
    threads = G;
    blocks = T;
    if (b > 2048) lds = (size_t)threads * 8 * sizeof(double);
  }
  hipLaunchKernelGGL(rotate_quantize_kernel, dim3((unsigned)blocks), dim3(threads), lds, stream, x,
                     ldx, T, K, logb, G, act_bits, c_b, smooth, signs, codes, scales, precond);
  return hipGetLastError();
}

}  // namespace cbq
