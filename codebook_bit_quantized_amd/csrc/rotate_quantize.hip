// Fused block Walsh-Hadamard rotation + per-token absmax quantisation.
//
// CodeQuant2, Figure 1: the rotation that smooths activation outliers is fused into
// the model; Tables 1 and 9: activations are quantised to 4 or 8 bits (A4W4, A8W4).
//
// Each thread owns 32 consecutive channels of one token (four 16-byte loads).  A
// token takes G lanes, G the power of two >= K/32 when K <= 1024 (then 64/G tokens
// share a wave), else a whole workgroup of ceil(K/2048) waves.  Between 1024 and
// 2048 channels with K/32 not a power of two, tokens of K/32 lanes are packed back to
// back in 512-lane workgroups (a token may straddle two waves; its absmax then meets in
// LDS), which keeps all but K/32 - 1 lanes of a workgroup busy; workgroups of eight
// waves, four to a CU, drift out of step, so one's loads overlap another's arithmetic.  The transform runs
// in fp64, which is exact for bf16 inputs whose nonzero exponents in a block spread
// at most 45 - log2(b) binades: five butterfly stages inside the thread, then one
// lane exchange per further stage (DPP for lane distances 1, 2 and 8, ds_swizzle for
// 4 and 16, a permute for 32) and LDS exchanges across waves beyond 64 lanes.
//
// Optionally, before the rotation, each channel is multiplied by an fp32 smoothing
// factor (one fp32 rounding; the exactness bound then becomes 29 - log2(b) binades)
// and/or negated by a random sign bit (CodeQuant2, Figure 1: per-channel scales and a
// rotation folded into the weights smooth the outliers; Table 5 caption: a fixed random rotation with
// SmoothQuant scaling).
//
// The quantiser follows one fixed IEEE fp32 sequence: v = fp32(u), M = max|v|,
// s = M / Q, r = fp32(v / s), q = clamp(rint_even(r)).  The quotient is formed as
// fp64(v) * fp64(1 / s) and then rounded to fp32: for fp32 v and s the exact quotient
// is never an fp32 rounding midpoint and lies at least 2^-49 (relative) away from
// one, while the fp64 product is within 2^-52 of it, so the fp32 rounding, and hence
// q, is that of the correctly rounded division.
#include <atomic>

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

// one butterfly stage between lanes j and j ^ M (M lanes = 32 * M channels apart): the
// lower lane keeps v + p, the upper one v - p, which is the negative of the butterfly's
// p - v.  Each value is one fma(p, +-1, v) accumulating into v (the product by +-1 is
// exact, so it rounds the same sum an add would).  Partners always carry the same sign
// (they differ only in the stage's own lane bit), so after the lane stages a lane's
// values are the transform times (-1)^(number of upper stages), i.e. the parity of its
// lane bits inside the block; the quantiser takes that sign into its multiplier.
template <int M>
__device__ __forceinline__ void lane_stage(double* v, bool upper) {
  const double sgn = upper ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double p = xor_lane_f64<M>(v[i]);
    v[i] = __builtin_fma(p, sgn, v[i]);
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
    if (signs != nullptr && active) {
      const uint32_t sg = reinterpret_cast<const uint32_t*>(signs)[j];
#pragma unroll
      for (int i = 0; i < 32; ++i) f[i] = (sg >> i) & 1u ? -f[i] : f[i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (double)f[i];
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
        v[c + i] += upper ? -p : p;       // upper lanes keep the negated butterfly
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
  // rint by the magic-number add: r + 1.5 * 2^23 rounds r (|r| <= 128) to the nearest
  // integer, ties to even, and leaves q = rint(r) in the low bits of the sum's pattern
  // (0x4B400000 + q); the clamp is applied to the sum, whose bounds are exact, and the
  // codes are packed from those low bits
  const float Q = act_bits == 4 ? 7.0f : 127.0f;
  const float lo = act_bits == 4 ? -8.0f : -127.0f;
  constexpr float kMagic = 12582912.0f;
  const float s = amax / Q;
  // the lane's values carry the sign (-1)^popcount(its lane bits inside the block) from
  // the lane stages: fold it into the (exactly negated) multiplier, so fp32(u * rs) is the
  // quotient of the transform itself and the clamp sees the right sign
  const int gth_q = b >> 5;
  const bool neg = gth_q > 1 && (__builtin_popcount((unsigned)j & (unsigned)(gth_q - 1)) & 1);
  const double rs = amax > 0.0f ? (neg ? -1.0 : 1.0) / (double)s : 0.0;
  uint32_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = (float)((double)u[i] * rs);
    q[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(r + kMagic, kMagic + lo, kMagic + Q));
  }
  // the low byte of each q[i] is the code as an int8; byte permutes gather them
  auto low_bytes = [&](int i0, int i1, int i2, int i3) {   // bytes (q[i0], q[i1], q[i2], q[i3])
    const uint32_t lo = __builtin_amdgcn_perm(q[i1], q[i0], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(q[i3], q[i2], 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  };
  if (active) {
    if (act_bits == 4) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // byte b holds code 2b in its low nibble and code 2b + 1 in its high one
        const uint32_t ev = low_bytes(8 * k, 8 * k + 2, 8 * k + 4, 8 * k + 6);
        const uint32_t od = low_bytes(8 * k + 1, 8 * k + 3, 8 * k + 5, 8 * k + 7);
        w[k] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
      }
      *reinterpret_cast<u32x4*>(codes + t * (K / 2) + (int64_t)j * 16) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = low_bytes(4 * k, 4 * k + 1, 4 * k + 2, 4 * k + 3);
      u32x4* dst = reinterpret_cast<u32x4*>(codes + t * K + (int64_t)j * 32);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
    if (j == 0) scales[t] = amax > 0.0f ? s * c_b : 0.0f;
  }
}

namespace {

// Exchange between 16-lane rows: a pair (A, B) of one lane and the pair of the lane 16
// (SWAP32: 32) lanes away.  The lane in the even row (lower half) gets its partner's A in
// place of its own B; the partner gets this lane's B in place of its own A.  Each lane then
// holds (A of the even-row lane, A or B of the odd-row lane at the same place) and both
// compute the butterfly (A + B, A - B) in the same registers.
template <bool SWAP32>
__device__ __forceinline__ void swap_butterfly(double& a, double& b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  uint32_t alo = (uint32_t)ua, ahi = (uint32_t)(ua >> 32);
  uint32_t blo = (uint32_t)ub, bhi = (uint32_t)(ub >> 32);
  if constexpr (SWAP32) {
    const auto lo = __builtin_amdgcn_permlane32_swap(alo, blo, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(ahi, bhi, false, false);
    alo = lo[0]; blo = lo[1]; ahi = hi[0]; bhi = hi[1];
  } else {
    const auto lo = __builtin_amdgcn_permlane16_swap(alo, blo, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(ahi, bhi, false, false);
    alo = lo[0]; blo = lo[1]; ahi = hi[0]; bhi = hi[1];
  }
  const double A = __builtin_bit_cast(double, ((uint64_t)ahi << 32) | alo);
  const double B = __builtin_bit_cast(double, ((uint64_t)bhi << 32) | blo);
  a = A + B;
  b = A - B;
}

}  // namespace

// Tokens of K/32 >= 16 lanes packed back to back (at most 32 tokens a workgroup), Hadamard
// blocks of b = 32 << g channels (0 <= g <= 6).  A workgroup of W lanes (512, or a smaller
// multiple of 64 that fits long tokens better) holds W >> g blocks:
// block row r = lane mod (64 >> g) of each wave, and the block's 1 << g lanes are 64 >> g
// lanes apart (jj = lane >> (6 - g) is the lane's place in its block), so the last one or
// two lane stages of every block are at lane distances 16 and 32 and run as half-swaps:
// each lane sends half its values and keeps half, and both lanes of a pair finish the
// butterfly in place, which also trades the transformed channel bit (on the lane) for a
// channel bit held in a register.  The channels a lane loads are chosen so that after the
// trades its 32 registers hold 32 consecutive channels, 32 * jj onwards in the block:
//   channel bits 0-2     -> register bits 0-2 throughout;
//   g = 1: bit 3 -> register bit 3, bit 4 -> the lane (distance 32), bit 5 -> register bit 4;
//   g >= 2: bits 3 and 4 -> the lanes at distances 16 and 32, bits 5 .. g + 2 -> the lanes
//           at distances 64 >> g .. 8 (exchanged by DPP / swizzle with the sign folded into
//           the quantiser as in the general kernel), bits g + 3 and g + 4 -> register bits
//           3 and 4.
// In-thread stages run first, over all five register bits, then the DPP stages, then the
// half-swaps.  The workgroup loops over groups of tokens, loading the next group before
// working on the current one, so one group's loads overlap the previous group's arithmetic.
template <int g>
__global__ void __launch_bounds__(512)
rotate_quantize_packed_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t T, int K,
                              int act_bits, float c_b, uint8_t* __restrict__ codes,
                              float* __restrict__ scales, int64_t n_groups) {
  constexpr int rows = 64 >> g;              // blocks per wave
  constexpr int b = 32 << g;                 // channels per block
  __shared__ uint32_t s_amax[3][32];         // per-token absmax (float bits), three rotating sets

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & (rows - 1);
  const int jj = g == 0 ? 0 : lane >> (6 - g);
  const int bpt = K >> (5 + g);              // blocks per token
  const int bw = wave * rows + r;            // block within the workgroup
  const int lt = bw / bpt, bt = bw - lt * bpt;
  const int tpb = ((int)blockDim.x >> g) / bpt;   // tokens per group
  const bool in_group = lt < tpb;
  // channel of register 8h + m (m < 8) inside the token: c0 + ch(h) + m
  int c0;
  if constexpr (g == 0) c0 = 0;
  else if constexpr (g == 1) c0 = 16 * jj;
  else c0 = 8 * (jj >> (g - 2)) + 32 * (jj & ((1 << (g - 2)) - 1));
  c0 += bt * b;
  auto ch = [](int h) { return g == 0 ? 8 * h : g == 1 ? 8 * (h & 1) + 32 * (h >> 1) : (b / 4) * h; };

  auto load = [&](int64_t it, u32x4 (&p)[4]) {
    const int64_t t = it * tpb + lt;
    const bool act = in_group && t < T;
    const uint16_t* src = x + (act ? t * ldx + c0 : 0);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      p[h] = act ? *reinterpret_cast<const u32x4*>(src + ch(h)) : u32x4{0, 0, 0, 0};
  };

  if (tid < 32) s_amax[0][tid] = 0u;
  __syncthreads();

  const float Q = act_bits == 4 ? 7.0f : 127.0f;
  const float lo = act_bits == 4 ? -8.0f : -127.0f;
  constexpr float kMagic = 12582912.0f;
  // sign carried by the DPP stages (g >= 3): the parity of the lane's upper-lane bits
  const bool neg = g >= 3 && (__builtin_popcount((unsigned)jj & ((1u << (g >= 3 ? g - 2 : 0)) - 1u)) & 1);

  u32x4 nxt[4];
  int64_t it = blockIdx.x;
  load(it, nxt);
  for (int par = 0; it < n_groups; it += gridDim.x, par = par == 2 ? 0 : par + 1) {
    u32x4 p[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) p[h] = nxt[h];
    if (it + gridDim.x < n_groups) load(it + gridDim.x, nxt);
    const int64_t t = it * tpb + lt;
    const bool active = in_group && t < T;

    double v[32];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * h + 2 * i] = (double)__builtin_bit_cast(float, p[h][i] << 16);
        v[8 * h + 2 * i + 1] = (double)__builtin_bit_cast(float, p[h][i] & 0xFFFF0000u);
      }
    }
    // in-thread stages over the five register bits
#pragma unroll
    for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (!(i & hs)) {
          const double a = v[i], c = v[i + hs];
          v[i] = a + c;
          v[i + hs] = a - c;
        }
      }
    }
    // lane stages below distance 16 (g >= 3)
    if constexpr (g >= 6) lane_stage<1>(v, (lane & 1) != 0);
    if constexpr (g >= 5) lane_stage<2>(v, (lane & 2) != 0);
    if constexpr (g >= 4) lane_stage<4>(v, (lane & 4) != 0);
    if constexpr (g >= 3) lane_stage<8>(v, (lane & 8) != 0);
    // half-swaps: distance 16 with register bit 3, distance 32 with register bit 4
    if constexpr (g >= 2) {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (!(i & 8)) swap_butterfly<false>(v[i], v[i + 8]);
    }
    if constexpr (g >= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) swap_butterfly<true>(v[i], v[i + 16]);
    }

    // absmax: the lane, its block's lanes, then the token's blocks through LDS
    float u[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      u[i] = (float)v[i];
      amax = fmaxf(amax, fabsf(u[i]));
    }
    if constexpr (g >= 6) amax = fmaxf(amax, xor_lane_f32<1>(amax));
    if constexpr (g >= 5) amax = fmaxf(amax, xor_lane_f32<2>(amax));
    if constexpr (g >= 4) amax = fmaxf(amax, xor_lane_f32<4>(amax));
    if constexpr (g >= 3) amax = fmaxf(amax, xor_lane_f32<8>(amax));
    if constexpr (g >= 2) amax = fmaxf(amax, xor_lane_f32<16>(amax));
    if constexpr (g >= 1) amax = fmaxf(amax, xor_lane_f32<32>(amax));
    const int nx = par == 2 ? 0 : par + 1;
    if (tid < 32) s_amax[nx][tid] = 0u;      // the set after this one; its last readers are done
    if (in_group && jj == 0) atomicMax(&s_amax[par][lt], __builtin_bit_cast(uint32_t, amax));
    __syncthreads();
    amax = in_group ? __builtin_bit_cast(float, s_amax[par][lt]) : 0.0f;

    const float s = amax / Q;
    const double rs = amax > 0.0f ? (neg ? -1.0 : 1.0) / (double)s : 0.0;
    uint32_t q[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float rq = (float)((double)u[i] * rs);
      q[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(rq + kMagic, kMagic + lo, kMagic + Q));
    }
    auto low_bytes = [&](int i0, int i1, int i2, int i3) {
      const uint32_t l = __builtin_amdgcn_perm(q[i1], q[i0], 0x0C0C0400u);
      const uint32_t hgh = __builtin_amdgcn_perm(q[i3], q[i2], 0x0C0C0400u);
      return __builtin_amdgcn_perm(hgh, l, 0x05040100u);
    };
    if (active) {
      const int64_t cpos = (int64_t)bt * b + 32 * jj;     // first channel of this lane's run
      if (act_bits == 4) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t ev = low_bytes(8 * k, 8 * k + 2, 8 * k + 4, 8 * k + 6);
          const uint32_t od = low_bytes(8 * k + 1, 8 * k + 3, 8 * k + 5, 8 * k + 7);
          w[k] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
        }
        *reinterpret_cast<u32x4*>(codes + t * (K / 2) + cpos / 2) = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = low_bytes(4 * k, 4 * k + 1, 4 * k + 2, 4 * k + 3);
        u32x4* dst = reinterpret_cast<u32x4*>(codes + t * K + cpos);
        dst[0] = u32x4{w[0], w[1], w[2], w[3]};
        dst[1] = u32x4{w[4], w[5], w[6], w[7]};
      }
      if (bt == 0 && jj == 0) scales[t] = amax > 0.0f ? s * c_b : 0.0f;
    }
  }
}

// Compute units of the current device, looked up once per device.
hipError_t device_cu_count(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) { *out = c; return hipSuccess; }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

hipError_t launch_rotate_quantize(const uint16_t* x, int64_t T, int K, int64_t ldx, int b,
                                  int act_bits, const float* smooth, const uint8_t* signs,
                                  uint8_t* codes, float* scales, uint32_t* precond,
                                  hipStream_t stream) {
  const int nthr = K / 32;
  int logb = 0;
  while ((1 << logb) < b) ++logb;
  const float c_b = (float)(1.0 / std::sqrt((double)b));
  // The packed kernel's workgroup: 512 lanes, or, where 512 would leave more than a tenth
  // of them idle (one long token a workgroup), the multiple of 64 up to 512 that leaves the
  // fewest idle; the share of its lanes that hold channels, against the general kernel's
  // (G lanes per token, G a power of two up to 64, else whole waves).
  auto use_of = [&](int w) { return (double)(w / nthr * nthr) / w; };
  int wg = 512;
  if (use_of(512) < 0.9)
    for (int w = 448; w >= 64; w -= 64)
      if (w >= nthr && use_of(w) > use_of(wg)) wg = w;
  const double packed_use = use_of(wg);
  int g_lanes = 1;
  while (g_lanes < nthr && g_lanes < 64) g_lanes <<= 1;
  if (nthr > 64) g_lanes = (nthr + 63) / 64 * 64;
  const double general_use = (double)nthr / g_lanes;
  // (On equal use, workgroups of 320 lanes measured slower than the general kernel at
  // K = 9728, those of 448 and 512 faster at K = 14336 and 2048.)
  const bool packed = packed_use > general_use || (packed_use == general_use && wg >= 448);
  if (nthr >= 16 && b >= 32 && b <= 2048 && packed && smooth == nullptr && signs == nullptr &&
      precond == nullptr) {
    // packed tokens, plain rotation: groups of tpb tokens, each workgroup looping over
    // about the same number of groups.  Two workgroups are resident per CU (116 VGPRs);
    // a grid of three per CU measured fastest (32768 x 1408: 40.1 us warm, against 43.4
    // for two per CU and 42.5 for one group per workgroup)
    const int g = logb - 5;
    const int64_t tpb = (wg >> g) / (K >> logb);
    const int64_t n_groups = (T + tpb - 1) / tpb;
    int cus = 0;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)(3 * 512 / wg) * cus;
    const int64_t per = (n_groups + slots - 1) / slots;
    const int64_t blocks = (n_groups + per - 1) / per;
#define CBQ_RQ_PACKED(G_)                                                                      \
  case G_:                                                                                    \
    hipLaunchKernelGGL(rotate_quantize_packed_kernel<G_>, dim3((unsigned)blocks), dim3(wg), 0, \
                       stream, x, ldx, T, K, act_bits, c_b, codes, scales, n_groups);         \
    break;
    switch (g) {
      CBQ_RQ_PACKED(0)
      CBQ_RQ_PACKED(1)
      CBQ_RQ_PACKED(2)
      CBQ_RQ_PACKED(3)
      CBQ_RQ_PACKED(4)
      CBQ_RQ_PACKED(5)
      CBQ_RQ_PACKED(6)
      default: return hipErrorInvalidValue;
    }
#undef CBQ_RQ_PACKED
    return hipGetLastError();
  }
  int G, threads;
  int64_t blocks;
  size_t lds = 0;
  if (nthr > 32 && nthr < 64) {
    G = 0;                                   // packed: K/32 lanes per token
    threads = 512;
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
