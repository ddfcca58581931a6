// Index regrouping for the GEMM kernels (cbq_prepack_weights): the blocked layout puts
// every 16-row x 128-channel tile of a weight matrix in 256*bits contiguous bytes, in the
// order the GEMM waves load them (lane 16j + r holds row r's indices of channels
// 32j .. 32j+31 of the chunk), so a wave's index load is one coalesced block instead of
// sixteen short pieces of sixteen rows.  Each unit is the 4*bits bytes of 32
// consecutive indices of one row, byte-aligned in both layouts (K % 32 == 0).  2- and
// 4-bit units are copied as they are.  3-bit units are re-encoded so the kernels build
// their byte selectors with one mask or one shift and a mask: group g < 3 (indices
// 8g .. 8g+7) becomes dword g, byte b holding index 8g+2b in bits 0-2 and 8g+2b+1 in
// bits 3-5; group 3's pair b (i_{24+2b} | i_{25+2b} << 3) is spread over bits 6-7 of
// byte b of the three dwords, two bits each, lowest first.
#include "cbq_internal.hpp"

namespace cbq {

// one thread per 32-index unit of the blocked layout
template <int BITS>
__global__ void __launch_bounds__(256)
prepack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t units,
               int N, int K, int kchunks) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  // u = ((e * N/16 + G) * kchunks + c) * 64 + 16 j + r
  const int slot = (int)(u & 63);
  const int64_t t = u >> 6;
  const int c = (int)(t % kchunks);
  const int64_t eg = t / kchunks;               // e * N/16 + G
  const int r = slot & 15, j = slot >> 4;
  const int64_t row = eg * 16 + r;               // e * N + n
  const int k0 = c * 128 + j * 32;
  uint32_t w[BITS];
  if (k0 < K) {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src + row * ((int64_t)K * BITS / 8) +
                                                          (int64_t)k0 * BITS / 8);
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = s[i];
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = 0u;    // channels past K: index 0, never used
  }
  if constexpr (BITS == 3) {
    // index k of the LSB-first unit: bits 3k .. 3k+2 of w[0] | w[1] << 32 | w[2] << 64
    auto idx = [&](int k) -> uint32_t {
      const int bit = 3 * k, wi = bit >> 5, sh = bit & 31;
      const uint32_t lo = w[wi] >> sh;
      const uint32_t hi = (sh > 29 && wi < 2) ? (w[wi + 1] << (32 - sh)) : 0u;
      return (lo | hi) & 7u;
    };
    uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < 3; ++g)
#pragma unroll
      for (int b = 0; b < 4; ++b) o[g] |= (idx(8 * g + 2 * b) | (idx(8 * g + 2 * b + 1) << 3)) << (8 * b);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t pr = idx(24 + 2 * b) | (idx(25 + 2 * b) << 3);
#pragma unroll
      for (int i = 0; i < 3; ++i) o[i] |= ((pr >> (2 * i)) & 3u) << (8 * b + 6);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) w[i] = o[i];
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(dst + u * 4 * BITS);
#pragma unroll
  for (int i = 0; i < BITS; ++i) d[i] = w[i];
}

hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int E, int N, int K, int bits,
                          hipStream_t stream) {
  const int kchunks = (K + 127) / 128;
  const int64_t units = (int64_t)E * (N / 16) * kchunks * 64;
  const dim3 grid((unsigned)((units + 255) / 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL(prepack_kernel<2>, grid, dim3(256), 0, stream, src, dst, units, N, K, kchunks); break;
    case 3: hipLaunchKernelGGL(prepack_kernel<3>, grid, dim3(256), 0, stream, src, dst, units, N, K, kchunks); break;
    default: hipLaunchKernelGGL(prepack_kernel<4>, grid, dim3(256), 0, stream, src, dst, units, N, K, kchunks); break;
  }
  return hipGetLastError();
}

}  // namespace cbq
