// Host codebook-LUT GEMM (plain C++; shared by cpu_lut.cpp and the C ABI).
#pragma once
#include <stdint.h>

namespace cbq {

// True when the host CPU has the instructions the kernel uses (AVX2, FMA, F16C, BMI2).
bool cpu_lut_supported();

// out[t][n] = scales[t] * sum_k q[t][k] * codebook[n][idx(n, k)] for one weight set
// (E = 1).  Host pointers; rows are split over n_threads threads (0: all cores).  The
// AVX-512 variant runs when use_avx512 is set and the CPU has AVX-512F.
void cpu_lut_gemm_impl(const uint8_t* codes, const float* scales, int act_bits, int64_t T,
                       int64_t N, int K, int bits, const uint8_t* idx, const uint16_t* codebook,
                       float* out, int64_t ldo, int n_threads, bool use_avx512);

}  // namespace cbq
