// Codebook-LUT GEMM on host cores (x86-64, AVX2).
//
// CodeQuant abstract and the AI Radio episode ("Improvements"): the method comes with
// dedicated LUT kernels for GPU and CPU, which look products up instead of computing
// them.  As on the GPU, the table held in registers is each weight row's codebook,
// split into its low and high bytes: vpshufb looks up 32 indices per instruction in
// each 16-entry byte table, two unpacks rebuild the fp16 centroids, F16C widens them
// and FMAs multiply them by the activation codes (exact integers; each product is exact
// in fp32, only the fp32 summation order differs from the definition).  The weights are
// dequantised once per row and reused by up to 8 tokens held in registers.
//
// Index unpacking: 4-bit nibbles with byte shuffles; 3- and 2-bit fields with BMI2
// pdep (eight indices per 24 or 16 bits).  On CPUs with AVX-512 a second variant
// looks 16 weights up per vpermps in an fp32 copy of the row's codebook and computes
// 4 rows x up to 4 tokens per pass.  Rows are split over a persistent thread pool.
#include "cpu_lut.hpp"

#include <immintrin.h>
#include <unistd.h>

#include <algorithm>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace cbq {

bool cpu_lut_supported() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
         __builtin_cpu_supports("f16c") && __builtin_cpu_supports("bmi2");
}

namespace {

// 32 consecutive indices of a row (starting at index k, k % 32 == 0) as bytes 0..31.
template <int BITS>
__attribute__((target("avx2,bmi2"))) inline __m256i load_indices(const uint8_t* row, int k) {
  if constexpr (BITS == 4) {
    const __m128i p = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + k / 2));
    const __m128i m = _mm_set1_epi8(0x0F);
    const __m128i lo = _mm_and_si128(p, m);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(p, 4), m);
    return _mm256_set_m128i(_mm_unpackhi_epi8(lo, hi), _mm_unpacklo_epi8(lo, hi));
  } else {
    constexpr int GB = BITS == 3 ? 3 : 2;                 // bytes per 8 indices
    constexpr uint64_t MASK = BITS == 3 ? 0x0707070707070707ull : 0x0303030303030303ull;
    const uint8_t* p = row + (int64_t)k * BITS / 8;
    uint64_t q[4];
    for (int g = 0; g < 4; ++g) {
      uint64_t f = 0;
      for (int b = 0; b < GB; ++b) f |= (uint64_t)p[g * GB + b] << (8 * b);
      q[g] = _pdep_u64(f, MASK);
    }
    return _mm256_set_epi64x((long long)q[3], (long long)q[2], (long long)q[1], (long long)q[0]);
  }
}

// One row against TB tokens.  Each token keeps NA independent partial sums (more for
// fewer tokens) so the FMA latency chain never limits the loop; at most 8 accumulators.
template <int BITS, int TB>
__attribute__((target("avx2,fma,f16c,bmi2")))
inline void row_tokens(const float* a, const float* scales, int64_t t0, int K, const uint8_t* row,
                       __m256i tlo, __m256i thi, float* out, int64_t ldo, int64_t n) {
  constexpr int NA = TB <= 2 ? 4 : (TB <= 4 ? 2 : 1);
  __m256 acc[TB][NA];
#pragma GCC unroll 8
  for (int t = 0; t < TB; ++t)
#pragma GCC unroll 4
    for (int p = 0; p < NA; ++p) acc[t][p] = _mm256_setzero_ps();
  for (int k = 0; k < K; k += 32) {
    const __m256i ix = load_indices<BITS>(row, k);
    const __m256i vlo = _mm256_shuffle_epi8(tlo, ix);
    const __m256i vhi = _mm256_shuffle_epi8(thi, ix);
    const __m256i h0 = _mm256_unpacklo_epi8(vlo, vhi);     // k 0..7  | k 16..23
    const __m256i h1 = _mm256_unpackhi_epi8(vlo, vhi);     // k 8..15 | k 24..31
    const __m256 w[4] = {_mm256_cvtph_ps(_mm256_castsi256_si128(h0)),
                         _mm256_cvtph_ps(_mm256_castsi256_si128(h1)),
                         _mm256_cvtph_ps(_mm256_extracti128_si256(h0, 1)),
                         _mm256_cvtph_ps(_mm256_extracti128_si256(h1, 1))};
#pragma GCC unroll 8
    for (int t = 0; t < TB; ++t) {
      const float* at = a + (t0 + t) * (int64_t)K + k;
#pragma GCC unroll 4
      for (int i = 0; i < 4; ++i)
        acc[t][i % NA] = _mm256_fmadd_ps(w[i], _mm256_loadu_ps(at + 8 * i), acc[t][i % NA]);
    }
  }
#pragma GCC unroll 8
  for (int t = 0; t < TB; ++t) {
    __m256 v = acc[t][0];
#pragma GCC unroll 4
    for (int p = 1; p < NA; ++p) v = _mm256_add_ps(v, acc[t][p]);
    const __m128 s4 = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    const __m128 s2 = _mm_add_ps(s4, _mm_movehl_ps(s4, s4));
    const __m128 s1 = _mm_add_ss(s2, _mm_shuffle_ps(s2, s2, 1));
    out[(t0 + t) * ldo + n] = scales[t0 + t] * _mm_cvtss_f32(s1);
  }
}

template <int BITS>
__attribute__((target("avx2,fma,f16c,bmi2")))
void rows_kernel(const float* a, const float* scales, int64_t T, int64_t n0, int64_t n1, int K,
                 const uint8_t* idx, const uint16_t* codebook, float* out, int64_t ldo) {
  constexpr int L = 1 << BITS;
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  for (int64_t n = n0; n < n1; ++n) {
    alignas(16) uint8_t lo[16] = {0}, hi[16] = {0};
    for (int c = 0; c < L; ++c) {
      lo[c] = (uint8_t)(codebook[n * L + c] & 0xFF);
      hi[c] = (uint8_t)(codebook[n * L + c] >> 8);
    }
    const __m256i tlo = _mm256_broadcastsi128_si256(_mm_load_si128(reinterpret_cast<const __m128i*>(lo)));
    const __m256i thi = _mm256_broadcastsi128_si256(_mm_load_si128(reinterpret_cast<const __m128i*>(hi)));
    const uint8_t* row = idx + n * row_bytes;
    int64_t t0 = 0;
    for (; t0 + 8 <= T; t0 += 8) row_tokens<BITS, 8>(a, scales, t0, K, row, tlo, thi, out, ldo, n);
    switch (T - t0) {
      case 1: row_tokens<BITS, 1>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 2: row_tokens<BITS, 2>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 3: row_tokens<BITS, 3>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 4: row_tokens<BITS, 4>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 5: row_tokens<BITS, 5>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 6: row_tokens<BITS, 6>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      case 7: row_tokens<BITS, 7>(a, scales, t0, K, row, tlo, thi, out, ldo, n); break;
      default: break;
    }
  }
}

// AVX-512 variant: each row's codebook is widened once into an fp32 table of 16 lanes,
// and vpermps looks up 16 weights per instruction, already as fp32.  A micro-kernel takes
// 4 rows x TB tokens: per 32 channels, 8 lookups and 2 TB activation loads feed 8 TB FMAs,
// so every activation load serves four rows.
template <int BITS>
__attribute__((target("avx512f,bmi2"))) inline __m512i load_indices16(const uint8_t* row, int k) {
  constexpr uint64_t MASK = BITS == 3 ? 0x0707070707070707ull : 0x0303030303030303ull;
  constexpr int GB = BITS;                                  // bytes per 8 indices
  const uint8_t* p = row + (int64_t)k * BITS / 8;
  uint64_t f0 = 0, f1 = 0;
  for (int b = 0; b < GB; ++b) {
    f0 |= (uint64_t)p[b] << (8 * b);
    f1 |= (uint64_t)p[GB + b] << (8 * b);
  }
  const __m128i bytes = _mm_set_epi64x((long long)_pdep_u64(f1, MASK), (long long)_pdep_u64(f0, MASK));
  return _mm512_cvtepu8_epi32(bytes);
}

// Indices k .. k+31 of a row as two vectors of 16 dwords.
template <int BITS>
__attribute__((target("avx512f,bmi2"))) inline void load_indices32(const uint8_t* row, int k,
                                                                   __m512i& i0, __m512i& i1) {
  if constexpr (BITS == 4) {
    const __m128i p = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + k / 2));
    const __m128i m = _mm_set1_epi8(0x0F);
    const __m128i lo = _mm_and_si128(p, m);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(p, 4), m);
    i0 = _mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi));
    i1 = _mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi));
  } else {
    i0 = load_indices16<BITS>(row, k);
    i1 = load_indices16<BITS>(row, k + 16);
  }
}

// Rows n .. n+3 against tokens t0 .. t0+TB-1.  One token keeps two partial sums per row
// (the 16-channel halves) so the FMA latency never limits the loop; more tokens keep one.
template <int BITS, int TB>
__attribute__((target("avx512f,bmi2")))
inline void block512(const float* a, const float* scales, int64_t t0, int K, const uint8_t* row0,
                     int64_t row_bytes, const __m512* tab, float* out, int64_t ldo, int64_t n) {
  constexpr int NA = TB == 1 ? 2 : 1;
  __m512 acc[4][TB][NA];
#pragma GCC unroll 4
  for (int r = 0; r < 4; ++r)
#pragma GCC unroll 4
    for (int t = 0; t < TB; ++t)
#pragma GCC unroll 2
      for (int q = 0; q < NA; ++q) acc[r][t][q] = _mm512_setzero_ps();
  for (int k = 0; k < K; k += 32) {
    __m512 w0[4], w1[4];
#pragma GCC unroll 4
    for (int r = 0; r < 4; ++r) {
      __m512i i0, i1;
      load_indices32<BITS>(row0 + r * row_bytes, k, i0, i1);
      w0[r] = _mm512_permutexvar_ps(i0, tab[r]);
      w1[r] = _mm512_permutexvar_ps(i1, tab[r]);
    }
#pragma GCC unroll 4
    for (int t = 0; t < TB; ++t) {
      const float* at = a + (t0 + t) * (int64_t)K + k;
      const __m512 a0 = _mm512_loadu_ps(at);
#pragma GCC unroll 4
      for (int r = 0; r < 4; ++r) acc[r][t][0] = _mm512_fmadd_ps(w0[r], a0, acc[r][t][0]);
      const __m512 a1 = _mm512_loadu_ps(at + 16);
#pragma GCC unroll 4
      for (int r = 0; r < 4; ++r) acc[r][t][NA - 1] = _mm512_fmadd_ps(w1[r], a1, acc[r][t][NA - 1]);
    }
  }
#pragma GCC unroll 4
  for (int r = 0; r < 4; ++r)
#pragma GCC unroll 4
    for (int t = 0; t < TB; ++t) {
      __m512 v = acc[r][t][0];
      if constexpr (NA == 2) v = _mm512_add_ps(v, acc[r][t][1]);
      out[(t0 + t) * ldo + n + r] = scales[t0 + t] * _mm512_reduce_add_ps(v);
    }
}

template <int BITS>
__attribute__((target("avx512f,bmi2,f16c")))
void rows_kernel512(const float* a, const float* scales, int64_t T, int64_t n0, int64_t n1, int K,
                    const uint8_t* idx, const uint16_t* codebook, float* out, int64_t ldo) {
  constexpr int L = 1 << BITS;
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  for (int64_t n = n0; n < n1; n += 4) {               // n1 - n0 is a multiple of 4
    __m512 tab[4];
    for (int r = 0; r < 4; ++r) {
      alignas(64) float ctab[16] = {0};
      for (int c = 0; c < L; ++c) ctab[c] = _cvtsh_ss(codebook[(n + r) * L + c]);
      tab[r] = _mm512_load_ps(ctab);
    }
    const uint8_t* row0 = idx + n * row_bytes;
    int64_t t0 = 0;
    for (; t0 + 4 <= T; t0 += 4) block512<BITS, 4>(a, scales, t0, K, row0, row_bytes, tab, out, ldo, n);
    switch (T - t0) {
      case 1: block512<BITS, 1>(a, scales, t0, K, row0, row_bytes, tab, out, ldo, n); break;
      case 2: block512<BITS, 2>(a, scales, t0, K, row0, row_bytes, tab, out, ldo, n); break;
      case 3: block512<BITS, 3>(a, scales, t0, K, row0, row_bytes, tab, out, ldo, n); break;
      default: break;
    }
  }
}

// A fixed set of worker threads, started on the first multi-threaded call and kept for
// the life of the process: a call hands each worker one range of rows and waits.
class Pool {
 public:
  static Pool& get() {
    static Pool p;
    return p;
  }
  int size() const { return (int)workers_.size() + 1; }
  // The pool's threads exist only in the process that started them (not after a fork).
  bool usable() const { return pid_ == getpid(); }
  // Runs job(0) .. job(n - 1), n <= size(), job(0) on the calling thread.
  void run(int n, const std::function<void(int)>& job) {
    std::unique_lock<std::mutex> call(call_mu_);        // one call at a time
    {
      std::lock_guard<std::mutex> lk(mu_);
      job_ = &job;
      n_ = n;
      pending_ = n - 1;
      ++gen_;
    }
    cv_.notify_all();
    job(0);
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, [&] { return pending_ == 0; });
    job_ = nullptr;
  }

 private:
  Pool() : pid_(getpid()) {
    const int hw = (int)std::max(1u, std::thread::hardware_concurrency());
    for (int i = 1; i < hw; ++i) workers_.emplace_back([this, i] { loop(i); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& w : workers_) w.join();
  }
  void loop(int i) {
    uint64_t seen = 0;
    for (;;) {
      const std::function<void(int)>* job;
      int n;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        job = job_;
        n = n_;
      }
      if (i < n) {
        (*job)(i);
        std::lock_guard<std::mutex> lk(mu_);
        if (--pending_ == 0) done_.notify_one();
      }
    }
  }
  pid_t pid_;
  std::vector<std::thread> workers_;
  std::mutex mu_, call_mu_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* job_ = nullptr;
  int n_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

}  // namespace

void cpu_lut_gemm_impl(const uint8_t* codes, const float* scales, int act_bits, int64_t T,
                       int64_t N, int K, int bits, const uint8_t* idx, const uint16_t* codebook,
                       float* out, int64_t ldo, int n_threads, bool use_avx512) {
  // activation codes -> fp32 (exact small integers), natural channel order
  std::vector<float> a((size_t)(T * K));
  const int64_t cb = (int64_t)K * act_bits / 8;
  for (int64_t t = 0; t < T; ++t) {
    const uint8_t* c = codes + t * cb;
    float* d = a.data() + t * K;
    if (act_bits == 8) {
      for (int k = 0; k < K; ++k) d[k] = (float)(int8_t)c[k];
    } else {
      for (int k = 0; k < K; k += 2) {
        const int lo = c[k / 2] & 0xF, hi = c[k / 2] >> 4;
        d[k] = (float)(lo >= 8 ? lo - 16 : lo);
        d[k + 1] = (float)(hi >= 8 ? hi - 16 : hi);
      }
    }
  }
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::min<int64_t>(nt, std::max<int64_t>(1, N / 16));
  const bool wide = use_avx512 && __builtin_cpu_supports("avx512f");
  auto run = [&](int64_t n0, int64_t n1) {
    if (wide) {
      switch (bits) {
        case 2: rows_kernel512<2>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
        case 3: rows_kernel512<3>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
        default: rows_kernel512<4>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
      }
      return;
    }
    switch (bits) {
      case 2: rows_kernel<2>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
      case 3: rows_kernel<3>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
      default: rows_kernel<4>(a.data(), scales, T, n0, n1, K, idx, codebook, out, ldo); break;
    }
  };
  if (nt <= 1) {
    run(0, N);
    return;
  }
  Pool& pool = Pool::get();
  if (pool.usable()) nt = std::min(nt, pool.size());
  const int64_t per = ((N + nt - 1) / nt + 3) / 4 * 4;   // whole 4-row blocks per thread
  auto part = [&](int i) {
    const int64_t n0 = i * per, n1 = std::min<int64_t>(N, n0 + per);
    if (n0 < n1) run(n0, n1);
  };
  if (pool.usable()) {
    pool.run(nt, part);
    return;
  }
  std::vector<std::thread> threads;                       // a forked child: plain threads
  for (int i = 1; i < nt; ++i) threads.emplace_back(part, i);
  part(0);
  for (auto& th : threads) th.join();
}

}  // namespace cbq
