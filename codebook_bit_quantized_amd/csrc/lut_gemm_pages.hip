// The codebook LUT GEMM in the two table forms of the pages' kernel design, for 4-bit
// codebooks and A4 activations (CBQ_PATH_PAGES_PRODUCTS, CBQ_PATH_PAGES_BUCKETS): kept to
// measure them against the register-table MFMA path, never chosen by CBQ_PATH_AUTO.  Meant
// for experts of a few rows (decode); correct for any row count.
//
// CodeQuant2, Figure 4: a table is built once and the GEMM then reads products from it in
// shared memory instead of multiplying; the AI Radio episode ("Improvements"): a
// multiplication table, whose cost is shared-memory bank conflicts.
//
//  - Product table: per weight row the products |a| * C[c] of the nine code magnitudes
//    |a| = 0..8 and the 16 centroids (fp32, exact: a 4-bit integer times an fp16 value),
//    one copy per 16-row tile shared by the tile's waves; the code's sign is put back
//    after the lookup (sign folding).  One LDS read and one fp32 add per (token, weight).
//    Entry (w, |a|, c) of row r sits at dword ((w * 9 + |a|) * 16 + c) * 16 + r, so the
//    16 rows of a read fall in distinct banks and only the four lanes that share a row can
//    conflict (when their centroid indices differ but agree modulo the bank stride).
//  - Bucketed activations: per weight row, 16 integer buckets S[c] that sum the codes
//    whose weight has index c (lane-private, in LDS: one ds_add per weight for two tokens,
//    packed as S0 + 65536 * S1 and split exactly afterwards), then
//    y = scale * sum_c C[c] * S[c]: 16 products per row and token at the end.
//
// Lane l serves row 16*G + (l & 15) and channel slice (l >> 4) * 32 of each 128-channel
// chunk (the unit order of the blocked index layout); the waves of a workgroup split K and
// their partial sums meet in LDS in wave order.  Each wave keeps the next chunk's loads in
// flight while it works on the current one, and issues the first two before the product
// table is built.
#include "cbq_internal.hpp"

namespace cbq {

namespace {
constexpr int NA = 9;   // code magnitudes 0..8

// MODE 0 (products) takes four tokens a pass, MODE 1 (buckets) two (one packed dword).
template <int MODE>
constexpr int pages_tokens() { return MODE == 0 ? 4 : 2; }

// Largest K split (waves a workgroup) launch_lut_pages picks: 16, or 8 for the product
// form with two weight sets (which needs more than 128 VGPRs a lane to keep its loads and
// lookups in flight).
template <int MODE, int NW>
constexpr int pages_max_split() { return MODE == 0 && NW == 2 ? 8 : 16; }

template <int NW, int TB>
struct PagesChunk {
  uint32_t wi[NW][4];   // 32 weight indices of this lane's slice, per weight set
  uint32_t ac[TB][4];   // 32 activation codes of this lane's slice, per token
};

template <int NW, int TB>
__device__ __forceinline__ void pages_load(PagesChunk<NW, TB>& b, const __amdgpu_buffer_rsrc_t* wres,
                                           uint32_t wlane, uint32_t chunk_step,
                                           __amdgpu_buffer_rsrc_t cres, const uint32_t* aoff, int nt,
                                           int K, int g, int c, int c_end) {
  // past c_end (or past K) the offsets are out of range: the loads return zeros
  const bool ok = c < c_end && c * 128 + g * 32 < K;
#pragma unroll
  for (int w = 0; w < NW; ++w) buf_load<16>(wres[w], ok ? wlane : kOffNone, b.wi[w], (uint32_t)c * chunk_step);
#pragma unroll
  for (int t = 0; t < TB; ++t)
    buf_load<16>(cres, ok && t < nt ? aoff[t] : kOffNone, b.ac[t], (uint32_t)c * 64u);
}

// The signed 4-bit code k of a 32-code slice.
__device__ __forceinline__ int code4(const uint32_t* ac, int k) {
  return ((int)(ac[k >> 3] << (28 - (k & 7) * 4))) >> 28;
}

template <int MODE, int NW, int TB>
__device__ __forceinline__ void pages_chunk(const PagesChunk<NW, TB>& b, const uint32_t* tab_row,
                                            uint32_t* bk, int nt, float (&acc)[NW][TB]) {
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    uint32_t ix[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) ix[w] = (b.wi[w][k >> 3] >> ((k & 7) * 4)) & 15u;
    if constexpr (MODE == 0) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t >= nt) break;
        const int a = code4(b.ac[t], k);
        const uint32_t mag = (uint32_t)(a < 0 ? -a : a);
        const uint32_t sgn = (uint32_t)a & 0x80000000u;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t v = tab_row[((w * NA + mag) * 16 + ix[w]) * 16];
          acc[w][t] += __builtin_bit_cast(float, v ^ sgn);
        }
      }
    } else {
      static_assert(TB == 2, "the bucket form packs two tokens a dword");
      const int a0 = code4(b.ac[0], k);
      const int a1 = nt > 1 ? code4(b.ac[1], k) : 0;
      const uint32_t pv = (uint32_t)a0 + ((uint32_t)a1 << 16);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        __hip_atomic_fetch_add(&bk[(w * 16 + ix[w]) * 64], pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}
}  // namespace

// MODE 0: product tables; MODE 1: buckets.  NW: 1 (fp32 out) or 2 (gate, up; SwiGLU).
template <int MODE, int NW>
__global__ void __launch_bounds__((64 * pages_max_split<MODE, NW>()))
lut_pages_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                 const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
                 GemmW w0, GemmW w1, int64_t n_rows, int N, int K, int splitk, int blocked,
                 void* __restrict__ out, int64_t ldo) {
  constexpr int TB = pages_tokens<MODE>();
  // LDS: [splitk][NW][TB][16] partial sums, then MODE 0: [NW][NA][16][16] product table
  // (w, |a|, c, row); MODE 1: [splitk][NW][16][64] buckets (wave, w, c, lane)
  extern __shared__ float lds[];
  float* const red = lds;
  uint32_t* const tab = reinterpret_cast<uint32_t*>(lds + splitk * NW * TB * 16);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = gridDim.y - 1 - blockIdx.y;
  int64_t r0, me;
  if (offsets) {
    r0 = offsets[e];
    me = offsets[e + 1] - r0;
  } else {
    r0 = 0;
    me = n_rows;
  }
  if (me <= 0) return;                        // uniform over the workgroup

  const int nl = lane & 15, g = lane >> 4;
  const int n = blockIdx.x * 16 + nl;
  const bool nvalid = n < N;
  const int nn = nvalid ? n : 0;
  const int64_t row_bytes = index_row_bytes(K, 4, blocked != 0);
  const uint32_t chunk_step = blocked ? 1024u : 64u;
  const uint32_t wlane = !nvalid ? kOffNone
                         : blocked ? (uint32_t)((int64_t)(n - nl) * row_bytes) + (uint32_t)(lane * 16)
                                   : (uint32_t)((int64_t)n * row_bytes) + (uint32_t)(g * 16);
  __amdgpu_buffer_rsrc_t wres[NW];
  wres[0] = make_rsrc(w0.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
  if constexpr (NW == 2) wres[1] = make_rsrc(w1.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(codes, 0x7FFFFFFFu);
  const int64_t code_bytes = K / 2;

  const int nchunks = (K + 127) >> 7;
  const int cpw = (nchunks + splitk - 1) / splitk;
  const int c_begin = wave * cpw, c_end = min(nchunks, c_begin + cpw);

  // the rows' fp16 codebooks (16 per row), as fp32
  float cbf[NW][16];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint16_t* cb = (w == 0 ? w0.codebook : w1.codebook) + ((int64_t)e * N + nn) * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c) cbf[w][c] = (float)__builtin_bit_cast(_Float16, cb[c]);
  }
  const uint32_t* const tab_row = tab + nl;
  // MODE 1: this lane's buckets, bucket (w, c) at dword ((wave * NW + w) * 16 + c) * 64 + lane
  uint32_t* const bk = tab + (size_t)wave * NW * 16 * 64 + lane;

  PagesChunk<NW, TB> b0, b1;
  uint32_t aoff[TB];
  int nt = 0;
  // the token offsets of the pass starting at row t0, and its first two chunks' loads
  auto start_pass = [&](int64_t t0) {
    nt = (int)min<int64_t>(me - t0, TB);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      uint32_t o = kOffNone;
      if (t < nt) {
        const int64_t r = r0 + t0 + t;
        const int64_t tok = row_token ? (int64_t)row_token[r] : r;
        o = (uint32_t)(tok * code_bytes) + (uint32_t)(g * 16);
      }
      aoff[t] = o;
    }
    pages_load(b0, wres, wlane, chunk_step, cres, aoff, nt, K, g, c_begin, c_end);
    pages_load(b1, wres, wlane, chunk_step, cres, aoff, nt, K, g, c_begin + 1, c_end);
  };
  start_pass(0);
  if constexpr (MODE == 0) {
    // lane group g writes the centroids c = g (mod 4) of its row: entry
    // ((w * NA + |a|) * 4 + j) * 4 + g for c = 4j + g, by wave (w * NA + |a|) * 4 + j
    // modulo splitk (a power of two)
    float cg[NW][4];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        cg[w][j] = g == 0 ? cbf[w][4 * j] : g == 1 ? cbf[w][4 * j + 1] : g == 2 ? cbf[w][4 * j + 2]
                                                                             : cbf[w][4 * j + 3];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = (w * NA + a) * 4 + j;
          if ((q & (splitk - 1)) == wave)
            tab[(q * 4 + g) * 16 + nl] = __builtin_bit_cast(uint32_t, (float)a * cg[w][j]);
        }
    lds_barrier();
  }
  for (int64_t t0 = 0;;) {
    if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < NW * 16; ++i) bk[i * 64] = 0u;
    }
    float acc[NW][TB];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[w][t] = 0.0f;
    for (int c = c_begin; c < c_end; c += 2) {
      pages_chunk<MODE>(b0, tab_row, bk, nt, acc);
      pages_load(b0, wres, wlane, chunk_step, cres, aoff, nt, K, g, c + 2, c_end);
      if (c + 1 < c_end) {
        pages_chunk<MODE>(b1, tab_row, bk, nt, acc);
        pages_load(b1, wres, wlane, chunk_step, cres, aoff, nt, K, g, c + 3, c_end);
      }
    }
    if constexpr (MODE == 1) {
      // S0 = the low 16 bits as a signed value, S1 = (X - S0) / 65536: exact while every
      // bucket sum stays within int16 (at most 4,096 codes a lane, |code| <= 8); then
      // sum_c C[c] * S[c] in fp64 (exact products)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const uint32_t x = bk[(w * 16 + c) * 64];
          const int v0 = (int16_t)(x & 0xFFFFu);
          const int v1 = (int16_t)((x - (uint32_t)v0) >> 16);
          s0 += (double)cbf[w][c] * (double)v0;
          s1 += (double)cbf[w][c] * (double)v1;
        }
        acc[w][0] = (float)s0;
        acc[w][1] = (float)s1;
      }
    }
    // the 4 channel slices of a row (lanes nl, nl+16, nl+32, nl+48), then the waves in order
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        float v = acc[w][t];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[w][t] = v;
      }
    if (splitk > 1) {
      if (lane < 16) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int t = 0; t < TB; ++t) red[((wave * NW + w) * TB + t) * 16 + lane] = acc[w][t];
      }
      lds_barrier();
      if (wave == 0) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int t = 0; t < TB; ++t) {
            float v = red[(w * TB + t) * 16 + nl];
            for (int u = 1; u < splitk; ++u) v += red[((u * NW + w) * TB + t) * 16 + nl];
            acc[w][t] = v;
          }
      }
    }
    if (wave == 0 && g == 0 && nvalid) {
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        if (t >= nt) break;
        const int64_t r = r0 + t0 + t;
        const int64_t tok = row_token ? (int64_t)row_token[r] : r;
        const float sc = scales[tok];
        if constexpr (NW == 2) {
          const float gv = acc[0][t] * sc, uv = acc[1][t] * sc;
          reinterpret_cast<uint16_t*>(out)[r * ldo + n] = f32_to_bf16_rne(silu_mul(gv, uv));
        } else {
          reinterpret_cast<float*>(out)[r * ldo + n] = acc[0][t] * sc;
        }
      }
    }
    t0 += TB;
    if (t0 >= me) break;
    if (splitk > 1) lds_barrier();   // red is rewritten by the next pass
    start_pass(t0);
  }
}

template <int MODE, int NW>
static hipError_t launch_pg(const GemmArgs& a, int splitk, hipStream_t stream) {
  constexpr int TB = pages_tokens<MODE>();
  const int E = a.offsets ? a.E : 1;
  dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)E);
  size_t lds = (size_t)splitk * NW * TB * 16 * sizeof(float);
  lds += MODE == 0 ? (size_t)NW * NA * 16 * 16 * sizeof(uint32_t)
                   : (size_t)splitk * NW * 16 * 64 * sizeof(uint32_t);
  hipLaunchKernelGGL((lut_pages_kernel<MODE, NW>), grid, dim3(64 * splitk), lds, stream, a.codes,
                     a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, a.N, a.K, splitk,
                     a.blocked, a.out, a.ldo);
  return hipGetLastError();
}

hipError_t launch_lut_pages(const GemmArgs& a, int mode, hipStream_t stream) {
  // K split over the waves of a workgroup (a power of two, at most 8 or 16) while the grid holds
  // fewer than 8,192 waves and each wave keeps at least two chunks (one ring round).  LDS per workgroup:
  // the product table 9 KB per weight set; the buckets 4 KB per wave and weight set.  The
  // caller keeps K <= 16384, so a lane sums at most 4,096 codes into a bucket.
  const int E = a.offsets ? a.E : 1;
  const int64_t active = a.offsets ? (a.n_rows < E ? a.n_rows : E) : 1;
  const int64_t tiles = (int64_t)((a.N + 15) / 16) * (active > 0 ? active : 1);
  const int nchunks = (a.K + 127) / 128;
  int splitk = 1;
  const int max_split = mode == 0 ? (a.n_w == 2 ? pages_max_split<0, 2>() : pages_max_split<0, 1>())
                                  : (a.n_w == 2 ? pages_max_split<1, 2>() : pages_max_split<1, 1>());
  while (splitk < max_split && tiles * splitk < 8192 && splitk * 2 <= nchunks) splitk *= 2;
  if (mode == 0) return a.n_w == 2 ? launch_pg<0, 2>(a, splitk, stream) : launch_pg<0, 1>(a, splitk, stream);
  return a.n_w == 2 ? launch_pg<1, 2>(a, splitk, stream) : launch_pg<1, 1>(a, splitk, stream);
}

}  // namespace cbq
