// Codebook-LUT GEMM, decode path (few rows per expert; HBM-bound on the indices).
//
// CodeQuant2, Figure 4: the LUT kernel precomputes a table once and then replaces
// multiplications by table lookups; Figure 3: one codebook per weight row.  Here the
// one-time precomputation is each row's 2^bits-entry fp16 table, split into low and
// high bytes and kept in VGPRs for the whole K sweep; a lookup is a v_perm_b32 byte
// permute (four weights per permute), which never touches LDS and so cannot bank-
// conflict.  The dequantised weights go straight into the B operand of a 16x16x32
// fp16 MFMA whose A operand holds up to 16 tokens' activation codes (exact in fp16),
// so the integer x centroid products are exact and accumulate in fp32.
//
// Layout.  A workgroup owns NG groups of 16 output rows n of one expert (NG = 2 for a
// single matrix with 2- or 3-bit tables, else 1) and `splitk` waves.  Lane l serves
// row n0 + 16q + (l & 15) of group q and channel slice (l >> 4) * 32 of each
// 128-channel chunk, i.e. one 4*bits-byte load per chunk per matrix and group.  Token
// rows of the expert are processed in blocks of 32 (two 16-row MFMA sub-tiles sharing
// each dequantised weight; the groups share each converted activation fragment).
//  - An expert with at most 32 rows (decode) is split along K: wave w takes a range
//    of chunks, and the partial sums are reduced through LDS in wave order
//    (deterministic).  This multiplies the loads in flight per output row.
//  - A larger expert is split along rows: wave w takes row blocks w, w + splitk, ...
//    over all of K; the waves of a workgroup read the same index bytes at about the
//    same time, so the repeats are served by the caches.
#include <type_traits>

#include "cbq_internal.hpp"

namespace cbq {

template <int BITS>
__device__ __forceinline__ void load_idx(const uint8_t* p, bool ok, uint32_t* w) {
  if constexpr (BITS == 4) {
    u32x4 v = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BITS == 3) {
    u32x3 v = ok ? *reinterpret_cast<const u32x3*>(p) : u32x3{0, 0, 0};
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else {
    u32x2 v = ok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0, 0};
    w[0] = v[0]; w[1] = v[1];
  }
}

template <int ABITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, bool ok, uint32_t* c) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 a = ok ? q[0] : u32x4{0, 0, 0, 0};
  c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
  if constexpr (ABITS == 8) {
    u32x4 b = ok ? q[1] : u32x4{0, 0, 0, 0};
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
  }
}

// LT: weights looked up in LDS pair tables (2- and 3-bit codebooks), shared by the
// workgroup's waves (they serve the same rows); otherwise in per-row register tables.
// BLK: 3-bit indices in the blocked layout's re-encoded units (cbq_prepack_weights).
template <int BITS, int ABITS, int NW, int MSUB, int NG, bool LT, int DEPTH, bool BLK>
__global__ void __launch_bounds__(NW == 2 ? 512 : 1024, BITS <= 3 ? 4 : 3)
lut_decode_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                  const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
                  GemmW w0, GemmW w1, int64_t n_rows, int N, int K, int splitk, int max_rows,
                  int blocked, void* __restrict__ out, int64_t ldo) {
  // [(splitk-1) * NG * NW * MSUB][64] f32x4 of split-K partial sums, then (LT) the pair
  // tables: [NG * NW][NE entries][16 rows] dwords
  extern __shared__ f32x4 red[];
  constexpr int NE = LT ? PairTab<BITS>::NE : 1;
  uint32_t* const ptab = reinterpret_cast<uint32_t*>(red + (size_t)(splitk - 1) * NG * NW * MSUB * 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Experts in reverse order: the shared experts come last in the row order and always
  // hold every token, the most rows of any expert, so their longer waves start first
  // instead of forming the tail of the grid.
  const int e = gridDim.y - 1 - blockIdx.y;
  int64_t r0, me;
  if (offsets) {
    r0 = offsets[e];
    me = offsets[e + 1] - r0;
  } else {
    r0 = 0;
    me = n_rows;
  }
  if (me <= 0 || (max_rows >= 0 && me > max_rows)) return;

  const int nl = lane & 15, g = lane >> 4;
  constexpr int L = 1 << BITS;
  // bytes per row of the expert's index block; the rows layout keeps each row's bitstream,
  // the blocked one each 16-row x 128-channel tile in 256*BITS contiguous bytes
  const int64_t row_bytes = index_row_bytes(K, BITS, blocked != 0);
  const uint32_t chunk_step = blocked ? 256u * BITS : 16u * BITS;
  const int64_t code_bytes = (int64_t)K * ABITS / 8;

  // row group q of this workgroup: rows (blockIdx.x * NG + q) * 16 + 0..15
  int nrow[NG];
  bool nvalid[NG];
  uint32_t wlane[NG];
  RowTable<BITS> tab[NG][NW];   // register tables (unused with LT)
  uint32_t trow[NG][NW];        // LT: dword of entry 0 of this lane's row in each table
  __amdgpu_buffer_rsrc_t wres[NW];
  wres[0] = make_rsrc(w0.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
  if constexpr (NW == 2) wres[1] = make_rsrc(w1.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int n = (blockIdx.x * NG + q) * 16 + nl;
    nrow[q] = n;
    nvalid[q] = n < N;
    const int nn = nvalid[q] ? n : 0;
    wlane[q] = !nvalid[q] ? kOffNone
               : blocked ? (uint32_t)((n - nl) * row_bytes) + (uint32_t)(lane * 4 * BITS)
                         : (uint32_t)(n * row_bytes) + (uint32_t)(g * 4 * BITS);
    if constexpr (LT) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        trow[q][w] = (uint32_t)((q * NW + w) * NE * 16 + nl);
        // the 4 lanes of each row in one wave build its table; tables go round the waves
        if ((q * NW + w) % splitk == wave) {
          const uint32_t* src = reinterpret_cast<const uint32_t*>(
              (w == 0 ? w0.codebook : w1.codebook) + ((int64_t)e * N + nn) * L);
          uint32_t cb[L / 2];
#pragma unroll
          for (int i = 0; i < L / 2; ++i) cb[i] = src[i];
          pair_build<BITS, 4, 16>(ptab, trow[q][w], cb, g);
        }
      }
    } else {
      tab[q][0].load(w0.codebook + ((int64_t)e * N + nn) * L);
      if constexpr (NW == 2) tab[q][1].load(w1.codebook + ((int64_t)e * N + nn) * L);
    }
  }
  // tables built by other waves of the workgroup must be complete before any lookup
  // (a wave's own LDS writes precede its reads in order, so one wave needs no barrier)
  if (LT && splitk > 1) lds_barrier();
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(codes, 0x7FFFFFFFu);

  const int nchunks = (K + 127) >> 7;
  const bool rowsplit = splitk > 1 && me > 16 * MSUB;   // uniform over the workgroup
  const bool ksplit = splitk > 1 && !rowsplit;
  const int cpw = ksplit ? (nchunks + splitk - 1) / splitk : nchunks;
  const int c_begin = ksplit ? wave * cpw : 0;
  const int c_end = min(nchunks, c_begin + cpw);
  const int64_t mb_first = rowsplit ? (int64_t)wave * 16 * MSUB : 0;
  const int64_t mb_step = rowsplit ? (int64_t)splitk * 16 * MSUB : 16 * MSUB;

  for (int64_t mb = mb_first; mb < me; mb += mb_step) {
    f32x4 acc[NG][NW][MSUB];
    uint32_t aoff[MSUB];     // byte offset of this lane's activation row per sub-tile
#pragma unroll
    for (int s = 0; s < MSUB; ++s) {
#pragma unroll
      for (int q = 0; q < NG; ++q)
#pragma unroll
        for (int w = 0; w < NW; ++w) acc[q][w][s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int64_t m = mb + s * 16 + nl;
      uint32_t o = kOffNone;
      if (m < me) {
        const int64_t r = r0 + m;
        const int64_t tok = row_token ? (int64_t)row_token[r] : r;
        o = (uint32_t)(tok * code_bytes) + (uint32_t)(g * 4 * ABITS);
      }
      aoff[s] = o;
    }
    const int nsub = (int)min<int64_t>((me - mb + 15) >> 4, MSUB);

    // The K sweep for NSUB live token sub-tiles, a compile-time count: an expert with
    // fewer rows than MSUB sub-tiles hold issues no loads, conversions or MFMAs for the
    // empty ones.  A ring of DEPTH chunks of raw data is loaded DEPTH chunks ahead, so a
    // wave of few chunks (the split-K waves of small grids) has all its loads in flight.
    auto sweep = [&](auto nsub_c) {
      constexpr int NSUB = decltype(nsub_c)::value;
      struct Slot {
        uint32_t w[NG][NW][BITS];
        uint32_t a[NSUB][ABITS];
      };
      Slot ring[DEPTH];
      auto load = [&](int c, Slot& d) {
        const bool ok = c < c_end && c * 128 + g * 32 < K;
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int w = 0; w < NW; ++w)
            buf_load<4 * BITS>(wres[w], ok ? wlane[q] : kOffNone, d.w[q][w], (uint32_t)c * chunk_step);
        const uint32_t cs = (uint32_t)(c * 128 * ABITS / 8);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
#pragma unroll
          for (int h = 0; h < ABITS / 4; ++h)
            buf_load<16>(cres, ok ? aoff[s] + 16 * h : kOffNone, &d.a[s][4 * h], cs);
        }
      };
      // the activation fragments are converted once per chunk and shared by the row
      // groups and weight matrices
      auto chunk = [&](const Slot& cur) {
        uint32_t ad[NSUB][16];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) codes32_to_f16_ord<ABITS, LT>(cur.a[s], ad[s]);
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          uint32_t bd[NW][16];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            if constexpr (LT) pair_lookup32<BITS, 16, BLK>(ptab, trow[q][w], cur.w[q][w], bd[w]);
            else dequant32<BITS, BLK>(tab[q][w], cur.w[q][w], bd[w]);
          }
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int w = 0; w < NW; ++w) {
                const f16x8 A = as_f16x8(ad[s][4 * j], ad[s][4 * j + 1], ad[s][4 * j + 2], ad[s][4 * j + 3]);
                const f16x8 B = as_f16x8(bd[w][4 * j], bd[w][4 * j + 1], bd[w][4 * j + 2], bd[w][4 * j + 3]);
                acc[q][w][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[q][w][s], 0, 0, 0);
              }
        }
      };
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) load(c_begin + i, ring[i]);
      int c = c_begin;
      for (; c + DEPTH - 1 < c_end; c += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
          chunk(ring[i]);
          load(c + DEPTH + i, ring[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < DEPTH - 1; ++i)
        if (c + i < c_end) chunk(ring[i]);
    };
    static_assert(MSUB == 1 || MSUB == 2, "one or two token sub-tiles");
    if (MSUB == 2 && nsub == 2) sweep(std::integral_constant<int, MSUB>{});
    else sweep(std::integral_constant<int, 1>{});

    // ordered split-K reduction
    if (ksplit) {
      if (wave > 0) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int s = 0; s < MSUB; ++s)
              red[((((wave - 1) * NG + q) * NW + w) * MSUB + s) * 64 + lane] = acc[q][w][s];
      }
      __syncthreads();
      if (wave == 0) {
        for (int v = 1; v < splitk; ++v)
#pragma unroll
          for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
              for (int s = 0; s < MSUB; ++s)
                acc[q][w][s] += red[((((v - 1) * NG + q) * NW + w) * MSUB + s) * 64 + lane];
      }
    }

    // epilogue: lane holds D[m = 4*(lane>>4) + i][n = lane & 15]
    if (wave == 0 || rowsplit) {
#pragma unroll
      for (int s = 0; s < MSUB; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = mb + s * 16 + 4 * g + i;
          if (m >= me) continue;
          const int64_t r = r0 + m;
          const int64_t tok = row_token ? (int64_t)row_token[r] : r;
          const float sc = scales[tok];
#pragma unroll
          for (int q = 0; q < NG; ++q) {
            if (!nvalid[q]) continue;
            if constexpr (NW == 2) {
              const float gv = acc[q][0][s][i] * sc, uv = acc[q][1][s][i] * sc;
              reinterpret_cast<uint16_t*>(out)[r * ldo + nrow[q]] = f32_to_bf16_rne(silu_mul(gv, uv));
            } else {
              reinterpret_cast<float*>(out)[r * ldo + nrow[q]] = acc[q][0][s][i] * sc;
            }
          }
        }
      }
    }
    if (ksplit) __syncthreads();
  }
}

template <int BITS, int ABITS, int NW, int MSUB, int NG, bool LT, int DEPTH, bool BLK>
static hipError_t launch_t2(const GemmArgs& a, int max_rows, int splitk, hipStream_t stream) {
  const int E = a.offsets ? a.E : 1;
  dim3 grid((unsigned)((a.N + 16 * NG - 1) / (16 * NG)), (unsigned)E);
  const size_t lds = (size_t)(splitk - 1) * NG * NW * MSUB * 64 * sizeof(f32x4) +
                     (LT ? (size_t)NG * NW * PairTab<BITS>::NE * 16 * sizeof(uint32_t) : 0);
  hipLaunchKernelGGL((lut_decode_kernel<BITS, ABITS, NW, MSUB, NG, LT, DEPTH, BLK>), grid, dim3(64 * splitk), lds,
                     stream, a.codes, a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows,
                     a.N, a.K, splitk, max_rows, a.blocked, a.out, a.ldo);
  return hipGetLastError();
}

template <int BITS, int ABITS, int NW, int MSUB, int NG, bool LT, int DEPTH>
static hipError_t launch_t(const GemmArgs& a, int max_rows, int splitk, hipStream_t stream) {
  if constexpr (BITS == 3) {
    if (a.blocked) return launch_t2<BITS, ABITS, NW, MSUB, NG, LT, DEPTH, true>(a, max_rows, splitk, stream);
  }
  return launch_t2<BITS, ABITS, NW, MSUB, NG, LT, DEPTH, false>(a, max_rows, splitk, stream);
}

// Row groups per wave: a single matrix with 2- or 3-bit tables (8 VGPRs per row)
// takes two, which halves the activation conversions; the gate/up pair and 4-bit
// tables (32 VGPRs per row) keep one, as more registers would cost occupancy.
static int decode_groups(int bits, int n_w) { return (n_w == 1 && bits <= 3) ? 2 : 1; }

// Calls of at most 16 rows (no expert can hold more) take one 16-token sub-tile and a
// deeper ring: six chunks for a single 4-bit matrix, four for the gate/up pair and for
// two row groups (what the registers hold); larger calls two sub-tiles and two chunks.
template <int BITS, int ABITS, bool LT>
static hipError_t launch_b(const GemmArgs& a, int max_rows, int splitk, hipStream_t s) {
  const bool small = a.n_rows <= 16;
  if (a.n_w == 2)
    return small ? launch_t<BITS, ABITS, 2, 1, 1, LT, 4>(a, max_rows, splitk, s)
                 : launch_t<BITS, ABITS, 2, 2, 1, LT, 2>(a, max_rows, splitk, s);
  if constexpr (BITS <= 3)
    return small ? launch_t<BITS, ABITS, 1, 1, 2, LT, 4>(a, max_rows, splitk, s)
                 : launch_t<BITS, ABITS, 1, 2, 2, LT, 2>(a, max_rows, splitk, s);
  else
    return small ? launch_t<BITS, ABITS, 1, 1, 1, LT, 6>(a, max_rows, splitk, s)
                 : launch_t<BITS, ABITS, 1, 2, 1, LT, 2>(a, max_rows, splitk, s);
}

// Where 2- and 3-bit codebooks are looked up by default, as measured on the decode GEMMs:
// LDS pair tables (one lookup per two weights) for 2-bit codebooks and for 3-bit ones in
// the row layout; register tables for 3-bit codebooks in the blocked layout, whose
// re-encoded units make the register selectors one mask or one shift and a mask.  4-bit
// pair tables would take 256 entries a row, so 4-bit tables stay in registers.
template <int BITS, int ABITS>
static hipError_t launch_b(const GemmArgs& a, int max_rows, int splitk, hipStream_t s) {
  if constexpr (BITS <= 3) {
    const bool lds = a.tables == kTablesLds ||
                     (a.tables == kTablesDefault && !(BITS == 3 && a.blocked));
    if (lds) return launch_b<BITS, ABITS, true>(a, max_rows, splitk, s);
  }
  return launch_b<BITS, ABITS, false>(a, max_rows, splitk, s);
}

hipError_t launch_lut_decode(const GemmArgs& a, int max_rows, hipStream_t stream) {
  // Split K (small experts) or rows (large) only while the grid holds fewer than 2,048
  // waves, and never below four 128-channel chunks per wave.  Measured on the decode
  // shapes, fewer and longer waves win: a wave's index loads are then spread over more
  // chunks, and a split costs a reduction through LDS.
  const int E = a.offsets ? a.E : 1;
  const int64_t active = a.offsets ? (a.n_rows < E ? a.n_rows : E) : 1;
  const int ng = decode_groups(a.bits, a.n_w);
  const int64_t tiles = (int64_t)((a.N + 16 * ng - 1) / (16 * ng)) * (active > 0 ? active : 1);
  const int nchunks = (a.K + 127) / 128;
  int splitk = 1;
  while (splitk < 16 && tiles * splitk < 2048 && splitk * 8 <= nchunks) splitk *= 2;
  if (a.n_w == 2 && splitk > 8) splitk = 8;
  const int ab = a.act_bits;
  switch (a.bits * 10 + (ab == 8 ? 8 : 4)) {
    case 44: return launch_b<4, 4>(a, max_rows, splitk, stream);
    case 48: return launch_b<4, 8>(a, max_rows, splitk, stream);
    case 34: return launch_b<3, 4>(a, max_rows, splitk, stream);
    case 38: return launch_b<3, 8>(a, max_rows, splitk, stream);
    case 24: return launch_b<2, 4>(a, max_rows, splitk, stream);
    case 28: return launch_b<2, 8>(a, max_rows, splitk, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cbq
