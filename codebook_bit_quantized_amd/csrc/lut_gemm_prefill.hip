// Codebook GEMM, prefill path (many rows per expert: a dense contraction).
//
// Once an expert has enough rows, each dequantised weight is reused by many tokens,
// so the work becomes MFMA-bound: weights are dequantised tile by tile into LDS as
// fp16 (exact: the centroids are fp16) with the same per-row register tables as the
// decode path, activation codes are converted to fp16 (exact), and 32x32x16 fp16
// MFMAs accumulate in fp32.  Products are exact; only the fp32 summation order
// differs from the plain definition.
//
// Tile: 128 rows (tokens of one expert) x 128 columns x 64 channels per step, 256
// threads as 2x2 waves of 64x64.  For the gate/up pair the 128 columns are 64 gate
// rows and the same 64 up rows, so the SwiGLU epilogue finds g and u in one lane.
// Thread t dequantises 32 weights of column t/2 and converts 32 codes of row t/2 per
// step; LDS is double-buffered so the next step's loads overlap this step's MFMAs.
// Workgroup (x, y) takes column tile x and the y-th 128-row tile in expert order,
// skipping experts with at most min_rows rows (those go to the decode path).
#include "cbq_internal.hpp"

namespace cbq {

namespace {
constexpr int BM = 128;
constexpr int BNC = 128;   // columns per tile
constexpr int BK = 64;
constexpr int LDW = BK + 8; // fp16 per LDS row (padding staggers the banks)

template <int BITS>
__device__ __forceinline__ void load_idx_p(const uint8_t* p, bool ok, uint32_t* w) {
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
__device__ __forceinline__ void load_codes_p(const uint8_t* p, bool ok, uint32_t* c) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 a = ok ? q[0] : u32x4{0, 0, 0, 0};
  c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
  if constexpr (ABITS == 8) {
    u32x4 b = ok ? q[1] : u32x4{0, 0, 0, 0};
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
  }
}
}  // namespace

template <int BITS, int ABITS, int NW>
__global__ void __launch_bounds__(256)
mfma_prefill_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
                    GemmW w0, GemmW w1, int64_t n_rows, int E, int N, int K, int min_rows,
                    void* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNC * LDW];
  __shared__ int64_t s_r0, s_me, s_m0;
  __shared__ int s_e;

  const int tid = threadIdx.x;
  if (tid == 0) {
    int64_t ty = blockIdx.y;
    int found = -1;
    int64_t r0 = 0, me = 0, m0 = 0;
    if (!offsets) {
      if (ty * BM < n_rows) { found = 0; r0 = 0; me = n_rows; m0 = ty * BM; }
    } else {
      for (int e = 0; e < E; ++e) {
        const int64_t a = offsets[e], c = offsets[e + 1] - offsets[e];
        if (c <= min_rows) continue;
        const int64_t nt = (c + BM - 1) / BM;
        if (ty < nt) { found = e; r0 = a; me = c; m0 = ty * BM; break; }
        ty -= nt;
      }
    }
    s_e = found; s_r0 = r0; s_me = me; s_m0 = m0;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int64_t r0 = s_r0, me = s_me, m0 = s_m0;

  constexpr int NCOL = (NW == 2) ? BNC / 2 : BNC;    // weight rows per matrix in the tile
  const int n0 = blockIdx.x * NCOL;
  constexpr int L = 1 << BITS;
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  const int64_t code_bytes = (int64_t)K * ABITS / 8;

  // ---- loader roles ----
  const int col = tid >> 1, khalf = tid & 1;
  const int wsel = (NW == 2) ? (col / NCOL) : 0;
  const int n = n0 + ((NW == 2) ? (col % NCOL) : col);
  const bool nvalid = n < N;
  const GemmW W = (NW == 2 && wsel == 1) ? w1 : w0;
  RowTable<BITS> tab;
  tab.load(W.codebook + ((int64_t)e * N + (nvalid ? n : 0)) * L);
  const uint8_t* wrow = W.idx + ((int64_t)e * N + (nvalid ? n : 0)) * row_bytes;

  const int arow = tid >> 1;
  const bool avalid = m0 + arow < me;
  const int64_t ar = r0 + m0 + (avalid ? arow : 0);
  const int64_t atok = row_token ? (int64_t)row_token[ar] : ar;
  const uint8_t* crow = codes + atok * code_bytes;

  uint32_t wv[BITS], av[ABITS];
  auto gload = [&](int kt) {
    const int kb = kt * BK + khalf * 32;
    const bool kok = kb < K;
    load_idx_p<BITS>(wrow + (int64_t)kb * BITS / 8, nvalid && kok, wv);
    load_codes_p<ABITS>(crow + (int64_t)kb * ABITS / 8, avalid && kok, av);
  };
  auto lstore = [&](int buf) {
    uint32_t d[16];
    dequant32<BITS>(tab, wv, d);
    u32x4* bp = reinterpret_cast<u32x4*>(&Bs[buf][col * LDW + khalf * 32]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bp[j] = u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
    codes32_to_f16<ABITS>(av, d);
    u32x4* ap = reinterpret_cast<u32x4*>(&As[buf][arow * LDW + khalf * 32]);
#pragma unroll
    for (int j = 0; j < 4; ++j) ap[j] = u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
  };

  // ---- MFMA roles ----
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int cb[2];
  if constexpr (NW == 2) { cb[0] = wn * 32; cb[1] = NCOL + wn * 32; }   // gate, up
  else { cb[0] = wn * 64; cb[1] = wn * 64 + 32; }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(&As[buf][(wm * 64 + i * 32 + lr) * LDW + kk * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(&Bs[buf][(cb[j] + lr) * LDW + kk * 16 + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][v] = D[8*(v/4) + 4*(lane/32) + v%4][lane%32] ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int mloc = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int64_t m = m0 + mloc;
      if (m >= me) continue;
      const int64_t r = r0 + m;
      const int64_t tok = row_token ? (int64_t)row_token[r] : r;
      const float sc = scales[tok];
      if constexpr (NW == 2) {
        const int nn = n0 + wn * 32 + lr;
        if (nn < N) {
          const float gv = acc[i][0][v] * sc, uv = acc[i][1][v] * sc;
          reinterpret_cast<uint16_t*>(out)[r * ldo + nn] = f32_to_bf16_rne(silu_mul(gv, uv));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nn = n0 + cb[j] + lr;
          if (nn < N) reinterpret_cast<float*>(out)[r * ldo + nn] = acc[i][j][v] * sc;
        }
      }
    }
  }
}

template <int BITS, int ABITS>
static hipError_t launch_p(const GemmArgs& a, int min_rows, hipStream_t stream) {
  const int E = a.offsets ? a.E : 1;
  const int ncol = a.n_w == 2 ? BNC / 2 : BNC;
  const int64_t mtiles = (a.n_rows + BM - 1) / BM + (a.offsets ? E : 0);
  dim3 grid((unsigned)((a.N + ncol - 1) / ncol), (unsigned)mtiles);
  if (a.n_w == 2)
    hipLaunchKernelGGL((mfma_prefill_kernel<BITS, ABITS, 2>), grid, dim3(256), 0, stream, a.codes,
                       a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, E, a.N, a.K,
                       min_rows, a.out, a.ldo);
  else
    hipLaunchKernelGGL((mfma_prefill_kernel<BITS, ABITS, 1>), grid, dim3(256), 0, stream, a.codes,
                       a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, E, a.N, a.K,
                       min_rows, a.out, a.ldo);
  return hipGetLastError();
}

hipError_t launch_mfma_prefill(const GemmArgs& a, int min_rows, hipStream_t stream) {
  switch (a.bits * 10 + (a.act_bits == 8 ? 8 : 4)) {
    case 44: return launch_p<4, 4>(a, min_rows, stream);
    case 48: return launch_p<4, 8>(a, min_rows, stream);
    case 34: return launch_p<3, 4>(a, min_rows, stream);
    case 38: return launch_p<3, 8>(a, min_rows, stream);
    case 24: return launch_p<2, 4>(a, min_rows, stream);
    case 28: return launch_p<2, 8>(a, min_rows, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cbq
