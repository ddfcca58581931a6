// Codebook GEMM, prefill path (many rows per expert: a dense contraction).
//
// Once an expert has enough rows, every dequantised weight is reused by many tokens
// and the work becomes MFMA-bound.  Weights are dequantised with the same per-row
// register tables as the decode path (CodeQuant2, Figure 4: a one-time table
// precomputation followed by lookups), and go straight into the B operand of
// 32x32x16 fp16 MFMAs: the 32 consecutive indices one lane loads per 64-channel step
// are exactly the 4 x 8 values its B fragments need, so weights never pass through
// LDS.  Activation codes are converted to fp16 once per step into LDS and shared by
// the four waves.  Products are exact (int codes x fp16 centroids); only the fp32
// summation order differs from the plain definition.
//
// Tile: up to 256 rows of one expert x 256 columns x 64 channels per step.  Wave w
// owns 64 columns (for the gate/up pair: 32 gate rows and the same 32 up rows, so
// the SwiGLU epilogue finds g and u in one lane) and all rows of the tile, held as
// up to 8 x 2 accumulators of 32x32 (256 AGPRs, one wave per SIMD).  Only the
// 32-row sub-tiles that hold rows are computed, so an expert's last tile wastes
// fewer than 32 rows.  A is double-buffered in LDS and the next step's loads are
// issued before this step's MFMAs.
//
// A tile is one column range x the y-th 256-row slice in expert order, skipping
// experts with at most min_rows rows (those go to the decode path).
#include "cbq_internal.hpp"

namespace cbq {

namespace {
constexpr int BM = 256;     // rows per tile
constexpr int BK = 64;      // channels per step
constexpr int LDW = BK + 8; // fp16 per LDS row (padding staggers the banks)
constexpr int MSUB = BM / 32;

}  // namespace

// Everything a tile needs after scheduling; shared by the per-NMS K-loops.
template <int BITS, int ABITS>
struct TileCtx {
  __amdgpu_buffer_rsrc_t wres[2];   // this expert's index block of each matrix
  __amdgpu_buffer_rsrc_t cres;      // the activation codes
  uint32_t wrow_off[2];             // byte offset of this lane's weight rows
  uint32_t crow_off;                // byte offset of this thread's activation row
  bool nvalid[2];
  int nrow[2];
  RowTable<BITS> tab[2];
  bool avalid;
  int K, g, nl, tid, rows;
};

template <int BITS, int ABITS, int NW, int NMS>
__device__ __forceinline__ void tile_run(const TileCtx<BITS, ABITS>& c, uint16_t (*As)[BM * LDW],
                                         const float* s_scale, const uint32_t* s_rowoff,
                                         __amdgpu_buffer_rsrc_t ores) {
  const int K = c.K, g = c.g, nl = c.nl, tid = c.tid;
  f32x16 acc[NMS][2];
#pragma unroll
  for (int i = 0; i < NMS; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][s][v] = 0.0f;
  const int nk = (K + BK - 1) / BK;
  // Raw loads run two steps ahead in a ring of two slots; the step loop is unrolled
  // by two so every slot index is a compile-time constant.
  uint32_t rw[2][2][BITS];     // [slot][matrix] raw indices
  uint32_t ra[2][ABITS * 2];   // [slot] raw activation codes
  uint32_t bdA[2][16], bdB[2][16];  // dequantised weights, alternating between steps
  f16x8 af[NMS];               // A fragments of the current 16-channel sub-step

  auto gload = [&](int kt, uint32_t (&w)[2][BITS], uint32_t* a) {
    const bool live = kt < nk;
    const int kb = kt * BK + g * 32;
    const bool kok = live && kb < K;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      buf_load<4 * BITS>(c.wres[s], (c.nvalid[s] && kok) ? c.wrow_off[s] + (uint32_t)(kb * BITS / 8) : kOffNone, w[s]);
    const int ka = kt * BK;
    const bool ok0 = live && c.avalid, ok1 = ok0 && ka + 32 < K;
    const uint32_t ab = c.crow_off + (uint32_t)(ka * ABITS / 8);
#pragma unroll
    for (int i = 0; i < ABITS / 4; ++i)       // first 32 codes
      buf_load<16>(c.cres, ok0 ? ab + 16 * i : kOffNone, a + 4 * i);
#pragma unroll
    for (int i = 0; i < ABITS / 4; ++i)       // second 32 codes
      buf_load<16>(c.cres, ok1 ? ab + 16 * (ABITS / 4 + i) : kOffNone, a + 4 * (ABITS / 4 + i));
  };
  auto astore = [&](int buf, const uint32_t* a) {
    uint32_t d[16];
    u32x4* ap = reinterpret_cast<u32x4*>(&As[buf][tid * LDW]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      codes32_to_f16<ABITS>(a + h * ABITS, d);
#pragma unroll
      for (int j = 0; j < 4; ++j) ap[h * 4 + j] = u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
    }
  };
  auto frag = [&](int buf, int kk, int ms) {
    return *reinterpret_cast<const f16x8*>(&As[buf][(ms * 32 + nl) * LDW + g * 32 + kk * 8]);
  };
  // One step: MFMAs on LDS buffer `buf` with weights `bd`, while step kt+1 is
  // prepared from ring slot (wn, an) into `bn` and the other LDS buffer, and ring slot
  // (wf, af_raw) is refilled with step kt+2.  Sub-steps 0-2 run before the barrier
  // (with the activation conversion and the first matrix's dequantisation); sub-step
  // 3 runs after it from fragments already in registers, so the next step's first
  // fragment reads (which need the barrier) overlap MFMAs instead of stalling.
  // Piece j (0..3) of one lane's 32-index dequantisation: indices 8j..8j+7.
  auto dq_piece = [&](const RowTable<BITS>& t, const uint32_t (&w)[BITS], uint32_t* d, int j) {
    if constexpr (BITS == 4) {
      dequant4(t, w[j], d + 4 * j);
    } else if constexpr (BITS == 3) {
      const uint32_t f = j == 0 ? w[0] : j == 1 ? __builtin_amdgcn_alignbit(w[1], w[0], 24)
                       : j == 2 ? __builtin_amdgcn_alignbit(w[2], w[1], 16) : (w[2] >> 8);
      dequant3(t, f, d + 4 * j);
    } else {
      uint32_t tmp[8];
      dequant2(t, w[j >> 1], tmp);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[4 * j + i] = tmp[4 * (j & 1) + i];
    }
  };
  // Piece p (0..7) of the activation conversion: codes 8p..8p+7 -> one 16-byte LDS store.
  auto a_piece = [&](int buf, const uint32_t* a, int p) {
    uint32_t d[4];
    const int h = p >> 2, j = p & 3;
    if constexpr (ABITS == 4) codes4_to_f16(a[h * 4 + j], d);
    else codes8_to_f16(a[h * 8 + 2 * j], a[h * 8 + 2 * j + 1], d);
    u32x4* ap = reinterpret_cast<u32x4*>(&As[buf][tid * LDW]);
    ap[p] = u32x4{d[0], d[1], d[2], d[3]};
  };
  // One step: MFMAs on LDS buffer `buf` with weights `bd`, while step kt+1 is
  // prepared from ring slot (wn, an) into `bn` and the other LDS buffer, and ring slot
  // (wf, af_raw) is refilled with step kt+2.  The preparation is cut into pieces that
  // are placed between the MFMA pairs in program order (scheduling fences keep them
  // there), so the vector ALU work issues while the matrix cores are busy.
  auto step = [&](int kt, int buf, uint32_t (&bd)[2][16], uint32_t (&bn)[2][16],
                  uint32_t (&wn)[2][BITS], uint32_t* an, uint32_t (&wf)[2][BITS], uint32_t* af_raw) {
    gload(kt + 2, wf, af_raw);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PRE = 3 * NMS;     // MFMA pairs before the barrier
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      const f16x8 b0 = as_f16x8(bd[0][4 * kk], bd[0][4 * kk + 1], bd[0][4 * kk + 2], bd[0][4 * kk + 3]);
      const f16x8 b1 = as_f16x8(bd[1][4 * kk], bd[1][4 * kk + 1], bd[1][4 * kk + 2], bd[1][4 * kk + 3]);
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        acc[ms][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b0, acc[ms][0], 0, 0, 0);
        acc[ms][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b1, acc[ms][1], 0, 0, 0);
        af[ms] = frag(buf, kk + 1, ms);
        const int i = kk * NMS + ms;
#pragma unroll
        for (int p = (12 * i + PRE - 1) / PRE; p < (12 * (i + 1) + PRE - 1) / PRE; ++p) {
          if (p < 8) a_piece(buf ^ 1, an, p);
          else dq_piece(c.tab[0], wn[0], bn[0], p - 8);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    {
      const f16x8 b0 = as_f16x8(bd[0][12], bd[0][13], bd[0][14], bd[0][15]);
      const f16x8 b1 = as_f16x8(bd[1][12], bd[1][13], bd[1][14], bd[1][15]);
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        acc[ms][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b0, acc[ms][0], 0, 0, 0);
        acc[ms][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b1, acc[ms][1], 0, 0, 0);
        af[ms] = frag(buf ^ 1, 0, ms);
#pragma unroll
        for (int p = (4 * ms + NMS - 1) / NMS; p < (4 * (ms + 1) + NMS - 1) / NMS; ++p)
          dq_piece(c.tab[1], wn[1], bn[1], p);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  gload(0, rw[0], ra[0]);
  gload(1, rw[1], ra[1]);
  astore(0, ra[0]);
#pragma unroll
  for (int s = 0; s < 2; ++s) dequant32<BITS>(c.tab[s], rw[0][s], bdA[s]);
  lds_barrier();
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) af[ms] = frag(0, 0, ms);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, 0, bdA, bdB, rw[1], ra[1], rw[0], ra[0]);       // prepare kt+1 from slot 1
    step(kt + 1, 1, bdB, bdA, rw[0], ra[0], rw[1], ra[1]);   // prepare kt+2 from slot 0
  }
  if (kt < nk) step(kt, 0, bdA, bdB, rw[1], ra[1], rw[0], ra[0]);

  // ---- epilogue: acc[ms][s][v] = D[ms*32 + 8*(v/4) + 4*g + v%4][nl] ----
  // Stores go through a buffer resource: rows past the tile (kOffNone) and columns
  // past N (kOffCol) carry out-of-range offsets and are dropped without branches.
  constexpr uint32_t ESZ = NW == 2 ? 2 : 4;
  uint32_t coff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) coff[s] = c.nvalid[s] ? (uint32_t)c.nrow[s] * ESZ : kOffCol;
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m0 = ms * 32 + 8 * q + 4 * g;            // rows m0 .. m0+3 of this lane
      const u32x4 ro = *reinterpret_cast<const u32x4*>(&s_rowoff[m0]);
      const f32x4 sc = *reinterpret_cast<const f32x4*>(&s_scale[m0]);
      if constexpr (NW == 2) {
        // bf16 h of rows m0..m0+3; lanes nl and nl ^ 1 hold columns 2p and 2p + 1 of
        // the same rows, so each pair trades one value per two rows and stores whole
        // dwords: the even lane rows m0 + j, the odd lane rows m0 + j + 1 (j = 0, 2).
        uint32_t hb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * q + j;
          const float gv = acc[ms][0][v] * sc[j], uv = acc[ms][1][v] * sc[j];
          hb[j] = f32_to_bf16_rne(silu_mul_fast(gv, uv));
        }
        const bool odd = (nl & 1) != 0;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const uint32_t send = odd ? hb[j] : hb[j + 1];
          const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
          const uint32_t word = odd ? (recv | (hb[j + 1] << 16)) : (hb[j] | (recv << 16));
          const uint32_t off = odd ? ro[j + 1] + coff[0] - 2u : ro[j] + coff[0];
          __builtin_amdgcn_raw_buffer_store_b32(word, ores, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * q + j;
#pragma unroll
          for (int s = 0; s < 2; ++s) buf_store_f32(ores, ro[j] + coff[s], acc[ms][s][v] * sc[j]);
        }
      }
    }
  }
}

template <int BITS, int ABITS, int NW>
__global__ void __launch_bounds__(256, 1)
mfma_prefill_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
                    GemmW w0, GemmW w1, int64_t n_rows, int E, int N, int K, int min_rows,
                    void* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDW];
  __shared__ __attribute__((aligned(16))) float s_scale[BM];
  __shared__ __attribute__((aligned(16))) uint32_t s_rowoff[BM];   // byte offset of each row in out
  __shared__ int64_t s_r0, s_me, s_m0;
  __shared__ int s_e;

  const int tid = threadIdx.x;
  // ---- workgroup -> tile (M-tile ty, column tile tcol) ----
  // The hardware deals workgroups to the 8 XCDs round-robin by linear id, so XCD x
  // gets ids x, x + 8, ...; those ids work through rounds of gridDim.x column tiles
  // of one M-tile each, so the column tiles of an M-tile (same activation rows) share
  // one L2.  Rounds 2P and 2P + 1 of XCD x take the M-tile pair (2s, 2s + 1),
  // s = 8P + (x + P) % 8: consecutive M-tiles (usually of one expert: same weights)
  // stay on one XCD, and the pair slot rotates with P to spread the work.  (The host
  // makes the M-tile slots a multiple of 16.)
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
  const uint32_t q = (lin / 8) / gridDim.x;
  const uint32_t P = q / 2;
  const int64_t ty = 2 * (8 * (int64_t)P + (lin % 8 + P) % 8) + (q & 1);
  const int tcol = (int)((lin / 8) % gridDim.x);
  // ---- M-tile -> (expert, first row): wave 0 scans the experts' tile counts ----
  if (tid < 64) {
    if (!offsets) {
      if (tid == 0) {
        const bool ok = ty * BM < n_rows;
        s_e = ok ? 0 : -1; s_r0 = 0; s_me = n_rows; s_m0 = ty * BM;
      }
    } else {
      if (tid == 0) s_e = -1;
      int64_t before = 0;                            // tiles of earlier 64-expert chunks
      for (int base = 0; base < E; base += 64) {
        const int ex = base + tid;
        int64_t a = 0, cnt = 0;
        if (ex < E) { a = offsets[ex]; cnt = offsets[ex + 1] - a; }
        const int64_t nt = cnt > min_rows ? (cnt + BM - 1) / BM : 0;
        int64_t incl = nt;                           // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int64_t o = __shfl_up(incl, d);
          if (tid >= d) incl += o;
        }
        const int64_t lo = before + incl - nt;
        if (nt > 0 && ty >= lo && ty < lo + nt) {
          s_e = ex; s_r0 = a; s_me = cnt; s_m0 = (ty - lo) * BM;
        }
        before += __shfl(incl, 63);
        if (before > ty) break;
      }
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int64_t r0 = s_r0, me = s_me, m0 = s_m0;
  const int rows = (int)((me - m0) < BM ? (me - m0) : BM);
  const int nms = (rows + 31) >> 5;                  // 32-row sub-tiles holding rows

  TileCtx<BITS, ABITS> c;
  c.K = K;
  c.tid = tid;
  c.rows = rows;
  // ---- activation loader: thread t owns tile row t ----
  c.avalid = tid < rows;
  int64_t atok = 0;
  constexpr uint32_t ESZ = NW == 2 ? 2 : 4;
  s_rowoff[tid] = kOffNone;
  s_scale[tid] = 0.0f;
  if (c.avalid) {
    const int64_t r = r0 + m0 + tid;
    atok = row_token ? (int64_t)row_token[r] : r;
    s_scale[tid] = scales[atok];
    s_rowoff[tid] = (uint32_t)(r * ldo * ESZ);
  }
  c.cres = make_rsrc(codes, 0x7FFFFFFFu);
  c.crow_off = (uint32_t)(atok * ((int64_t)K * ABITS / 8));

  // ---- weight rows of this lane ----
  const int lane = tid & 63, wave = tid >> 6;
  c.nl = lane & 31;
  c.g = lane >> 5;
  constexpr int NCOL = (NW == 2) ? 128 : 256;        // weight rows per matrix per tile
  const int n0 = tcol * NCOL;
  if constexpr (NW == 2) { c.nrow[0] = c.nrow[1] = n0 + wave * 32 + c.nl; }   // gate, up
  else { c.nrow[0] = n0 + wave * 64 + c.nl; c.nrow[1] = c.nrow[0] + 32; }
  constexpr int L = 1 << BITS;
  const int64_t row_bytes = (int64_t)K * BITS / 8;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const GemmW& W = (NW == 2 && s == 1) ? w1 : w0;
    c.nvalid[s] = c.nrow[s] < N;
    const int64_t rowi = (int64_t)e * N + (c.nvalid[s] ? c.nrow[s] : 0);
    c.tab[s].load(W.codebook + rowi * L);
    c.wres[s] = make_rsrc(W.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
    c.wrow_off[s] = (uint32_t)((c.nvalid[s] ? c.nrow[s] : 0) * row_bytes);
  }

  // output buffer: every row of this call (n_rows) x ldo elements
  const __amdgpu_buffer_rsrc_t ores = make_rsrc(out, (uint32_t)(n_rows * ldo * ESZ));
  switch (nms) {
    case 1: tile_run<BITS, ABITS, NW, 1>(c, As, s_scale, s_rowoff, ores); break;
    case 2: tile_run<BITS, ABITS, NW, 2>(c, As, s_scale, s_rowoff, ores); break;
    case 3: tile_run<BITS, ABITS, NW, 3>(c, As, s_scale, s_rowoff, ores); break;
    case 4: tile_run<BITS, ABITS, NW, 4>(c, As, s_scale, s_rowoff, ores); break;
    case 5: tile_run<BITS, ABITS, NW, 5>(c, As, s_scale, s_rowoff, ores); break;
    case 6: tile_run<BITS, ABITS, NW, 6>(c, As, s_scale, s_rowoff, ores); break;
    case 7: tile_run<BITS, ABITS, NW, 7>(c, As, s_scale, s_rowoff, ores); break;
    default: tile_run<BITS, ABITS, NW, 8>(c, As, s_scale, s_rowoff, ores); break;
  }
}

template <int BITS, int ABITS>
static hipError_t launch_p(const GemmArgs& a, int min_rows, hipStream_t stream) {
  const int E = a.offsets ? a.E : 1;
  const int ncol = a.n_w == 2 ? 128 : 256;
  int64_t mtiles = (a.n_rows + BM - 1) / BM + (a.offsets ? E : 0);   // M-tile slots
  mtiles = (mtiles + 15) / 16 * 16;                  // a multiple of 16 (XCD pairs)
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
