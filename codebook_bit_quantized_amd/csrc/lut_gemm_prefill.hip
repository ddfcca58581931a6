// Codebook GEMM, prefill path (many rows per expert: a dense contraction).
//
// Once an expert has enough rows, every dequantised weight is reused by many tokens
// and the work becomes MFMA-bound.  Weights are dequantised with the same per-row
// register tables as the decode path (CodeQuant2, Figure 4: a table built once, then
// read instead of multiplying), and go straight into the B operand of
// 32x32x16 fp16 MFMAs: the 32 consecutive indices one lane loads per 64-channel step
// are exactly the 4 x 8 values its B fragments need, so weights never pass through
// LDS.  Activation codes are converted to fp16 once per step into LDS and shared by
// the four waves.  Products are exact (int codes x fp16 centroids); only the fp32
// summation order differs from the plain definition.
//
// Tile: up to BM rows of one expert x 256 columns x 64 channels per step, four waves.
// Wave w owns 64 columns (for the gate/up pair: 32 gate rows and the same 32 up rows,
// so the SwiGLU epilogue finds g and u in one lane) and all rows of the tile, held as
// up to BM/32 x 2 accumulators of 32x32.  For 2- and 3-bit codebooks BM = 128: 128
// accumulator registers, 256 registers a wave, so two workgroups share each CU (two
// waves per SIMD) and one workgroup's epilogue, prologue and waits overlap the other's
// MFMAs.  For 4-bit codebooks, whose dequantisation is the heaviest vector work, BM =
// 256 spreads each dequantised weight over twice the rows (one workgroup a CU).  Only
// the 32-row sub-tiles that hold rows are computed, so an expert's last tile wastes
// fewer than 32 rows.  A is double-buffered in LDS (converted by one or two threads per
// row) and the next step's loads are issued before this step's MFMAs.
//
// A tile is one column range x one BM-row slice of an expert, skipping experts with at
// most min_rows rows (those go to the decode path); an expert's slices go to the XCDs in
// runs that share its weights in one L2.
#include <algorithm>

#include "cbq_internal.hpp"

namespace cbq {

namespace {
// Rows per tile: 256 (one thread per row, one workgroup a CU) for 4-bit codebooks, whose
// dequantisation is the heaviest vector work and is best spread over the most rows;
// 128 (two threads per row, two workgroups a CU) for 2- and 3-bit codebooks.
template <int BITS>
constexpr int tile_rows() { return BITS == 4 ? 256 : 128; }
constexpr int XG = 4;       // consecutive M-tiles kept on one XCD
static_assert(XG == 1 || XG == 2 || XG == 4, "the kernel counts the padding of runs of 2 and 4 only");
constexpr int BK = 64;      // channels per step
constexpr int LDW = BK + 8; // fp16 per LDS row (padding staggers the banks)

}  // namespace

// Everything a tile needs after scheduling; shared by the per-NMS K-loops.  LT: the
// weights are looked up in LDS pair tables (2- and 3-bit codebooks); otherwise in the
// per-row register tables.
template <int BITS, int ABITS, bool LT>
struct TileCtx {
  __amdgpu_buffer_rsrc_t wres[2];   // this expert's index block of each matrix
  __amdgpu_buffer_rsrc_t cres;      // the activation codes
  uint32_t wrow_off[2];             // byte offset of this lane's first 32 indices of each matrix
  uint32_t wstep;                   // bytes between a lane's index slices of consecutive steps
  uint32_t crow_off;                // byte offset of this thread's activation row
  bool nvalid[2];
  int nrow[2];
  RowTable<BITS> tab[2];            // register tables (unused with LT)
  const uint32_t* ptab;             // LDS pair tables (LT)
  uint32_t trow[2];                 // dword of entry 0 of this lane's row in each table
  bool avalid;
  int K, g, nl, tid, rows;
  // K split of the gate/up pair (4-bit tiles): the tile stores its unscaled fp32 sums of g
  // and u at byte offset poff[s] (+ the row's offset) of the workspace instead of h
  bool partial = false;
  uint32_t poff[2];
};

// NS: 32-column weight slots per wave (2; 1 for a single matrix in 128-column tiles).
template <int BITS, int ABITS, int NW, int NMS, bool LT, bool BLK, int BM, int NS>
__device__ __forceinline__ void tile_run(const TileCtx<BITS, ABITS, LT>& c, uint16_t (*As)[BM * LDW],
                                         const float* s_scale, const uint32_t* s_rowoff,
                                         __amdgpu_buffer_rsrc_t ores) {
  const int K = c.K, g = c.g, nl = c.nl, tid = c.tid;
  constexpr int TPR = 256 / BM;            // threads per tile row (1 or 2)
  constexpr int NPA = 8 / TPR;             // activation pieces per thread and step
  static_assert(NS == 2 || NW == 1, "the gate/up pair takes both slots");
  f32x16 acc[NMS][NS];
#pragma unroll
  for (int i = 0; i < NMS; ++i)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][s][v] = 0.0f;
  const int nk = (K + BK - 1) / BK;
  // Raw loads run two steps ahead in a ring of two slots; the step loop is unrolled
  // by two so every slot index is a compile-time constant.
  uint32_t rw[2][NS][BITS];    // [ring slot][weight slot] raw indices
  uint32_t ra[2][ABITS * 2 / TPR];   // [slot] raw activation codes (this thread's part of its row)
  uint32_t bdA[NS][16], bdB[NS][16];  // dequantised weights, alternating between steps
  f16x8 af[NMS];               // A fragments of the current 16-channel sub-step

  auto gload = [&](int kt, uint32_t (&w)[NS][BITS], uint32_t* a) {
    const bool live = kt < nk;
    const int kb = kt * BK + g * 32;
    const bool kok = live && kb < K;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      buf_load<4 * BITS>(c.wres[s], (c.nvalid[s] && kok) ? c.wrow_off[s] + (uint32_t)kt * c.wstep : kOffNone, w[s]);
#pragma unroll
    for (int hh = 0; hh < 2 / TPR; ++hh) {    // this thread's 32-code halves of the step
      const int ka = kt * BK + 32 * ((tid % TPR) + hh);
      const bool okh = live && c.avalid && ka < K;
      const uint32_t ab = c.crow_off + (uint32_t)(ka * ABITS / 8);
#pragma unroll
      for (int i = 0; i < ABITS / 4; ++i)
        buf_load<16>(c.cres, okh ? ab + 16 * i : kOffNone, a + ABITS * hh + 4 * i);
    }
  };
  auto astore = [&](int buf, const uint32_t* a) {
    uint32_t d[16];
    u32x4* ap = reinterpret_cast<u32x4*>(&As[buf][(tid / TPR) * LDW]) + 4 * (tid % TPR);
#pragma unroll
    for (int h = 0; h < 2 / TPR; ++h) {
      codes32_to_f16_ord<ABITS, LT>(a + h * ABITS, d);
#pragma unroll
      for (int j = 0; j < 4; ++j) ap[h * 4 + j] = u32x4{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
    }
  };
  auto frag = [&](int buf, int kk, int ms) {
    return *reinterpret_cast<const f16x8*>(&As[buf][(ms * 32 + nl) * LDW + g * 32 + kk * 8]);
  };
  // Piece j (0..3) of one lane's 32-index dequantisation of matrix slot s: indices 8j..8j+7.
  auto dq_piece = [&](int s, const uint32_t (&w)[BITS], uint32_t* d, int j) {
    const RowTable<BITS>& t = c.tab[s];
    if constexpr (LT) {
      pair_lookup8<BITS, 32, BLK>(c.ptab, c.trow[s], w, j, d + 4 * j);
    } else if constexpr (BITS == 4) {
      dequant4(t, w[j], d + 4 * j);
    } else if constexpr (BITS == 3 && BLK) {
      dequant3_blk(t, j < 3 ? w[j] : group3_blk(w), d + 4 * j);
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
  // Piece p (0 .. NPA-1) of this thread's conversion: codes 8p..8p+7 of its 64 / TPR ->
  // one 16-byte LDS store.
  auto a_piece = [&](int buf, const uint32_t* a, int p) {
    uint32_t d[4];
    codes8_group<ABITS, LT>(a + (p >> 2) * ABITS, p & 3, d);
    u32x4* ap = reinterpret_cast<u32x4*>(&As[buf][(tid / TPR) * LDW]) + 4 * (tid % TPR);
    ap[p] = u32x4{d[0], d[1], d[2], d[3]};
  };
  // One step: MFMAs on LDS buffer `buf` with weights `bd`, while step kt+1 is
  // prepared from ring slot (wn, an) into `bn` and the other LDS buffer, and ring slot
  // (wf, af_raw) is refilled with step kt+2.  The preparation is cut into NPA + 4 pieces
  // (activation conversion, then the first matrix's dequantisation) placed between the
  // MFMA pairs of sub-steps 0-2 in program order (scheduling fences keep them there), so
  // the vector ALU work issues while the matrix cores are busy.  Sub-step 3 runs after
  // the barrier from fragments already in registers, beside the second matrix's
  // dequantisation, so the next step's first fragment reads (which need the barrier)
  // overlap MFMAs instead of stalling.
  auto step = [&](int kt, int buf, uint32_t (&bd)[NS][16], uint32_t (&bn)[NS][16],
                  uint32_t (&wn)[NS][BITS], uint32_t* an, uint32_t (&wf)[NS][BITS], uint32_t* af_raw) {
    gload(kt + 2, wf, af_raw);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PRE = 3 * NMS;     // MFMA pairs before the barrier
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      const f16x8 b0 = as_f16x8(bd[0][4 * kk], bd[0][4 * kk + 1], bd[0][4 * kk + 2], bd[0][4 * kk + 3]);
      const f16x8 b1 = as_f16x8(bd[NS - 1][4 * kk], bd[NS - 1][4 * kk + 1], bd[NS - 1][4 * kk + 2],
                                bd[NS - 1][4 * kk + 3]);
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        acc[ms][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b0, acc[ms][0], 0, 0, 0);
        if constexpr (NS == 2)
          acc[ms][NS - 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b1, acc[ms][NS - 1], 0, 0, 0);
        af[ms] = frag(buf, kk + 1, ms);
        const int i = kk * NMS + ms;
        constexpr int NP = NPA + 4;
#pragma unroll
        for (int p = (NP * i + PRE - 1) / PRE; p < (NP * (i + 1) + PRE - 1) / PRE; ++p) {
          if (p < NPA) a_piece(buf ^ 1, an, p);
          else dq_piece(0, wn[0], bn[0], p - NPA);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    {
      const f16x8 b0 = as_f16x8(bd[0][12], bd[0][13], bd[0][14], bd[0][15]);
      const f16x8 b1 = as_f16x8(bd[NS - 1][12], bd[NS - 1][13], bd[NS - 1][14], bd[NS - 1][15]);
#pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        acc[ms][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b0, acc[ms][0], 0, 0, 0);
        if constexpr (NS == 2)
          acc[ms][NS - 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ms], b1, acc[ms][NS - 1], 0, 0, 0);
        af[ms] = frag(buf ^ 1, 0, ms);
        if constexpr (NS == 2) {
#pragma unroll
          for (int p = (4 * ms + NMS - 1) / NMS; p < (4 * (ms + 1) + NMS - 1) / NMS; ++p)
            dq_piece(NS - 1, wn[NS - 1], bn[NS - 1], p);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  gload(0, rw[0], ra[0]);
  gload(1, rw[1], ra[1]);
  astore(0, ra[0]);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (LT) pair_lookup32<BITS, 32, BLK>(c.ptab, c.trow[s], rw[0][s], bdA[s]);
    else dequant32<BITS, BLK>(c.tab[s], rw[0][s], bdA[s]);
  }
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
  uint32_t coff[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) coff[s] = c.nvalid[s] ? (uint32_t)c.nrow[s] * ESZ : kOffCol;
#pragma unroll
  for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m0 = ms * 32 + 8 * q + 4 * g;            // rows m0 .. m0+3 of this lane
      const u32x4 ro = *reinterpret_cast<const u32x4*>(&s_rowoff[m0]);
      const f32x4 sc = *reinterpret_cast<const f32x4*>(&s_scale[m0]);
      bool part = false;
      if constexpr (NW == 2 && BM == 256) part = c.partial;
      if (part) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int s = 0; s < 2; ++s) buf_store_f32(ores, ro[j] + c.poff[s], acc[ms][s][4 * q + j]);
      } else if constexpr (NW == 2) {
        // bf16 h of rows m0..m0+3; lanes nl and nl ^ 1 hold columns 2p and 2p + 1 of
        // the same rows, so each pair trades one value per two rows and stores whole
        // dwords: the even lane rows m0 + j, the odd lane rows m0 + j + 1 (j = 0, 2).
        uint32_t hb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * q + j;
          const float gv = acc[ms][0][v] * sc[j], uv = acc[ms][NS - 1][v] * sc[j];
          hb[j] = f32_to_bf16_rne(silu_mul(gv, uv));
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
          for (int s = 0; s < NS; ++s) buf_store_f32(ores, ro[j] + coff[s], acc[ms][s][v] * sc[j]);
        }
      }
    }
  }
}

// BLK: 3-bit indices in the blocked layout's re-encoded units (cbq_prepack_weights).
// NS: 32-column weight slots per wave (1: a single matrix in 128-column tiles, twice the
// workgroups and half the accumulators, so two workgroups share each CU at BM = 256 too).
template <int BITS, int ABITS, int NW, bool LT, bool BLK, int NS, int BM = tile_rows<BITS>()>
__global__ void __launch_bounds__(256, (BM == 128 || NS == 1) ? 2 : 1)
mfma_prefill_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
                    GemmW w0, GemmW w1, int64_t n_rows, int E, int N, int K, int min_rows,
                    int blocked, void* __restrict__ out, int64_t ldo, float* __restrict__ ws,
                    int tc0) {
  // K split z of gridDim.z (single matrix): z = 0 writes out, z >= 1 writes its partial
  // sums to ws + (z - 1) * n_rows * N (pitch N); a reduction adds them after.  The gate/up
  // pair with 256-row tiles, tc0 >= 0: column tiles tcol >= tc0 split in two, in calls of at
  // most 8 M-tiles (one per XCD) only; the grid has ncol - tc0 extra column tiles, right of
  // the ncol real ones, for the second halves.  Both halves write their unscaled sums of g
  // and u to ws, planes [half][g or u][n_rows][N - 128 tc0], and mfma_swiglu_reduce_kernel
  // forms h from them.
  // LDS pair tables: per wave, two matrix slots of 32 rows, NE entries each
  constexpr int NE = LT ? PairTab<BITS>::NE : 1;
  __shared__ __attribute__((aligned(16))) uint32_t Tab[LT ? 4 * 2 * NE * 32 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDW];
  __shared__ __attribute__((aligned(16))) float s_scale[BM];
  __shared__ __attribute__((aligned(16))) uint32_t s_rowoff[BM];   // byte offset of each row in out
  __shared__ int64_t s_r0, s_me, s_m0, s_ttot;
  __shared__ uint32_t s_pad;
  __shared__ uint64_t s_nruns;
  __shared__ int s_e;

  const int tid = threadIdx.x;
  // ---- workgroup -> (M-tile, column tile tcol) ----
  // The hardware deals workgroups to the 8 XCDs round-robin by linear id, so XCD x
  // gets ids x, x + 8, ...; those ids work through rounds of gridDim.x column tiles
  // of one M-tile each, so the column tiles of an M-tile (same activation rows) share
  // one L2.  Each expert's M-tiles are cut into runs of G consecutive tiles (its last
  // run may be shorter; no run spans two experts), and rounds G*P .. G*P + G - 1 of
  // XCD x take the tiles of run 8P + x: one L2 fetches an expert's weights once per run.
  // G is the largest power of two <= XG with 8G <= T, the call's M-tile count (counted
  // first), so a call of few tiles still spreads them over all eight XCDs, and with at
  // most T / 4 slots of padding.  Rounds past the end of a short run, or past the call's
  // last run, have no work.  (The host makes the slots a multiple of 8 G' for a power of
  // two G' >= G and leaves room for a partial run per expert.)
  if (tid < 64) {
    // the call's M-tiles, the slots that runs of 2 and of 4 tiles would leave empty at
    // the end of each expert (16-bit fields; they only steer the run length below), and
    // the call's runs of 2 and of 4 tiles (32-bit fields)
    int64_t tot = 0;
    uint32_t pad = 0;
    uint64_t nruns = 0;
    if (!offsets) {
      tot = n_rows > min_rows ? (n_rows + BM - 1) / BM : 0;
      pad = (uint32_t)((-tot) & 1) | ((uint32_t)((-tot) & 3) << 16);
    } else {
      for (int base = 0; base < E; base += 64) {
        const int ex = base + tid;
        int64_t cnt = 0;
        if (ex < E) cnt = offsets[ex + 1] - offsets[ex];
        int64_t nt = cnt > min_rows ? (cnt + BM - 1) / BM : 0;
        uint32_t pd = (uint32_t)((-nt) & 1) | ((uint32_t)((-nt) & 3) << 16);
        uint64_t nr = (uint64_t)((nt + 1) >> 1) | ((uint64_t)((nt + 3) >> 2) << 32);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          nt += __shfl_xor(nt, d);
          pd += __shfl_xor(pd, d);
          nr += __shfl_xor(nr, d);
        }
        tot += nt;
        pad += pd;
        nruns += nr;
      }
    }
    if (tid == 0) { s_ttot = tot; s_pad = pad; s_nruns = nruns; }
  }
  __syncthreads();
  const int64_t ttot = s_ttot;
  uint32_t G = 1;                                    // a power of two, so it divides the
  while (2 * G <= XG && 8 * 2 * G <= ttot) G *= 2;   // rounds per XCD
  // shorter runs where padding each expert's last run would leave more than a quarter
  // of the slots empty (experts of one or two tiles): empty slots between the busy ones
  // would crowd the busy workgroups onto fewer CUs.  (Any power of two up to the
  // host's bound is a valid choice; this one only steers the placement.)
  while (G > 1 && (int64_t)(G == 4 ? s_pad >> 16 : s_pad & 0xFFFFu) > ttot / 4) G >>= 1;
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
  const uint32_t q = (lin / 8) / gridDim.x;
  const uint32_t P = q / G;
  const uint32_t x8 = lin % 8;                       // the XCD
  int64_t run = 8 * (int64_t)P + x8;                 // run of this slot, before the exchange
  const int64_t rr = q % G;                          // tile of the run
  // Inside each whole block of 16 runs, XCD x takes runs 8 (x / 4) + (x mod 4) + 4a in its
  // rounds a = 0, 1 of the block, so the block's two aligned groups of 8 consecutive runs
  // each stay on four XCDs: an expert of 8 runs (the shared experts, which come first in
  // the scan below) is fetched by four L2s instead of eight, and every XCD still takes two
  // of its runs.  (Groups kept on XCD pairs fetched 2 MB less but gave four XCDs all the
  // shared runs, and the gate/up 3.5 % more time.)  Slots past the last whole block keep
  // the plain order, so every run of the call has a slot.
  if (offsets) {
    const uint64_t nr = s_nruns;
    const int64_t runs = G == 1 ? ttot : G == 2 ? (int64_t)(uint32_t)nr : (int64_t)(nr >> 32);
    if (run < runs / 16 * 16)
      run = (run & ~(int64_t)15) + 8 * (x8 >> 2) + 4 * ((run >> 3) & 1) + (x8 & 3);
  }
  int tcol = (int)((lin / 8) % gridDim.x);
  // The gate/up pair's tail split: with at most 8 M-tiles each XCD holds at most one, and
  // works through its column tiles in rounds of its CUs; the host picks tc0 so that the
  // column tiles of the last, partly filled round split in K and fill it.  The second
  // halves follow the first ones in the XCD's order, ahead of the slots with no work.
  bool tsplit = false;
  int half = 0;
  if constexpr (NW == 2 && BM == 256) {
    const int ncol = (N + 127) / 128;
    if (tc0 >= 0 && tcol >= tc0) {
      if (ttot > 8) {
        if (tcol >= ncol) return;                    // no split: no second halves
      } else {
        tsplit = true;
        if (tcol >= ncol) { half = 1; tcol -= ncol - tc0; }
      }
    }
  }
  // ---- (run, tile of the run) -> (expert, first row): wave 0 scans the experts' run counts ----
  if (tid < 64) {
    if (!offsets) {
      if (tid == 0) {                                // one matrix of n_rows rows: runs are contiguous
        const int64_t ty = run * G + rr;
        const bool ok = ty * BM < n_rows;
        s_e = ok ? 0 : -1; s_r0 = 0; s_me = n_rows; s_m0 = ty * BM;
      }
    } else {
      if (tid == 0) s_e = -1;
      int64_t before = 0;                            // runs of earlier 64-expert chunks
      for (int base = 0; base < E; base += 64) {
        const int ex = E - 1 - (base + tid);         // the last experts (shared) first
        int64_t a = 0, cnt = 0;
        if (ex >= 0) { a = offsets[ex]; cnt = offsets[ex + 1] - a; }
        const int64_t nt = cnt > min_rows ? (cnt + BM - 1) / BM : 0;
        const int64_t nr = (nt + G - 1) / G;         // the expert's runs
        int64_t incl = nr;                           // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int64_t o = __shfl_up(incl, d);
          if (tid >= d) incl += o;
        }
        const int64_t lo = before + incl - nr;
        if (nr > 0 && run >= lo && run < lo + nr) {
          const int64_t tile = (run - lo) * G + rr;  // past the expert's last tile: no work
          if (tile < nt) { s_e = ex; s_r0 = a; s_me = cnt; s_m0 = tile * BM; }
        }
        before += __shfl(incl, 63);
        if (before > run) break;
      }
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int64_t r0 = s_r0, me = s_me, m0 = s_m0;
  const int rows = (int)((me - m0) < BM ? (me - m0) : BM);
  const int nms = (rows + 31) >> 5;                  // 32-row sub-tiles holding rows
  // this split's channels [k0, k0 + Kl): whole 64-channel steps, the last split takes the
  // tail (single matrix only; the gate/up pair is never split, and its code keeps none of this)
  int split = 0, k0 = 0, Kl = K;
  int64_t pitch = ldo;
  if constexpr (NW == 1) {
    const int nsplit = (int)gridDim.z;
    split = (int)blockIdx.z;
    const int sps = ((K + BK - 1) / BK + nsplit - 1) / nsplit;
    k0 = split * sps * BK;
    Kl = K - k0 < sps * BK ? K - k0 : sps * BK;
    if (Kl <= 0) return;                             // uniform over the workgroup
    if (split > 0) pitch = N;
  } else if constexpr (BM == 256) {
    if (tsplit) {                                    // two halves; the host splits K >= 2048 only
      split = half;
      const int sps = ((K + BK - 1) / BK + 1) / 2;
      k0 = split * sps * BK;
      Kl = K - k0 < sps * BK ? K - k0 : sps * BK;
    }
  }

  TileCtx<BITS, ABITS, LT> c;
  c.K = Kl;
  c.tid = tid;
  c.rows = rows;
  // ---- activation loader: threads 2i and 2i + 1 own the two 32-code halves of tile row i ----
  const int arow = tid / (256 / BM);                 // one or two threads per tile row
  c.avalid = arow < rows;
  int64_t atok = 0;
  constexpr uint32_t ESZ = NW == 2 ? 2 : 4;
  const int64_t rowb = tsplit ? (int64_t)(N - tc0 * 128) * 4 : pitch * ESZ;   // bytes between rows
  if (tid < BM) {                                    // thread t < BM: row t's scale and output offset
    uint32_t ro = kOffNone;
    float sv = 0.0f;
    if (tid < rows) {
      const int64_t r = r0 + m0 + tid;
      const int64_t tk = row_token ? (int64_t)row_token[r] : r;
      sv = scales[tk];
      ro = (uint32_t)(r * rowb);
    }
    s_rowoff[tid] = ro;
    s_scale[tid] = sv;
  }
  if (c.avalid) {
    const int64_t r = r0 + m0 + arow;
    atok = row_token ? (int64_t)row_token[r] : r;
  }
  c.cres = make_rsrc(codes, 0x7FFFFFFFu);
  c.crow_off = (uint32_t)(atok * ((int64_t)K * ABITS / 8) + (int64_t)k0 * ABITS / 8);

  // ---- weight rows of this lane ----
  const int lane = tid & 63, wave = tid >> 6;
  c.nl = lane & 31;
  c.g = lane >> 5;
  constexpr int NCOL = (NW == 2) ? 128 : 128 * NS;   // weight rows per matrix per tile
  const int n0 = tcol * NCOL;
  if constexpr (NW == 2) { c.nrow[0] = c.nrow[1] = n0 + wave * 32 + c.nl; }   // gate, up
  else if constexpr (NS == 2) { c.nrow[0] = n0 + wave * 64 + c.nl; c.nrow[1] = c.nrow[0] + 32; }
  else { c.nrow[0] = c.nrow[1] = n0 + wave * 32 + c.nl; }
  constexpr int L = 1 << BITS;
  // bytes per row of the expert's index block (rows layout: each row's bitstream; blocked
  // layout: 16-row x 128-channel tiles of 256*BITS bytes, a step of 64 channels being half
  // a tile, so 128*BITS bytes apart in either half)
  const int64_t row_bytes = index_row_bytes(K, BITS, blocked != 0);
  c.wstep = blocked ? 128u * BITS : 8u * BITS;
  c.ptab = Tab;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const GemmW& W = (NW == 2 && s == 1) ? w1 : w0;
    c.nvalid[s] = c.nrow[s] < N;
    const int64_t rowi = (int64_t)e * N + (c.nvalid[s] ? c.nrow[s] : 0);
    if constexpr (LT) {
      // this wave's tables only hold its own rows: built and read by the wave itself,
      // so no barrier is needed (a wave's LDS accesses complete in order)
      uint32_t cb[L / 2];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(W.codebook + rowi * L);
#pragma unroll
      for (int i = 0; i < L / 2; ++i) cb[i] = src[i];
      c.trow[s] = (uint32_t)((wave * 2 + s) * NE * 32 + c.nl);
      pair_build<BITS, 2, 32>(Tab, c.trow[s], cb, c.g);
    } else {
      c.tab[s].load(W.codebook + rowi * L);
    }
    c.wres[s] = make_rsrc(W.idx + (int64_t)e * N * row_bytes, (uint32_t)(N * row_bytes));
    const int nr = c.nvalid[s] ? c.nrow[s] : 0;
    c.wrow_off[s] = (blocked ? (uint32_t)((nr & ~15) * row_bytes) + (uint32_t)((c.g * 16 + (nr & 15)) * 4 * BITS)
                             : (uint32_t)(nr * row_bytes) + (uint32_t)(c.g * 4 * BITS)) +
                    (uint32_t)(k0 / BK) * c.wstep;
  }

  // output buffer: every row of this call (n_rows) x ldo elements, or this split's slice
  // of the partial sums (n_rows x N), or the gate/up pair's four partial planes
  __amdgpu_buffer_rsrc_t ores;
  if (tsplit) {
    const int64_t plane = n_rows * (int64_t)(N - tc0 * 128) * 4;
    ores = make_rsrc(ws, (uint32_t)(4 * plane));
    c.partial = true;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      c.poff[s] = c.nvalid[s] ? (uint32_t)((2 * split + s) * plane + (int64_t)(c.nrow[s] - tc0 * 128) * 4)
                              : kOffCol;
  } else if (split == 0) {
    ores = make_rsrc(out, (uint32_t)(n_rows * ldo * ESZ));
  } else {
    ores = make_rsrc(ws + (int64_t)(split - 1) * n_rows * N, (uint32_t)(n_rows * N * 4));
  }
  switch (nms) {
    case 1: tile_run<BITS, ABITS, NW, 1, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
    case 2: tile_run<BITS, ABITS, NW, 2, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
    case 3: tile_run<BITS, ABITS, NW, 3, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
    case 4: tile_run<BITS, ABITS, NW, 4, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
    default:
      if constexpr (BM == 256) {
        switch (nms) {
          case 5: tile_run<BITS, ABITS, NW, 5, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
          case 6: tile_run<BITS, ABITS, NW, 6, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
          case 7: tile_run<BITS, ABITS, NW, 7, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
          default: tile_run<BITS, ABITS, NW, 8, LT, BLK, BM, NS>(c, As, s_scale, s_rowoff, ores); break;
        }
      }
      break;
  }
}

// Adds the partial sums of K splits 1 .. nsplit-1 (ws, pitch N) to split 0's rows in out,
// in split order, for the rows the MFMA path computed: rows of experts with more than
// min_rows rows.  One row per workgroup pass.
__global__ void __launch_bounds__(256)
mfma_split_reduce_kernel(float* __restrict__ out, int64_t ldo, const float* __restrict__ ws,
                         int nsplit, int64_t n_rows, int N, const int32_t* __restrict__ offsets,
                         int E, int min_rows) {
  for (int64_t r = blockIdx.x; r < n_rows; r += gridDim.x) {
    if (offsets) {
      // the expert holding row r: the last e with offsets[e] <= r
      int lo = 0, hi = E;                            // offsets[lo] <= r < offsets[hi] if inside
      if (r < offsets[0] || r >= offsets[E]) continue;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid;
      }
      if (offsets[lo + 1] - offsets[lo] <= min_rows) continue;
    }
    float* o = out + r * ldo;
    for (int n = threadIdx.x; n < N; n += blockDim.x) {
      float v = o[n];
      for (int s = 1; s < nsplit; ++s) v += ws[((int64_t)(s - 1) * n_rows + r) * N + n];
      o[n] = v;
    }
  }
}

// h for the gate/up pair's split column tiles (columns c0 .. N-1): g and u are the sums of
// both K halves' partials (lower half first), then scaled and passed through SwiGLU as in
// the kernel's own epilogue.  Runs only where the kernel split, i.e. in calls of at most 8
// M-tiles (counted again here from the offsets), and only on rows the MFMA path computed.
__global__ void __launch_bounds__(256)
mfma_swiglu_reduce_kernel(uint16_t* __restrict__ out, int64_t ldo, const float* __restrict__ ws,
                          int64_t n_rows, int N, int c0, const float* __restrict__ scales,
                          const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets,
                          int E, int min_rows, int bm) {
  __shared__ int64_t s_tot;
  if (threadIdx.x < 64) {
    int64_t tot = 0;
    if (!offsets) {
      tot = n_rows > min_rows ? (n_rows + bm - 1) / bm : 0;
    } else {
      for (int base = 0; base < E; base += 64) {
        const int ex = base + (int)threadIdx.x;
        const int64_t cnt = ex < E ? offsets[ex + 1] - offsets[ex] : 0;
        int64_t nt = cnt > min_rows ? (cnt + bm - 1) / bm : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) nt += __shfl_xor(nt, d);
        tot += nt;
      }
    }
    if (threadIdx.x == 0) s_tot = tot;
  }
  __syncthreads();
  if (s_tot > 8) return;
  const int W = N - c0;
  const int64_t plane = n_rows * (int64_t)W;
  for (int64_t r = blockIdx.x; r < n_rows; r += gridDim.x) {
    if (offsets) {
      if (r < offsets[0] || r >= offsets[E]) continue;
      int lo = 0, hi = E;                            // the expert holding row r
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid;
      }
      if (offsets[lo + 1] - offsets[lo] <= min_rows) continue;
    } else if (n_rows <= min_rows) {
      return;
    }
    const int64_t tk = row_token ? (int64_t)row_token[r] : r;
    const float sc = scales[tk];
    const float* p = ws + r * W;
    uint16_t* o = out + r * ldo + c0;
    // four columns a thread: N is a multiple of 16 and c0 of 128, so W is a multiple of 4,
    // the planes and rows start on 16-byte boundaries, and (ldo % 4 == 0) the four bf16 of
    // h form one aligned 8-byte store
    for (int n = 4 * (int)threadIdx.x; n < W; n += 4 * (int)blockDim.x) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(p + n), g1 = *reinterpret_cast<const f32x4*>(p + 2 * plane + n);
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(p + plane + n), u1 = *reinterpret_cast<const f32x4*>(p + 3 * plane + n);
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_mul((g0[i] + g1[i]) * sc, (u0[i] + u1[i]) * sc));
      *reinterpret_cast<u32x2*>(o + n) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    }
  }
}

size_t mfma_split_workspace_bytes(int n_w, int bits, int64_t n_rows, int N, int K) {
  if (bits != 4 || n_rows <= 0) return 0;
  if (n_w == 1) return K >= 4096 ? (size_t)n_rows * (size_t)N * sizeof(float) : 0;
  // the gate/up pair: four planes of at most 16 column tiles (128 columns each), for calls
  // of 512 to 4096 rows (fewer rows fill too few row tiles to gain from the split)
  if (K < 2048 || n_rows < 512 || n_rows > 4096) return 0;
  return 4 * (size_t)n_rows * (size_t)std::min(N, 16 * 128) * sizeof(float);
}

template <int BITS, int ABITS, bool LT, bool BLK>
static hipError_t launch_p2(const GemmArgs& a, int min_rows, hipStream_t stream) {
  constexpr int BM = tile_rows<BITS>();
  const int E = a.offsets ? a.E : 1;
  // M-tile slots: an expert of r rows takes ceil(r / BM) <= r / BM + 1 tiles, and only
  // experts of more than min_rows rows get any, at most n_rows / (min_rows + 1) of them.
  // The kernel's run length G follows from the call's tile count by the rule below; taken
  // at this upper bound it bounds the kernel's G (powers of two, so whole runs of this
  // length are whole runs of the kernel's), and each expert's last run leaves at most
  // G - 1 slots unused
  const int64_t big = a.offsets ? std::min<int64_t>(E, a.n_rows / (min_rows + 1)) : 0;
  const int64_t mt = (a.n_rows + BM - 1) / BM + big;
  int64_t G = 1;
  while (2 * G <= XG && 8 * 2 * G <= mt) G *= 2;
  const int64_t slots = mt + big * (G - 1);
  const int64_t mtiles = (slots + 8 * G - 1) / (8 * G) * (8 * G);   // whole runs on every XCD
  auto grid_for = [&](int ncol) { return dim3((unsigned)((a.N + ncol - 1) / ncol), (unsigned)mtiles); };
  if (a.n_w == 2) {
    // 256-row tiles (4-bit codebooks) run one workgroup per CU.  In calls of few M-tiles
    // each XCD works through its tile's column tiles in rounds of its CUs; when the last
    // round would be at most half full, the column tiles in it split K in two with the
    // workspace, so both halves fill that round, and a second pass forms their h.
    int tc0 = -1, extra = 0;
    if constexpr (BM == 256) {
      int cus = 0;
      if (a.ws != nullptr && mfma_split_workspace_bytes(2, BITS, a.n_rows, a.N, a.K) > 0 && mt <= 16 &&
          device_cu_count(&cus) == hipSuccess) {
        const int per = cus / 8;                     // CUs per XCD
        const int ntc = (a.N + 127) / 128;
        const int tl = per > 0 ? ntc % per : 0;      // column tiles of the last round
        const size_t need = 16 * (size_t)a.n_rows * (size_t)(a.N - (ntc - tl) * 128);
        if (tl > 0 && 2 * tl <= per && need <= mfma_split_workspace_bytes(2, BITS, a.n_rows, a.N, a.K) &&
            a.ws_bytes >= need) {
          tc0 = ntc - tl;
          extra = tl;
        }
      }
    }
    dim3 grid = grid_for(128);
    grid.x += (unsigned)extra;                       // the split column tiles' second halves
    hipLaunchKernelGGL((mfma_prefill_kernel<BITS, ABITS, 2, LT, BLK, 2>), grid, dim3(256), 0, stream,
                       a.codes, a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, E, a.N, a.K,
                       min_rows, a.blocked, a.out, a.ldo, static_cast<float*>(a.ws), tc0);
    if (extra > 0) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const unsigned blocks = (unsigned)(a.n_rows < 4096 ? a.n_rows : 4096);
      hipLaunchKernelGGL(mfma_swiglu_reduce_kernel, dim3(blocks), dim3(256), 0, stream,
                         static_cast<uint16_t*>(a.out), a.ldo, static_cast<const float*>(a.ws), a.n_rows,
                         a.N, tc0 * 128, a.scales, a.row_token, a.offsets, E, min_rows, BM);
    }
    return hipGetLastError();
  }
  if constexpr (BM == 256) {
    // a single matrix whose 256-column tiles would leave CUs idle (fewer than two
    // workgroups per CU even with every M-tile slot filled) takes 128-column tiles; with
    // a workspace it also splits K in two, so both workgroup slots of each CU fill, and
    // adds the second half's partial sums in a second, ordered pass
    if ((int64_t)((a.N + 255) / 256) * mt < 2 * 256) {
      const size_t need = mfma_split_workspace_bytes(a.n_w, BITS, a.n_rows, a.N, a.K);
      const int nsplit = (need > 0 && a.ws != nullptr && a.ws_bytes >= need &&
                          (int64_t)((a.N + 127) / 128) * mt < 2 * 256) ? 2 : 1;
      dim3 grid = grid_for(128);
      grid.z = (unsigned)nsplit;
      hipLaunchKernelGGL((mfma_prefill_kernel<BITS, ABITS, 1, LT, BLK, 1>), grid, dim3(256), 0, stream,
                         a.codes, a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, E, a.N, a.K,
                         min_rows, a.blocked, a.out, a.ldo, static_cast<float*>(a.ws), -1);
      if (nsplit > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned blocks = (unsigned)(a.n_rows < 4096 ? a.n_rows : 4096);
        hipLaunchKernelGGL(mfma_split_reduce_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<float*>(a.out), a.ldo, static_cast<const float*>(a.ws), nsplit,
                           a.n_rows, a.N, a.offsets, E, min_rows);
      }
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((mfma_prefill_kernel<BITS, ABITS, 1, LT, BLK, 2>), grid_for(256), dim3(256), 0, stream,
                     a.codes, a.scales, a.offsets, a.row_token, a.w[0], a.w[1], a.n_rows, E, a.N, a.K,
                     min_rows, a.blocked, a.out, a.ldo, nullptr, -1);
  return hipGetLastError();
}

// 3-bit weights in the blocked layout take the kernels for its re-encoded units.
template <int BITS, int ABITS, bool LT>
static hipError_t launch_p(const GemmArgs& a, int min_rows, hipStream_t stream) {
  if constexpr (BITS == 3) {
    if (a.blocked) return launch_p2<BITS, ABITS, LT, true>(a, min_rows, stream);
  }
  return launch_p2<BITS, ABITS, LT, false>(a, min_rows, stream);
}

hipError_t launch_mfma_prefill(const GemmArgs& a, int min_rows, hipStream_t stream) {
  // 2- and 3-bit codebooks: register tables unless the LDS pair tables are asked for (the
  // pair tables take fewer vector instructions but add LDS traffic to the activation
  // tiles' reads, and measured slightly slower here); 4-bit tables stay in registers
  const bool lt = a.tables == kTablesLds;
  switch (a.bits * 10 + (a.act_bits == 8 ? 8 : 4)) {
    case 44: return launch_p<4, 4, false>(a, min_rows, stream);
    case 48: return launch_p<4, 8, false>(a, min_rows, stream);
    case 34: return lt ? launch_p<3, 4, true>(a, min_rows, stream) : launch_p<3, 4, false>(a, min_rows, stream);
    case 38: return lt ? launch_p<3, 8, true>(a, min_rows, stream) : launch_p<3, 8, false>(a, min_rows, stream);
    case 24: return lt ? launch_p<2, 4, true>(a, min_rows, stream) : launch_p<2, 4, false>(a, min_rows, stream);
    case 28: return lt ? launch_p<2, 8, true>(a, min_rows, stream) : launch_p<2, 8, false>(a, min_rows, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cbq
