// Device-side building blocks shared by the GEMM kernels (gfx950, wave64).
//
// Per-row codebook tables live in VGPRs and are looked up with v_perm_b32 byte
// permutes, so the table the LUT kernel builds once and then reads (CodeQuant2,
// Figure 4) costs no LDS bandwidth and has no bank conflicts (the
// problem the AI Radio episode's "Improvements" section describes for an
// LDS-resident table).
//
// A row's 2^bits fp16 centroids are split into a low-byte table and a high-byte
// table; a lookup selects the low and high bytes of up to four weights with one
// permute each and interleaves them into fp16 pairs.
//
// K order inside a group of eight consecutive weights.  Every dequantiser and every
// activation converter below emits four dwords per group in the same order
//     D0 = (k0, k2)  D1 = (k4, k6)  D2 = (k1, k3)  D3 = (k5, k7)
// (low half first).  Because weights and activations are permuted identically, the
// dot product over the group is unchanged; only the fp32 summation order differs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cbq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// v_perm_b32: byte i of the result = byte sel[i] of the 8-byte value {hi:lo}
// (0..3 from lo, 4..7 from hi; 12 gives 0x00).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, float c) {
  f16x2 v = __builtin_bit_cast(f16x2, a);
  f16x2 k = {(_Float16)c, (_Float16)c};
  return __builtin_bit_cast(uint32_t, v + k);
}

__device__ __forceinline__ f16x8 as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(f16x8, v);
}

// ---------------------------------------------------------------------------
// Per-row codebook tables in registers.
//   lo[i] = low bytes of entries 4i..4i+3, hi[i] = their high bytes.
template <int BITS> struct RowTable {
  static constexpr int L = 1 << BITS;
  static constexpr int NT = (L + 3) / 4;
  uint32_t lo[NT], hi[NT];

  // cb: pointer to the row's 2^BITS fp16 patterns (4-byte aligned).
  __device__ __forceinline__ void load(const uint16_t* cb) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(cb);
    if constexpr (BITS == 2) {
      uint32_t a = w[0], b = w[1];
      lo[0] = perm(b, a, 0x06040200u);
      hi[0] = perm(b, a, 0x07050301u);
    } else {
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        uint32_t a = w[2 * i], b = w[2 * i + 1];
        lo[i] = perm(b, a, 0x06040200u);
        hi[i] = perm(b, a, 0x07050301u);
      }
    }
  }
};

// 4-bit: one dword of eight nibble indices -> D0..D3.
__device__ __forceinline__ void dequant4(const RowTable<4>& t, uint32_t x, uint32_t* d) {
  const uint32_t s7e = x & 0x07070707u;
  const uint32_t s7o = (x >> 4) & 0x07070707u;
  const uint32_t be = ((x >> 1) & 0x04040404u) | 0x03020100u;   // byte i -> i + 4*bit3
  const uint32_t bo = ((x >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t le = perm(perm(t.lo[3], t.lo[2], s7e), perm(t.lo[1], t.lo[0], s7e), be);
  const uint32_t he = perm(perm(t.hi[3], t.hi[2], s7e), perm(t.hi[1], t.hi[0], s7e), be);
  const uint32_t lo = perm(perm(t.lo[3], t.lo[2], s7o), perm(t.lo[1], t.lo[0], s7o), bo);
  const uint32_t ho = perm(perm(t.hi[3], t.hi[2], s7o), perm(t.hi[1], t.hi[0], s7o), bo);
  d[0] = perm(he, le, 0x05010400u);   // (k0, k2)
  d[1] = perm(he, le, 0x07030602u);   // (k4, k6)
  d[2] = perm(ho, lo, 0x05010400u);   // (k1, k3)
  d[3] = perm(ho, lo, 0x07030602u);   // (k5, k7)
}

// 3-bit: eight indices in the low 24 bits of f -> D0..D3.
__device__ __forceinline__ void dequant3(const RowTable<3>& t, uint32_t f, uint32_t* d) {
  uint32_t ta = (f & 0x3Fu) | ((f << 10) & 0x3F0000u);          // i0,i1 | i2,i3 << 16
  uint32_t sa = (ta | (ta << 5)) & 0x07070707u;                  // bytes i0 i1 i2 i3
  uint32_t tb = ((f >> 12) & 0x3Fu) | ((f >> 2) & 0x3F0000u);
  uint32_t sb = (tb | (tb << 5)) & 0x07070707u;                  // bytes i4 i5 i6 i7
  const uint32_t la = perm(t.lo[1], t.lo[0], sa), ha = perm(t.hi[1], t.hi[0], sa);
  const uint32_t lb = perm(t.lo[1], t.lo[0], sb), hb = perm(t.hi[1], t.hi[0], sb);
  d[0] = perm(ha, la, 0x06020400u);   // (k0, k2)
  d[1] = perm(hb, lb, 0x06020400u);   // (k4, k6)
  d[2] = perm(ha, la, 0x07030501u);   // (k1, k3)
  d[3] = perm(hb, lb, 0x07030501u);   // (k5, k7)
}

// 2-bit: one dword of sixteen indices -> two groups (D0..D3 of indices 0..7, then 8..15).
__device__ __forceinline__ void dequant2(const RowTable<2>& t, uint32_t x, uint32_t* d) {
  const uint32_t y0 = x & 0x03030303u;          // bytes: i0 i4 i8 i12
  const uint32_t y1 = (x >> 2) & 0x03030303u;   // i1 i5 i9 i13
  const uint32_t y2 = (x >> 4) & 0x03030303u;   // i2 i6 i10 i14
  const uint32_t y3 = (x >> 6) & 0x03030303u;   // i3 i7 i11 i15
  // selector for a pair (a, b): bytes (a, a+4, b, b+4) = (a | b << 16) * 0x101 + 0x04000400
#define CBQ_SEL2(v) (__umul24((v), 0x101u) + 0x04000400u)
  d[0] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y2, y0, 0x0C040C00u)));   // (k0, k2)
  d[1] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y2, y0, 0x0C050C01u)));   // (k4, k6)
  d[2] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y3, y1, 0x0C040C00u)));   // (k1, k3)
  d[3] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y3, y1, 0x0C050C01u)));   // (k5, k7)
  d[4] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y2, y0, 0x0C060C02u)));   // (k8, k10)
  d[5] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y2, y0, 0x0C070C03u)));   // (k12, k14)
  d[6] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y3, y1, 0x0C060C02u)));   // (k9, k11)
  d[7] = perm(t.hi[0], t.lo[0], CBQ_SEL2(perm(y3, y1, 0x0C070C03u)));   // (k13, k15)
#undef CBQ_SEL2
}

// 3-bit units of the blocked layout (cbq_prepack_weights).  Group g < 3 (indices
// 8g .. 8g+7 of the unit) is dword g: byte b holds index 8g+2b in bits 0-2 and 8g+2b+1 in
// bits 3-5.  Group 3's six-bit pairs are spread over the spare top bits: pair b's bits
// 2i .. 2i+1 are bits 6-7 of byte b of dword i.  This gathers group 3 into the same form.
__device__ __forceinline__ uint32_t group3_blk(const uint32_t* w) {
  return ((w[0] >> 6) & 0x03030303u) | ((w[1] >> 4) & 0x0C0C0C0Cu) | ((w[2] >> 2) & 0x30303030u);
}

// 3-bit, one group in the blocked form (only bits 0-5 of each byte are read) -> D0..D3:
// the even indices' and the odd indices' selectors are one mask and one shift-and-mask.
__device__ __forceinline__ void dequant3_blk(const RowTable<3>& t, uint32_t x, uint32_t* d) {
  const uint32_t se = x & 0x07070707u;                 // bytes i0 i2 i4 i6
  const uint32_t so = (x >> 3) & 0x07070707u;          // bytes i1 i3 i5 i7
  const uint32_t le = perm(t.lo[1], t.lo[0], se), he = perm(t.hi[1], t.hi[0], se);
  const uint32_t lo = perm(t.lo[1], t.lo[0], so), ho = perm(t.hi[1], t.hi[0], so);
  d[0] = perm(he, le, 0x05010400u);   // (k0, k2)
  d[1] = perm(he, le, 0x07030602u);   // (k4, k6)
  d[2] = perm(ho, lo, 0x05010400u);   // (k1, k3)
  d[3] = perm(ho, lo, 0x07030602u);   // (k5, k7)
}

// Dequantise 32 consecutive indices (one lane's slice: 4*BITS bytes already loaded
// into w[0..BITS-1]) into 16 dwords: group j (indices 8j..8j+7) -> d[4j..4j+3].  BLK:
// the slice is a unit of the blocked layout (which re-encodes 3-bit units).
template <int BITS, bool BLK = false>
__device__ __forceinline__ void dequant32(const RowTable<BITS>& t, const uint32_t* w, uint32_t* d) {
  if constexpr (BITS == 3 && BLK) {
    dequant3_blk(t, w[0], d + 0);
    dequant3_blk(t, w[1], d + 4);
    dequant3_blk(t, w[2], d + 8);
    dequant3_blk(t, group3_blk(w), d + 12);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dequant4(t, w[j], d + 4 * j);
  } else if constexpr (BITS == 3) {
    dequant3(t, w[0], d + 0);
    dequant3(t, __builtin_amdgcn_alignbit(w[1], w[0], 24), d + 4);
    dequant3(t, __builtin_amdgcn_alignbit(w[2], w[1], 16), d + 8);
    dequant3(t, w[2] >> 8, d + 12);
  } else {
    dequant2(t, w[0], d + 0);
    dequant2(t, w[1], d + 8);
  }
}

// ---------------------------------------------------------------------------
// Activation codes -> fp16 in the same group order.
// A4: one dword of eight two's-complement nibbles.  (0x6400 | u) is fp16 1024 + u.
__device__ __forceinline__ void codes4_to_f16(uint32_t x, uint32_t* d) {
  const uint32_t xb = x ^ 0x88888888u;          // nibble v -> v + 8
  const uint32_t e = xb & 0x0F0F0F0Fu;
  const uint32_t o = (xb >> 4) & 0x0F0F0F0Fu;
  d[0] = pk_add_f16(perm(0x64646464u, e, 0x04010400u), -1032.0f);
  d[1] = pk_add_f16(perm(0x64646464u, e, 0x04030402u), -1032.0f);
  d[2] = pk_add_f16(perm(0x64646464u, o, 0x04010400u), -1032.0f);
  d[3] = pk_add_f16(perm(0x64646464u, o, 0x04030402u), -1032.0f);
}

// A8: two dwords holding eight int8 codes k0..k7.
__device__ __forceinline__ void codes8_to_f16(uint32_t x0, uint32_t x1, uint32_t* d) {
  const uint32_t b0 = x0 ^ 0x80808080u, b1 = x1 ^ 0x80808080u;   // c -> c + 128
  d[0] = pk_add_f16(perm(0x64646464u, b0, 0x04020400u), -1152.0f);   // (k0, k2)
  d[1] = pk_add_f16(perm(0x64646464u, b1, 0x04020400u), -1152.0f);   // (k4, k6)
  d[2] = pk_add_f16(perm(0x64646464u, b0, 0x04030401u), -1152.0f);   // (k1, k3)
  d[3] = pk_add_f16(perm(0x64646464u, b1, 0x04030401u), -1152.0f);   // (k5, k7)
}

// 32 consecutive codes (16 bytes for A4, 32 for A8, in c[0..ABITS-1]) -> 16 dwords.
template <int ABITS>
__device__ __forceinline__ void codes32_to_f16(const uint32_t* c, uint32_t* d) {
  if constexpr (ABITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) codes4_to_f16(c[j], d + 4 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) codes8_to_f16(c[2 * j], c[2 * j + 1], d + 4 * j);
  }
}

// ---------------------------------------------------------------------------
// Natural pair order.  The LDS pair tables below give each weight pair in index order,
// (k0, k1) (k2, k3) (k4, k5) (k6, k7) per group of eight, so a GEMM that reads them takes
// its activation fragments from these converters instead.
// A4: for byte j the permute gives (b, 0x64, b, 0x64); masking to (0x640L, 0x64H0) makes
// the low half fp16 1024 + L and the high half 1024 + 16 H; one packed fma scales the high
// half by 1/16 and removes both offsets (each step exact in fp16).
__device__ __forceinline__ void codes4_to_f16_nat(uint32_t x, uint32_t* d) {
  const uint32_t xb = x ^ 0x88888888u;          // nibble v -> v + 8
  const f16x2 mul = {(_Float16)1.0f, (_Float16)0.0625f};
  const f16x2 add = {(_Float16)-1032.0f, (_Float16)-72.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = perm(0x64646464u, xb, 0x04000400u + 0x00010001u * (uint32_t)j) & 0xFFF0FF0Fu;
    d[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, t), mul, add));
  }
}

// A8, natural order: (k0, k1) (k2, k3) from x0, (k4, k5) (k6, k7) from x1.
__device__ __forceinline__ void codes8_to_f16_nat(uint32_t x0, uint32_t x1, uint32_t* d) {
  const uint32_t b0 = x0 ^ 0x80808080u, b1 = x1 ^ 0x80808080u;   // c -> c + 128
  d[0] = pk_add_f16(perm(0x64646464u, b0, 0x04010400u), -1152.0f);
  d[1] = pk_add_f16(perm(0x64646464u, b0, 0x04030402u), -1152.0f);
  d[2] = pk_add_f16(perm(0x64646464u, b1, 0x04010400u), -1152.0f);
  d[3] = pk_add_f16(perm(0x64646464u, b1, 0x04030402u), -1152.0f);
}

// Eight codes (group p of 32: one dword for A4, two for A8) -> four dwords, in the pair
// order NAT (natural) or the grouped order of the register dequantisers.
template <int ABITS, bool NAT>
__device__ __forceinline__ void codes8_group(const uint32_t* c, int p, uint32_t* d) {
  if constexpr (ABITS == 4) {
    if constexpr (NAT) codes4_to_f16_nat(c[p], d);
    else codes4_to_f16(c[p], d);
  } else {
    if constexpr (NAT) codes8_to_f16_nat(c[2 * p], c[2 * p + 1], d);
    else codes8_to_f16(c[2 * p], c[2 * p + 1], d);
  }
}

template <int ABITS, bool NAT>
__device__ __forceinline__ void codes32_to_f16_ord(const uint32_t* c, uint32_t* d) {
#pragma unroll
  for (int p = 0; p < 4; ++p) codes8_group<ABITS, NAT>(c, p, d + 4 * p);
}

// ---------------------------------------------------------------------------
// LDS pair tables for 2- and 3-bit codebooks (CodeQuant2, Figure 4: the kernel's table
// sits in on-chip shared memory).  Two consecutive indices 2j, 2j+1 of a row form the
// 2*BITS-bit field v = i_2j | i_2j+1 << BITS of its bitstream; entry v of the row's table
// is the dword C[v & (L-1)] | C[v >> BITS] << 16, both weights as an fp16 pair in index
// order.  A lookup is one field extract, one address add and one ds_read_b32 per two
// weights, against about five vector instructions for the register tables.  The tables
// of R rows are interleaved (entry v of row r at dword v*R + r), so lanes that read
// different rows read different banks.
template <int BITS>
struct PairTab {
  static constexpr int L = 1 << BITS;
  static constexpr int NE = L * L;   // entries per row
};

// Field j (0..15) of the 32 indices a lane holds in w[0..BITS-1] (LSB-first).
template <int BITS>
__device__ __forceinline__ uint32_t pair_field(const uint32_t* w, int j) {
  constexpr int FB = 2 * BITS;
  const int off = j * FB, wi = off >> 5, sh = off & 31;
  if (sh + FB <= 32) return __builtin_amdgcn_ubfe(w[wi], (uint32_t)sh, (uint32_t)FB);
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], (uint32_t)sh) & ((1u << FB) - 1u);
}

// Pairs 4p .. 4p+3 of the lane's 32 indices -> d[0..3], from the table row whose entry 0
// is dword `row` of `tab` (entries R dwords apart).  BLK: a 3-bit unit of the blocked
// layout, whose pair 4p + b is bits 0-5 of byte b of group p.
template <int BITS, int R, bool BLK = false>
__device__ __forceinline__ void pair_lookup8(const uint32_t* tab, uint32_t row, const uint32_t* w,
                                             int p, uint32_t* d) {
  if constexpr (BITS == 3 && BLK) {
    const uint32_t x = p < 3 ? w[p] : group3_blk(w);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = tab[row + __builtin_amdgcn_ubfe(x, 8u * q, 6u) * R];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = tab[row + pair_field<BITS>(w, 4 * p + q) * R];
  }
}

template <int BITS, int R, bool BLK = false>
__device__ __forceinline__ void pair_lookup32(const uint32_t* tab, uint32_t row, const uint32_t* w,
                                              uint32_t* d) {
#pragma unroll
  for (int p = 0; p < 4; ++p) pair_lookup8<BITS, R, BLK>(tab, row, w, p, d + 4 * p);
}

// This lane's share of one row's table: P lanes (sub = 0 .. P-1) build the row, lane sub
// the entries whose high index is sub*H .. sub*H + H - 1 (H = L / P), from the row's
// codebook cb (L fp16 in L/2 dwords).  Entry rows are R dwords apart from `row` on.
template <int BITS, int P, int R>
__device__ __forceinline__ void pair_build(uint32_t* tab, uint32_t row, const uint32_t* cb, int sub) {
  constexpr int L = 1 << BITS;
  constexpr int H = L / P;
  static_assert(H >= 1 && H * P == L, "P must divide L");
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int q = sub * H + h;                 // high index: C[q] in the upper half
    uint32_t cw = cb[0];
#pragma unroll
    for (int k = 1; k < L / 2; ++k) cw = (q >> 1) == k ? cb[k] : cw;
    const uint32_t hv = (q & 1) ? (cw >> 16) : cw;
    uint32_t* dst = tab + row + (uint32_t)(q * L) * R;
#pragma unroll
    for (int lo = 0; lo < L; ++lo)
      dst[lo * R] = perm(hv, cb[lo >> 1], (lo & 1) ? 0x05040302u : 0x05040100u);
  }
}

// Buffer-resource loads.  A load whose byte offset is at or past num_records returns
// zeros without faulting, so a disabled load is just an out-of-range offset and no
// select has to touch the loaded registers (which would force an early wait).
constexpr uint32_t kOffNone = 0x80000000u;
// Second sentinel for offsets built as row part + column part: rows use kOffNone,
// columns kOffCol, so no sum of the two wraps below 2^30 (buffers stay < 1 GiB).
constexpr uint32_t kOffCol = 0x40000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// off: per-lane byte offset (kOffNone disables the load); soff: wave-uniform byte
// offset added on top (kept in an SGPR, so advancing it costs no vector ALU work).
template <int BYTES>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w,
                                         uint32_t soff = 0) {
  if constexpr (BYTES == 16) {
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BYTES == 12) {
    u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off, soff, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else if constexpr (BYTES == 8) {
    u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    w[0] = v[0]; w[1] = v[1];
  } else {
    static_assert(BYTES == 4, "unsupported load width");
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
  }
}

__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

__device__ __forceinline__ void buf_store_u16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for its outstanding global loads (prefetches
// included) at each barrier; this one waits only for the wave's own LDS traffic.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// small numeric helpers
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, ((uint32_t)h) << 16);
}

// SiLU(g) * u in fp32 for the SwiGLU epilogue of every GEMM path: g * u * rcp(1 + exp(-g))
// with the hardware exp2 (of -g * log2 e) and reciprocal, each within a few fp32 ulps.
// The result is rounded to bf16 (2^16 fp32 ulps apart), so it lies within one bf16 step
// of the exactly rounded value.  Both GEMM paths call this one function, so equal fp32
// (g, u) give equal bf16 h whichever path computed them.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace cbq
