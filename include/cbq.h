/*
 * cbq.h - codebook-LUT MoE expert path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libcbq.so.  Four calls make one MoE FFN layer of the CodeQuant /
 * CodeQuant2 method: activations rotated by a Walsh-Hadamard transform and
 * quantised per token to int4/int8, top-k routing, expert matmuls whose weights are
 * packed 2/3/4-bit indices into per-output-row fp16 codebooks, and the weighted
 * combine of expert outputs.
 *
 * Conventions shared by every call
 *  - Every tensor pointer is DEVICE memory owned by the caller; the library never
 *    allocates, frees or retains device memory.  Pointers must stay valid until the
 *    work queued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    queued asynchronously; no call synchronises the host with the device.
 *  - Arguments are validated on the host before any HIP call.  A violation returns
 *    CBQ_EINVAL / CBQ_EUNSUPPORTED / CBQ_EWORKSPACE and queues nothing; a failed
 *    launch returns CBQ_EHIP.  cbq_last_error() then describes the failure (the
 *    message is per calling thread).  No C++ exception crosses this interface.
 *  - Empty work (zero tokens or rows) is a successful no-op.  Results for non-finite
 *    inputs are unspecified.
 *  - The library keeps no mutable global state; calls on different streams may run
 *    concurrently.
 *  - bf16 / fp16 tensors are passed as uint16_t bit patterns.
 */
#ifndef CBQ_H
#define CBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CBQ_OK = 0,
  CBQ_EINVAL = -1,        /* bad pointer, size, layout or alignment */
  CBQ_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  CBQ_EWORKSPACE = -3,    /* workspace missing or too small */
  CBQ_EHIP = -4           /* a HIP runtime call or kernel launch failed */
};

/* GEMM epilogues */
enum {
  CBQ_EPI_F32 = 0,          /* out = fp32 [n_rows][ldo]: y = scale * acc */
  CBQ_EPI_SWIGLU_BF16 = 1   /* n_w == 2: out = bf16 [n_rows][ldo]: h = silu(g) * u */
};

/* GEMM inner paths */
enum {
  CBQ_PATH_AUTO = 0,  /* per expert: LUT path when its row count <= CBQ_AUTO_MAX_LUT_ROWS,
                         else the MFMA path; decided on the device */
  CBQ_PATH_LUT = 1,   /* register codebook lookup feeding 16x16x32 MFMA; an expert's weights
                         are streamed from HBM once (K split over waves for experts of at most
                         32 rows, row blocks of 32 split over waves for larger ones) */
  CBQ_PATH_MFMA = 2,  /* 256-row tiles: weights dequantised in registers straight into the
                         B operand of 32x32x16 fp16 MFMAs, activation codes converted to fp16
                         once per tile step in LDS */
  /* The table forms of CodeQuant2, Figure 4 (a table built once, then products read from
     shared memory instead of multiplied; the AI Radio episode, "Improvements", calls it a
     multiplication table).  4-bit codebooks, act_bits == 4 and K <= 16384 only (else
     CBQ_EUNSUPPORTED), no table flags; meant for experts of a few rows, correct for any.  Never chosen by
     CBQ_PATH_AUTO: kept to measure them against CBQ_PATH_LUT. */
  CBQ_PATH_PAGES_PRODUCTS = 3, /* per weight row, an LDS table of the products |a| * C[c] of
                                  the nine code magnitudes and 16 centroids, exact in fp32;
                                  the code's sign applied after the lookup; fp32 sums */
  CBQ_PATH_PAGES_BUCKETS = 4   /* per weight row and token, 16 integer buckets in LDS that
                                  sum the activation codes by weight index, then
                                  sum_c C[c] * bucket[c] (fp64, rounded to fp32 per lane) */
};

/* Flags added to a path to choose where 2- and 3-bit codebooks are looked up (4-bit ones
   always use the register tables).  By default the LUT path uses LDS pair tables (two
   weights per lookup, the table the pages' kernel keeps in shared memory) for 2-bit
   codebooks and for 3-bit ones in the row layout, and per-row register tables (byte
   permutes) for 3-bit codebooks in the blocked layout; the MFMA path uses the register
   tables: the faster placement of each as measured.  Results agree within fp32
   summation order; kept to compare the two placements. */
#define CBQ_PATH_REG_TABLES 0x10
#define CBQ_PATH_LDS_TABLES 0x20

#define CBQ_AUTO_MAX_LUT_ROWS 32

/* Index layouts of cbq_weights.idx */
enum {
  CBQ_LAYOUT_ROWS = 0,     /* one LSB-first bitstream per row (the format the method defines) */
  CBQ_LAYOUT_BLOCKED = 1   /* the same indices regrouped (3-bit units re-encoded) by cbq_prepack_weights */
};

/*
 * One weight matrix type for E experts (E = 1 for a dense linear).
 * Reading of CodeQuant2, Figure 3 (right): a centroid matrix with one codebook per
 * weight row and a per-row assignment of every weight to one of its centroids.
 *  idx      : layout CBQ_LAYOUT_ROWS: [E][N][K*bits/8] bytes.  Row n of expert e is an
 *             LSB-first bitstream: the index of weight k occupies bits [k*bits, (k+1)*bits).
 *             Layout CBQ_LAYOUT_BLOCKED: see cbq_prepack_weights.
 *  codebook : [E][N][1 << bits] fp16 bit patterns; entry c of row n is the value
 *             of every weight of that row whose index is c (order not assumed).
 *  W[e][n][k] = codebook[e][n][idx(e, n, k)].
 *  bits in {2, 3, 4}; K % 32 == 0; N % 16 == 0; both pointers 16-byte aligned.
 */
typedef struct {
  const uint8_t* idx;
  const uint16_t* codebook;
  int32_t E, N, K, bits;
  int32_t layout;          /* CBQ_LAYOUT_* */
} cbq_weights;

/*
 * cbq_prepack_weights - regroup a weight set's indices for the GEMM kernels (an offline
 * step, like the codebook construction).  The values are unchanged: W[e][n][k] is the
 * same matrix, so the GEMM's results are those of the row layout, bit for bit.
 *
 * CBQ_LAYOUT_BLOCKED: with Kp = K rounded up to a multiple of 128, rows are taken in
 * groups of 16 and channels in chunks of 128; the 32 indices of row 16G + r, channels
 * 128c + 32j .. 128c + 32j + 31, are the 4*bits bytes of that row's bitstream at
 * channel 128c + 32j (zeros past K), stored at byte
 *     ((e * N/16 + G) * Kp/128 + c) * 256*bits + (16j + r) * 4*bits.
 * So one 16-row x 128-channel tile is 256*bits contiguous bytes, which a 64-lane wave
 * reads in one fully coalesced load (a row stream would give it sixteen 16*bits-byte
 * pieces 1/8 K*bits bytes apart).  2- and 4-bit units keep their bytes.  A 3-bit unit
 * (indices i0 .. i31, 12 bytes) is re-encoded so the kernels form their byte selectors
 * with one mask or one shift and a mask: dword g (g = 0, 1, 2) holds i(8g+2b) in bits
 * 8b .. 8b+2 and i(8g+2b+1) in bits 8b+3 .. 8b+5 (b = 0..3); the six-bit pair
 * p_b = i(24+2b) | i(25+2b) << 3 goes to bits 8b+6 .. 8b+7 of the three dwords, bits
 * 2w .. 2w+1 of p_b in dword w.
 *
 *  src : a CBQ_LAYOUT_ROWS weight set (device pointers).
 *  dst : device buffer of cbq_prepack_bytes(src) bytes, 16-byte aligned, not
 *        overlapping src->idx.  The blocked weight set is {dst, src->codebook, E, N, K,
 *        bits, CBQ_LAYOUT_BLOCKED}.
 */
size_t cbq_prepack_bytes(const cbq_weights* src);
int cbq_prepack_weights(const cbq_weights* src, uint8_t* dst, void* stream);

/*
 * cbq_rotate_quantize - Hadamard rotation fused with per-token absmax quantisation.
 * Passage: CodeQuant2, Figure 1 (rotation fused into the model to smooth activation
 * outliers) and Tables 1 and 9 (A4W4 / A8W4 activation settings); CodeQuant
 * abstract (rotation-based outlier smoothing).
 *
 *  x          : bf16 [T][ldx] (ldx >= K, ldx % 8 == 0, 16-byte aligned); row t holds
 *               one token's K channels.
 *  had_block  : 0 -> rotation block b = K & -K (largest power of two dividing K);
 *               otherwise b itself (a power of two dividing K; 1 = no rotation).
 *  act_bits   : 4 (codes in [-8, 7], Q = 7) or 8 (codes in [-127, 127], Q = 127).
 *  codes      : [T][K*act_bits/8] bytes, 16-byte aligned.  A4: two's-complement
 *               nibbles, channel 2j in the low nibble of byte j; A8: int8.
 *  scales     : fp32 [T].
 *  precond_violations : optional device uint32 counter (NULL to skip the check);
 *               incremented once per (token, block) whose nonzero bf16 exponents
 *               spread more than 45 - log2(b) binades, the bound under which the
 *               fp64 transform below is exact.
 *
 *  Computes u = (I_{K/b} (x) H_b) x exactly (Sylvester order, H[i][j] =
 *  (-1)^popcount(i & j), no normalisation), then in IEEE fp32:
 *  v = fp32(u); M = max|v|; s = M / Q; q = clamp(rint_even(v / s));
 *  scale = s * fp32(1/sqrt(b)).  A token with M == 0 gets codes 0 and scale 0.
 *  Requires 1 <= K, K % 32 == 0, K <= 16384.
 */
int cbq_rotate_quantize(const uint16_t* x, int64_t T, int32_t K, int64_t ldx,
                        int32_t had_block, int32_t act_bits, uint8_t* codes, float* scales,
                        uint32_t* precond_violations, void* stream);

/*
 * cbq_rotate_quantize_ex - cbq_rotate_quantize with per-channel transforms before the
 * rotation.  Passage: CodeQuant2, Figure 1 (per-channel scales and a rotation, folded
 * into the weights, smooth the activation outliers) and Table 5 caption (the base
 * setting is a fixed random rotation with SmoothQuant scaling).
 *
 *  smooth : optional fp32 [K] multipliers m (16-byte aligned): channel c becomes
 *           fp32(x_c * m_c), one fp32 rounding (a SmoothQuant factor 1/s_c).
 *  signs  : optional [K/8] bytes (4-byte aligned), LSB-first bit c set -> channel c is
 *           negated (a random-sign Hadamard, H D).
 *  Then u = (I (x) H_b) v exactly and the quantiser of cbq_rotate_quantize.  With smooth,
 *  the values have 24 significant bits and the fp64 transform is exact when a block's
 *  nonzero exponents spread at most 29 - log2(b) binades (the precondition counter
 *  tests that bound).  NULL, NULL gives cbq_rotate_quantize exactly.
 */
int cbq_rotate_quantize_ex(const uint16_t* x, int64_t T, int32_t K, int64_t ldx, int32_t had_block,
                           int32_t act_bits, const float* smooth, const uint8_t* signs,
                           uint8_t* codes, float* scales, uint32_t* precond_violations,
                           void* stream);

/*
 * cbq_rotate_quantize_dense - a dense K x K rotation before the quantiser.  Passage:
 * CodeQuant2, Figure 1 (a rotation fused into the model smooths activation outliers);
 * CodeQuant abstract (the rotation may be learned).  R stands for such a learned
 * rotation (orthonormal, so the scale carries no normalisation factor).
 *
 *  x          : bf16 [T][ldx] (ldx >= K, ldx % 8 == 0, 16-byte aligned).
 *  R          : bf16 [K][K] (16-byte aligned): u[j] = sum_k R[j][k] * x[k].
 *  act_bits   : 4 or 8, codes and scales as in cbq_rotate_quantize (8-byte aligned codes).
 *  precond_violations : optional device uint32 counter; incremented once per token
 *               whose nonzero exponents spread more than 37 - ceil(log2 K) binades
 *               minus the widest spread of a row of R, the bound under which the fp64
 *               sums below are exact in any order.
 *  ws, ws_bytes : device workspace of at least cbq_rotate_dense_workspace(T, K) bytes,
 *               16-byte aligned; it holds fp32(u) between the two passes.
 *
 *  Computes u = R x exactly (bf16 products are exact in fp64; inside the bound so are
 *  the sums), then v = fp32(u); M = max|v|; s = M / Q; q = clamp(rint_even(v / s));
 *  scale = s.  A token with M == 0 gets codes 0 and scale 0.
 *  Requires K % 64 == 0, 64 <= K <= 16384, T < 2^31.
 */
size_t cbq_rotate_dense_workspace(int64_t T, int32_t K);
int cbq_rotate_quantize_dense(const uint16_t* x, int64_t T, int32_t K, int64_t ldx,
                              const uint16_t* R, int32_t act_bits, uint8_t* codes, float* scales,
                              uint32_t* precond_violations, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * cbq_moe_route_gather - top-k routing and per-expert row lists.
 * Passage: the AI Radio episode on CodeQuant (introduction: a router sends each input
 * to the right expert of the mixture).
 *
 *  logits         : fp32 [T][E] router logits (1 <= E <= 256), 16-byte aligned rows
 *                   are not required.
 *  topk           : 1 <= topk <= min(E, 8).
 *  renormalize    : 1 -> weights are a softmax over the k selected logits;
 *                   0 -> the selected entries of a softmax over all E logits.
 *  n_shared       : 0 <= n_shared <= 8 always-on experts (weight 1) after the routed ones.
 *  topk_ids       : int32 [T][topk]: the k largest logits, descending, ties to the
 *                   lower expert id.
 *  topk_w         : fp32 [T][topk] routing weights.
 *  expert_offsets : int32 [E + n_shared + 1]: rows of expert e are
 *                   [expert_offsets[e], expert_offsets[e+1]); the last entry is
 *                   T*topk + n_shared*T.
 *  sorted_tokens  : int32 [T*topk + n_shared*T]: the token of every row, tokens
 *                   ascending inside an expert; shared expert s owns rows
 *                   T*topk + s*T + t.
 *  slot_of        : int32 [T][topk]: the row of token t's j-th choice.
 *  ws, ws_bytes   : device workspace of at least cbq_route_workspace(...) bytes, 4-byte
 *                   aligned (per-chunk expert counts; fully rewritten by every call, so it
 *                   needs no clearing); may be NULL when that size is 0 (T == 0).
 *  All integer outputs are deterministic (no dependence on atomic ordering).
 *  Requires T <= 2^24.
 */
size_t cbq_route_workspace(int64_t T, int32_t E, int32_t topk, int32_t n_shared);
int cbq_moe_route_gather(const float* logits, int64_t T, int32_t E, int32_t topk,
                         int32_t renormalize, int32_t n_shared, int32_t* topk_ids,
                         float* topk_w, int32_t* expert_offsets, int32_t* sorted_tokens,
                         int32_t* slot_of, void* ws, size_t ws_bytes, void* stream);

/*
 * cbq_moe_route_gather_noalloc - cbq_moe_route_gather without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 *  Arguments and outputs as cbq_moe_route_gather; the per-chunk expert counts go to a
 *  scratch array of 256 KiB inside the library (one per GPU, held until the process
 *  ends), which covers every size the routing accepts (T <= 2^24, E <= 256).  The call
 *  allocates nothing; its first call on a device looks the array's address up once.
 *  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 *  different streams, or from different threads) race and give undefined results;
 *  calls ordered on one stream are safe.  The array needs no clearing (each call
 *  rewrites the part it reads).  Outputs are bit-identical to cbq_moe_route_gather's.
 */
int cbq_moe_route_gather_noalloc(const float* logits, int64_t T, int32_t E, int32_t topk,
                                 int32_t renormalize, int32_t n_shared, int32_t* topk_ids,
                                 float* topk_w, int32_t* expert_offsets, int32_t* sorted_tokens,
                                 int32_t* slot_of, void* stream);

/*
 * cbq_codebook_lut_gemm - grouped expert GEMM with codebook weights.
 * Passage: CodeQuant2, Figure 4 (the kernel builds a table once, then reads products
 * from on-chip memory instead of multiplying) and Figure 3 (per-row centroid codebooks); the
 * AI Radio episode, "Improvements" (products looked up instead of recomputed;
 * shared-memory bank conflicts).
 *
 *  codes, scales   : quantised activations from cbq_rotate_quantize: codes
 *                    [T][K*act_bits/8] (16-byte aligned), scales fp32 [T].
 *  n_rows          : number of GEMM rows R.
 *  expert_offsets  : int32 [W->E + 1] row ranges per expert (device), or NULL: all
 *                    R rows use expert 0.
 *  row_token       : int32 [R]: row r reads token row_token[r] of codes/scales
 *                    (sorted_tokens of the router), or NULL: row r reads token r.
 *                    Every entry of a row inside an expert range must lie in [0, T),
 *                    T the number of token rows of codes and scales.  The call is not
 *                    told T, so it cannot check this: an entry outside that range
 *                    makes the kernels read outside codes and scales (caller's
 *                    contract, like the extents of every other buffer).
 *  W, n_w          : n_w == 1: one weight set; n_w == 2: {gate, up} with equal
 *                    E/N/K/bits (host pointer to the array; read during the call only).
 *  epilogue        : CBQ_EPI_F32 (n_w == 1): out[r][n] = scale[t_r] * sum_k q[t_r][k] W[e][n][k]
 *                    as fp32.  CBQ_EPI_SWIGLU_BF16 (n_w == 2): g, u as above, then
 *                    out[r][n] = bf16_rne(silu(g) * u).
 *  path            : CBQ_PATH_AUTO / CBQ_PATH_LUT / CBQ_PATH_MFMA, optionally with one
 *                    table flag, or CBQ_PATH_PAGES_PRODUCTS / CBQ_PATH_PAGES_BUCKETS.
 *                    Products are exact on every path; the paths differ only in the
 *                    fp32 summation order.
 *                    The SwiGLU epilogue is one fp32 formula on every path
 *                    (g * u * rcp(1 + exp(-g)) with the hardware exp2 and reciprocal),
 *                    so the bf16 h of two paths differs only where that summation
 *                    order moves g or u across a bf16 rounding boundary: mostly by one
 *                    bf16 step, by more only where g or u nearly cancels (the fp32
 *                    order changes them by units in the last place of their partial
 *                    sums, large against a small h).
 *  out, ldo        : fp32 or bf16 [R][ldo], ldo >= N, ldo % 4 == 0, 16-byte aligned.
 *  ws, ws_bytes    : optional device workspace (16-byte aligned; NULL / 0: none).  The GEMM
 *                    needs none.  cbq_gemm_workspace(...) is nonzero only for 4-bit
 *                    codebooks on the MFMA or AUTO path: one weight set with K >= 4096
 *                    (n_rows * N * 4 bytes), or the gate/up pair with K >= 2048 and
 *                    512 <= n_rows <= 4096 (16 * n_rows * min(N, 2048) bytes).  Given that many
 *                    bytes, an MFMA call whose 256-row tiles would leave CUs idle splits K
 *                    in two: a single matrix keeps the second half's partial sums there
 *                    and adds them to out in a second pass; the pair (in calls of at most
 *                    8 row tiles) splits the column tiles of its last, at most half-full
 *                    round of workgroups, keeps both halves' sums of g and u there, and a
 *                    second pass forms their h.  The order is fixed, so the result is
 *                    deterministic and differs from the unsplit call only in the fp32
 *                    summation order.  The workspace is scratch: its contents after the
 *                    call are unspecified, and calls that share one must not overlap.
 *  Rows of experts with no rows, and rows outside every expert range, are not written.
 *  Limits (CBQ_EUNSUPPORTED beyond them): the output is smaller than 1 GiB, one
 *  expert's index block and the codes array are smaller than 2 GiB each (the codes
 *  limit is checked only when row_token is NULL; otherwise it is the caller's).
 */
size_t cbq_gemm_workspace(const cbq_weights* W, int32_t n_w, int64_t n_rows, int32_t act_bits,
                          int32_t path);
int cbq_codebook_lut_gemm(const uint8_t* codes, const float* scales, int32_t act_bits,
                          int64_t n_rows, const int32_t* expert_offsets,
                          const int32_t* row_token, const cbq_weights* W, int32_t n_w,
                          int32_t epilogue, int32_t path, void* out, int64_t ldo, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * cbq_moe_combine - weighted sum of the expert outputs per token.
 * Passage: the AI Radio episode on CodeQuant, introduction (a mixture of experts
 * with a router); the weighting follows the router's softmax.
 *
 *  expert_out : fp32 [T*topk + n_shared*T][H] in row order (16-byte aligned, H % 4 == 0).
 *  slot_of, topk_w : from cbq_moe_route_gather.
 *  y          : fp32 [T][H]: y[t] = sum_j topk_w[t][j] * expert_out[slot_of[t][j]]
 *               (j ascending) + sum_s expert_out[T*topk + s*T + t].
 */
int cbq_moe_combine(const float* expert_out, const int32_t* slot_of, const float* topk_w,
                    int64_t T, int32_t topk, int32_t H, int32_t n_shared, float* y,
                    void* stream);

/*
 * cbq_kmeans_codebooks - offline codebook construction, one 1-D K-means per weight row.
 * Passage: CodeQuant2, Figure 3 (right: K-means initialises the centroid matrix and the
 * per-row assignment matrices); CodeQuant abstract (weight outliers absorbed into
 * cluster centroids).
 *
 *  w          : bf16 [R][ldw] weight rows (ldw >= K); row r is clustered on its own.
 *  bits       : 2, 3 or 4: L = 2^bits clusters per row.
 *  max_iters  : 0 .. 1000 centroid updates at most.
 *  idx        : [R][K*bits/8] bytes, 4-byte aligned: the assignments as the LSB-first
 *               bitstream cbq_weights uses.
 *  codebook   : fp16 [R][L]: the centroids.
 *  iters_done : optional int32 [R]: the number of updates made per row.
 *
 *  Per row: sort the values (-0 before +0); initial centroids are the values at
 *  ranks floor((2j + 1) K / (2L)); each round assigns every weight to the centroid
 *  with the smallest fp64 |w - c| (ties to the lower index) and stops if no
 *  assignment changed, else replaces every non-empty cluster's centroid by its mean
 *  (fp64 sum / count, one division).  The centroids are then rounded once to fp16
 *  and the weights are assigned against those fp16 values.  The sums are exact (so
 *  the result is deterministic) for rows whose nonzero exponents spread at most
 *  45 - ceil(log2 K) binades.  Requires K % 32 == 0, 32 <= K <= 16384.
 *  The output (idx, codebook, E = 1, N = R) is a ready cbq_weights set.
 */
int cbq_kmeans_codebooks(const uint16_t* w, int64_t R, int32_t K, int64_t ldw, int32_t bits,
                         int32_t max_iters, uint8_t* idx, uint16_t* codebook,
                         int32_t* iters_done, void* stream);

/*
 * cbq_refit_codebooks - output-aware refit of clustered rows' centroids on calibration
 * activations, assignments fixed.  Passage: the AI Radio episode on CodeQuant (the
 * centroids are fine-tuned to minimise the error of the layer's output, looking at how
 * the weights meet the activations); CodeQuant2, Figure 1 (right: centroids tuned after
 * clustering).
 *
 *  w        : bf16 [R][ldw] original weight rows (ldw >= K).
 *  idx      : [R][K*bits/8] the rows' assignments (LSB-first bitstream, as cbq_weights).
 *  x        : bf16 [n][ldx] calibration activations (1 <= n <= 256, ldx >= K).
 *  codebook : fp16 [R][2^bits], 2-byte aligned; read as the current centroids and
 *             overwritten with the refit ones.
 *
 *  Per row, with P[i][j] = sum over k assigned to j of x[i][k] and y = x w: solve
 *  (P^T P) c = P^T y over the non-empty clusters by Cholesky in index order; a cluster
 *  whose pivot is at most 1e-12 of the largest diagonal entry keeps its centroid (its
 *  share P c moves to the right-hand side) and the factorisation restarts without it;
 *  empty clusters keep theirs.  The sums run in fp64; each new centroid is rounded once
 *  to fp16.  Requires K % 32 == 0, 32 <= K <= 16384, bits in 2..4.
 */
int cbq_refit_codebooks(const uint16_t* w, int64_t R, int32_t K, int64_t ldw, int32_t bits,
                        const uint8_t* idx, const uint16_t* x, int32_t n, int64_t ldx,
                        uint16_t* codebook, void* stream);

/*
 * cbq_cpu_lut_gemm - the same codebook-LUT GEMM on host cores (x86-64 with AVX2, FMA,
 * F16C and BMI2).  Passage: CodeQuant abstract (dedicated kernels for GPU and CPU) and the
 * AI Radio episode, "Improvements" (a CPU speedup from looking products up).
 *
 *  All pointers are HOST memory; the call is synchronous and returns when out is
 *  written.  codes/scales as for cbq_codebook_lut_gemm (row t reads token t);
 *  W: one weight set (E = 1) with host pointers; out fp32 [T][ldo], ldo >= N.
 *  out[t][n] = scales[t] * sum_k q[t][k] * C[n][idx(n, k)]: every product is exact in
 *  fp32, the fp32 summation order differs from the definition.
 *  n_threads: rows are split over that many threads (0 = all hardware threads).
 *  flags: 0, or CBQ_CPU_NO_AVX512 to keep to the AVX2 kernel on a CPU with AVX-512F
 *  (which otherwise gets a variant looking up 16 fp32 centroids per instruction).
 *  CBQ_EUNSUPPORTED when the CPU lacks the instructions.
 */
#define CBQ_CPU_NO_AVX512 1
int cbq_cpu_lut_gemm(const uint8_t* codes, const float* scales, int32_t act_bits, int64_t T,
                     const cbq_weights* W, float* out, int64_t ldo, int32_t n_threads,
                     int32_t flags);

/* Name of a status code, and the calling thread's message for its last failure. */
const char* cbq_status_string(int status);
const char* cbq_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int cbq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CBQ_H */
