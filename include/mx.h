/*
 * mx.h -- C ABI of libmx355, the MXFP4 quantize-then-contract path on AMD
 * MI355X (gfx950).
 *
 * The path is the one the pages train a mixture-of-experts LLM with
 * ("Training an MoE LLM in MXFP4: How We Closed the Gap to BF16", Abstract):
 * hybrid 1D/2D block quantization to MXFP4 -- E2M1 elements with one UE8M0
 * power-of-two scale per block ("AMD's ALTO Gets 4-Bit MoE Training to
 * Within 0.007 of BF16", section "What ALTO Actually Does") -- an optional
 * randomized Hadamard transform (RHT) along the reduction dimension,
 * round-to-nearest-even or stochastic rounding, and the expert GEMM over the
 * quantized operands, accumulated in FP32.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, never frees, never synchronises and keeps no state; it
 *     is safe to call from several host threads on different streams.
 *   - Every call validates its arguments on the host first.  On any status
 *     other than MX_OK nothing was launched.  Kernels run asynchronously on
 *     `stream` (0 = the null stream); a device fault surfaces at the caller's
 *     next synchronisation.
 *   - Element code nibble (OCP MX v1.0, FP4 E2M1): bit 3 sign, bits 2..1
 *     exponent, bit 0 mantissa; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.  Two
 *     codes per byte, the even element in the low nibble.
 *   - Scale byte (UE8M0): value 2^(byte - 127); 0xFF marks a block whose amax
 *     is NaN or Inf (after the RHT, when one is applied); such a block's codes
 *     are all 0.
 *   - Block scale: X = floor(log2(amax)) - 2, clamped to [-127, 127], so amax
 *     maps into [4, 8) and values in (6, 8) * 2^X saturate to 6 (OCP MX v1.0).
 *   - Round to nearest: ties go to the even code; |v| > 6 saturates to 6; the
 *     sign bit is kept when the magnitude rounds to 0.
 *   - Stochastic rounding (SR): with v = x / 2^X, lo <= |v| < hi neighbours on
 *     the E2M1 grid and D = floor(2^16 (|v| - lo) / (hi - lo)), the magnitude
 *     rounds up iff r16 < D, where r16 is 16 random bits of Philox4x32-10
 *     (Salmon et al., SC'11): for element index i, counter
 *     (g lo, g hi, stream_id, 0) with g = i >> 3, key (seed lo, seed hi),
 *     output word (i & 7) >> 1, its low half for even i, high half for odd i.
 *     The element index is index_base + the element's position in the
 *     quantized logical matrix (row-major, blocks along its last axis), so a
 *     tensor quantized in row slices, each with its own index_base, gives
 *     bit-identical results to the whole tensor.
 *   - RHT of a 32-block: y = c * H32 * (s .* x), H32 the Sylvester Hadamard
 *     matrix (H[i][j] = (-1)^popcount(i & j)), s_j = -1 where bit j of
 *     sign_mask is set, c = fp32(2^-2.5); computed in fp32 as butterfly stages
 *     h = 1, 2, 4, 8, 16 (pairs (i, i+h) -> (a+b, a-b)) then one multiply by
 *     c.  The stage order is part of the contract.  Inverse: butterflies,
 *     times c, then the sign flips.
 */
#ifndef MX355_MX_H
#define MX355_MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_NULL = 1,         /* a required pointer is NULL                  */
    MX_ERR_SHAPE = 2,        /* a size is negative / not a multiple of 32 / inconsistent */
    MX_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned             */
    MX_ERR_DTYPE = 4,        /* unsupported element type                     */
    MX_ERR_UNSUPPORTED = 5,  /* a valid but unimplemented option combination */
    MX_ERR_LAUNCH = 6        /* the HIP runtime rejected a kernel launch     */
} mx_status;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;
typedef enum { MX_RNE = 0, MX_SR = 1 } mx_round;

/* Scale storage orders (flags).
 * Row-major, the default: the scale of block c of row r of an R x C grid of
 *   32-element blocks is byte r*C + c.
 * MX_SCALES_STAGED: the order the grouped GEMM's K loop consumes.  Blocks
 *   8s .. 8s+7 of a row form stage s (256 elements of K); stages are stored
 *   one after another, each holding 8 bytes for every row: the scale of
 *   block 8s + j of row r is byte (s*R + r)*8 + j.  Slots of blocks past the
 *   row's last block are padding, left unwritten by the quantizers and
 *   ignored by the GEMM.  In the column-wise grouped layout each group's
 *   padded blocks start a stage of their own: block j of group g is slot
 *   j % 8 of stage S_g + j / 8, with S_g the sum over the groups before g of
 *   ceil(B / 8) and B a group's padded block count (ceil32(n) / 32).
 *   It holds the same bytes as the row-major order.  It exists so that one K
 *   stage of a 256-row GEMM tile is 2 KiB of contiguous memory, read by a
 *   few whole-line requests, instead of 256 separate 8-byte pieces, one
 *   memory request each.
 * MX_SCALES_B_2D: the GEMM's B operand has 2D (32x32) scales.
 * MX_GROUPS_PAD256 (column-wise quantize only): each group's token segment
 *   is zero-padded to a multiple of 256 tokens instead of 32, so every K
 *   stage of the weight-gradient GEMM starts on a whole 128-byte line of
 *   codes (its group offsets are then the 256-padded starts). */
enum { MX_SCALES_B_2D = 1, MX_SCALES_STAGED = 2, MX_GROUPS_PAD256 = 4 };

/* HIP stream handle (hipStream_t) passed as an opaque pointer. */
typedef void* mx_stream;

/* Library version (monotone integer). */
int mx_version(void);

/* Human-readable name of a status code (static storage). */
const char* mx_status_str(mx_status s);

/* The RHT sign mask for a seed: word 0 of Philox4x32-10 at counter 0 under
 * key (seed lo, seed hi).  Bit j set means element j of every 32-block has
 * its sign flipped before the Walsh-Hadamard butterflies: the random-sign
 * diagonal of the randomized Hadamard transform the recipe applies before
 * quantizing (Abstract of "Training an MoE LLM in MXFP4: How We Closed the
 * Gap to BF16").  Host function; no device work, cannot fail. */
uint32_t mx_rht_sign_mask(uint64_t seed);

/* Randomized Hadamard transform of every 32-block along the last axis.
 * x: [rows x cols] row-major, type xt (fp32 or bf16); y: [rows x cols] fp32.
 * cols % 32 == 0; rows >= 0 (0 launches nothing).  x and y may not overlap.
 * inverse != 0 applies the inverse transform.
 * Pages: the RHT the recipe layers on the quantizer (Abstract of "Training an
 * MoE LLM in MXFP4"). */
mx_status mx_rht(const void* x, mx_dtype xt, float* y, int64_t rows, int64_t cols,
                 uint32_t sign_mask, int inverse, mx_stream stream);

/* 1x32 MXFP4 quantization (the "1D" half of the hybrid scheme, used for
 * activations and gradients).
 *
 * block_axis = 1 (row-wise): x [rows x cols], cols % 32 == 0.  Blocks of 32
 *   run along cols.  codes [rows x cols/2] with rows codes_ld bytes apart
 *   (0 = cols/2; else at least cols/2 and a multiple of 16, so the rows can
 *   be padded to whole 128-byte lines for the GEMM), scales [rows x cols/32].
 *   group_offsets and row_index must be NULL, num_groups 0, kp 0 (a
 *   row_index here returns MX_ERR_UNSUPPORTED).
 * block_axis = 0 (column-wise, grouped): the rows of x (tokens) are split
 *   into num_groups groups by group_offsets (DEVICE int32[num_groups+1],
 *   non-decreasing, [0] = 0, [num_groups] = rows; produced on the device by
 *   routing).  Each group is zero-padded to a multiple of 32 tokens and the
 *   result is written transposed, so the token axis is contiguous:
 *   Q [cols x kp] with Q[c][P_g + r] = x[off_g + r][c], P_g the padded start
 *   of group g.  codes [cols x kp/2], scales [cols x kp/32].  kp (a multiple
 *   of 32) is the capacity of that axis; the caller guarantees
 *   kp >= sum_g ceil32(n_g) (rows + 31 * num_groups always suffices).
 *   Positions beyond the padded total are not written.  codes_ld: 0 or kp/2.
 *   row_index (optional, DEVICE int32[rows]): the rows are gathered, so the
 *   token at grouped position p is x[row_index[p]] (x itself may have any
 *   number of rows; every index must be a valid row of it).  This fuses the
 *   permutation of tokens into expert order with the quantization: no
 *   permuted copy of x is written.  NULL: position p is x[p].
 *   One row of x must span at most 4 GiB - 1 bytes (else MX_ERR_SHAPE).
 * block_axis | MX_SCALES_STAGED: the scales in the staged order.  Row-wise:
 *   R = rows, scales holds ceil(cols/256) * rows * 8 bytes.  Column-wise:
 *   per-group stages, R = cols, scales holds (kp/256 + num_groups) * cols * 8
 *   bytes.  Padding slots are not written.
 * block_axis = 0 | MX_GROUPS_PAD256 (may be combined with the staged flag):
 *   groups padded to multiples of 256 tokens (ceil256 in place of ceil32
 *   above; kp >= sum_g ceil256(n_g), rows + 255 * num_groups always
 *   suffices).  Row-wise: MX_ERR_SHAPE.
 * use_rht != 0 applies the RHT (sign_mask) to each block before quantizing.
 * rnd: MX_RNE or MX_SR (seed, stream_id, index_base as above; index_base %
 *   32 == 0).
 * x may be fp32 or bf16; pointers 16-byte aligned except scales (any).
 * Pages: hybrid 1D/2D quantization, RHT and SR (Abstract of "Training an MoE
 * LLM in MXFP4"); E2M1 + UE8M0 ("What ALTO Actually Does"). */
mx_status mx_quantize_1d(const void* x, mx_dtype xt, int64_t rows, int64_t cols,
                         int block_axis, const int32_t* group_offsets, int32_t num_groups,
                         int64_t kp, const int32_t* row_index, int use_rht, uint32_t sign_mask, mx_round rnd,
                         uint64_t seed, uint32_t stream_id, uint64_t index_base,
                         uint8_t* codes, int64_t codes_ld, uint8_t* scales, mx_stream stream);

/* Both 1x32 quantizations of one token-major tensor from a single read: the
 * column-wise, grouped layout (per-group padded, transposed, with the
 * optional RHT; the weight-gradient operand) and the row-wise layout (1x32
 * blocks along cols, never with the RHT; the data-gradient or forward
 * operand).  The expert tensors dominate memory traffic as well as compute
 * ("What ALTO Actually Does", news digest "AMD's ALTO Gets 4-Bit MoE
 * Training to Within 0.007 of BF16"), and the recipe quantizes the same
 * activation and gradient tensors once per GEMM that consumes them
 * (Abstract of "Training an MoE LLM in MXFP4": 1D blocks, RHT and SR).
 * The outputs are bit for bit those of
 *   mx_quantize_1d(x, block_axis = 0, group_offsets, num_groups, kp, NULL,
 *                  use_rht, sign_mask, col_rnd, seed, col_stream_id,
 *                  col_index_base, col_codes, 0, col_scales) and
 *   mx_quantize_1d(x, block_axis = 1, ..., use_rht = 0, row_rnd, seed,
 *                  row_stream_id, row_index_base, row_codes, row_codes_ld,
 *                  row_scales);
 * the rows of x are the grouped positions (no row gather).  Row-wise codes
 * [rows x cols/2] at pitch row_codes_ld (0 = cols/2), scales
 * [rows x cols/32].  layout_flags: 0, or MX_SCALES_STAGED (both outputs'
 * scales in the staged order: column-wise [kp/256 + num_groups][cols][8],
 * row-wise [ceil(cols/256)][rows][8]) and/or MX_GROUPS_PAD256 (the
 * column-wise output's groups padded to 256 tokens), exactly as those flags
 * act in the two mx_quantize_1d calls above; other bits:
 * MX_ERR_UNSUPPORTED.  Arguments, layouts and errors otherwise as
 * mx_quantize_1d. */
mx_status mx_quantize_1d_dual(const void* x, mx_dtype xt, int64_t rows, int64_t cols,
                              const int32_t* group_offsets, int32_t num_groups, int64_t kp, int use_rht,
                              uint32_t sign_mask, mx_round col_rnd, uint32_t col_stream_id,
                              uint64_t col_index_base, uint8_t* col_codes, uint8_t* col_scales,
                              mx_round row_rnd, uint32_t row_stream_id, uint64_t row_index_base,
                              uint8_t* row_codes, int64_t row_codes_ld, uint8_t* row_scales, uint64_t seed,
                              int layout_flags, mx_stream stream);

/* 32x32 MXFP4 quantization, round to nearest even (the "2D" half of the
 * hybrid scheme, used for weights).  w: batch x [rows x cols], rows % 32 ==
 * 0, cols % 32 == 0.  One pass writes the as-given layout (codes
 * [batch x rows x cols/2], scales [batch x rows/32 x cols/32]) and/or the
 * transposed layout (codes_t [batch x cols x rows/2], scales_t
 * [batch x cols/32 x rows/32]); a 32x32 block has the same scale and codes in
 * both, so the transposed pair is exactly the quantization of w^T.  Either
 * pair may be NULL (not both).  codes_ld / codes_t_ld: bytes from one code
 * row to the next in each layout (0 = cols/2 and rows/2; else at least that
 * and a multiple of 16); a batch entry spans rows (cols) such rows.  An
 * empty input (batch, rows or cols 0) returns MX_OK before any pointer is
 * checked.
 * Pages: "What ALTO Actually Does" (UE8M0 per block), Abstract (hybrid
 * 1D/2D). */
mx_status mx_quantize_2d(const void* w, mx_dtype wt, int64_t batch, int64_t rows, int64_t cols,
                         uint8_t* codes, int64_t codes_ld, uint8_t* scales, uint8_t* codes_t,
                         int64_t codes_t_ld, uint8_t* scales_t, mx_stream stream);

/* Study variants of the row-wise 1x32 quantizer, for measuring
 * operator-level SNR: outlier clipping and macro-block scaling.  Both are
 * named among the techniques that improved operator-level SNR yet failed
 * end to end (Abstract of "Training an MoE LLM in MXFP4"; "The Numbers" in
 * the news digest "AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of
 * BF16"); the pages define neither.  The readings:
 *   - clip_ratio rho in (0, 1]: a block's scale is chosen for
 *     fl32(rho * amax) instead of amax, X = floor(log2(fl32(rho * amax)))
 *     - 2, so its largest values saturate at +-6 * 2^X while the others get
 *     a finer grid; rho = 1 is mx_quantize_1d's rule; rho = 0 selects a
 *     search instead: a block takes X - 1 rather than the rule's X when
 *     that strictly lowers its squared round-to-nearest-even error, each
 *     candidate's error summed in fp64 in its own units (eight elements in
 *     order per quarter of the block, then the four quarters in order),
 *     X - 1 winning iff S(X - 1) < 4 S(X);
 *   - macro_block Bm (0 = none; else a multiple of 32 dividing cols): each
 *     Bm consecutive elements of a row (after the RHT, when on) are
 *     multiplied by r = fl32(6 / amax_M), their fp32 macro scale (r = 1
 *     when amax_M is 0 or not finite, or 6 / amax_M is not finite), and the
 *     products y' = fl32(y * r) are quantized in 1x32 blocks as usual.  A
 *     decoded element is deq(code, scale) / r (mx_dequantize_1d_ex).
 * x [rows x cols] (fp32 or bf16), row-major, 16-byte aligned; codes
 * [rows x cols/2] (contiguous, 16-byte aligned), scales [rows x cols/32];
 * macro_r [rows x cols/Bm] fp32 (written; required when Bm > 0).
 * use_rht, sign_mask, rnd, seed, stream_id and index_base as in
 * mx_quantize_1d (row-wise).  Device pointers owned by the caller.
 * Errors: MX_ERR_DTYPE, MX_ERR_UNSUPPORTED (rnd), MX_ERR_SHAPE (sizes,
 * clip_ratio outside [0, 1], macro_block), MX_ERR_NULL, MX_ERR_ALIGN,
 * MX_ERR_LAUNCH.  rows == 0 launches nothing. */
mx_status mx_quantize_1d_ex(const void* x, mx_dtype xt, int64_t rows, int64_t cols, int use_rht,
                            uint32_t sign_mask, mx_round rnd, uint64_t seed, uint32_t stream_id,
                            uint64_t index_base, float clip_ratio, int64_t macro_block, uint8_t* codes,
                            uint8_t* scales, float* macro_r, mx_stream stream);

/* Decode of mx_quantize_1d_ex's output to fp32: y = deq(code, scale) / r,
 * the quotient rounded once (r = 1 when macro_block is 0; macro_r may then
 * be NULL); a 0xFF scale decodes to NaN.  codes [rows x cols/2] contiguous,
 * y [rows x cols] fp32, both 16-byte aligned.  Errors as
 * mx_quantize_1d_ex. */
mx_status mx_dequantize_1d_ex(const uint8_t* codes, const uint8_t* scales, const float* macro_r,
                              int64_t rows, int64_t cols, int64_t macro_block, float* y,
                              mx_stream stream);

/* 32x32 quantization of a weight tensor with weight de-oscillation: a
 * hysteresis band against the previous step's quantized weights.
 * Pages: "What ALTO Actually Does" (news digest "AMD's ALTO Gets 4-Bit MoE
 * Training to Within 0.007 of BF16") describes the oscillation: the
 * optimizer moves a full-precision master weight while the GEMM consumes
 * its quantized value, so a weight near a rounding boundary can alternate
 * between two levels under updates much smaller than a level step; the
 * Abstract of "Training an MoE LLM in MXFP4" names a simplified
 * de-oscillation scheme without giving its rule.  The rule here: the tile's
 * scale byte comes from its amax as in mx_quantize_2d, except that when
 * that is one below the previous byte p (p != 0xFF) and the amax is at
 * least (4 - margin64 / 16) 2^(p - 127), the tile keeps p (its elements
 * still fit without clipping; the digest's case of a block whose shared
 * scale, set by an outlier, moves every value of the block); if the byte
 * then equals the previous one (neither 0xFF), an element keeps its
 * previous code c while
 * its scaled value v = w / 2^X lies strictly inside
 * (q - f (q - q_dn), q + f (q_up - q)), q the value of c on the signed E2M1
 * grid {-6, ..., -0.5, 0, 0.5, ..., 6} (both zero codes are 0), q_dn / q_up
 * its neighbours there (the band is open past +-6), f = 1/2 + margin64 / 64;
 * otherwise it takes its round-to-nearest-even code (at the tile's byte),
 * as does every element of a tile whose scale changed.  margin64 = 0
 * leaves every decoded value equal to mx_quantize_2d's.
 * w: batch x [rows x cols] (fp32 master weights, or bf16), rows % 32 == 0,
 * cols % 32 == 0; margin64 in [0, 31].
 * prev_codes / prev_scales: the as-given layout written for the previous
 * step (rows prev_codes_ld bytes apart, 0 = cols/2); they may be the very
 * buffers codes / scales (in-place update, then with the same pitch).
 * codes / scales: the as-given layout (required); codes_t / scales_t: the
 * transposed layout (optional pair), as in mx_quantize_2d.
 * flips (optional, uint16 [batch x rows/32 x cols/32], 2-byte aligned): per
 * tile, the number of elements whose decoded value differs from the
 * previous one (a 0xFF scale on either side counts all 1024).
 * Device pointers owned by the caller; code pointers 16-byte aligned.
 * Errors: MX_ERR_DTYPE, MX_ERR_SHAPE (sizes, margin64, pitches, an in-place
 * call with a different pitch), MX_ERR_NULL, MX_ERR_ALIGN, MX_ERR_LAUNCH.
 * An empty input returns MX_OK before any pointer is checked. */
mx_status mx_quantize_2d_deosc(const void* w, mx_dtype wt, int64_t batch, int64_t rows, int64_t cols,
                               const uint8_t* prev_codes, int64_t prev_codes_ld, const uint8_t* prev_scales,
                               int margin64, uint8_t* codes, int64_t codes_ld, uint8_t* scales, uint8_t* codes_t,
                               int64_t codes_t_ld, uint8_t* scales_t, uint16_t* flips, mx_stream stream);

/* Exact decode of MXFP4: each E2M1 element times the UE8M0 power-of-two
 * scale its block shares (the format named in "What ALTO Actually Does",
 * news digest "AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of
 * BF16"), i.e.
 * y = (-1)^s * E2M1[m] * 2^(byte - 127); a block with scale byte 0xFF
 * decodes to NaN.
 * codes batch x [rows x cols/2], rows codes_ld bytes apart (0 = cols/2;
 * else at least that and a multiple of 16); block_rows = 1 (scales [rows x cols/32]) or
 * 32 (scales [rows/32 x cols/32], rows % 32 == 0); y batch x [rows x cols],
 * yt fp32 or bf16 (every decoded value is exact in both, except 6*2^(>=127)
 * which overflows to Inf).  cols % 32 == 0.  Pointers are device pointers
 * owned by the caller; codes and y 16-byte aligned, scales any.
 * Errors: MX_ERR_DTYPE (yt), MX_ERR_SHAPE (sizes, block_rows, codes_ld),
 * MX_ERR_NULL, MX_ERR_ALIGN, MX_ERR_LAUNCH.  An empty input returns MX_OK
 * before any pointer is checked. */
mx_status mx_dequantize(const uint8_t* codes, int64_t codes_ld, const uint8_t* scales, int64_t batch, int64_t rows,
                        int64_t cols, int block_rows, void* y, mx_dtype yt, mx_stream stream);

/* Grouped MXFP4 GEMM with FP32 accumulation: per group,
 *   C = alpha * deq(A) . deq(B)^T,
 * both operands K-contiguous (codes [. x K/2], scales [. x K/32]).
 * Both operands enter as MXFP4 codes and scales: the contraction consumes
 * the quantized values, never the master values ("What ALTO Actually Does").
 * a_ld, b_ld: bytes from one code row of A (of B) to the next; 0 means K/2
 * (contiguous rows).  Otherwise at least K/2 and a multiple of 16.  Rows
 * padded to a multiple of 128 bytes are read as whole cache lines, which is
 * markedly faster when K/2 is not a multiple of 128.  Scales are always
 * contiguous.
 *
 * group_dim_k = 0 (forward / data gradient): groups split the M rows of C by
 *   group_offsets (DEVICE int32[num_groups+1], [0] = 0, [num_groups] = M).
 *   Row m of group g reads A row a_row_index[m] (DEVICE int32[M]; NULL = m)
 *   and multiplies B_g = b_codes + g*N*b_ld ([N x K]); MX_SCALES_B_2D in
 *   scale_flags selects 2D scales [N/32 x K/32] per group (else 1D
 *   [N x K/32]).  C [M x N].
 * group_dim_k = 1 (weight gradient): groups split K by group_offsets (DEVICE,
 *   multiples of 32, [num_groups] <= K); A [M x K], B [N x K], 1D scales;
 *   C [num_groups x M x N]; a group with an empty K range writes zeros.
 * scale_flags: MX_SCALES_B_2D and/or MX_SCALES_STAGED.  Staged: with groups
 *   along K, A's and B's scales are in the staged order with per-group
 *   stages (R = M, resp. N; group g's blocks are those of its K range, as
 *   mx_quantize_1d(block_axis = 0 | MX_SCALES_STAGED) writes them when
 *   group_offsets are its padded group starts); needs num_groups < 64.  With
 *   groups along M, A's scales are staged (R = M, one stage grid over K);
 *   needs MX_SCALES_B_2D and no row index.  Staged scale pointers 4-byte
 *   aligned, and (K/256 + num_groups + 1) * 8 * R below 4 GiB.
 * K % 32 == 0, N % 32 == 0, M >= 0; ct = MX_BF16 (round to nearest even) or
 * MX_F32.  Code and C pointers 16-byte aligned.  The kernel addresses each
 * operand with 32-bit byte offsets: N*b_ld (one B group) and, without a row
 * index, M*a_ld must not exceed 4 GiB - 1 (else MX_ERR_SHAPE); with a row
 * index the indexed rows must lie within the first 4 GiB of a_codes.
 * Errors: MX_ERR_DTYPE (ct), MX_ERR_SHAPE (sizes, row pitches, num_groups
 * < 1, group_dim_k), MX_ERR_UNSUPPORTED (group_dim_k = 1 with 2D B scales or a row
 * index; unknown scale_flags bits; staged scales outside the cases above),
 * MX_ERR_NULL, MX_ERR_ALIGN, MX_ERR_LAUNCH.  M == 0 launches nothing. */
mx_status mx_grouped_gemm(const uint8_t* a_codes, int64_t a_ld, const uint8_t* a_scales,
                          const int32_t* a_row_index,
                          const uint8_t* b_codes, int64_t b_ld, const uint8_t* b_scales, int scale_flags,
                          const int32_t* group_offsets, int32_t num_groups, int group_dim_k,
                          int64_t M, int64_t N, int64_t K, float alpha,
                          void* c, mx_dtype ct, mx_stream stream);

/* mx_grouped_gemm with groups splitting M (group_dim_k = 0) and the output
 * also emitted as the next layer's MXFP4 operand: with y = RNE_bf16(alpha *
 * A . B^T) per row, c_codes [M x N/2] and c_scales [M x N/32] are the
 * row-wise 1x32 quantization of y along N, round to nearest even, bit for
 * bit what mx_quantize_1d(y, MX_BF16, M, N, block_axis = 1, use_rht = 0,
 * MX_RNE) writes.  The quantizer is fused into the GEMM's epilogue, so y
 * need not make a round trip through memory: the expert layers dominate
 * memory traffic as well as compute ("What ALTO Actually Does", news digest
 * "AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of BF16").
 * c: bf16 [M x N] as in mx_grouped_gemm, or NULL to write only the MXFP4
 * output.  c_codes_ld: the code rows' pitch in bytes (0 = N/2, else >= N/2
 * and a multiple of 16); the bytes between N/2 and the pitch are not
 * written.  c (when given) and c_codes 16-byte aligned; c_scales any.
 * Arguments and errors otherwise as mx_grouped_gemm; additionally
 * MX_ERR_NULL (c_codes or c_scales NULL), MX_ERR_SHAPE (c_codes_ld below
 * N/2, or M * c_codes_ld above 4 GiB - 1) and MX_ERR_ALIGN (c_codes_ld not
 * a multiple of 16). */
mx_status mx_grouped_gemm_q(const uint8_t* a_codes, int64_t a_ld, const uint8_t* a_scales,
                            const int32_t* a_row_index,
                            const uint8_t* b_codes, int64_t b_ld, const uint8_t* b_scales, int scale_flags,
                            const int32_t* group_offsets, int32_t num_groups,
                            int64_t M, int64_t N, int64_t K, float alpha,
                            void* c, uint8_t* c_codes, int64_t c_codes_ld, uint8_t* c_scales,
                            mx_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MX355_MX_H */
