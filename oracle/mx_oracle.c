/*
 * mx_oracle.c -- plain CPU oracle for the MXFP4 quantize-then-contract path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  It exists so that tests, the smoke check and the
 * CPU-baseline leg of the bench can compare the GPU library against a slow,
 * obviously-correct implementation written from the definitions.  It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * What it follows
 *   - "Training an MoE LLM in MXFP4: How We Closed the Gap to BF16", Abstract:
 *     MXFP4 training with hybrid 1D/2D block quantization, a randomized
 *     Hadamard transform (RHT) and stochastic rounding (SR); the experiments
 *     ran "simulated" MXFP4 kernels, i.e. quantize -> dequantize -> a
 *     high-precision GEMM, which is what oracle_grouped_gemm does in FP64.
 *   - "AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of BF16",
 *     section "What ALTO Actually Does": the format is E2M1 elements with one
 *     UE8M0 scale per block; the expert GEMM consumes the quantized operands,
 *     not the master values; one outlier sets the shared scale of its whole
 *     block.
 *   - OCP Microscaling Formats (MX) Specification v1.0: E2M1 magnitudes
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}, E8M0 scale with bias 127 (0xFF = NaN),
 *     block size 32, shared exponent floor(log2(amax)) - 2 for E2M1
 *     (2 = the largest exponent of an E2M1 normal), saturating conversion.
 *   - Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
 *     3", SC'11: Philox4x32 with 10 rounds.
 *
 * Readings where the sources are silent (each is listed in the design notes):
 *   - the RHT of one 32-block is y = c * H32 * (s .* x) in fp32, H32 the
 *     Sylvester (natural-order) Hadamard matrix, s the sign vector given by
 *     the bits of a 32-bit mask (bit j flips element j), c = fp32(2^-2.5),
 *     butterfly stages in the order h = 1, 2, 4, 8, 16, then one multiply by
 *     c.  fp32 sums are not associative, so this order is part of the
 *     contract.  The inverse is butterflies, times c, then the sign flips.
 *   - ties of round-to-nearest go to the even code; |v| > 6 saturates to 6;
 *     the sign bit is kept for results of magnitude 0.
 *   - SR rounds the magnitude up with probability D / 2^16,
 *     D = floor(2^16 * (|v| - lo) / (hi - lo)), by the rule r16 < D, where
 *     r16 is 16 random bits taken from Philox4x32-10 for that element.
 *   - the random bits of element i (its 64-bit index in the quantized
 *     logical matrix plus a caller base) come from the Philox call with
 *     counter (g lo, g hi, stream, 0), g = i >> 3, key (seed lo, seed hi):
 *     word (i & 7) >> 1, low half when i is even, high half when odd.
 *   - a block whose amax is NaN or Inf gets scale byte 0xFF; its codes are
 *     written as 0 and carry no meaning.
 *
 * Build: plain C99, -O2 -ffp-contract=off, no fast-math.  Every float step
 * that decides a code is done in the precision the contract names (fp32 for
 * the RHT, exact double arithmetic elsewhere).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

/* E2M1 magnitude for each 3-bit magnitude code (OCP MX v1.0, FP4 E2M1). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int oracle_version(void) { return 1; }

double oracle_decode(uint8_t code, uint8_t scale_byte);

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11).                               */
/* ------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;  /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;  /* Weyl key bumps    */
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The RHT sign mask: word 0 of Philox4x32-10 at counter 0 under key = seed. */
uint32_t oracle_rht_sign_mask(uint64_t seed)
{
    uint32_t ctr[4] = {0, 0, 0, 0};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[0];
}

/* 16 random bits for element index i (see the header comment). */
uint32_t oracle_sr_bits(uint64_t seed, uint32_t stream, uint64_t i)
{
    uint64_t g = i >> 3;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream, 0};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    uint32_t word = w[(i & 7) >> 1];
    return (i & 1) ? (word >> 16) : (word & 0xFFFFu);
}

/* ------------------------------------------------------------------ */
/* Randomized Hadamard transform of one 32-block, fp32.                */
/* ------------------------------------------------------------------ */
static float rht_c32(void)
{
    /* fp32 nearest to 2^-2.5 = 1/sqrt(32); 1/sqrt(32) is computed in double
     * and rounded once (a test checks this is the nearest fp32). */
    return (float)(1.0 / sqrt(32.0));
}

static void fwht32_f32(float t[32])
{
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float a = t[i], b = t[i + h];
            volatile float s = a + b;   /* volatile: one rounding per op */
            volatile float d = a - b;
            t[i] = s;
            t[i + h] = d;
        }
    }
}

static void flip_signs(float t[32], uint32_t mask)
{
    for (int j = 0; j < 32; ++j)
        if ((mask >> j) & 1u) t[j] = -t[j];
}

/* y = c * H * (s .* x)  (inverse != 0: x = s .* (c * H * y)) */
void oracle_rht_block(const float in[32], float out[32], uint32_t mask, int inverse)
{
    float t[32];
    const float c = rht_c32();
    memcpy(t, in, sizeof(t));
    if (!inverse) flip_signs(t, mask);
    fwht32_f32(t);
    for (int j = 0; j < 32; ++j) {
        volatile float p = t[j] * c;
        t[j] = p;
    }
    if (inverse) flip_signs(t, mask);
    memcpy(out, t, sizeof(t));
}

/* ------------------------------------------------------------------ */
/* Element widening.  dtype 0 = fp32, 1 = bf16 (exact widening).       */
/* ------------------------------------------------------------------ */
static float load_elem(const void* x, int dtype, int64_t idx)
{
    if (dtype == 0) return ((const float*)x)[idx];
    uint16_t h = ((const uint16_t*)x)[idx];
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------ */
/* Scale, rounding and encoding of one block.                           */
/* ------------------------------------------------------------------ */

/* UE8M0 scale byte for a block amax: X = floor(log2 amax) - 2 clamped to
 * [-127, 127]; 0 for amax = 0; 0xFF for NaN / Inf.  floor(log2) comes from
 * frexp, which is exact. */
uint8_t oracle_scale_byte(double amax)
{
    if (isnan(amax) || isinf(amax)) return 0xFF;
    if (amax == 0.0) return 0;
    int e;
    (void)frexp(amax, &e);          /* amax = f * 2^e, f in [0.5, 1) */
    int floor_log2 = e - 1;
    int X = floor_log2 - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    return (uint8_t)(X + 127);
}

/* Round-to-nearest, ties to the even code, saturating at 6.  A >= 0. */
int oracle_rtne_mag(double A)
{
    if (A >= 6.0) return 7;
    int m0 = 0;
    while (m0 < 7 && E2M1_MAG[m0 + 1] <= A) ++m0;
    double lo = E2M1_MAG[m0], hi = E2M1_MAG[m0 + 1];
    double dlo = A - lo, dhi = hi - A;   /* exact: A has <= 24 significant bits */
    if (dlo < dhi) return m0;
    if (dhi < dlo) return m0 + 1;
    return (m0 % 2 == 0) ? m0 : m0 + 1;  /* tie: the even code */
}

/* Stochastic rounding of the magnitude with 16 random bits.  A >= 0. */
int oracle_sr_mag(double A, uint32_t r16)
{
    if (A >= 6.0) return 7;
    int m0 = 0;
    while (m0 < 7 && E2M1_MAG[m0 + 1] <= A) ++m0;
    double lo = E2M1_MAG[m0], hi = E2M1_MAG[m0 + 1];
    double d = (A - lo) / (hi - lo);            /* exact: step is a power of 2 */
    uint32_t D = (uint32_t)floor(d * 65536.0);  /* exact */
    return (r16 < D) ? m0 + 1 : m0;
}

/* Quantize one block of n values v[] (already transformed).  rnd: 0 RTNE,
 * 1 SR with random bits r16[].  Writes n 4-bit codes to code[] (one per
 * entry, not yet packed) and returns the scale byte. */
static uint8_t quantize_block(const float* v, int n, int rnd, const uint32_t* r16,
                              uint8_t* code)
{
    double amax = 0.0;
    int nonfinite = 0;
    for (int j = 0; j < n; ++j) {
        if (isnan(v[j]) || isinf(v[j])) nonfinite = 1;
        double a = fabs((double)v[j]);
        if (a > amax) amax = a;
    }
    if (nonfinite) {
        for (int j = 0; j < n; ++j) code[j] = 0;
        return 0xFF;
    }
    uint8_t byte = oracle_scale_byte(amax);
    int X = (int)byte - 127;
    for (int j = 0; j < n; ++j) {
        double s = ldexp((double)v[j], -X);       /* exact in double */
        double A = fabs(s);
        int m = (rnd == 0) ? oracle_rtne_mag(A) : oracle_sr_mag(A, r16[j]);
        int sign = signbit(v[j]) ? 1 : 0;
        code[j] = (uint8_t)((sign << 3) | m);
    }
    return byte;
}

/* ------------------------------------------------------------------ */
/* 1D quantize.                                                         */
/*                                                                      */
/* block_axis = 1: x [rows x cols]; the quantized logical matrix Q is   */
/*   x itself; 1x32 blocks along cols; codes [rows x cols/2], scales    */
/*   [rows x cols/32].                                                  */
/* block_axis = 0: the rows of x are split into groups by offsets       */
/*   off[0..G] (off[0] = 0, off[G] = rows); each group is zero-padded   */
/*   to a multiple of group_pad rows (32, or 256 so that every 256-     */
/*   token K stage of the weight gradient starts a group's segment on a  */
/*   whole 128-byte line of codes); Q = [cols x kp] with Q[c][P_g + r] = */
/*   x[off[g] + r][c], P_g the padded start of group g; 32-blocks run   */
/*   along Q's rows (i.e. down the token axis of one group).  codes     */
/*   [cols x kp/2], scales [cols x kp/32]; positions of Q beyond the    */
/*   padded total are not written.                                      */
/* Element index for SR = index_base + (q_row * q_cols + q_col).        */
/* Only logical rows [q_row_begin, q_row_end) are produced (the Python  */
/* wrapper splits the work over threads).                               */
/* ------------------------------------------------------------------ */
int oracle_quantize_1d(const void* x, int dtype, int64_t rows, int64_t cols,
                       int block_axis, const int32_t* off, int32_t num_groups,
                       int64_t kp, int32_t group_pad, int use_rht, uint32_t mask, int rnd,
                       uint64_t seed, uint32_t stream, uint64_t index_base,
                       uint8_t* codes, uint8_t* scales,
                       int64_t q_row_begin, int64_t q_row_end)
{
    if (cols <= 0 || rows < 0) return 1;
    int64_t q_cols;
    if (block_axis == 1) {
        if (cols % 32) return 2;
        q_cols = cols;
    } else {
        q_cols = kp;
        if (kp % 32 || group_pad <= 0 || group_pad % 32) return 2;
    }
    float v[32], t[32];
    uint32_t r16[32];
    uint8_t code[32];
    for (int64_t q = q_row_begin; q < q_row_end; ++q) {
        for (int64_t b = 0; b < q_cols / 32; ++b) {
            int valid = 1;
            if (block_axis == 1) {
                for (int j = 0; j < 32; ++j)
                    v[j] = load_elem(x, dtype, q * cols + b * 32 + j);
            } else {
                /* find the group whose padded range holds block b */
                int64_t p = 0;
                int g = -1;
                for (int gg = 0; gg < num_groups; ++gg) {
                    int64_t n = (int64_t)off[gg + 1] - off[gg];
                    int64_t np = (n + group_pad - 1) / group_pad * group_pad;
                    if (b * 32 >= p && b * 32 < p + np) { g = gg; break; }
                    p += np;
                }
                if (g < 0) { valid = 0; }
                else {
                    int64_t n = (int64_t)off[g + 1] - off[g];
                    for (int j = 0; j < 32; ++j) {
                        int64_t r = b * 32 - p + j;
                        v[j] = (r < n) ? load_elem(x, dtype, ((int64_t)off[g] + r) * cols + q)
                                       : 0.0f;
                    }
                }
            }
            if (!valid) continue;   /* beyond the padded total: not written */
            if (use_rht) {
                oracle_rht_block(v, t, mask, 0);
                memcpy(v, t, sizeof(v));
            }
            if (rnd == 1)
                for (int j = 0; j < 32; ++j)
                    r16[j] = oracle_sr_bits(seed, stream,
                                            index_base + (uint64_t)(q * q_cols + b * 32 + j));
            uint8_t byte = quantize_block(v, 32, rnd, r16, code);
            scales[q * (q_cols / 32) + b] = byte;
            for (int j = 0; j < 16; ++j)
                codes[q * (q_cols / 2) + b * 16 + j] =
                    (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Study variants of the row-wise 1x32 quantizer: outlier clipping and   */
/* macro-block scaling.                                                  */
/*                                                                      */
/* Both are named, without definitions, among the techniques that raised */
/* operator-level SNR but failed end to end (Abstract of "Training an   */
/* MoE LLM in MXFP4"; "The Numbers" in the news digest).  The readings: */
/*   - outlier clipping with ratio rho in (0, 1]: a block's scale is    */
/*     chosen for fl32(rho * amax) instead of amax, X = floor(log2(     */
/*     fl32(rho * amax))) - 2, so the block's largest values saturate   */
/*     at +-6 * 2^X (clipped) while the rest get a finer grid; rho = 1  */
/*     is the plain quantizer;                                           */
/*   - macro-block scaling with size Bm (a multiple of 32 dividing the  */
/*     row, 0 = none): a second, fp32 scale per Bm consecutive elements */
/*     of a row.  Its multiplier r = fl32(6 / amax_M) (1 when amax_M is */
/*     0 or not finite, or when the quotient is not finite) maps the    */
/*     macro-block's largest magnitude to 6 up to one rounding; the     */
/*     elements y' = fl32(y * r) are then quantized in 1x32 blocks as   */
/*     usual, and decode to deq(code, scale) / r.                       */
/*   - clip_ratio = 0 selects a search instead of a fixed ratio: a block */
/*     takes the exponent X - 1 (clipping its largest values) instead of */
/*     the rule's X when that strictly lowers its squared round-to-     */
/*     nearest-even error.  Each candidate's error is summed in its own */
/*     units, sum (v_j - q_j)^2 with v_j = y_j / 2^X and q_j the RTNE    */
/*     value: every difference is exact in fp32 and its square in fp64; */
/*     the sum is taken in fp64 as s_k = ((d_8k^2 + d_8k+1^2) + ...) over */
/*     the eight elements of each quarter k, then ((s_0 + s_1) + s_2) +  */
/*     s_3.  X - 1 wins iff S(X - 1) < 4 S(X) (the same error in the     */
/*     input's units; the factor 4 is exact).  Not taken when the rule   */
/*     gives byte 0 (no lower exponent).                                 */
/* The RHT (when on) comes first, so amax_M is over transformed values. */
/* Element index for SR as in oracle_quantize_1d (row-wise).            */
/* macro_r [rows x cols/Bm] (written when Bm > 0).                      */
/* ------------------------------------------------------------------ */
int oracle_quantize_1d_ex(const void* x, int dtype, int64_t rows, int64_t cols,
                          int use_rht, uint32_t mask, int rnd, uint64_t seed, uint32_t stream,
                          uint64_t index_base, float clip_ratio, int64_t macro_block,
                          uint8_t* codes, uint8_t* scales, float* macro_r,
                          int64_t r_begin, int64_t r_end)
{
    if (cols <= 0 || cols % 32 || rows < 0) return 2;
    if (!(clip_ratio >= 0.0f && clip_ratio <= 1.0f)) return 2;
    if (macro_block < 0 || (macro_block > 0 && (macro_block % 32 || cols % macro_block))) return 2;
    float y[32], t[32];
    uint32_t r16[32];
    uint8_t code[32];
    for (int64_t row = r_begin; row < r_end; ++row) {
        float r = 1.0f;
        for (int64_t b = 0; b < cols / 32; ++b) {
            /* a new macro-block starts: its multiplier from the transformed amax */
            if (macro_block > 0 && (b * 32) % macro_block == 0) {
                float amax = 0.0f;
                int nonfinite = 0;
                for (int64_t bb = b; bb < b + macro_block / 32; ++bb) {
                    for (int j = 0; j < 32; ++j) t[j] = load_elem(x, dtype, row * cols + bb * 32 + j);
                    if (use_rht) { oracle_rht_block(t, y, mask, 0); memcpy(t, y, sizeof(t)); }
                    for (int j = 0; j < 32; ++j) {
                        if (isnan(t[j]) || isinf(t[j])) nonfinite = 1;
                        else if (fabsf(t[j]) > amax) amax = fabsf(t[j]);
                    }
                }
                r = 1.0f;
                if (!nonfinite && amax > 0.0f) {
                    volatile float q = 6.0f / amax;          /* one fp32 rounding */
                    if (!isinf(q)) r = q;
                }
                macro_r[row * (cols / macro_block) + (b * 32) / macro_block] = r;
            }
            for (int j = 0; j < 32; ++j) y[j] = load_elem(x, dtype, row * cols + b * 32 + j);
            if (use_rht) { oracle_rht_block(y, t, mask, 0); memcpy(y, t, sizeof(y)); }
            if (macro_block > 0)
                for (int j = 0; j < 32; ++j) { volatile float p = y[j] * r; y[j] = p; }
            if (rnd == 1)
                for (int j = 0; j < 32; ++j)
                    r16[j] = oracle_sr_bits(seed, stream, index_base + (uint64_t)(row * cols + b * 32 + j));
            /* the block scale from the clipped amax */
            double amax = 0.0;
            int nonfinite = 0;
            for (int j = 0; j < 32; ++j) {
                if (isnan(y[j]) || isinf(y[j])) nonfinite = 1;
                if (fabs((double)y[j]) > amax) amax = fabs((double)y[j]);
            }
            uint8_t byte;
            if (nonfinite) {
                byte = 0xFF;
                for (int j = 0; j < 32; ++j) code[j] = 0;
            } else {
                if (clip_ratio > 0.0f) {
                    volatile float ca = clip_ratio * (float)amax;   /* fl32(rho * amax) */
                    byte = oracle_scale_byte((double)ca);
                } else {
                    byte = oracle_scale_byte(amax);
                    if (byte > 0) {
                        double S[2];
                        for (int cand = 0; cand < 2; ++cand) {
                            int Xc = (int)byte - cand - 127;
                            double part[4];
                            for (int k = 0; k < 4; ++k) {
                                double acc = 0.0;
                                for (int e = 0; e < 8; ++e) {
                                    double v = ldexp((double)y[8 * k + e], -Xc);
                                    double q = E2M1_MAG[oracle_rtne_mag(fabs(v))];
                                    double d = fabs(v) - q;           /* sign-free: |v - sign(v) q| */
                                    acc = acc + d * d;
                                }
                                part[k] = acc;
                            }
                            S[cand] = ((part[0] + part[1]) + part[2]) + part[3];
                        }
                        if (S[1] < 4.0 * S[0]) byte = (uint8_t)(byte - 1);
                    }
                }
                int X = (int)byte - 127;
                for (int j = 0; j < 32; ++j) {
                    double A = fabs(ldexp((double)y[j], -X));
                    int m = (rnd == 0) ? oracle_rtne_mag(A) : oracle_sr_mag(A, r16[j]);
                    code[j] = (uint8_t)(((signbit(y[j]) ? 1 : 0) << 3) | m);
                }
            }
            scales[row * (cols / 32) + b] = byte;
            for (int j = 0; j < 16; ++j)
                codes[row * (cols / 2) + b * 16 + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* Decode of oracle_quantize_1d_ex's output to fp32: deq(code, scale) / r,
 * the division rounded once to fp32 (r = 1 without macro-blocks). */
int oracle_dequantize_1d_ex(const uint8_t* codes, const uint8_t* scales, const float* macro_r,
                            int64_t rows, int64_t cols, int64_t macro_block, float* y,
                            int64_t r_begin, int64_t r_end)
{
    if (cols % 32 || (macro_block > 0 && (macro_block % 32 || cols % macro_block))) return 2;
    for (int64_t row = r_begin; row < r_end; ++row)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[row * (cols / 2) + c / 2];
            uint8_t code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double v = oracle_decode(code, scales[row * (cols / 32) + c / 32]);
            double r = macro_block > 0 ? (double)macro_r[row * (cols / macro_block) + c / macro_block] : 1.0;
            y[row * cols + c] = (float)(v / r);    /* a double quotient of floats, rounded once */
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* 2D quantize, 32x32 blocks, RTNE.  w [batch x rows x cols].           */
/* codes [batch x rows x cols/2], scales [batch x rows/32 x cols/32];   */
/* codes_t [batch x cols x rows/2], scales_t [batch x cols/32 x rows/32]*/
/* (either pair may be NULL).  Only tiles with tile-row index in        */
/* [tr_begin, tr_end) of every batch entry are produced.                */
/* ------------------------------------------------------------------ */
static void put_nibble(uint8_t* base, int64_t elem, uint8_t code)
{
    uint8_t* p = base + elem / 2;
    if (elem % 2 == 0) *p = (uint8_t)((*p & 0xF0) | code);
    else *p = (uint8_t)((*p & 0x0F) | (code << 4));
}

int oracle_quantize_2d(const void* w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                       int64_t tr_begin, int64_t tr_end)
{
    if (rows % 32 || cols % 32) return 2;
    float v[1024];
    uint8_t code[1024];
    for (int64_t bt = 0; bt < batch; ++bt) {
        for (int64_t tr = tr_begin; tr < tr_end; ++tr) {
            for (int64_t tc = 0; tc < cols / 32; ++tc) {
                for (int i = 0; i < 32; ++i)
                    for (int j = 0; j < 32; ++j)
                        v[i * 32 + j] = load_elem(w, dtype,
                                                  bt * rows * cols + (tr * 32 + i) * cols + tc * 32 + j);
                uint8_t byte = quantize_block(v, 1024, 0, NULL, code);
                if (scales) scales[bt * (rows / 32) * (cols / 32) + tr * (cols / 32) + tc] = byte;
                if (scales_t) scales_t[bt * (rows / 32) * (cols / 32) + tc * (rows / 32) + tr] = byte;
                for (int i = 0; i < 32; ++i)
                    for (int j = 0; j < 32; ++j) {
                        int64_t r = tr * 32 + i, c = tc * 32 + j;
                        if (codes)
                            put_nibble(codes + bt * rows * (cols / 2), r * cols + c, code[i * 32 + j]);
                        if (codes_t)
                            put_nibble(codes_t + bt * rows * (cols / 2), c * rows + r, code[i * 32 + j]);
                    }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* 2D quantize with weight de-oscillation (hysteresis against the        */
/* previous step's quantized weights).                                   */
/*                                                                      */
/* "AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of BF16", section */
/* "What ALTO Actually Does": the optimizer moves a full-precision      */
/* master weight while the GEMM consumes its quantized value, so a     */
/* weight sitting near a rounding boundary can alternate between two   */
/* levels from updates far smaller than a level step.  The pages name a */
/* simplified de-oscillation scheme (Abstract of "Training an MoE LLM  */
/* in MXFP4") but give no formula; the reading implemented here is a   */
/* hysteresis band:                                                    */
/*   - the tile's scale byte comes from its amax as in                 */
/*     oracle_quantize_2d, except that a tile whose amax has dropped    */
/*     just below the previous scale's range keeps the previous byte:   */
/*     when the rule gives exactly one less than the previous byte p    */
/*     (p != 0xFF) and amax >= (4 - margin64/16) 2^(p - 127), the tile  */
/*     keeps p.  Its elements then fit without clipping (amax / 2^X_p   */
/*     < 4), and an amax that hovers around a power of two no longer    */
/*     moves every value of the tile; upward crossings are never held   */
/*     back (they would saturate the tile's largest values);            */
/*   - if it equals the previous step's byte for that tile (and neither */
/*     is 0xFF), each element keeps its previous code c_p while its     */
/*     scaled value v = w / 2^X lies strictly inside                    */
/*       (q_p - f (q_p - q_dn),  q_p + f (q_up - q_p)),                */
/*     q_p the value of c_p on the signed E2M1 grid                     */
/*     {-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, ..., 6} (both zero     */
/*     codes are the point 0), q_dn and q_up its neighbours on that     */
/*     grid (none past +-6: the band is open on that side), and         */
/*     f = 1/2 + margin64/64, margin64 in [0, 31].  f = 1/2 is exactly  */
/*     the rounding interval of q_p, so margin64 = 0 changes no value;  */
/*     a larger margin widens the band by margin64/64 of a grid step on */
/*     each side;                                                        */
/*   - otherwise the element takes its round-to-nearest-even code;      */
/*   - a tile whose scale changed is quantized as without hysteresis.  */
/* flips (optional): per tile, the number of elements whose value       */
/* (code and scale, decoded) differs from the previous one; a NaN      */
/* scale on either side counts every element.                          */
/* prev_codes [batch x rows x cols/2], prev_scales [batch x rows/32 x   */
/* cols/32] (the as-given layout of the previous call); outputs as in   */
/* oracle_quantize_2d plus flips [batch x rows/32 x cols/32].           */
/* ------------------------------------------------------------------ */
static const double SIGNED_GRID[15] = {-6.0, -4.0, -3.0, -2.0, -1.5, -1.0, -0.5, 0.0,
                                       0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* position of a code on the signed grid */
static int signed_grid_index(uint8_t code)
{
    int m = code & 7;
    if (m == 0) return 7;
    return (code & 8) ? 7 - m : 7 + m;
}

int oracle_quantize_2d_deosc(const void* w, int dtype, int64_t batch, int64_t rows, int64_t cols,
                             const uint8_t* prev_codes, const uint8_t* prev_scales, int margin64,
                             uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                             uint16_t* flips, int64_t tr_begin, int64_t tr_end)
{
    if (rows % 32 || cols % 32) return 2;
    if (margin64 < 0 || margin64 > 31) return 2;
    const double f = 0.5 + margin64 / 64.0;
    float v[1024];
    uint8_t code[1024];
    for (int64_t bt = 0; bt < batch; ++bt) {
        for (int64_t tr = tr_begin; tr < tr_end; ++tr) {
            for (int64_t tc = 0; tc < cols / 32; ++tc) {
                for (int i = 0; i < 32; ++i)
                    for (int j = 0; j < 32; ++j)
                        v[i * 32 + j] = load_elem(w, dtype,
                                                  bt * rows * cols + (tr * 32 + i) * cols + tc * 32 + j);
                uint8_t byte = quantize_block(v, 1024, 0, NULL, code);
                int64_t sidx = bt * (rows / 32) * (cols / 32) + tr * (cols / 32) + tc;
                uint8_t pbyte = prev_scales[sidx];
                if (pbyte != 0xFF && byte != 0xFF && byte + 1 == pbyte) {
                    double amax = 0.0;
                    for (int k = 0; k < 1024; ++k)
                        if (fabs((double)v[k]) > amax) amax = fabs((double)v[k]);
                    if (amax >= ldexp(4.0 - margin64 / 16.0, (int)pbyte - 127)) {
                        byte = pbyte;                       /* the previous scale is kept */
                        for (int k = 0; k < 1024; ++k) {
                            double A = fabs(ldexp((double)v[k], -((int)byte - 127)));
                            code[k] = (uint8_t)(((signbit(v[k]) ? 1 : 0) << 3) | oracle_rtne_mag(A));
                        }
                    }
                }
                const uint8_t* pc = prev_codes + bt * rows * (cols / 2);
                int hyst = (byte == pbyte && byte != 0xFF);
                int nflip = 0;
                for (int i = 0; i < 32; ++i)
                    for (int j = 0; j < 32; ++j) {
                        int64_t e = (tr * 32 + i) * cols + tc * 32 + j;
                        uint8_t pb = pc[e / 2];
                        uint8_t cp = (e % 2 == 0) ? (pb & 0xF) : (pb >> 4);
                        uint8_t* c = &code[i * 32 + j];
                        if (hyst && *c != cp) {
                            int k = signed_grid_index(cp);
                            double q = SIGNED_GRID[k];
                            double lo = (k == 0) ? -INFINITY : q - f * (q - SIGNED_GRID[k - 1]);
                            double hi = (k == 14) ? INFINITY : q + f * (SIGNED_GRID[k + 1] - q);
                            double sv = ldexp((double)v[i * 32 + j], -((int)byte - 127));
                            if (sv > lo && sv < hi) *c = cp;
                        }
                        double now = oracle_decode(*c, byte), before = oracle_decode(cp, pbyte);
                        if (!(now == before)) ++nflip;
                    }
                if (scales) scales[sidx] = byte;
                if (scales_t) scales_t[bt * (rows / 32) * (cols / 32) + tc * (rows / 32) + tr] = byte;
                if (flips) flips[sidx] = (uint16_t)nflip;
                for (int i = 0; i < 32; ++i)
                    for (int j = 0; j < 32; ++j) {
                        int64_t r = tr * 32 + i, cc = tc * 32 + j;
                        if (codes)
                            put_nibble(codes + bt * rows * (cols / 2), r * cols + cc, code[i * 32 + j]);
                        if (codes_t)
                            put_nibble(codes_t + bt * rows * (cols / 2), cc * rows + r, code[i * 32 + j]);
                    }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantize.                                                           */
/* ------------------------------------------------------------------ */
double oracle_decode(uint8_t code, uint8_t scale_byte)
{
    if (scale_byte == 0xFF) return NAN;
    double mag = E2M1_MAG[code & 7];
    double v = ldexp(mag, (int)scale_byte - 127);
    return (code & 8) ? -v : v;
}

/* codes [batch x rows x cols/2]; scales per block_rows (1 -> [rows x cols/32],
 * 32 -> [rows/32 x cols/32]) for each batch entry; y [batch x rows x cols]
 * in double.  Only rows [r_begin, r_end) of every batch entry. */
int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t batch,
                      int64_t rows, int64_t cols, int block_rows, double* y,
                      int64_t r_begin, int64_t r_end)
{
    if (cols % 32) return 2;
    if (block_rows != 1 && block_rows != 32) return 2;
    if (block_rows == 32 && rows % 32) return 2;
    int64_t srows = rows / block_rows;
    for (int64_t bt = 0; bt < batch; ++bt)
        for (int64_t r = r_begin; r < r_end; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                uint8_t byte = codes[bt * rows * (cols / 2) + r * (cols / 2) + c / 2];
                uint8_t code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                uint8_t s = scales[bt * srows * (cols / 32) + (r / block_rows) * (cols / 32) + c / 32];
                y[bt * rows * cols + r * cols + c] = oracle_decode(code, s);
            }
    return 0;
}

/* Round a double to the nearest bf16 (ties to the even significand), in one
 * rounding from the double's exact value; returned as its bits.  bf16 has 8
 * significant bits and fp32's exponent range: the spacing of bf16 values in
 * [2^k, 2^(k+1)) is 2^(k-7), and 2^-133 below 2^-126 (subnormals).
 * Magnitudes that round to 2^128 or above give Inf; NaN stays NaN.  Used
 * only to state what a bf16 output must be. */
uint16_t oracle_round_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    int k = e - 1;                      /* floor(log2 a) */
    if (k < -126) k = -126;
    double n = ldexp(a, 7 - k);         /* a / spacing: exact (power-of-two scaling) */
    double fl = floor(n);
    double frac = n - fl;               /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = ldexp(fl, k - 7);        /* the rounded magnitude, exact */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                 /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* oracle_round_bf16 over an array: out[i] = round(v[i]) for i in [0, n). */
void oracle_round_bf16_array(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);
}

/* ------------------------------------------------------------------ */
/* Grouped GEMM over dequantized operands, FP64, k ascending.            */
/*                                                                      */
/* C = alpha * deq(A) . deq(B)^T for each group; both operands are      */
/* K-contiguous: A codes [. x K/2], B codes [. x K/2].                  */
/* group_dim_k = 0: groups split M by off[0..G]; output row m of group  */
/*   g uses A row a_row_index[m] (or m when NULL) and B_g = B + g*N*K/2 */
/*   (B_g is [N x K]); b_scale_2d selects [N/32 x K/32] per group       */
/*   instead of [N x K/32].  C [M x N].                                  */
/* group_dim_k = 1: groups split K by off[0..G] (multiples of 32);      */
/*   A [M x K], B [N x K], both with 1D scales; C [G x M x N].          */
/* The rows computed are listed in (row_group, row_m) pairs so that     */
/* callers can sample; c_out receives n_rows x N doubles.               */
/* ------------------------------------------------------------------ */
int oracle_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                        const int32_t* a_row_index,
                        const uint8_t* b_codes, const uint8_t* b_scales, int b_scale_2d,
                        const int32_t* off, int32_t num_groups, int group_dim_k,
                        int64_t M, int64_t N, int64_t K, double alpha,
                        const int32_t* row_group, const int64_t* row_m, int64_t n_rows,
                        double* c_out)
{
    if (K % 32 || N <= 0 || M < 0) return 2;
    (void)num_groups;
    for (int64_t t = 0; t < n_rows; ++t) {
        int g = row_group[t];
        int64_t m = row_m[t];
        int64_t k_begin = 0, k_end = K;
        const uint8_t* bc = b_codes;
        const uint8_t* bs = b_scales;
        int64_t arow = m;
        if (group_dim_k == 0) {
            bc = b_codes + (int64_t)g * N * (K / 2);
            bs = b_scales + (int64_t)g * (b_scale_2d ? (N / 32) * (K / 32) : N * (K / 32));
            arow = a_row_index ? a_row_index[m] : m;
        } else {
            k_begin = off[g];
            k_end = off[g + 1];
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = k_begin; k < k_end; ++k) {
                uint8_t ab = a_codes[arow * (K / 2) + k / 2];
                uint8_t acode = (k % 2 == 0) ? (ab & 0xF) : (ab >> 4);
                double av = oracle_decode(acode, a_scales[arow * (K / 32) + k / 32]);
                uint8_t bb = bc[n * (K / 2) + k / 2];
                uint8_t bcode = (k % 2 == 0) ? (bb & 0xF) : (bb >> 4);
                uint8_t bsb = b_scale_2d ? bs[(n / 32) * (K / 32) + k / 32] : bs[n * (K / 32) + k / 32];
                double bv = oracle_decode(bcode, bsb);
                acc += av * bv;
            }
            c_out[t * N + n] = alpha * acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Staged storage order of a scale matrix (no arithmetic: a permutation of
 * bytes).  This order is not from the pages; it is the order the library's
 * grouped GEMM reads one K stage of 256 elements in (include/mx.h,
 * MX_SCALES_STAGED), written here from that definition so the tests can
 * compare the library's staged output with the row-major oracle output.
 *
 * scales: rows x nblk, row-major (block b of row r at r * nblk + b).
 * gb: num_groups + 1 block offsets (non-decreasing, gb[0] = 0, gb[G] <=
 * nblk) splitting the blocks of every row into groups; num_groups = 0
 * means a single group of all nblk blocks.  Group g's blocks fill stages
 * of 8 of their own, numbered after those of the groups before it: block
 * gb[g] + i goes to slot i % 8 of stage S_g + i / 8, S_g = sum over g' < g
 * of ceil((gb[g'+1] - gb[g']) / 8), i.e. to out[((S_g + i/8) * rows + r) * 8
 * + i % 8].  Bytes of out no block maps to are left untouched.  Returns the
 * number of stages. */
int64_t oracle_stage_scales(const uint8_t* scales, int64_t rows, int64_t nblk, const int64_t* gb,
                            int32_t num_groups, uint8_t* out) {
    int64_t one[2] = {0, nblk};
    if (num_groups == 0) {
        gb = one;
        num_groups = 1;
    }
    int64_t stage0 = 0;
    for (int32_t g = 0; g < num_groups; ++g) {
        const int64_t n = gb[g + 1] - gb[g];
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t i = 0; i < n; ++i)
                out[((stage0 + i / 8) * rows + r) * 8 + i % 8] = scales[r * nblk + gb[g] + i];
        stage0 += (n + 7) / 8;
    }
    return stage0;
}
