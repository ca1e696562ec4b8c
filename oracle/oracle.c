/*
 * oracle.c -- plain, slow CPU oracle for the BF16 -> MXFP4 -> block-scaled FP8 path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or constant generator with the HIP
 * kernels: every value here is computed from the format definitions in double
 * precision, one element at a time, in the order the method states it.
 *
 * Method source: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs"
 * (technical summary, section 2 "Methodology"):
 *   - item 1, MXFP4 spec: 32-element blocks share one power-of-two UE8M0 scale,
 *     elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit);
 *   - item 1, FP8 target: E4M3 with 128-element blocks, reached by a direct
 *     FP4 -> FP8 conversion with no BF16 intermediate;
 *   - item 1, hierarchical scale alignment: the four 32-element MX scales of a
 *     128-element FP8 block are aligned to the largest one and each sub-block's
 *     exponent is shifted by the difference, keeping values numerically equal;
 *   - item 2, forward pass: codes packed two per uint8 container;
 *   - item 3, kernels: row layout (FPROP), transposed column layout (Wgrad) with
 *     transpose fused into the conversion, ragged per-expert token counts with no
 *     padding.
 * Readings where the page is silent (rounding, scale rule, nibble order, layouts)
 * follow the OCP Microscaling (MX) v1.0 conventions and are listed with each
 * function below:
 *   - shared exponent = floor(log2(amax)) - emax_elem, emax_elem = 2 for E2M1,
 *     stored biased by 127 and clamped to [0, 254]; an all-zero block gets 0;
 *   - E2M1: round to nearest, ties to even code, saturating at +-6;
 *   - E4M3 (OCP "E4M3FN": bias 7, no infinities): round to nearest, ties to even,
 *     used when a sub-block shift pushes a value into the subnormal range;
 *   - the sign of zero is kept (a negative value that rounds to 0 gives -0);
 *   - element 2i goes in the low nibble of byte i, element 2i+1 in the high nibble.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- value decoding ---------------------------------------------------- */

/* BF16 bits -> exact double.  BF16 is the top half of an IEEE binary32:
 * 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
static double bf16_value(uint16_t b)
{
    int sign = b >> 15;
    int e = (b >> 7) & 0xFF;
    int m = b & 0x7F;
    double mag;
    if (e == 0)
        mag = ldexp((double)m, -126 - 7);             /* subnormal */
    else
        mag = ldexp((double)(128 + m), e - 127 - 7);   /* normal; e == 255 not allowed */
    return sign ? -mag : mag;
}

static int bf16_negative(uint16_t b) { return b >> 15; }

/* Magnitude of an E2M1 code (low three bits): 2 exponent bits with bias 1,
 * 1 mantissa bit; exponent field 0 is subnormal (0 or 0.5). */
static double e2m1_magnitude(int code)
{
    int e = (code >> 1) & 3;
    int m = code & 1;
    if (e == 0)
        return ldexp((double)m, -1);
    return ldexp(1.0 + 0.5 * m, e - 1);
}

/* ---- generic binary minifloat rounding --------------------------------- */

/* Round the non-negative finite value v to the nearest value of a binary
 * minifloat with `mbits` mantissa bits and exponent bias `bias` (exponent field
 * 0 = subnormal, same quantum as the smallest normal binade), ties to the
 * encoding whose mantissa LSB is 0.  Returns the magnitude code
 * (exponent_field << mbits | mantissa).  Values above the largest code
 * `max_code` saturate to it. */
static int minifloat_round_nearest_even(double v, int mbits, int bias, int max_code)
{
    if (v == 0.0)
        return 0;
    int e2;
    frexp(v, &e2);               /* v = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;              /* v in [2^E, 2^(E+1)) */
    int emin = 1 - bias;         /* exponent of the smallest normal binade */
    if (E < emin)
        E = emin;                /* subnormals use the quantum of the first binade */
    double quantum = ldexp(1.0, E - mbits);
    double n = v / quantum;      /* exact: division by a power of two */
    double fl = floor(n);
    double frac = n - fl;
    long q = (long)fl;
    if (frac > 0.5 || (frac == 0.5 && (q & 1)))
        q += 1;
    long code;
    if (E == emin && q < (1L << mbits))
        code = q;                                            /* subnormal */
    else
        code = ((long)(E + bias) << mbits) + (q - (1L << mbits)); /* normal (q may carry) */
    if (code > max_code)
        code = max_code;
    return (int)code;
}

/* E2M1, saturating: largest magnitude code 7 (= 6.0). */
static int e2m1_encode(double y) { return minifloat_round_nearest_even(y, 1, 1, 7); }

/* OCP E4M3FN: bias 7, 3 mantissa bits, largest finite code 0x7E (= 448).
 * The FP4 -> FP8 conversions never exceed 6; the backward FP8 quantizer does
 * reach the saturation (see below). */
static int e4m3_encode(double v) { return minifloat_round_nearest_even(v, 3, 7, 0x7E); }

/* ---- step a1/a2: block amax and shared UE8M0 scale --------------------- */

/* Shared scale byte of a 32-element block whose largest magnitude is `amax`:
 * floor(log2(amax)) - 2 + 127, clamped to [0, 254]; 0 for an all-zero block. */
static int ue8m0_scale_for_amax(double amax)
{
    if (amax == 0.0)
        return 0;
    int e2;
    frexp(amax, &e2);            /* floor(log2(amax)) = e2 - 1 */
    int s = (e2 - 1) - 2 + 127;
    if (s < 0) s = 0;
    if (s > 254) s = 254;
    return s;
}

/* ---- public entry points (C linkage for ctypes) ------------------------ */

/* One 32-element block: x[0..31] BF16 bits -> 16 packed bytes + 1 scale byte. */
void oracle_quantize_block(const uint16_t *x, uint8_t *packed16, uint8_t *scale)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs(bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    int s = ue8m0_scale_for_amax(amax);
    *scale = (uint8_t)s;
    uint8_t codes[32];
    for (int i = 0; i < 32; ++i) {
        double y = ldexp(fabs(bf16_value(x[i])), 127 - s);   /* |x| / 2^(s-127), exact */
        int c = e2m1_encode(y);
        if (bf16_negative(x[i]))
            c |= 8;
        codes[i] = (uint8_t)c;
    }
    for (int i = 0; i < 16; ++i)
        packed16[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
}

/* Quantize rows [row_begin, row_end) of a row-major BF16 matrix with K columns
 * (K a multiple of 32).  codes: [*, K/2] bytes, scales: [*, K/32] bytes. */
void oracle_quantize_rows(const uint16_t *x, int64_t K, int64_t row_begin, int64_t row_end,
                          uint8_t *codes, uint8_t *scales)
{
    int64_t nb = K / 32;
    for (int64_t m = row_begin; m < row_end; ++m)
        for (int64_t j = 0; j < nb; ++j)
            oracle_quantize_block(x + m * K + 32 * j, codes + m * (K / 2) + 16 * j,
                                  scales + m * nb + j);
}

/* Unpack code k of a packed row: even k in the low nibble. */
static int code_at(const uint8_t *packed_row, int64_t k)
{
    uint8_t b = packed_row[k / 2];
    return (k & 1) ? (b >> 4) : (b & 15);
}

/* The FP8 byte of one E2M1 code whose MX scale is s and whose FP8 block scale is S
 * (S >= s): value e2m1(c) * 2^(s - S), rounded to E4M3, sign of the code kept. */
static uint8_t fp8_of_code(int c, int s, int S)
{
    double v = ldexp(e2m1_magnitude(c & 7), s - S);
    int b = e4m3_encode(v);
    if (c & 8)
        b |= 0x80;
    return (uint8_t)b;
}

/* Row layout (FPROP), rows [row_begin, row_end): each 128-element block along K
 * gets the UE8M0 scale S = max of its four MX scales; y: [*, K] E4M3 bytes,
 * y_scales: [*, K/128] UE8M0 bytes.  K a multiple of 128. */
void oracle_fp8_rows(const uint8_t *codes, const uint8_t *scales, int64_t K,
                     int64_t row_begin, int64_t row_end, uint8_t *y, uint8_t *y_scales)
{
    int64_t nb32 = K / 32, nb128 = K / 128;
    for (int64_t m = row_begin; m < row_end; ++m) {
        const uint8_t *crow = codes + m * (K / 2);
        const uint8_t *srow = scales + m * nb32;
        for (int64_t b = 0; b < nb128; ++b) {
            int S = 0;
            for (int j = 0; j < 4; ++j)
                if (srow[4 * b + j] > S)
                    S = srow[4 * b + j];
            y_scales[m * nb128 + b] = (uint8_t)S;
            for (int64_t k = 128 * b; k < 128 * (b + 1); ++k)
                y[m * K + k] = fp8_of_code(code_at(crow, k), srow[k / 32], S);
        }
    }
}

/* Column layout (Wgrad) for expert g, row blocks [blk_begin, blk_end) of that
 * expert.  Expert g owns rows [offs[g], offs[g+1]); M_g = offs[g+1] - offs[g];
 * its rows are cut into ceil(M_g/128) blocks of 128 (the last one partial).
 * For block b and column k the FP8 scale is the max of the MX scales of group
 * k/32 over the rows of the block that exist.  Output for expert g is the
 * transpose [K, M_g] at byte offset K*offs[g]; element (k, m') at k*M_g + m'.
 * Scales for expert g are [nblocks_g, K] at byte offset K*B_g, where B_g is the
 * number of row blocks of experts 0..g-1. */
void oracle_fp8_cols(const uint8_t *codes, const uint8_t *scales, const int32_t *offs,
                     int32_t g, int64_t K, int64_t blk_begin, int64_t blk_end,
                     uint8_t *yT, uint8_t *yT_scales)
{
    int64_t nb32 = K / 32;
    int64_t Bg = 0;
    for (int32_t h = 0; h < g; ++h)
        Bg += ((int64_t)offs[h + 1] - offs[h] + 127) / 128;
    int64_t row0 = offs[g];
    int64_t Mg = (int64_t)offs[g + 1] - offs[g];
    uint8_t *outT = yT + K * row0;
    uint8_t *outS = yT_scales + K * Bg;
    for (int64_t b = blk_begin; b < blk_end; ++b) {
        int64_t mlo = 128 * b;
        int64_t mhi = mlo + 128 < Mg ? mlo + 128 : Mg;
        for (int64_t j = 0; j < nb32; ++j) {
            int S = 0;
            for (int64_t m = mlo; m < mhi; ++m) {
                int s = scales[(row0 + m) * nb32 + j];
                if (s > S)
                    S = s;
            }
            for (int64_t k = 32 * j; k < 32 * (j + 1); ++k) {
                outS[b * K + k] = (uint8_t)S;
                for (int64_t m = mlo; m < mhi; ++m) {
                    const uint8_t *crow = codes + (row0 + m) * (K / 2);
                    int s = scales[(row0 + m) * nb32 + j];
                    outT[k * Mg + m] = fp8_of_code(code_at(crow, k), s, S);
                }
            }
        }
    }
}

/* ---- backward FP8 quantizer: BF16 -> E4M3 with 1x128 blocks ------------ */
/* Technical summary, section 2 (Methodology): the backward pass of the asymmetric
 * flow (item 2) stays on the standard FP8 path for gradients, in the E4M3 format with
 * 128-element blocks (item 1).  The page does not fix
 * the block scale; the reading here follows the rest of this path and OCP MX: one
 * UE8M0 byte per 128 elements along the row, shared exponent
 * floor(log2(amax)) - emax_elem with emax_elem = 8 for E4M3 (its largest normal is
 * 448 = 1.75 * 2^8), biased by 127 and clamped to [0, 254], 0 for an all-zero
 * block.  Elements are |x| / 2^(S-127) rounded to E4M3FN, ties to even, into the
 * subnormals, saturating at 448 (the block maximum lands in [256, 512), so values
 * above 448 occur and clamp); the sign is kept, -0 included. */
static int ue8m0_scale_for_amax_e4m3(double amax)
{
    if (amax == 0.0)
        return 0;
    int e2;
    frexp(amax, &e2);            /* floor(log2(amax)) = e2 - 1 */
    int s = (e2 - 1) - 8 + 127;
    if (s < 0) s = 0;
    if (s > 254) s = 254;
    return s;
}

/* One 128-element block: x[0..127] BF16 bits -> 128 E4M3 bytes + 1 scale byte. */
void oracle_fp8q_block(const uint16_t *x, uint8_t *y128, uint8_t *scale)
{
    double amax = 0.0;
    for (int i = 0; i < 128; ++i) {
        double a = fabs(bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    int s = ue8m0_scale_for_amax_e4m3(amax);
    *scale = (uint8_t)s;
    for (int i = 0; i < 128; ++i) {
        double v = ldexp(fabs(bf16_value(x[i])), 127 - s);    /* |x| / 2^(s-127), exact */
        int b = e4m3_encode(v);
        if (bf16_negative(x[i]))
            b |= 0x80;
        y128[i] = (uint8_t)b;
    }
}

/* Row layout, rows [row_begin, row_end) of a row-major BF16 matrix with K columns
 * (K a multiple of 128): y [*, K] E4M3 bytes, y_scales [*, K/128] UE8M0 bytes. */
void oracle_fp8q_rows(const uint16_t *x, int64_t K, int64_t row_begin, int64_t row_end,
                      uint8_t *y, uint8_t *y_scales)
{
    int64_t nb = K / 128;
    for (int64_t m = row_begin; m < row_end; ++m)
        for (int64_t b = 0; b < nb; ++b)
            oracle_fp8q_block(x + m * K + 128 * b, y + m * K + 128 * b, y_scales + m * nb + b);
}

/* Column layout for the Wgrad gradient of expert g, row blocks [blk_begin, blk_end)
 * of that expert: the transposed counterpart of oracle_fp8q_rows over the same
 * ragged segments and the same output layout as oracle_fp8_cols.  For block b and
 * column k the 1x128 block runs along the token dimension: rows
 * [128b, min(128b+128, M_g)) of the expert (a partial last block uses only its
 * rows).  Its UE8M0 scale comes from the amax over those rows (rule above) and is
 * stored at yT_scales[K*B_g + b*K + k]; element (k, m') goes to
 * yT[K*offs[g] + k*M_g + m']. */
void oracle_fp8q_cols(const uint16_t *x, const int32_t *offs, int32_t g, int64_t K,
                      int64_t blk_begin, int64_t blk_end, uint8_t *yT, uint8_t *yT_scales)
{
    int64_t Bg = 0;
    for (int32_t h = 0; h < g; ++h)
        Bg += ((int64_t)offs[h + 1] - offs[h] + 127) / 128;
    int64_t row0 = offs[g];
    int64_t Mg = (int64_t)offs[g + 1] - offs[g];
    uint8_t *outT = yT + K * row0;
    uint8_t *outS = yT_scales + K * Bg;
    for (int64_t b = blk_begin; b < blk_end; ++b) {
        int64_t mlo = 128 * b;
        int64_t mhi = mlo + 128 < Mg ? mlo + 128 : Mg;
        for (int64_t k = 0; k < K; ++k) {
            double amax = 0.0;
            for (int64_t m = mlo; m < mhi; ++m) {
                double a = fabs(bf16_value(x[(row0 + m) * K + k]));
                if (a > amax)
                    amax = a;
            }
            int s = ue8m0_scale_for_amax_e4m3(amax);
            outS[b * K + k] = (uint8_t)s;
            for (int64_t m = mlo; m < mhi; ++m) {
                uint16_t xb = x[(row0 + m) * K + k];
                int e = e4m3_encode(ldexp(fabs(bf16_value(xb)), 127 - s));
                if (bf16_negative(xb))
                    e |= 0x80;
                outT[k * Mg + m] = (uint8_t)e;
            }
        }
    }
}

/* ---- FP8 grouped GEMM, forward (row layout) ---------------------------- */
/* Technical summary, section 2: the GEMMs stay in FP8 on the standard block-scaled
 * pipeline (item 1: E4M3 with 128-element blocks; the precision-decoupling framing:
 * compute in FP8, store and communicate in FP4); the forward expert GEMM consumes the
 * row-layout FP8 activations.  Reading (the page fixes no GEMM formula): each expert g
 * owns rows [offs[g], offs[g+1]) of A and a weight W_g [N, K] in the same format as the
 * activations (E4M3 with one UE8M0 scale per 1x128 block along K, per output feature;
 * a 128x128-block weight scale is the case where 128 consecutive features repeat it),
 * and
 *     y[m, n] = bf16( sum_k A[m,k] 2^(sA[m,k/128]-127) * W_g[n,k] 2^(sW_g[n,k/128]-127) )
 * with the sum taken exactly (here: fp64, whose rounding over K <= 2^16 terms is far
 * below the BF16 step) and one round-to-nearest-even to BF16 at the end. */

/* E4M3FN byte -> exact double: bias 7, exponent field 0 is subnormal (m * 2^-9).
 * The NaN bytes 0x7F / 0xFF are not valid inputs. */
static double e4m3_value(uint8_t b)
{
    int e = (b >> 3) & 0xF, m = b & 7;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (b & 0x80) ? -v : v;
}

/* Round half to even at integer granularity (q >= 0). */
static double round_half_even(double q)
{
    double f = floor(q), r = q - f;
    if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0))
        f += 1.0;
    return f;
}

/* double -> BF16 bits, one rounding to nearest even from the exact value (no binary32
 * intermediate): 8 significant bits for normals (exponent field 1..254), steps of
 * 2^-133 below 2^-126 (subnormals), Inf above the largest finite value. */
static uint16_t bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e;
    double f = frexp(a, &e);            /* a = f 2^e, f in [0.5, 1) */
    int E = e - 1 + 127;                /* biased exponent of a */
    if (E <= 0) {                       /* subnormal range: units of 2^-133 */
        double q = round_half_even(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)q);          /* q = 128 is the smallest normal */
    }
    double q = round_half_even(f * 256.0);              /* 128 .. 256 */
    if (q == 256.0) {
        q = 128.0;
        ++E;
    }
    if (E >= 255)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)(E << 7) | (uint16_t)(q - 128.0));
}

/* y = the GEMM above at `count` points (ms[i], ns[i]); exact[i] gets the fp64 sum,
 * y_bf16[i] its BF16 rounding, absum[i] = sum_k |term| (for error bounds).  A [*, K],
 * sA [*, K/128], W [G, N, K], sW [G, N, K/128] row-major.  Rows must lie in
 * [0, offs[G]). */
void oracle_fp8_gemm_at(const uint8_t *a, const uint8_t *sa, const uint8_t *w, const uint8_t *sw,
                        const int32_t *offs, int32_t G, int64_t N, int64_t K,
                        const int64_t *ms, const int64_t *ns, int64_t count,
                        double *exact, uint16_t *y_bf16, double *absum)
{
    int64_t kb = K / 128;
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        int32_t g = 0;
        while (g + 1 < G && (int64_t)offs[g + 1] <= m)
            ++g;
        const uint8_t *ar = a + m * K, *sar = sa + m * kb;
        const uint8_t *wr = w + ((int64_t)g * N + n) * K, *swr = sw + ((int64_t)g * N + n) * kb;
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double x = ldexp(e4m3_value(ar[k]), (int)sar[k / 128] - 127);
            double y = ldexp(e4m3_value(wr[k]), (int)swr[k / 128] - 127);
            s += x * y;
            t += fabs(x * y);
        }
        exact[i] = s;
        y_bf16[i] = bf16_round(s);
        if (absum)
            absum[i] = t;
    }
}

/* ---- FP8 grouped GEMM, weight gradient (column layouts) ---------------- */
/* Technical summary, section 2: the GEMMs stay in FP8 (item 1), and the column
 * conversion (item 3: the transpose fused into the Wgrad conversion, ragged experts)
 * produces the weight-gradient GEMM's operands.  Reading: for expert g with M_g tokens,
 * the weight gradient contracts over the expert's tokens,
 *     dW[g, n, k] = bf16( sum_{m < M_g} dY_g[m, n] X_g[m, k] )
 * where both operands come in the column layout of oracle_fp8_cols / oracle_fp8q_cols:
 * dyT holds expert g as [N, M_g] at byte N*offs[g] with scales [nb_g, N] at byte N*B_g
 * (entry (b, n) scales tokens 128b .. 128b+127 of row n), and xT likewise with K.
 * B_g is the number of 128-token blocks of the experts before g; a partial last block
 * scales only the tokens it has.  An expert with no tokens has dW_g = 0.  The sum is
 * taken in fp64 and rounded once to BF16 (nearest even), as for the forward GEMM. */

/* 128-token blocks of the experts before g. */
static int64_t blocks_before(const int32_t *offs, int32_t g)
{
    int64_t b = 0;
    for (int32_t e = 0; e < g; ++e)
        b += ((int64_t)offs[e + 1] - offs[e] + 127) / 128;
    return b;
}

/* dW at `count` points (gs[i], ns[i], ks[i]); exact / y_bf16 / absum as in
 * oracle_fp8_gemm_at (absum = sum_m |term|). */
void oracle_fp8_wgrad_at(const uint8_t *dyT, const uint8_t *dyT_scales, const uint8_t *xT,
                         const uint8_t *xT_scales, const int32_t *offs, int32_t G, int64_t N,
                         int64_t K, const int64_t *gs, const int64_t *ns, const int64_t *ks,
                         int64_t count, double *exact, uint16_t *y_bf16, double *absum)
{
    (void)G;
    for (int64_t i = 0; i < count; ++i) {
        int32_t g = (int32_t)gs[i];
        int64_t n = ns[i], k = ks[i];
        int64_t m0 = offs[g], Mg = (int64_t)offs[g + 1] - offs[g], Bg = blocks_before(offs, g);
        const uint8_t *dy = dyT + N * m0 + n * Mg;          /* row n of expert g's [N, M_g] */
        const uint8_t *xx = xT + K * m0 + k * Mg;           /* row k of expert g's [K, M_g] */
        double s = 0.0, t = 0.0;
        for (int64_t m = 0; m < Mg; ++m) {
            int64_t b = m / 128;
            double u = ldexp(e4m3_value(dy[m]), (int)dyT_scales[N * (Bg + b) + n] - 127);
            double v = ldexp(e4m3_value(xx[m]), (int)xT_scales[K * (Bg + b) + k] - 127);
            s += u * v;
            t += fabs(u * v);
        }
        exact[i] = s;
        y_bf16[i] = bf16_round(s);
        if (absum)
            absum[i] = t;
    }
}

/* ---- NVFP4 variant quantizer ------------------------------------------- */
/* Page "Train models faster with JAX and MaxText using NVFP4 on NVIDIA Blackwell",
 * section on the NVFP4 pre-training recipe: E2M1 values in 16-element microblocks, one
 * E4M3 scale per block (mantissa bits, not a power of two) under one FP32 scale per
 * tensor; activations and weights round to nearest even.  Reading (the page gives no
 * formulas), in FP32 the way the recipe's GPU implementation computes it:
 *   amax_t = max |x| over the tensor (the routed rows);
 *   t      = FP32(2688 / amax_t), 2688 = 6 * 448 (E2M1 max times E4M3 max), so the
 *            largest block maps to the largest E4M3 scale; 1 for an all-zero tensor,
 *            FLT_MAX where the quotient overflows;
 *   block  : amax_b over its 16 elements; S = E4M3(FP32(FP32(amax_b / 6) * t)), nearest
 *            even with subnormals, saturating at 448;
 *            e = FP32(t / E4M3value(S)) (0 when S is 0, FLT_MAX where it overflows);
 *   element: y = FP32(x * e); code = E2M1(|y|) nearest even, saturating at 6, sign of x
 *            kept (a negative that rounds to 0 is 0x8).
 * A value decodes as E2M1value(code) * E4M3value(S) / t.  Inputs are finite. */

/* The tensor's FP32 encode scale for its largest magnitude. */
static float nvfp4_encode_scale(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    float t = 2688.0f / amax;
    return t > FLT_MAX ? FLT_MAX : t;
}

/* One 16-element block with the tensor's encode scale t: 8 packed bytes + 1 E4M3
 * scale byte. */
void oracle_nvfp4_block(const uint16_t *x, float t, uint8_t *packed8, uint8_t *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf((float)bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    float sb = amax / 6.0f;
    sb = sb * t;
    int S = e4m3_encode((double)sb);
    *scale = (uint8_t)S;
    float e = 0.0f;
    if (S != 0) {
        e = t / (float)e4m3_value((uint8_t)S);
        if (e > FLT_MAX)
            e = FLT_MAX;
    }
    uint8_t codes[16];
    for (int i = 0; i < 16; ++i) {
        float y = (float)bf16_value(x[i]) * e;
        int c = fabsf(y) >= 6.0f ? 7 : e2m1_encode((double)fabsf(y));
        if (signbit(y))
            c |= 8;
        codes[i] = (uint8_t)c;
    }
    for (int i = 0; i < 8; ++i)
        packed8[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
}

/* max |x| over rows [row_begin, row_end) of a BF16 matrix with K columns. */
float oracle_nvfp4_amax(const uint16_t *x, int64_t K, int64_t row_begin, int64_t row_end)
{
    float amax = 0.0f;
    for (int64_t i = row_begin * K; i < row_end * K; ++i) {
        float a = fabsf((float)bf16_value(x[i]));
        if (a > amax)
            amax = a;
    }
    return amax;
}

float oracle_nvfp4_encode_scale(float amax) { return nvfp4_encode_scale(amax); }

/* Rows [row_begin, row_end) with the tensor's encode scale t (K a multiple of 16):
 * codes [*, K/2], scales [*, K/16]. */
void oracle_nvfp4_rows(const uint16_t *x, int64_t K, int64_t row_begin, int64_t row_end, float t,
                       uint8_t *codes, uint8_t *scales)
{
    int64_t nb = K / 16;
    for (int64_t m = row_begin; m < row_end; ++m)
        for (int64_t j = 0; j < nb; ++j)
            oracle_nvfp4_block(x + m * K + 16 * j, t, codes + m * (K / 2) + 8 * j, scales + m * nb + j);
}

/* ---- NVFP4 with stochastic rounding (gradient quantizers) --------------- */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds on a 128-bit
 * counter (c0, c1, c2, c3) under a 64-bit key (k0, k1).  A round multiplies c0 and c2
 * by the two round constants into 64-bit products, and the new counter is
 * (hi(c2 product) ^ c1 ^ k0, lo(c2 product), hi(c0 product) ^ c3 ^ k1, lo(c0 product));
 * the key grows by the two Weyl constants after every round. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p2 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t n0 = (uint32_t)(p2 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p2;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0;
        c[1] = n1;
        c[2] = n2;
        c[3] = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    for (int i = 0; i < 4; ++i)
        out[i] = c[i];
}

/* The 16 random bits of element (row m, column k) of a [*, K] matrix under `seed`: the
 * elements are numbered row-major, n = m K + k; the Philox counter is the index of n's
 * 8-element chunk, (n / 8 low word, high word, 0, 0), the key (seed low word, high
 * word), and element j = n % 8 of the chunk takes half j % 2 (0: low) of output word
 * j / 2. */
unsigned oracle_sr_bits16(uint64_t seed, int64_t K, int64_t m, int64_t k)
{
    uint64_t n = (uint64_t)(m * K + k);
    uint64_t chunk = n / 8;
    uint32_t ctr[4] = {(uint32_t)chunk, (uint32_t)(chunk >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    int j = (int)(n % 8);
    return (w[j / 2] >> (16 * (j % 2))) & 0xFFFFu;
}

/* E2M1 magnitude code of a >= 0, rounded stochastically with the 16-bit random r: at or
 * above 6 the code of 6; otherwise, between the neighbouring E2M1 values lo <= a < hi,
 * hi with probability (a - lo) / (hi - lo), taken when r < 65536 (a - lo) / (hi - lo)
 * (exact: the gaps are powers of two).  Values on the grid never move. */
int oracle_e2m1_encode_sr(double a, unsigned r)
{
    if (a >= 6.0)
        return 7;
    int c = 0;
    while (c < 7 && e2m1_magnitude(c + 1) <= a)
        ++c;
    double lo = e2m1_magnitude(c), hi = e2m1_magnitude(c + 1);
    double f = (a - lo) / (hi - lo);
    return (double)r < 65536.0 * f ? c + 1 : c;
}

/* Rows [row_begin, row_end) as oracle_nvfp4_rows, the element codes rounded
 * stochastically instead of to nearest even (block scales unchanged). */
void oracle_nvfp4_rows_sr(const uint16_t *x, int64_t K, int64_t row_begin, int64_t row_end, float t,
                          uint64_t seed, uint8_t *codes, uint8_t *scales)
{
    int64_t nb = K / 16;
    for (int64_t m = row_begin; m < row_end; ++m)
        for (int64_t j = 0; j < nb; ++j) {
            const uint16_t *xb = x + m * K + 16 * j;
            uint8_t unused[8];
            oracle_nvfp4_block(xb, t, unused, scales + m * nb + j);
            uint8_t S = scales[m * nb + j];
            float e = 0.0f;
            if (S != 0) {
                e = t / (float)e4m3_value(S);
                if (e > FLT_MAX)
                    e = FLT_MAX;
            }
            uint8_t c[16];
            for (int i = 0; i < 16; ++i) {
                float y = (float)bf16_value(xb[i]) * e;
                int code = oracle_e2m1_encode_sr((double)fabsf(y), oracle_sr_bits16(seed, K, m, 16 * j + i));
                if (signbit(y))
                    code |= 8;
                c[i] = (uint8_t)code;
            }
            for (int i = 0; i < 8; ++i)
                codes[m * (K / 2) + 8 * j + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
        }
}

/* ---- small helpers exported for the pins ------------------------------- */

int oracle_e2m1_encode(double y) { return e2m1_encode(y); }
int oracle_e4m3_encode(double v) { return e4m3_encode(v); }
double oracle_e2m1_magnitude(int code) { return e2m1_magnitude(code); }
double oracle_bf16_value(uint16_t b) { return bf16_value(b); }
int oracle_scale_for_amax(double amax) { return ue8m0_scale_for_amax(amax); }
uint8_t oracle_fp8_of_code(int c, int s, int S) { return fp8_of_code(c, s, S); }
int oracle_scale_for_amax_e4m3(double amax) { return ue8m0_scale_for_amax_e4m3(amax); }
double oracle_e4m3_value(uint8_t b) { return e4m3_value(b); }
uint16_t oracle_bf16_round(double v) { return bf16_round(v); }
