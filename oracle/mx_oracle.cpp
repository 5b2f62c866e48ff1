/*
 * mx_oracle.cpp -- plain, slow CPU oracle for the MXFP8 microscaled hot path.
 *
 * C++ kept to plain functions over arrays (no classes, templates or library
 * algorithms), so that each step reads as the definition it follows; the
 * functions have C linkage for the ctypes wrappers in oracle/__init__.py.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the package's smoke check and the bench's
 * CPU-baseline leg do.  It shares no code, header, table or constant
 * generator with the HIP kernels.
 *
 * Everything is computed in IEEE binary64 from the definitions:
 *
 *   - MX block quantisation: a block of 32 consecutive elements (or a 32x32
 *     weight tile) shares one E8M0 scale that is recomputed from the data on
 *     every call.  Sources: torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8 / HiF8
 *     architecture overview" (the MXFP8 bullet: 32 elements share one e8m0
 *     scale, dynamic quantisation, BF16 output); MindSpeed RFC "add
 *     MXFP8-32x32 quantisation support to FSDP", sections 1.1, 3.1 and 3.3.3
 *     (block size [1,32,32], forward and backward share one FP8 weight and
 *     differ only in the scale).
 *   - The scale rule is "rceil": the scale exponent is the smallest integer e
 *     with amax <= 448 * 2^e, i.e. ceil(log2(amax / 448)); the tutorial's
 *     step-3 log names the recipe "mxfp8_rceil".  Elements are divided by
 *     2^e, rounded to nearest (ties to even) and saturated to E4M3 (the RFC,
 *     section 3.3.1, fixes the element type to E4M3).
 *   - The number formats E4M3 (OCP OFP8 "E4M3FN": bias 7, max 448, no
 *     infinities, S.1111.111 = NaN) and E8M0 (unsigned power-of-two exponent,
 *     bias 127, 0xFF = NaN) are named, not defined, by the pages; they are
 *     written out here from the OCP definitions.
 *
 * Readings taken where the pages are silent (each also listed with its
 * justification in the design notes of the repository):
 *   R1  amax == 0: the exponent is clamped to its smallest value, -127, so the
 *       scale byte is 0x00.
 *   R2  the exponent is clamped to the finite E8M0 range [-127, 127].
 *   R3  a block holding a NaN or an infinity gets scale byte 0xFF (NaN) and
 *       every payload byte 0x7F (E4M3 NaN).
 *   R4  the sign of a zero result is kept (-0 and tiny negatives give 0x80).
 *   R5  BF16 subnormal inputs are not flushed.
 *   R6  saturation clamps to +-448 (unreachable for finite blocks: every
 *       |x| <= amax <= 448 * 2^e).
 *   R7  column-axis output is written transposed: q_t[c][r], s_t[c][r/32].
 *   R8  the 32x32 forward and backward scales are two views of one tile
 *       array s[R/32][C/32].
 *   R22 E5M2 payload (an allowed element type besides E4M3): the scale
 *       keeps the rceil rule with E5M2's largest finite value, the smallest
 *       e with amax <= 57344 * 2^e; elements round to nearest-even E5M2
 *       (OCP "E5M2": bias 15, 0x7C = infinity, 0x7D..0x7F = NaN), saturating
 *       at +-57344 (unreachable for finite blocks); a NaN/Inf block gets
 *       scale 0xFF and payload 0x7F (an E5M2 NaN) as in R3.
 *   R20 MoE backward, per-group column blocks: along the token axis, blocks
 *       of 32 restart at every group offset and a group's last block holds
 *       only its remaining rows; its amax covers those rows alone.  The
 *       transposed output gives group g the column range starting at
 *       P_g = 128 * (floor(o_g / 128) + g), i.e. a capacity of
 *       128 * (floor(T / 128) + G) columns (every range starts on a whole
 *       128-byte line, and its scales on a whole 4-byte word); every column
 *       that holds no token (the rest of a partial block, the gaps between
 *       groups) belongs to an all-zero block: payload 0x00, scale 0x00 (R1).
 *
 * Threading: OpenMP over independent rows / blocks only; no element's
 * arithmetic is split or reordered.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>

extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* BF16: 1 sign, 8 exponent bits (bias 127), 7 mantissa bits; the top half of
 * an IEEE binary32.  Exact in binary64. */
double orc_bf16_value(uint16_t bits)
{
    int s = bits >> 15;
    int E = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double mag;
    if (E == 0xFF)
        mag = m ? NAN : INFINITY;
    else if (E == 0)
        mag = ldexp((double)m, -126 - 7);          /* subnormal: 0.m * 2^-126 */
    else
        mag = ldexp(1.0 + m / 128.0, E - 127);
    return s ? -mag : mag;
}

/* OCP E4M3: S.EEEE.MMM, bias 7.  E=0 is subnormal (2^-6 * M/8); E=15,M=7 is
 * NaN; there is no infinity.  Largest finite value 0x7E = 448. */
double orc_e4m3_value(uint8_t code)
{
    int s = code >> 7;
    int E = (code >> 3) & 0xF;
    int M = code & 0x7;
    double mag;
    if (E == 15 && M == 7)
        return NAN;
    if (E == 0)
        mag = ldexp(M / 8.0, -6);
    else
        mag = ldexp(1.0 + M / 8.0, E - 7);
    return s ? -mag : mag;
}

/* OCP E5M2: S.EEEEE.MM, bias 15.  E=0 is subnormal (2^-14 * M/4); E=31 is
 * infinity (M=0) or NaN (M!=0).  Largest finite value 0x7B = 57344. */
double orc_e5m2_value(uint8_t code)
{
    int s = code >> 7;
    int E = (code >> 2) & 0x1F;
    int M = code & 0x3;
    double mag;
    if (E == 31)
        mag = M ? NAN : INFINITY;
    else if (E == 0)
        mag = ldexp(M / 4.0, -14);
    else
        mag = ldexp(1.0 + M / 4.0, E - 15);
    return s ? -mag : mag;
}

/* E8M0: unsigned exponent, value 2^(b-127); 0xFF is NaN. */
double orc_e8m0_value(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Round a binary64 value to E4M3: nearest representable value, ties to the
 * even mantissa, saturating to +-448 (R6), NaN -> 0x7F, sign of zero kept
 * (R4).  The grid of E4M3 magnitudes has spacing 2^-9 below 2^-6 (subnormal
 * range) and 2^(floor(log2|v|) - 3) above. */
uint8_t orc_e4m3_round(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    int p; /* a lies on the grid k * 2^p */
    if (a < 0x1p-6) {
        p = -9;
    } else {
        int ex;
        frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
        p = (ex - 1) - 3;       /* three fraction bits below the leading one */
    }
    double k = nearbyint(ldexp(a, -p)); /* default rounding mode: ties to even */
    double r = ldexp(k, p);             /* the rounded magnitude, <= 448 here */
    if (r == 0.0)
        return sign;
    if (r < 0x1p-6) /* subnormal code: r = M * 2^-9 */
        return sign | (uint8_t)ldexp(r, 9);
    int ex;
    double f = frexp(r, &ex); /* r = f * 2^ex = (2f) * 2^(ex-1) */
    int E = (ex - 1) + 7;
    int M = (int)((2.0 * f - 1.0) * 8.0);
    return sign | (uint8_t)((E << 3) | M);
}

/* Round a binary64 value to E5M2 (R22): nearest representable value, ties
 * to the even mantissa, saturating to +-57344, NaN -> 0x7F, sign of zero
 * kept.  Grid spacing 2^-16 below 2^-14 (subnormals), 2^(floor(log2|v|) - 2)
 * above. */
uint8_t orc_e5m2_round(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 57344.0)
        return sign | 0x7B;
    int p;
    if (a < 0x1p-14) {
        p = -16;
    } else {
        int ex;
        frexp(a, &ex);
        p = (ex - 1) - 2;       /* two fraction bits below the leading one */
    }
    double k = nearbyint(ldexp(a, -p));
    double r = ldexp(k, p);
    if (r == 0.0)
        return sign;
    if (r < 0x1p-14) /* subnormal code: r = M * 2^-16 */
        return sign | (uint8_t)ldexp(r, 16);
    int ex;
    double f = frexp(r, &ex);
    int E = (ex - 1) + 15;
    int M = (int)((2.0 * f - 1.0) * 4.0);
    return sign | (uint8_t)((E << 2) | M);
}

/* The smallest integer e with amax <= emax_value * 2^e, i.e. the ceiling of
 * log2(amax / emax_value), clamped to [-127, 127] (R1, R2). */
static int rceil_for(double amax, double emax_value)
{
    if (amax == 0.0)
        return -127;
    int e = (int)ceil(log2(amax / emax_value));
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    /* make the log2 estimate exactly the definition */
    while (e > -127 && amax <= ldexp(emax_value, e - 1))
        e--;
    while (e < 127 && amax > ldexp(emax_value, e))
        e++;
    return e;
}

/* rceil: the smallest integer e with amax <= 448 * 2^e, i.e. the ceiling of
 * log2(amax / 448), clamped to [-127, 127] (R1, R2). */
int orc_rceil_exponent(double amax)
{
    return rceil_for(amax, 448.0);
}

/* The same rule for E5M2 elements (R22): amax <= 57344 * 2^e. */
int orc_rceil_exponent_e5m2(double amax)
{
    return rceil_for(amax, 57344.0);
}

/* Element types of the payload. */
enum { ELEM_E4M3 = 0, ELEM_E5M2 = 1 };

static double elem_value(int elem, uint8_t code)
{
    return elem == ELEM_E5M2 ? orc_e5m2_value(code) : orc_e4m3_value(code);
}

/* ------------------------------------------------------------------------ */
/* One MX block                                                              */
/* ------------------------------------------------------------------------ */

/* Quantise n values (already decoded to binary64) sharing one scale into
 * payload elements of type elem.  Writes n codes, returns the scale byte. */
static uint8_t quant_block_elem(int elem, int n, const double *v, uint8_t *codes)
{
    for (int i = 0; i < n; i++) {
        if (!isfinite(v[i])) { /* R3 */
            for (int j = 0; j < n; j++)
                codes[j] = 0x7F;
            return 0xFF;
        }
    }
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    int e = elem == ELEM_E5M2 ? orc_rceil_exponent_e5m2(amax) : orc_rceil_exponent(amax);
    for (int i = 0; i < n; i++) {
        double w = ldexp(v[i], -e); /* exact power-of-two scaling */
        codes[i] = elem == ELEM_E5M2 ? orc_e5m2_round(w) : orc_e4m3_round(w);
    }
    return (uint8_t)(e + 127);
}


/* ------------------------------------------------------------------------ */
/* Quantisation modes.  x is BF16 [R, C] row-major.                          */
/* ------------------------------------------------------------------------ */

/* 1x32 along the row (the contraction axis of a TN GEMM):
 * q[R][C], s[R][C/32].  Requires C % 32 == 0.  elem: payload type. */
void orc_quant_row_elem(const uint16_t *x, int64_t R, int64_t C, int elem, uint8_t *q, uint8_t *s)
{
    int64_t nb = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++) {
        double v[32];
        for (int64_t j = 0; j < nb; j++) {
            for (int i = 0; i < 32; i++)
                v[i] = orc_bf16_value(x[r * C + 32 * j + i]);
            s[r * nb + j] = quant_block_elem(elem, 32, v, q + r * C + 32 * j);
        }
    }
}

/* 32x1 along the column (blocks of 32 consecutive rows of one column),
 * written transposed (R7): q_t[C][R], s_t[C][R/32].  Requires R % 32 == 0. */
void orc_quant_col_elem(const uint16_t *x, int64_t R, int64_t C, int elem, uint8_t *q_t,
                        uint8_t *s_t)
{
    int64_t nb = R / 32;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; c++) {
        double v[32];
        for (int64_t i = 0; i < nb; i++) {
            for (int k = 0; k < 32; k++)
                v[k] = orc_bf16_value(x[(32 * i + k) * C + c]);
            s_t[c * nb + i] = quant_block_elem(elem, 32, v, q_t + c * R + 32 * i);
        }
    }
}

/* 32x32 tiles (RFC block size [1,32,32]): one scale per tile, payload in the
 * original layout: q[R][C], s[R/32][C/32] (R8).  Requires R, C % 32 == 0. */
void orc_quant_block32_elem(const uint16_t *x, int64_t R, int64_t C, int elem, uint8_t *q,
                            uint8_t *s)
{
    int64_t tr = R / 32, tc = C / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tr * tc; t++) {
        int64_t i = t / tc, j = t % tc;
        double v[1024];
        uint8_t codes[1024];
        for (int a = 0; a < 32; a++)
            for (int b = 0; b < 32; b++)
                v[32 * a + b] = orc_bf16_value(x[(32 * i + a) * C + 32 * j + b]);
        s[i * tc + j] = quant_block_elem(elem, 1024, v, codes);
        for (int a = 0; a < 32; a++)
            memcpy(q + (32 * i + a) * C + 32 * j, codes + 32 * a, 32);
    }
}

void orc_quant_row(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, uint8_t *s)
{
    orc_quant_row_elem(x, R, C, ELEM_E4M3, q, s);
}

void orc_quant_col(const uint16_t *x, int64_t R, int64_t C, uint8_t *q_t, uint8_t *s_t)
{
    orc_quant_col_elem(x, R, C, ELEM_E4M3, q_t, s_t);
}

void orc_quant_block32(const uint16_t *x, int64_t R, int64_t C, uint8_t *q, uint8_t *s)
{
    orc_quant_block32_elem(x, R, C, ELEM_E4M3, q, s);
}

/* ------------------------------------------------------------------------ */
/* GEMM: C[m][n] = sum_k A[m][k] * B[n][k] on the dequantised operands       */
/* ------------------------------------------------------------------------ */

/* How the B operand and its scales are laid out:
 *   0  B bytes [N][K], scales [N][K/32]           (1x32 blocks along K)
 *   1  B bytes [N][K], tile scales [N/32][K/32]   (32x32 weight, forward)
 *   2  B bytes [K][N], tile scales [K/32][N/32]   (the same 32x32 weight
 *      stored [out=K][in=N], contracted over its rows: backward data) */
static double b_value(int bkind, int elem, int64_t N, int64_t K, const uint8_t *b,
                      const uint8_t *sb, int64_t n, int64_t k)
{
    switch (bkind) {
    case 0:
        return elem_value(elem, b[n * K + k]) * orc_e8m0_value(sb[n * (K / 32) + k / 32]);
    case 1:
        return elem_value(elem, b[n * K + k]) * orc_e8m0_value(sb[(n / 32) * (K / 32) + k / 32]);
    default:
        return elem_value(elem, b[k * N + n]) * orc_e8m0_value(sb[(k / 32) * (N / 32) + n / 32]);
    }
}

/* ref[M][N] = sum_k a*b in binary64 and bound[M][N] = sum_k |a*b| (the
 * tolerance scale).  a: bytes [M][K] with scales [M][K/32].  Either output
 * pointer may be NULL.  Returns 0, or -1 on a shape the layout forbids. */
int orc_gemm_elem(int bkind, int a_elem, int b_elem, int64_t M, int64_t N, int64_t K,
                  const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                  double *ref, double *bound)
{
    if (K % 32 != 0 || M < 0 || N < 0)
        return -1;
    if (bkind != 0 && N % 32 != 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    /* dequantise B once: bt[n][k] */
    double *bt = (double *)malloc((size_t)N * (size_t)(K ? K : 1) * sizeof(double));
    if (!bt)
        return -2;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            bt[n * K + k] = b_value(bkind, b_elem, N, K, b, sb, n, k);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) {
        double *av = (double *)malloc((size_t)(K ? K : 1) * sizeof(double));
        if (!av)
            abort();
        for (int64_t k = 0; k < K; k++)
            av[k] = elem_value(a_elem, a[m * K + k]) * orc_e8m0_value(sa[m * (K / 32) + k / 32]);
        for (int64_t n = 0; n < N; n++) {
            const double *bv = bt + n * K;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = av[k] * bv[k];
                acc += p;
                mag += fabs(p);
            }
            if (ref)
                ref[m * N + n] = acc;
            if (bound)
                bound[m * N + n] = mag;
        }
        free(av);
    }
    free(bt);
    return 0;
}

/* E4M3 operands. */
int orc_gemm(int bkind, int64_t M, int64_t N, int64_t K,
             const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
             double *ref, double *bound)
{
    return orc_gemm_elem(bkind, ELEM_E4M3, ELEM_E4M3, M, N, K, a, sa, b, sb, ref, bound);
}

/* Grouped GEMM for MoE experts: rows offsets[g] .. offsets[g+1]-1 of the
 * token matrix a [T][K] are multiplied by expert g's weight b[g] ([N][K],
 * scales [N][K/32]); ref/bound are [T][N].  Empty groups contribute no rows.
 * Returns 0, or -1 if the offsets are not a non-decreasing cover of [0, T]. */
int orc_grouped_gemm(int64_t G, const int64_t *offsets, int64_t T, int64_t N, int64_t K,
                     const uint8_t *a, const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                     double *ref, double *bound)
{
    if (K % 32 != 0 || offsets[0] != 0 || offsets[G] != T)
        return -1;
    for (int64_t g = 0; g < G; g++)
        if (offsets[g + 1] < offsets[g])
            return -1;
    for (int64_t g = 0; g < G; g++) {
        int64_t r0 = offsets[g], rows = offsets[g + 1] - offsets[g];
        if (rows == 0)
            continue;
        int rc = orc_gemm(0, rows, N, K, a + r0 * K, sa + r0 * (K / 32),
                          b + g * N * K, sb + g * N * (K / 32),
                          ref ? ref + r0 * N : NULL, bound ? bound + r0 * N : NULL);
        if (rc)
            return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MoE backward                                                              */
/* ------------------------------------------------------------------------ */

/* First column of group g (R20). */
static int64_t group_col(int64_t g, int64_t o_g)
{
    return 128 * (o_g / 128 + g);
}

int64_t orc_grouped_col_capacity(int64_t T, int64_t G)
{
    return 128 * (T / 128 + G);
}

static int offsets_ok(int64_t G, const int64_t *offsets, int64_t T)
{
    if (G < 0 || offsets[0] != 0 || offsets[G] != T)
        return 0;
    for (int64_t g = 0; g < G; g++)
        if (offsets[g + 1] < offsets[g])
            return 0;
    return 1;
}

/* Column blocks per group (R20): x is BF16 [T][C]; q_t[C][cap] and
 * s_t[C][cap / 32] with cap = orc_grouped_col_capacity(T, G).  The last block
 * of a group is quantised from its remaining rows only.  elem is the payload
 * element type (E4M3 or E5M2, the block rule being the same with that
 * type's largest finite value).  Returns 0, or -1 on bad offsets, an unknown
 * element type or C % 32 != 0. */
int orc_quant_col_grouped_elem(const uint16_t *x, int64_t T, int64_t C, int64_t G,
                               const int64_t *offsets, int elem, uint8_t *q_t, uint8_t *s_t)
{
    if (!offsets_ok(G, offsets, T) || C % 32 != 0 || (elem != ELEM_E4M3 && elem != ELEM_E5M2))
        return -1;
    const int64_t cap = orc_grouped_col_capacity(T, G), nbc = cap / 32;
    memset(q_t, 0, (size_t)(C * cap));
    memset(s_t, 0, (size_t)(C * nbc));
    for (int64_t g = 0; g < G; g++) {
        const int64_t o = offsets[g], rows = offsets[g + 1] - offsets[g];
        const int64_t P = group_col(g, o);
        const int64_t nb = (rows + 31) / 32;
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < C; c++) {
            double v[32];
            uint8_t codes[32];
            for (int64_t j = 0; j < nb; j++) {
                const int n = (int)((rows - 32 * j) < 32 ? (rows - 32 * j) : 32);
                for (int k = 0; k < n; k++)
                    v[k] = orc_bf16_value(x[(o + 32 * j + k) * C + c]);
                s_t[c * nbc + P / 32 + j] = quant_block_elem(elem, n, v, codes);
                memcpy(q_t + c * cap + P + 32 * j, codes, (size_t)n);
            }
        }
    }
    return 0;
}

int orc_quant_col_grouped(const uint16_t *x, int64_t T, int64_t C, int64_t G,
                          const int64_t *offsets, uint8_t *q_t, uint8_t *s_t)
{
    return orc_quant_col_grouped_elem(x, T, C, G, offsets, ELEM_E4M3, q_t, s_t);
}

/* Per-expert weight gradient: for every group g,
 *   ref[g][m][n] = sum over the group's tokens t of A[m][t] * B[n][t]
 * where A = a [M][cap] (scales [M][cap/32]) and B = b [N][cap] are the
 * per-group column-quantised copies of (for MoE) the output gradient and the
 * expert input, token t of group g sitting at column P_g + (t - o_g) (R20).
 * An empty group gives ref = bound = 0.  ref/bound are [G][M][N].  a_elem /
 * b_elem are the payload element types of A and B (E4M3 or E5M2); -1 on an
 * unknown one. */
int orc_grouped_gemm_wgrad_elem(int64_t G, const int64_t *offsets, int64_t T, int64_t M,
                                int64_t N, int a_elem, int b_elem, const uint8_t *a,
                                const uint8_t *sa, const uint8_t *b, const uint8_t *sb,
                                double *ref, double *bound)
{
    if (!offsets_ok(G, offsets, T) || M < 0 || N < 0 ||
        (a_elem != ELEM_E4M3 && a_elem != ELEM_E5M2) || (b_elem != ELEM_E4M3 && b_elem != ELEM_E5M2))
        return -1;
    const int64_t cap = orc_grouped_col_capacity(T, G), nbc = cap / 32;
    for (int64_t g = 0; g < G; g++) {
        const int64_t o = offsets[g], rows = offsets[g + 1] - offsets[g];
        const int64_t P = group_col(g, o);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; m++) {
            for (int64_t n = 0; n < N; n++) {
                double acc = 0.0, mag = 0.0;
                for (int64_t t = 0; t < rows; t++) {
                    const int64_t k = P + t;
                    double p = elem_value(a_elem, a[m * cap + k]) * orc_e8m0_value(sa[m * nbc + k / 32]) *
                               elem_value(b_elem, b[n * cap + k]) * orc_e8m0_value(sb[n * nbc + k / 32]);
                    acc += p;
                    mag += fabs(p);
                }
                if (ref)
                    ref[(g * M + m) * N + n] = acc;
                if (bound)
                    bound[(g * M + m) * N + n] = mag;
            }
        }
    }
    return 0;
}

/* The same with E4M3 operands. */
int orc_grouped_gemm_wgrad(int64_t G, const int64_t *offsets, int64_t T, int64_t M, int64_t N,
                           const uint8_t *a, const uint8_t *sa, const uint8_t *b,
                           const uint8_t *sb, double *ref, double *bound)
{
    return orc_grouped_gemm_wgrad_elem(G, offsets, T, M, N, ELEM_E4M3, ELEM_E4M3, a, sa, b, sb, ref,
                                       bound);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

}  // extern "C"
