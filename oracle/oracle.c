/*
 * CPU oracle for the FP8 block-scaled NT GEMM (test infrastructure).
 *
 * This file is test infrastructure. Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load it. The product library never
 * links, loads or calls it, and it shares no code with the HIP path.
 *
 * What it computes, and where that is stated:
 *
 *   D[m,n] = bf16( sum_kb (sa[m,kb] * sb[n/128,kb]) * sum_{k in block kb} A[m,k] * B[n,k] )
 *
 *   - DeepGEMM fp8_gemm.cuh (DeepSeek/DeepGEMM mirror, commit 676329b8e2),
 *     fp8_gemm_kernel: the static check that fixes the K block at 128
 *     channels; the math warp-groups' per-stage loop, where the WGMMA batch
 *     of one 128-wide K block yields a partial sum that is then scaled by the
 *     product of the A-row scale and the B-block scale and added into
 *     final_accum; and the epilogue's round-to-nearest bf16 conversion.
 *   - Same kernel, B-scale staging: column n of B uses scale row n/128
 *     (the tile's scale row is (n_block*BLOCK_N)/BLOCK_K, a tile that
 *     straddles a 128-column boundary takes a second row, picked per
 *     8-column group).
 *   - Same file, Gemm::make_2d_tma_*_desc: A is [rows][K] with K contiguous,
 *     B is [N (x groups)][K] with K contiguous, D is [rows][N] row major.
 *
 * Precision: every e4m3 value is an integer multiple of 2^-9 of magnitude at
 * most 448, so a product is a multiple of 2^-18 below 2^18 and a 128-term
 * block sum needs fewer than 53 significant bits: the fp64 block sum is
 * exact.  The scale product of two fp32 numbers is exact in fp64 as well.
 * The only roundings are the fp64 accumulation over K blocks and the final
 * round to bf16, done once, straight from fp64, to nearest with ties to even.
 *
 * Readings where the pages are silent (each is also listed with the design
 * notes):
 *   - e4m3 is the OCP E4M3FN format (bias 7, no infinities, S.1111.111 is
 *     NaN, largest finite 448).  The page names only the type __nv_fp8_e4m3.
 *   - Quantization (not on the pages; fixed by the workload description):
 *     scale = amax/448 in fp32 with IEEE division, code = e4m3 round to
 *     nearest even of (x / scale) computed in fp32, saturated to +-448.
 *     A block whose amax is zero stores scale 0 and codes 0.
 *   - Grouped routing: a contiguous-grouped row r uses group layout[r] when
 *     0 <= layout[r] < G and is otherwise left untouched; a masked group g
 *     writes rows r < clamp(masked_m[g], 0, M_max) and leaves the rest
 *     untouched.
 *
 * Compile with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <omp.h>

/* ------------------------------------------------------------------ e4m3 */

/* OCP E4M3FN decode, written from the format's definition:
 * sign s, 4-bit exponent e (bias 7), 3-bit mantissa m.
 *   e == 0            : (-1)^s * (m/8) * 2^-6        (subnormal, and zero)
 *   e == 15 and m == 7: NaN
 *   otherwise         : (-1)^s * (1 + m/8) * 2^(e-7)                     */
double orc_e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Magnitudes of the finite non-negative codes 0x00..0x7E, filled once from
 * the decode above.  They increase strictly with the code. */
static double e4m3_grid[0x7F];

__attribute__((constructor)) static void fill_e4m3_grid(void)
{
    for (int c = 0; c <= 0x7E; ++c)
        e4m3_grid[c] = orc_e4m3_value((uint8_t)c);
}

/* Round an fp32 value to the nearest e4m3 value, ties to the even code,
 * saturating at +-448.  The nearest grid point is found by bisection on the
 * increasing table of magnitudes, then the two neighbours are compared; on
 * an exact tie the code with mantissa lsb 0 wins.  The sign is carried
 * separately, so -0 and small negatives map to 0x80.  NaN maps to the NaN
 * code with the input's sign. */
uint8_t orc_e4m3_from_float(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 0x7E;                  /* grid[lo] <= a < grid[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_grid[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double d_lo = a - e4m3_grid[lo], d_hi = e4m3_grid[hi] - a;
    int best;
    if (d_lo < d_hi)
        best = lo;
    else if (d_hi < d_lo)
        best = hi;
    else
        best = (lo & 1) == 0 ? lo : hi;
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------ bf16 */

/* Round an fp64 value to bf16 (8 significant bits, 8-bit exponent, bias
 * 127), to nearest with ties to even, keeping bf16 subnormals (spacing
 * 2^-133) and sending values past the largest finite bf16 to +-inf.
 * Returns the 16-bit pattern. */
uint16_t orc_bf16_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);                   /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                        /* exponent of the last kept bit */
    if (q < -133)
        q = -133;                         /* bf16 subnormal spacing */
    double scaled = ldexp(a, -q);         /* exact: power-of-two scaling */
    double r = nearbyint(scaled);         /* default mode: ties to even */
    double rounded = ldexp(r, q);
    if (rounded >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    float f = (float)rounded;             /* exact: <= 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)((bits >> 16) & 0x7FFF));
}

/* ------------------------------------------------------------- quantize */

/* Per-token quantization of x[M][K] (fp32, row major) into q[M][K] e4m3
 * codes and s[M][K/128] fp32 scales: one scale per row per 128-wide
 * K block. */
void orc_quantize_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s)
{
    int64_t KB = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const float* blk = x + m * K + kb * 128;
            float amax = 0.0f;
            for (int k = 0; k < 128; ++k) {
                float a = fabsf(blk[k]);
                if (a > amax)
                    amax = a;
            }
            float scale = amax / 448.0f;
            s[m * KB + kb] = scale;
            for (int k = 0; k < 128; ++k)
                q[m * K + kb * 128 + k] = (amax == 0.0f) ? 0 : orc_e4m3_from_float(blk[k] / scale);
        }
    }
}

/* The bf16 value with bit pattern b (1 sign, 8 exponent, 7 fraction bits)
 * is the fp32 value whose upper 16 bits are b and lower 16 bits are zero:
 * bf16 is fp32 with the fraction cut to 7 bits, same exponent range. */
float orc_bf16_value(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Per-token quantization of bf16 activations: each element converted
 * exactly to fp32, then quantized as orc_quantize_per_token does. */
void orc_quantize_per_token_bf16(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s)
{
    float* xf = (float*)malloc((size_t)(M * K) * sizeof(float));
    if (!xf)
        return;
    for (int64_t i = 0; i < M * K; ++i)
        xf[i] = orc_bf16_value(x[i]);
    orc_quantize_per_token(xf, M, K, q, s);
    free(xf);
}

/* Per-block quantization of x[N][K] into q[N][K] and s[ceil(N/128)][K/128]:
 * one scale per 128x128 block (the last row block is partial when N is not a
 * multiple of 128). */
void orc_quantize_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, float* s)
{
    int64_t KB = K / 128, NB = (N + 127) / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; ++nb) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            int64_t n_end = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
            float amax = 0.0f;
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int k = 0; k < 128; ++k) {
                    float a = fabsf(x[n * K + kb * 128 + k]);
                    if (a > amax)
                        amax = a;
                }
            float scale = amax / 448.0f;
            s[nb * KB + kb] = scale;
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int k = 0; k < 128; ++k) {
                    float v = x[n * K + kb * 128 + k];
                    q[n * K + kb * 128 + k] = (amax == 0.0f) ? 0 : orc_e4m3_from_float(v / scale);
                }
        }
    }
}

/* --------------------------------------------------- power-of-two scales */

/* Power-of-two (E8M0) block scales for the hardware block-scaled matrix
 * instruction (the Gluon tutorial page "TCGen05 Copy Instruction", its
 * section on tensor scales: per-block scales are handed to the scaled MMA
 * next to the operands and applied by it).  Byte b stands for 2^(b - 127);
 * 255 is NaN.  The recipe is not on the pages; the reading taken here keeps
 * the 1x128 / 128x128 blocks of the fp32 recipe and rounds the scale up to
 * a power of two: a block's exponent is the smallest e >= -127 with
 * amax <= 448 * 2^e, so x * 2^-e stays within the e4m3 range and no code
 * saturates.  Scales are stored one byte per block, rows of K/128 bytes
 * padded to a multiple of 4 (the padding is neither read nor written). */
double orc_e8m0_value(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* The exponent of the rule above, found by counting up from -127: plain and
 * slow, at most 248 steps for a finite amax. */
int orc_e8m0_exponent(float amax)
{
    int e = -127;
    while ((double)amax > ldexp(448.0, e))
        ++e;
    return e;
}

/* Codes of one block: e4m3 of x * 2^-e (exact in fp64; the fp32 value it is
 * rounded from is exact too, except below the fp32 normal range, where the
 * e4m3 result is a signed zero either way). */
static uint8_t e8m0_code(float v, int e)
{
    return orc_e4m3_from_float((float)ldexp((double)v, -e));
}

static int64_t e8m0_pitch(int64_t KB)
{
    return (KB + 3) / 4 * 4;
}

/* Per-token quantization with power-of-two scales: q[M][K] e4m3 codes,
 * s[M][KBp] exponent bytes, KBp = K/128 rounded up to a multiple of 4. */
void orc_quantize_per_token_e8m0(const float* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s)
{
    int64_t KB = K / 128, KBp = e8m0_pitch(KB);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const float* blk = x + m * K + kb * 128;
            float amax = 0.0f;
            for (int k = 0; k < 128; ++k) {
                float a = fabsf(blk[k]);
                if (a > amax)
                    amax = a;
            }
            int e = orc_e8m0_exponent(amax);
            s[m * KBp + kb] = (uint8_t)(e + 127);
            for (int k = 0; k < 128; ++k)
                q[m * K + kb * 128 + k] = e8m0_code(blk[k], e);
        }
    }
}

/* Per-block (128x128) quantization with power-of-two scales: q[N][K],
 * s[ceil(N/128)][KBp]. */
void orc_quantize_per_block_e8m0(const float* x, int64_t N, int64_t K, uint8_t* q, uint8_t* s)
{
    int64_t KB = K / 128, KBp = e8m0_pitch(KB), NB = (N + 127) / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; ++nb) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            int64_t n_end = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
            float amax = 0.0f;
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int k = 0; k < 128; ++k) {
                    float a = fabsf(x[n * K + kb * 128 + k]);
                    if (a > amax)
                        amax = a;
                }
            int e = orc_e8m0_exponent(amax);
            s[nb * KBp + kb] = (uint8_t)(e + 127);
            for (int64_t n = nb * 128; n < n_end; ++n)
                for (int k = 0; k < 128; ++k)
                    q[n * K + kb * 128 + k] = e8m0_code(x[n * K + kb * 128 + k], e);
        }
    }
}

/* ----------------------------------------------------------------- GEMM */

/* One output row of the block-scaled NT GEMM, straight from the definition:
 * for every column n, for every K block kb, the exact fp64 block dot product
 * S of A's row and B's row n, then V += (sa[kb] * sb[n/128][kb]) * S, and
 * finally D = bf16(V).
 *   a_row : K codes of one A row      sa_row : K/128 scales of that row
 *   b     : [N][K] codes              sb     : [ceil(N/128)][K/128] scales
 *   d_row : N bf16 outputs                                                 */
static void oracle_row_c(const uint8_t* a_row, const float* sa_row,
                         const uint8_t* b, const float* sb, const float* c_row,
                         int64_t N, int64_t K, uint16_t* d_row)
{
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_value((uint8_t)c);
    int64_t KB = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t* b_row = b + n * K;
        const float* sb_row = sb + (n / 128) * KB;
        double v = 0.0;
        for (int64_t kb = 0; kb < KB; ++kb) {
            double block = 0.0;
            for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
                block += dec[a_row[k]] * dec[b_row[k]];
            double scale = (double)sa_row[kb] * (double)sb_row[kb];
            v += scale * block;
        }
        if (c_row)
            v += (double)c_row[n];
        d_row[n] = orc_bf16_from_double(v);
    }
}

static void oracle_row(const uint8_t* a_row, const float* sa_row,
                       const uint8_t* b, const float* sb,
                       int64_t N, int64_t K, uint16_t* d_row)
{
    oracle_row_c(a_row, sa_row, b, sb, NULL, N, K, d_row);
}

/* Dense form: A[M][K], sa[M][K/128], B[N][K], sb[ceil(N/128)][K/128],
 * D[M][N]; every row is written. */
void orc_gemm_nt(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                 uint16_t* D, int64_t M, int64_t N, int64_t K)
{
    int64_t KB = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        oracle_row(A + m * K, sa + m * KB, B, sb, N, K, D + m * N);
}

/* Dense form with an fp32 addend C[M][N]: D = bf16(C + the dense sum),
 * the addend joining the fp64 sum before the single rounding (the matmul
 * accumulate case of the Triton Gluon tutorial page "TCGen05 Copy
 * Instruction": D = A @ B + C with C in fp32). */
void orc_gemm_nt_acc(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                     const float* C, uint16_t* D, int64_t M, int64_t N, int64_t K)
{
    int64_t KB = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        oracle_row_c(A + m * K, sa + m * KB, B, sb, C + m * N, N, K, D + m * N);
}

/* Dense form on a chosen list of rows; row i of out[nrows][N] receives
 * D[rows[i]]. */
void orc_gemm_nt_rows(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t* rows, int64_t nrows, uint16_t* out)
{
    int64_t KB = K / 128;
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i)
        oracle_row(A + rows[i] * K, sa + rows[i] * KB, B, sb, N, K, out + i * N);
}

/* Contiguous-grouped form: A[M_sum][K], sa[M_sum][K/128], B[G][N][K],
 * sb[G][ceil(N/128)][K/128], D[M_sum][N], layout[M_sum] int32 group ids.
 * Row r is computed with group layout[r] when that id lies in [0, G);
 * any other row of D is left as it was. */
void orc_gemm_grouped_contiguous(const uint8_t* A, const float* sa, const uint8_t* B,
                                 const float* sb, uint16_t* D, const int32_t* layout,
                                 int64_t M_sum, int64_t N, int64_t K, int64_t G)
{
    int64_t KB = K / 128, NB = (N + 127) / 128;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < M_sum; ++r) {
        int64_t g = layout[r];
        if (g < 0 || g >= G)
            continue;
        oracle_row(A + r * K, sa + r * KB, B + g * N * K, sb + g * NB * KB, N, K, D + r * N);
    }
}

/* Contiguous-grouped form on a chosen list of rows of A; out[i] receives the
 * row of D for rows[i], or is left as it was when that row is not routed. */
void orc_gemm_grouped_contiguous_rows(const uint8_t* A, const float* sa, const uint8_t* B,
                                      const float* sb, const int32_t* layout,
                                      int64_t M_sum, int64_t N, int64_t K, int64_t G,
                                      const int64_t* rows, int64_t nrows, uint16_t* out)
{
    int64_t KB = K / 128, NB = (N + 127) / 128;
    (void)M_sum;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        int64_t g = layout[r];
        if (g < 0 || g >= G)
            continue;
        oracle_row(A + r * K, sa + r * KB, B + g * N * K, sb + g * NB * KB, N, K, out + i * N);
    }
}

static int64_t masked_rows_of(const int32_t* masked_m, int64_t g, int64_t M_max)
{
    int64_t v = masked_m[g];
    if (v < 0)
        v = 0;
    if (v > M_max)
        v = M_max;
    return v;
}

/* Masked-grouped form: A[G][M_max][K], sa[G][M_max][K/128], B[G][N][K],
 * sb[G][ceil(N/128)][K/128], D[G][M_max][N], masked_m[G].  Rows
 * r < clamp(masked_m[g], 0, M_max) of slab g are computed with B[g];
 * the other rows of D are left as they were. */
void orc_gemm_grouped_masked(const uint8_t* A, const float* sa, const uint8_t* B,
                             const float* sb, uint16_t* D, const int32_t* masked_m,
                             int64_t G, int64_t M_max, int64_t N, int64_t K)
{
    int64_t KB = K / 128, NB = (N + 127) / 128;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t g = 0; g < G; ++g) {
        for (int64_t r = 0; r < M_max; ++r) {
            if (r >= masked_rows_of(masked_m, g, M_max))
                continue;
            int64_t row = g * M_max + r;
            oracle_row(A + row * K, sa + row * KB, B + g * N * K, sb + g * NB * KB, N, K,
                       D + row * N);
        }
    }
}

/* Masked-grouped form on a chosen list of flat rows (g * M_max + r). */
void orc_gemm_grouped_masked_rows(const uint8_t* A, const float* sa, const uint8_t* B,
                                  const float* sb, const int32_t* masked_m,
                                  int64_t G, int64_t M_max, int64_t N, int64_t K,
                                  const int64_t* rows, int64_t nrows, uint16_t* out)
{
    int64_t KB = K / 128, NB = (N + 127) / 128;
    (void)G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows[i];
        int64_t g = row / M_max, r = row % M_max;
        if (r >= masked_rows_of(masked_m, g, M_max))
            continue;
        oracle_row(A + row * K, sa + row * KB, B + g * N * K, sb + g * NB * KB, N, K,
                   out + i * N);
    }
}

/* Threads an OpenMP parallel region of this library uses. */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}

/* Set the thread count of later parallel regions (timing on one core). */
void orc_set_num_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}
