/*
 * dg_fp8.h - C ABI of the MI355X (gfx950) FP8 block-scaled NT GEMM library.
 *
 * The operation (DeepGEMM fp8_gemm.cuh, fp8_gemm_kernel: the 128-channel K
 * block fixed by its static check, the per-block WGMMA partial sum promoted
 * by the A-row scale times the B-block scale into final_accum, and the
 * round-to-nearest bf16 epilogue):
 *
 *   D[m,n] = bf16( sum_kb (sa[m,kb] * sb[n/128,kb]) * sum_{k in block kb} A[m,k] * B[n,k] )
 *
 * with kb = 0 .. K/128-1.  A and B are OCP E4M3FN codes (one byte each, bias
 * 7, largest finite 448), both K-contiguous ("NT": the layouts that
 * Gemm::make_2d_tma_a_desc / make_2d_tma_b_desc describe).  D is bf16 stored
 * as 16-bit patterns, row major, as make_2d_tma_d_desc describes.  Scales are
 * fp32: sa is one value per row per 128-wide K block, stored row major as
 * [rows][K/128] (the page's kernel keeps sa M-major; this library fixes the
 * row-major layout that its quantize helper writes), and sb is one value per
 * 128x128 block of B, stored [ceil(N/128)][K/128] (the layout the page's
 * B-scale staging reads).  Column n uses sb row n/128; when N is not a
 * multiple of 128 the last row covers a partial block.
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers to caller-owned, contiguous, row-major
 *     memory, each aligned to 16 bytes.  The library allocates nothing,
 *     frees nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream).  No call synchronizes; results are ready when the
 *     stream reaches them.
 *   - Arguments are checked on the host before anything is enqueued: sizes
 *     first, then pointers.  On an error the call returns a nonzero
 *     dg_status and writes nothing.  A call with no rows to compute (M, M_sum
 *     or M_max equal to 0) returns DG_OK without looking at its pointers.
 *   - Rows that a call does not route (M tail, padding rows of the
 *     contiguous form, rows past masked_m in the masked form) are never
 *     written.
 *   - Sizes that pass a call's rules but would need a grid of more than
 *     2^31 - 1 workgroups return DG_ERR_SHAPE, with nothing enqueued.
 *   - A launch failure reported by the HIP runtime returns DG_ERR_HIP.
 *   - Calls on different streams may run concurrently; they share nothing.
 */
#ifndef DG_FP8_H
#define DG_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_NULL = 1,        /* a required pointer is NULL                     */
    DG_ERR_SHAPE = 2,       /* a size is out of range (see each call)        */
    DG_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned              */
    DG_ERR_UNSUPPORTED = 4, /* valid arguments this build cannot run         */
    DG_ERR_HIP = 5          /* the HIP runtime reported an error              */
} dg_status;

/* Dense form.
 *   A  [M][K]  e4m3 codes          sa [M][K/128]          fp32
 *   B  [N][K]  e4m3 codes          sb [ceil(N/128)][K/128] fp32
 *   D  [M][N]  bf16 bits (output)
 * Sizes: M >= 0 (0 enqueues nothing), N > 0 with N % 8 == 0 (the page's
 * kernel asserts N % 8), K > 0 with K % 128 == 0 (its static check fixes the
 * 128-channel K block) and K < 2^24 (a tile's rows of K bytes are addressed
 * with 32-bit offsets).  All of M*K, N*K, M*N must be below 2^62. */
dg_status dg_fp8_gemm_nt(const uint8_t* A, const float* sa,
                         const uint8_t* B, const float* sb,
                         uint16_t* D, int64_t M, int64_t N, int64_t K,
                         void* stream);

/* Dense form with an fp32 addend: D = bf16(C + the dense form's sum), C
 * added before the single rounding to bf16.  The accumulate case of the
 * Triton Gluon tutorial page "TCGen05 Copy Instruction" (its matmul
 * accumulate section: D = A @ B + C with C held in fp32), applied to the
 * block-scaled product.
 *   C  [M][N]  fp32 (input, not modified), other arguments as in
 *   dg_fp8_gemm_nt; C and D must not overlap.  Same size rules, and
 *   N < 2^22 (DG_ERR_SHAPE otherwise). */
dg_status dg_fp8_gemm_nt_acc(const uint8_t* A, const float* sa,
                             const uint8_t* B, const float* sb,
                             const float* C, uint16_t* D,
                             int64_t M, int64_t N, int64_t K, void* stream);

/* Contiguous-grouped form (MoE experts with rows sorted by expert).
 *   A  [M_sum][K]  e4m3         sa [M_sum][K/128]               fp32
 *   B  [G][N][K]   e4m3         sb [G][ceil(N/128)][K/128]      fp32
 *   D  [M_sum][N]  bf16 bits    grouped_layout [M_sum] int32 (device)
 * Row r is computed with B[g], sb[g] for g = grouped_layout[r] when
 * 0 <= g < G; any other row (padding, id -1) is not written.  Groups are
 * padded to 128 rows, so M_sum % 128 == 0 and each aligned block of 128 rows
 * normally holds one group id >= 0; a block whose rows carry several ids is
 * computed once per id (each pass costs a whole block's work), so every row
 * still gets its own group's B.  The page's kernel takes the same per-row
 * int array (grouped_layout) and adds per-group offsets in its scheduler.
 * Sizes: M_sum >= 0, G >= 1, N and K as for the dense form. */
dg_status dg_fp8_gemm_grouped_contiguous(const uint8_t* A, const float* sa,
                                         const uint8_t* B, const float* sb,
                                         uint16_t* D, const int32_t* grouped_layout,
                                         int64_t M_sum, int64_t N, int64_t K, int64_t G,
                                         void* stream);

/* Masked-grouped form (MoE decode: a fixed slab of M_max rows per expert).
 *   A  [G][M_max][K]  e4m3      sa [G][M_max][K/128]            fp32
 *   B  [G][N][K]      e4m3      sb [G][ceil(N/128)][K/128]      fp32
 *   D  [G][M_max][N]  bf16 bits masked_m [G] int32 (device)
 * Rows r < clamp(masked_m[g], 0, M_max) of slab g are computed with B[g],
 * sb[g]; the other rows of D are not written, and a group with no valid row
 * does not read its B.  The page's tensor maps stack the G slabs of A and D
 * along rows (shape_m * kNumGroups).
 * Sizes: G >= 1, M_max >= 0, N and K as for the dense form. */
dg_status dg_fp8_gemm_grouped_masked(const uint8_t* A, const float* sa,
                                     const uint8_t* B, const float* sb,
                                     uint16_t* D, const int32_t* masked_m,
                                     int64_t G, int64_t M_max, int64_t N, int64_t K,
                                     void* stream);

/* Per-token quantization of activations: x [M][K] fp32 -> q [M][K] e4m3
 * codes and s [M][K/128] fp32, one scale per row per 128-wide K block.
 * scale = amax/448 (fp32 IEEE division), q = e4m3 of x/scale (fp32 IEEE
 * division, round to nearest even, saturated to +-448, sign kept); a block
 * with amax 0 stores scale 0 and codes 0.  Not on the pages: the recipe is
 * the workload's, and it fixes the sa layout the GEMM reads.
 * Sizes: M >= 0, K > 0 with K % 128 == 0. */
dg_status dg_quantize_fp8_per_token(const float* x, int64_t M, int64_t K,
                                    uint8_t* q, float* s, void* stream);

/* The same per-token quantization from bf16 activations: x [M][K] holds
 * bf16 bit patterns (a bf16 value is exactly the fp32 value with the same
 * upper 16 bits), converted exactly to fp32 and then quantized as above.
 * Sizes and layout of q and s as above. */
dg_status dg_quantize_fp8_per_token_bf16(const uint16_t* x, int64_t M, int64_t K,
                                         uint8_t* q, float* s, void* stream);

/* Per-block quantization of weights: x [N][K] fp32 -> q [N][K] and
 * s [ceil(N/128)][K/128], one scale per 128x128 block (the last row block is
 * partial when N % 128 != 0), same rounding as above.  For grouped B call it
 * on the flattened [G*N][K] when N % 128 == 0, else once per group.
 * Sizes: N >= 0, K > 0 with K % 128 == 0. */
dg_status dg_quantize_fp8_per_block(const float* x, int64_t N, int64_t K,
                                    uint8_t* q, float* s, void* stream);

/* ---- Power-of-two (E8M0) scales.
 * The same three forms with each block scale a power of two, held as one
 * E8M0 exponent byte (2^(b-127); 255 is NaN), for the hardware block-scaled
 * matrix instruction: the Gluon tutorial page "TCGen05 Copy Instruction",
 * section on tensor scales, hands per-block scales to the scaled MMA, which
 * applies them itself (here: v_mfma_scale_f32_16x16x128_f8f6f4, so no
 * per-block promotion step).  Blocks are the same 1x128 (A) and 128x128 (B)
 * blocks; the result is the dense form's definition with sa, sb replaced by
 * their powers of two.
 * Scale rows hold K/128 bytes padded to SP = K/128 rounded up to a multiple
 * of 4 (padding bytes are neither read nor written):
 *   dense:      sa [M][SP]            sb [ceil(N/128)][SP]
 *   contiguous: sa [M_sum][SP]        sb [G][ceil(N/128)][SP]
 *   masked:     sa [G][M_max][SP]     sb [G][ceil(N/128)][SP]
 * Everything else (operands, routing, sizes, errors) is as for the fp32-scale
 * entry point of the same form. */
dg_status dg_fp8_gemm_nt_e8m0(const uint8_t* A, const uint8_t* sa,
                              const uint8_t* B, const uint8_t* sb,
                              uint16_t* D, int64_t M, int64_t N, int64_t K, void* stream);
dg_status dg_fp8_gemm_grouped_contiguous_e8m0(const uint8_t* A, const uint8_t* sa,
                                              const uint8_t* B, const uint8_t* sb,
                                              uint16_t* D, const int32_t* grouped_layout,
                                              int64_t M_sum, int64_t N, int64_t K, int64_t G,
                                              void* stream);
dg_status dg_fp8_gemm_grouped_masked_e8m0(const uint8_t* A, const uint8_t* sa,
                                          const uint8_t* B, const uint8_t* sb,
                                          uint16_t* D, const int32_t* masked_m,
                                          int64_t G, int64_t M_max, int64_t N, int64_t K,
                                          void* stream);

/* Quantization with power-of-two scales (the recipe is not on the pages):
 * a block's exponent is the smallest e >= -127 with amax <= 448 * 2^e, its
 * byte e + 127, and q = e4m3 of x * 2^-e (an exact scaling; round to nearest
 * even, never past 448).  Per token: x [M][K] fp32 -> q [M][K],
 * s [M][SP].  Per block: x [N][K] fp32 -> q [N][K], s [ceil(N/128)][SP].
 * Sizes and errors as for the fp32-scale quantizers. */
dg_status dg_quantize_fp8_per_token_e8m0(const float* x, int64_t M, int64_t K,
                                         uint8_t* q, uint8_t* s, void* stream);
dg_status dg_quantize_fp8_per_block_e8m0(const float* x, int64_t N, int64_t K,
                                         uint8_t* q, uint8_t* s, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* dg_status_string(dg_status status);

#ifdef __cplusplus
}
#endif

#endif /* DG_FP8_H */
