// Internal launchers behind the C ABI (not exported).  Each enqueues its
// kernels on `stream` and returns DG_OK, DG_ERR_SHAPE when a size passes the
// C ABI's checks but exceeds what the kernel's grid or 32-bit offsets
// address (nothing is enqueued then), or DG_ERR_HIP when the launch fails.
// The C ABI layer has already validated sizes and pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_fp8.h"

namespace dg {

// Status of the launch just enqueued.
inline dg_status launched() { return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP; }

// DenseAcc: dense routing, D = bf16(C + A B^T scaled) with C fp32 [rows][N]
enum class Form : int { Dense = 0, Contiguous = 1, Masked = 2, DenseAcc = 3 };

struct GemmArgs {
    const uint8_t* A;     // e4m3 codes, K-contiguous rows
    const void* sa;       // fp32 [rows][K/128]; E8M0 bytes [rows][SP] with e8m0
    const uint8_t* B;     // [groups][N][K]
    const void* sb;       // fp32 [groups][ceil(N/128)][K/128]; E8M0 [groups][ceil(N/128)][SP]
    uint16_t* D;          // bf16 bits, [rows][N]
    const int32_t* aux;   // contiguous: group id per row; masked: valid rows per group
    int64_t rows;         // dense: M; contiguous: M_sum; masked: M_max (rows per slab)
    int64_t N, K, G;
    const float* C;       // DenseAcc: fp32 [rows][N] added before the bf16 rounding
    bool e8m0 = false;    // scales are E8M0 exponent bytes, SP = K/128 rounded up to 4
};

dg_status launch_gemm(Form form, const GemmArgs& args, hipStream_t stream);

dg_status launch_quantize_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream);
dg_status launch_quantize_per_token_bf16(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                                          float* s, hipStream_t stream);
dg_status launch_quantize_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream);
// Power-of-two scales: s holds E8M0 bytes, rows of K/128 padded to a multiple of 4.
dg_status launch_quantize_per_token_e8m0(const float* x, int64_t M, int64_t K, uint8_t* q,
                                          uint8_t* s, hipStream_t stream);
dg_status launch_quantize_per_block_e8m0(const float* x, int64_t N, int64_t K, uint8_t* q,
                                          uint8_t* s, hipStream_t stream);

}  // namespace dg
