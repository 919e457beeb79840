// The library's C ABI (declared in include/dg_fp8.h): host-side argument
// checks, then one enqueue on the caller's stream.  Nothing here touches the
// GPU before every check has passed, so a rejected call enqueues nothing.
#include "dg_fp8.h"

#include <hip/hip_runtime.h>

#include "launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 62;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool product_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxElems / a; }

// Checks shared by the three GEMM forms.
dg_status check_nk(int64_t N, int64_t K) {
    if (N <= 0 || N % 8 != 0) return DG_ERR_SHAPE;
    if (K <= 0 || K % 128 != 0) return DG_ERR_SHAPE;
    // a tile's rows (up to 256) of K bytes are addressed with 32-bit offsets
    if (K >= (int64_t(1) << 24)) return DG_ERR_SHAPE;
    if (!product_ok(N, K)) return DG_ERR_SHAPE;
    if (N > 0x7fffffffLL || K > 0x7fffffffLL) return DG_ERR_SHAPE;
    return DG_OK;
}

dg_status check_ptrs(const void* const* ptrs, int n) {
    for (int i = 0; i < n; ++i)
        if (ptrs[i] == nullptr) return DG_ERR_NULL;
    for (int i = 0; i < n; ++i)
        if (!aligned16(ptrs[i])) return DG_ERR_ALIGN;
    return DG_OK;
}

// The three forms, with fp32 scales or (e8) E8M0 exponent bytes; the size
// rules are the same for both.
dg_status gemm_dense(const uint8_t* A, const void* sa, const uint8_t* B, const void* sb,
                     uint16_t* D, int64_t M, int64_t N, int64_t K, void* stream, bool e8) {
    dg_status s = check_nk(N, K);
    if (s != DG_OK) return s;
    if (M < 0 || !product_ok(M, K) || !product_ok(M, N) || M > 0x7fffffffLL) return DG_ERR_SHAPE;
    if (M == 0) return DG_OK;
    const void* ptrs[] = {A, sa, B, sb, D};
    if ((s = check_ptrs(ptrs, 5)) != DG_OK) return s;
    dg::GemmArgs a{A, sa, B, sb, D, nullptr, M, N, K, 1};
    a.e8m0 = e8;
    return dg::launch_gemm(dg::Form::Dense, a, static_cast<hipStream_t>(stream));
}

dg_status gemm_contiguous(const uint8_t* A, const void* sa, const uint8_t* B, const void* sb,
                          uint16_t* D, const int32_t* grouped_layout, int64_t M_sum, int64_t N,
                          int64_t K, int64_t G, void* stream, bool e8) {
    dg_status s = check_nk(N, K);
    if (s != DG_OK) return s;
    if (G < 1 || G > 0x7fffffffLL || !product_ok(G, N * K)) return DG_ERR_SHAPE;
    if (M_sum < 0 || M_sum % 128 != 0 || M_sum > 0x7fffffffLL) return DG_ERR_SHAPE;
    if (!product_ok(M_sum, K) || !product_ok(M_sum, N)) return DG_ERR_SHAPE;
    if (M_sum == 0) return DG_OK;
    const void* ptrs[] = {A, sa, B, sb, D, grouped_layout};
    if ((s = check_ptrs(ptrs, 6)) != DG_OK) return s;
    dg::GemmArgs a{A, sa, B, sb, D, grouped_layout, M_sum, N, K, G};
    a.e8m0 = e8;
    return dg::launch_gemm(dg::Form::Contiguous, a, static_cast<hipStream_t>(stream));
}

dg_status gemm_masked(const uint8_t* A, const void* sa, const uint8_t* B, const void* sb,
                      uint16_t* D, const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N,
                      int64_t K, void* stream, bool e8) {
    dg_status s = check_nk(N, K);
    if (s != DG_OK) return s;
    if (G < 1 || G > 0x7fffffffLL || !product_ok(G, N * K)) return DG_ERR_SHAPE;
    if (M_max < 0 || M_max > 0x7fffffffLL) return DG_ERR_SHAPE;
    if (!product_ok(G * M_max, K) || !product_ok(G * M_max, N)) return DG_ERR_SHAPE;
    if (M_max == 0) return DG_OK;
    const void* ptrs[] = {A, sa, B, sb, D, masked_m};
    if ((s = check_ptrs(ptrs, 6)) != DG_OK) return s;
    dg::GemmArgs a{A, sa, B, sb, D, masked_m, M_max, N, K, G};
    a.e8m0 = e8;
    return dg::launch_gemm(dg::Form::Masked, a, static_cast<hipStream_t>(stream));
}

dg_status check_quantize(const void* x, int64_t rows, int64_t K, const void* q, const void* s,
                         bool blocks) {
    if (K <= 0 || K % 128 != 0 || rows < 0 || !product_ok(rows, K)) return DG_ERR_SHAPE;
    if (blocks && (rows + 127) / 128 > 65535) return DG_ERR_SHAPE;
    if (rows == 0) return DG_OK;
    const void* ptrs[] = {x, q, s};
    return check_ptrs(ptrs, 3);
}

}  // namespace

extern "C" {

dg_status dg_fp8_gemm_nt(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                         uint16_t* D, int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_dense(A, sa, B, sb, D, M, N, K, stream, false);
}

dg_status dg_fp8_gemm_nt_e8m0(const uint8_t* A, const uint8_t* sa, const uint8_t* B,
                              const uint8_t* sb, uint16_t* D, int64_t M, int64_t N, int64_t K,
                              void* stream) {
    return gemm_dense(A, sa, B, sb, D, M, N, K, stream, true);
}

dg_status dg_fp8_gemm_nt_acc(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                             const float* C, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             void* stream) {
    dg_status s = check_nk(N, K);
    if (s != DG_OK) return s;
    if (M < 0 || !product_ok(M, K) || !product_ok(M, N) || M > 0x7fffffffLL) return DG_ERR_SHAPE;
    if (N >= (1LL << 22)) return DG_ERR_SHAPE;  // 256 rows of fp32 C within 32-bit offsets
    if (M == 0) return DG_OK;
    const void* ptrs[] = {A, sa, B, sb, C, D};
    if ((s = check_ptrs(ptrs, 6)) != DG_OK) return s;
    dg::GemmArgs a{A, sa, B, sb, D, nullptr, M, N, K, 1, C};
    return dg::launch_gemm(dg::Form::DenseAcc, a, static_cast<hipStream_t>(stream));
}

dg_status dg_fp8_gemm_grouped_contiguous(const uint8_t* A, const float* sa, const uint8_t* B,
                                         const float* sb, uint16_t* D,
                                         const int32_t* grouped_layout, int64_t M_sum, int64_t N,
                                         int64_t K, int64_t G, void* stream) {
    return gemm_contiguous(A, sa, B, sb, D, grouped_layout, M_sum, N, K, G, stream, false);
}

dg_status dg_fp8_gemm_grouped_contiguous_e8m0(const uint8_t* A, const uint8_t* sa,
                                              const uint8_t* B, const uint8_t* sb, uint16_t* D,
                                              const int32_t* grouped_layout, int64_t M_sum,
                                              int64_t N, int64_t K, int64_t G, void* stream) {
    return gemm_contiguous(A, sa, B, sb, D, grouped_layout, M_sum, N, K, G, stream, true);
}

dg_status dg_fp8_gemm_grouped_masked(const uint8_t* A, const float* sa, const uint8_t* B,
                                     const float* sb, uint16_t* D, const int32_t* masked_m,
                                     int64_t G, int64_t M_max, int64_t N, int64_t K,
                                     void* stream) {
    return gemm_masked(A, sa, B, sb, D, masked_m, G, M_max, N, K, stream, false);
}

dg_status dg_fp8_gemm_grouped_masked_e8m0(const uint8_t* A, const uint8_t* sa, const uint8_t* B,
                                          const uint8_t* sb, uint16_t* D,
                                          const int32_t* masked_m, int64_t G, int64_t M_max,
                                          int64_t N, int64_t K, void* stream) {
    return gemm_masked(A, sa, B, sb, D, masked_m, G, M_max, N, K, stream, true);
}

dg_status dg_quantize_fp8_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                    void* stream) {
    const dg_status st = check_quantize(x, M, K, q, s, false);
    if (st != DG_OK || M == 0) return st;
    return dg::launch_quantize_per_token(x, M, K, q, s, static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_fp8_per_token_bf16(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                                         float* s, void* stream) {
    const dg_status st = check_quantize(x, M, K, q, s, false);
    if (st != DG_OK || M == 0) return st;
    return dg::launch_quantize_per_token_bf16(x, M, K, q, s, static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_fp8_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, float* s,
                                    void* stream) {
    const dg_status st = check_quantize(x, N, K, q, s, true);
    if (st != DG_OK || N == 0) return st;
    return dg::launch_quantize_per_block(x, N, K, q, s, static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_fp8_per_token_e8m0(const float* x, int64_t M, int64_t K, uint8_t* q,
                                         uint8_t* s, void* stream) {
    const dg_status st = check_quantize(x, M, K, q, s, false);
    if (st != DG_OK || M == 0) return st;
    return dg::launch_quantize_per_token_e8m0(x, M, K, q, s, static_cast<hipStream_t>(stream));
}

dg_status dg_quantize_fp8_per_block_e8m0(const float* x, int64_t N, int64_t K, uint8_t* q,
                                         uint8_t* s, void* stream) {
    const dg_status st = check_quantize(x, N, K, q, s, true);
    if (st != DG_OK || N == 0) return st;
    return dg::launch_quantize_per_block_e8m0(x, N, K, q, s, static_cast<hipStream_t>(stream));
}

const char* dg_status_string(dg_status status) {
    switch (status) {
        case DG_OK: return "ok";
        case DG_ERR_NULL: return "a required pointer is NULL";
        case DG_ERR_SHAPE: return "a size is out of range";
        case DG_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case DG_ERR_UNSUPPORTED: return "arguments are valid but not supported by this build";
        case DG_ERR_HIP: return "the HIP runtime reported an error";
    }
    return "unknown status";
}

}  // extern "C"
