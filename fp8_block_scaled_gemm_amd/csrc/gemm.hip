// FP8 block-scaled NT GEMM for gfx950 (dense, contiguous-grouped, masked-grouped).
//
// What is computed (DeepGEMM fp8_gemm.cuh, fp8_gemm_kernel): for each
// 128-wide K block kb, the partial product P = A_blk * B_blk^T of e4m3
// operands with fp32 accumulation, promoted into the fp32 accumulator as
// F += (sa[m,kb] * sb[n/128,kb]) * P; the epilogue rounds F to bf16 (nearest
// even) and stores the rows the call routes.
//
// How it maps to CDNA4:
//   - One v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3, C = 0) covers a whole
//     128-wide K block of a 16x16 sub-tile, so its result *is* the block
//     partial P and goes straight into the promotion FMA; no second set of
//     accumulators is kept.
//   - The MFMA takes B as its first operand and A as its second, so each lane
//     ends up with one output row and four consecutive output columns: one
//     scale product per lane and sub-tile, and 8-byte bf16 stores.
//   - A and B K-slabs (128 bytes per row per K block) are staged in LDS,
//     double buffered, each 16-byte chunk XOR-swizzled by (row & 7) so the
//     fragment reads are free of bank conflicts.
#include "device_common.h"
#include "launch.h"

namespace dg {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileConfig {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // rows / cols per wave
    static constexpr int TM = WM / 16, TN = WN / 16;            // 16x16 sub-tiles per wave
    static constexpr int kLoadsA = BM * 8 / kThreads;           // 16-byte chunks per thread
    static constexpr int kLoadsB = BN * 8 / kThreads;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16x16");
    static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "uneven staging");
    static_assert(BM <= kThreads, "one thread per row stages the A scales");
};

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in LDS.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// MFMA operand: lane (lr, lg) supplies 32 bytes of row `row`, chunks 2*lg and
// 2*lg+1.  A and B fragments use the same K assignment, so the dot product
// pairs matching K indices whatever order the instruction walks them in.
__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int lg) {
    const v4u lo = *reinterpret_cast<const v4u*>(base + lds_off(row, 2 * lg));
    const v4u hi = *reinterpret_cast<const v4u*>(base + lds_off(row, 2 * lg + 1));
    v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

__device__ __forceinline__ v4f mfma_block(const v8i& b, const v8i& a) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format 0 = e4m3 for both operands; zero scale operands select the
    // unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, zero, 0, 0, 0, 0, 0, 0);
}

template <class T, Form kForm>
__global__ __launch_bounds__(T::kThreads) void gemm_kernel(GemmArgs p, int m_blocks, int n_blocks) {
    __shared__ __align__(16) uint8_t smA[2][T::BM * 128];
    __shared__ __align__(16) uint8_t smB[2][T::BN * 128];
    __shared__ float smSA[2][T::BM];
    __shared__ int smRowOk[T::BM];
    __shared__ int smGroup;

    const int tid = threadIdx.x;
    const int64_t K = p.K, N = p.N;
    const int KB = (int)(K >> 7);
    const int NB = (int)((N + 127) >> 7);

    // ---- tile -> (group, m block, n block); m varies fastest so that
    // consecutive workgroups share one B slab
    int tile = blockIdx.x;
    int g = 0;
    if (kForm == Form::Masked) {
        g = tile / (m_blocks * n_blocks);
        tile -= g * m_blocks * n_blocks;
    }
    const int mb = tile % m_blocks, nb = tile / m_blocks;
    const int m0 = mb * T::BM, n0 = nb * T::BN;

    int valid;       // tile rows [0, valid) exist and may be routed
    int64_t arow0;   // A / sa / D row of tile row 0
    if (kForm == Form::Dense) {
        valid = (int)min<int64_t>(T::BM, p.rows - m0);
        arow0 = m0;
    } else if (kForm == Form::Masked) {
        const int64_t vm = min<int64_t>(max(p.aux[g], 0), p.rows);
        if (m0 >= vm) return;  // whole tile past masked_m: uniform exit
        valid = (int)min<int64_t>(T::BM, vm - m0);
        arow0 = (int64_t)g * p.rows + m0;
    } else {
        // contiguous: the tile's group is the id of its routed rows (ids
        // outside [0, G) are padding); one id per 128-row block
        valid = T::BM;
        arow0 = m0;
        if (tid == 0) smGroup = -1;
        __syncthreads();
        int id = -1;
        if (tid < T::BM) {
            id = p.aux[m0 + tid];
            if (id >= 0 && id < p.G) atomicMax(&smGroup, id);
        }
        __syncthreads();
        g = smGroup;
        if (g < 0) return;  // all padding: uniform exit
        if (tid < T::BM) smRowOk[tid] = (id == g);
    }
    const uint8_t* Bg = p.B + (int64_t)g * N * K;
    const float* sbg = p.sb + (int64_t)g * NB * KB;

    // ---- global -> registers -> LDS staging of one K block
    v4u ra[T::kLoadsA], rb[T::kLoadsB];
    float rsa = 0.f;
#define DG_LOAD_STAGE(kb_)                                                                        \
    do {                                                                                          \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsA; ++i) {                                  \
            const int c = tid + i * T::kThreads, r = min(c >> 3, valid - 1);                      \
            ra[i] = *reinterpret_cast<const v4u*>(p.A + (arow0 + r) * K + (kb_) * 128 +         \
                                                    (c & 7) * 16);                                \
        }                                                                                         \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsB; ++i) {                                  \
            const int c = tid + i * T::kThreads;                                                  \
            const int64_t n = min<int64_t>(n0 + (c >> 3), N - 1);                                 \
            rb[i] = *reinterpret_cast<const v4u*>(Bg + n * K + (kb_) * 128 + (c & 7) * 16);     \
        }                                                                                         \
        if (tid < T::BM) rsa = p.sa[(arow0 + min(tid, valid - 1)) * KB + (kb_)];                  \
    } while (0)
#define DG_STORE_STAGE(st_)                                                                       \
    do {                                                                                          \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsA; ++i) {                                  \
            const int c = tid + i * T::kThreads;                                                  \
            *reinterpret_cast<v4u*>(&smA[st_][lds_off(c >> 3, c & 7)]) = ra[i];                 \
        }                                                                                         \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsB; ++i) {                                  \
            const int c = tid + i * T::kThreads;                                                  \
            *reinterpret_cast<v4u*>(&smB[st_][lds_off(c >> 3, c & 7)]) = rb[i];                 \
        }                                                                                         \
        if (tid < T::BM) smSA[st_][tid] = rsa;                                                    \
    } while (0)

    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    DG_LOAD_STAGE(0);
    DG_STORE_STAGE(0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < KB) DG_LOAD_STAGE(kb + 1);

        v8i bf[T::TN];
        float sbv[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            bf[j] = lds_frag(smB[st], wn * T::WN + 16 * j + lr, lg);
            const int cb = min((n0 + wn * T::WN + 16 * j) >> 7, NB - 1);
            sbv[j] = sbg[cb * KB + kb];
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int r = wm * T::WM + 16 * i + lr;
            const v8i af = lds_frag(smA[st], r, lg);
            const float s_a = smSA[st][r];
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const v4f part = mfma_block(bf[j], af);
                const float s = s_a * sbv[j];
                acc[i][j] += s * part;
            }
        }

        if (kb + 1 < KB) DG_STORE_STAGE(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds row (16i + lr) and columns (16j + 4lg .. +3)
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int lrow = wm * T::WM + 16 * i + lr;
        bool ok = lrow < valid;
        if (kForm == Form::Contiguous) ok = ok && smRowOk[lrow];
        if (!ok) continue;
        uint16_t* drow = p.D + (arow0 + lrow) * N;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int64_t n = n0 + wn * T::WN + 16 * j + 4 * lg;
            if (n < N) {
                v2u packed;
                packed[0] = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
                packed[1] = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
                *reinterpret_cast<v2u*>(drow + n) = packed;
            }
        }
    }
}

#undef DG_LOAD_STAGE
#undef DG_STORE_STAGE

template <class T, Form kForm>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
    const int64_t m_blocks = (a.rows + T::BM - 1) / T::BM;
    const int64_t n_blocks = (a.N + T::BN - 1) / T::BN;
    const int64_t groups = (kForm == Form::Masked) ? a.G : 1;
    const int64_t grid = groups * m_blocks * n_blocks;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_kernel<T, kForm>), dim3((unsigned)grid), dim3(T::kThreads), 0, stream,
                       a, (int)m_blocks, (int)n_blocks);
    return hipGetLastError();
}

using Tile128 = TileConfig<128, 128, 2, 2>;

hipError_t launch_gemm(Form form, const GemmArgs& a, hipStream_t stream) {
    switch (form) {
        case Form::Dense: return launch_tiled<Tile128, Form::Dense>(a, stream);
        case Form::Contiguous: return launch_tiled<Tile128, Form::Contiguous>(a, stream);
        case Form::Masked: return launch_tiled<Tile128, Form::Masked>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
