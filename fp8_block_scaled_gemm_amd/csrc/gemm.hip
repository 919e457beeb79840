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
//   - A and B K-slabs (128 bytes per row per K block) go from global memory
//     straight into LDS (global_load_lds_dwordx4, no register staging),
//     double buffered.  Each 16-byte chunk of a row sits at chunk ^ (row & 7),
//     so the 16-lane groups of a fragment read hit distinct banks.
//   - Workgroups are dispatched round-robin over the 8 XCDs; the tile order
//     gives each XCD a contiguous range of tiles, grouped a few m-blocks at a
//     time, so that concurrent tiles on one XCD share A and B slabs in its L2.
#include "device_common.h"
#include "launch.h"

namespace dg {

constexpr int kNumXcds = 8;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct TileConfig {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // rows / cols per wave
    static constexpr int TM = WM / 16, TN = WN / 16;            // 16x16 sub-tiles per wave
    static constexpr int kGroupM = GROUP_M_;                    // m-blocks per raster group
    // one wave-wide direct load fills 1 KiB (8 rows) of a stage
    static constexpr int kLoadsA = BM / 8 / kWaves;
    static constexpr int kLoadsB = BN / 8 / kWaves;
    static constexpr int kStageA = BM * 128, kStageB = BN * 128;
    // a wave's columns never cross a 128-column scale block
    static constexpr bool kOneScaleB =
        (128 % WN == 0) && (BN % 128 == 0 || 128 % BN == 0);
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16x16");
    static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "uneven staging");
    static_assert(BM % 64 == 0 && BM / 64 <= kWaves, "one wave per 64 rows stages A scales");
};

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in a stage.
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-wide direct load: lane l's bytes from `src` land at
// dst + size*l in LDS (dst is wave-uniform).
__device__ __forceinline__ void load_lds_16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void load_lds_4(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
}

// Logical tile of workgroup `b` among `tiles`: XCD x (= b % 8) receives the
// contiguous range [x*per, (x+1)*per); returns -1 for the padding slots.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
    const int per = (tiles + kNumXcds - 1) / kNumXcds;
    const int t = (b % kNumXcds) * per + b / kNumXcds;
    return t < tiles ? t : -1;
}

// Operands are separate __restrict__ arguments so the compiler knows the
// scales are never written during the kernel and may use scalar loads.
template <class T, Form kForm>
__global__ __launch_bounds__(T::kThreads) void gemm_kernel(
    const uint8_t* __restrict__ A_, const float* __restrict__ sa_, const uint8_t* __restrict__ B_,
    const float* __restrict__ sb_, uint16_t* __restrict__ D_, const int32_t* __restrict__ aux_,
    int64_t rows_, int64_t N_, int64_t K_, int64_t G_, int m_blocks, int n_blocks) {
    struct {
        const uint8_t* __restrict__ A; const float* __restrict__ sa;
        const uint8_t* __restrict__ B; const float* __restrict__ sb;
        uint16_t* __restrict__ D; const int32_t* __restrict__ aux;
        int64_t rows, N, K, G;
    } p{A_, sa_, B_, sb_, D_, aux_, rows_, N_, K_, G_};
    __shared__ __align__(1024) uint8_t smA[2][T::kStageA];
    __shared__ __align__(1024) uint8_t smB[2][T::kStageB];
    __shared__ __align__(16) float smSA[2][T::BM];
    __shared__ int smRowOk[kForm == Form::Contiguous ? T::BM : 1];
    __shared__ int smGroup;

    const int tid = threadIdx.x;
    // wave-uniform in a scalar register, so that per-wave addresses (the B
    // scales) become scalar loads that do not wait on the vector queue
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t K = p.K, N = p.N;
    const int KB = (int)(K >> 7);
    const int NB = (int)((N + 127) >> 7);

    // ---- tile -> (group, m block, n block)
    const int tiles_per_group = m_blocks * n_blocks;
    const int groups = kForm == Form::Masked ? (int)p.G : 1;
    int tile = xcd_tile(blockIdx.x, groups * tiles_per_group);
    if (tile < 0) return;
    int g = 0;
    if (kForm == Form::Masked) {
        g = tile / tiles_per_group;
        tile -= g * tiles_per_group;
    }
    // raster: groups of kGroupM m-blocks, m fastest inside a group
    const int span = T::kGroupM * n_blocks;
    const int first_m = (tile / span) * T::kGroupM;
    const int gm = min(m_blocks - first_m, T::kGroupM);
    const int in_span = tile % span;
    const int mb = first_m + in_span % gm, nb = in_span / gm;
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

    // ---- per-lane sources of the direct loads (K block 0); a wave's load i
    // fills rows [8q, 8q+8) of a stage, q = wave + i * kWaves, and lane l
    // fetches the logical chunk that belongs at physical chunk l % 8
    const uint8_t* srcA[T::kLoadsA];
    const uint8_t* srcB[T::kLoadsB];
    {
        const int sub = lane >> 3, pchunk = lane & 7;
        const int lchunk = pchunk ^ sub;
#pragma unroll
        for (int i = 0; i < T::kLoadsA; ++i) {
            const int row = (wave + i * T::kWaves) * 8 + sub;
            srcA[i] = p.A + (arow0 + min(row, valid - 1)) * K + lchunk * 16;
        }
#pragma unroll
        for (int i = 0; i < T::kLoadsB; ++i) {
            const int row = (wave + i * T::kWaves) * 8 + sub;
            srcB[i] = Bg + min<int64_t>(n0 + row, N - 1) * K + lchunk * 16;
        }
    }
    const float* srcSA = p.sa + (arow0 + min(wave * 64 + lane, valid - 1)) * KB;

#define DG_ISSUE_LOADS(kb_, st_)                                                              \
    do {                                                                                      \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsA; ++i)                                \
            load_lds_16(srcA[i] + (kb_) * 128, &smA[st_][(wave + i * T::kWaves) * 1024]);    \
        _Pragma("unroll") for (int i = 0; i < T::kLoadsB; ++i)                                \
            load_lds_16(srcB[i] + (kb_) * 128, &smB[st_][(wave + i * T::kWaves) * 1024]);    \
        if (wave < T::BM / 64) load_lds_4(srcSA + (kb_), &smSA[st_][wave * 64]);              \
    } while (0)

    const int lr = lane & 15, lg = lane >> 4;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const int wrow = wm * T::WM, wcol = wn * T::WN;

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    DG_ISSUE_LOADS(0, 0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < KB) DG_ISSUE_LOADS(kb + 1, st ^ 1);

        const uint8_t* sA = smA[st];
        const uint8_t* sB = smB[st];
        v8i bf[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) bf[j] = lds_frag(sB, wcol + 16 * j + lr, lg);
        float sbv[T::kOneScaleB ? 1 : T::TN];
        if (T::kOneScaleB) {
            sbv[0] = sbg[min((n0 + wcol) >> 7, NB - 1) * KB + kb];
        } else {
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                sbv[j] = sbg[min((n0 + wcol + 16 * j) >> 7, NB - 1) * KB + kb];
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int r = wrow + 16 * i + lr;
            const v8i af = lds_frag(sA, r, lg);
            const float s_a = smSA[st][r];
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const v4f part = mfma_block(bf[j], af);
                const float s = s_a * sbv[T::kOneScaleB ? 0 : j];
                acc[i][j] += s * part;
            }
        }
        __syncthreads();
    }
#undef DG_ISSUE_LOADS

    // ---- epilogue: lane holds row (16i + lr) and columns (16j + 4lg .. +3)
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int lrow = wrow + 16 * i + lr;
        bool ok = lrow < valid;
        if (kForm == Form::Contiguous) ok = ok && smRowOk[lrow];
        if (!ok) continue;
        uint16_t* drow = p.D + (arow0 + lrow) * N;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int64_t n = n0 + wcol + 16 * j + 4 * lg;
            if (n < N) {
                v2u packed;
                packed[0] = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
                packed[1] = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
                *reinterpret_cast<v2u*>(drow + n) = packed;
            }
        }
    }
}

template <class T, Form kForm>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
    const int64_t m_blocks = (a.rows + T::BM - 1) / T::BM;
    const int64_t n_blocks = (a.N + T::BN - 1) / T::BN;
    const int64_t groups = (kForm == Form::Masked) ? a.G : 1;
    const int64_t tiles = groups * m_blocks * n_blocks;
    if (tiles == 0) return hipSuccess;
    const int64_t grid = (tiles + kNumXcds - 1) / kNumXcds * kNumXcds;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_kernel<T, kForm>), dim3((unsigned)grid), dim3(T::kThreads), 0, stream,
                       a.A, a.sa, a.B, a.sb, a.D, a.aux, a.rows, a.N, a.K, a.G, (int)m_blocks,
                       (int)n_blocks);
    return hipGetLastError();
}

// 256x256 tiles, 8 waves of 128x64 (two per SIMD).
using TileLarge = TileConfig<256, 256, 2, 4, 4>;
// 128x256 tiles, 4 waves of 128x64: contiguous groups are padded to 128 rows.
using TileRows128 = TileConfig<128, 256, 1, 4, 8>;

hipError_t launch_gemm(Form form, const GemmArgs& a, hipStream_t stream) {
    switch (form) {
        case Form::Dense: return launch_tiled<TileLarge, Form::Dense>(a, stream);
        case Form::Contiguous: return launch_tiled<TileRows128, Form::Contiguous>(a, stream);
        case Form::Masked: return launch_tiled<TileLarge, Form::Masked>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
