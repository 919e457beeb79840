// FP8 block-scaled NT GEMM for gfx950 (dense, contiguous-grouped, masked-grouped).
//
// What is computed (DeepGEMM fp8_gemm.cuh, fp8_gemm_kernel): for each
// 128-wide K block kb, the partial product P = A_blk * B_blk^T of e4m3
// operands with fp32 accumulation, promoted into the fp32 accumulator as
// F += (sa[m,kb] * sb[n/128,kb]) * P; the epilogue rounds F to bf16 (nearest
// even) and stores the rows the call routes.
//
// How it maps to CDNA4 (gfx950):
//   - One v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3, C = 0) covers a whole
//     128-wide K block of a 16x16 sub-tile, so its result *is* the block
//     partial P and goes straight into the promotion FMA; no second set of
//     accumulators is kept.
//   - The MFMA takes B as its first operand and A as its second, so each lane
//     owns one output row and four consecutive output columns: one scale
//     product per lane and sub-tile.
//   - A and B K-slabs (128 bytes per row per K block) are loaded straight
//     from memory into double-buffered LDS stages with bounds-checked buffer
//     loads (rows past the valid rows read as zero and touch no memory), and
//     fragments are read from there with ds_read_b128.  LDS bandwidth is the
//     scarce resource (256 bytes per clock without bank conflicts).  The
//     16-byte chunk c of stage row r sits at c ^ (r & 7), and lane (lr, lg)
//     of a fragment read takes chunks lg and lg + 4 of row lr: measured
//     conflict-free, where chunks 2 lg and 2 lg + 1 (any row swizzle tried)
//     cost two cycles per read.  Which K bytes a lane holds is free as long
//     as A and B fragments agree; lg, lg + 4 is also the instruction's own
//     order (K [16 g, 16 g + 16) and [64 + 16 g, +16) for lane group g).
//   - The output tile is staged through LDS in bf16 and written back in full
//     16-byte chunks per lane, whole row segments per store instruction
//     (scattered 8-byte fragment stores reach half the write bandwidth).
//   - Workgroups are dispatched round-robin over the 8 XCDs; the tile order
//     gives each XCD a contiguous range of tiles, grouped a few m-blocks at a
//     time, so that concurrent tiles on one XCD share A and B slabs in its L2.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

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
    // one wave-wide direct load fills 1 KiB (8 rows) of a stage; waves take
    // the 8-row groups round-robin (the B slab may end part way round)
    static constexpr int kLoadsA = BM / 8 / kWaves;
    static constexpr int kLoadsB = (BN / 8 + kWaves - 1) / kWaves;
    static constexpr int kLoadsBMin = BN / 8 / kWaves;  // loads of the wave with the fewest
    static constexpr int kStageA = BM * 128;
    static constexpr int kStageB = BN * 128;
    // every wave's columns lie in one 128-column scale block
    static constexpr bool kOneScaleB = BN % 128 == 0 && 128 % WN == 0;
    // LDS row pitch of the bf16 output tile: a power of two of 16-byte
    // chunks, at least 16, so the chunk swizzle c ^ (row & 15) stays in the row
    static constexpr int kPitchChunks = BN <= 128 ? 16 : 32;
    // the bf16 output tile reuses the stage memory on its way out
    static constexpr int kSmem = (2 * (kStageA + kStageB) > BM * kPitchChunks * 16)
                                     ? 2 * (kStageA + kStageB)
                                     : BM * kPitchChunks * 16;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16x16");
    static_assert(BM % (8 * kWaves) == 0 && BN % 8 == 0, "slabs are staged 8 rows at a time");
    static_assert(BN <= 256, "output tile pitch");
    static_assert(BM % 64 == 0 && kWaves % (BM / 64) == 0, "waves stage the A scales 64 rows each");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<size_t>((lds_ptr_t)p));
}

// Raw buffer resource (gfx9 V#): `bytes` readable from `base`, stride 0.
// Loads at offsets past `bytes` return zero and touch no memory.
__device__ __forceinline__ v4u buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4u r;
    r[0] = (uint32_t)a;
    r[1] = (uint32_t)(a >> 32) & 0xffffu;
    r[2] = bytes;
    r[3] = 0x00020000u;
    return r;
}

// One wave-wide direct load: lane l's bytes at buffer offset `off` land at
// dst + size*l in LDS (dst is wave-uniform, passed in M0).  Written as inline
// assembly on purpose: the compiler then does not track these LDS writes and
// cannot put a wait for the stage being filled in front of reads of the
// other stage (its alias tracking for such loads depends on control flow).
// The kernel orders them itself: every LDS read of a buffer is separated
// from the loads that refill it by a barrier (a compiler memory barrier as
// well), and a buffer is read only after the explicit vmcnt wait and barrier
// that publish it.  So the statements carry no memory clobber, and the
// compiler may still schedule unrelated LDS reads and arithmetic across them.
__device__ __forceinline__ void load_lds_16(const v4u& rsrc, uint32_t off, void* dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr(dst)), "v"(off), "s"(rsrc) : "m0");
}
__device__ __forceinline__ void load_lds_4(const v4u& rsrc, uint32_t off, void* dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_addr(dst)), "v"(off), "s"(rsrc) : "m0");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// The same with lgkmcnt = 0: every LDS access this wave issued has completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that is also a compiler barrier for memory accesses, but
// (unlike __syncthreads) waits for nothing: the kernel has already waited for
// exactly the loads the barrier publishes.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ v4f mfma_block(const v8i& b, const v8i& a) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format 0 = e4m3 for both operands; zero scale operands select the
    // unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, zero, 0, 0, 0, 0, 0, 0);
}

// acc + 2^(eb-127) * 2^(ea-127) * (B_blk A_blk^T) in one instruction.  Each
// lane passes one E8M0 byte per operand in bits 0-7 (opsel 0): operand 0's
// (eb) applies to B row (lane & 15) of the sub-tile, operand 1's (ea) to A
// row (lane & 15), each for the 32-wide K group (lane >> 4); a block's four
// groups share one scale, so every lane passes its row's block scale.
__device__ __forceinline__ v4f mfma_block_e8(const v8i& b, const v8i& a, const v4f& c, int eb,
                                              int ea) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, eb, 0, ea);
}

__device__ __forceinline__ v8i join(const v4u& lo, const v4u& hi) {
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Logical tile of workgroup `b` among `tiles`: XCD x (= b % 8) receives the
// contiguous range [x*per, (x+1)*per); -1 for the padding slots.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
    const int per = (tiles + kNumXcds - 1) / kNumXcds;
    const int t = (b % kNumXcds) * per + b / kNumXcds;
    return t < tiles ? t : -1;
}

// Where one output tile lives.  Every field is wave-uniform.
struct TileInfo {
    int g;              // group (0 for dense)
    int m0, n0;         // first row within the group's row space, first column
    int valid;          // tile rows [0, valid) exist and may be routed
    int64_t arow0;      // A / sa / D row of tile row 0
    uint64_t ok0, ok1;  // contiguous form: routed-row masks, tile rows 0-63 / 64-127
};

// Masked form: work units are (group, m-block) pairs times n-blocks; a
// pair's cost is the number of 64-row chunks of its m-block that hold valid
// rows.  Pairs are ranked by cost, highest first (ties by pair index); rank r
// goes to XCD r % 8, so every XCD gets a balanced share, runs its pairs
// longest first, and keeps all n-blocks of a pair (which share the A rows) in
// its own L2.  Workgroup b runs on XCD b % 8 as that XCD's (b / 8)-th tile.
// Pairs without valid rows rank last and are skipped.  Every lane of the
// wave computes the same answer from the masked_m array.
template <class T>
__device__ __forceinline__ bool masked_slot(int b, int m_blocks, int n_blocks, int64_t rows,
                                            int G, const int32_t* __restrict__ masked_m,
                                            int lane, int& g, int& mb, int& nb) {
    constexpr int kLevels = T::BM / 64 + 1;  // costs 0 .. BM/64
    const int P = G * m_blocks;
    const int k = b / kNumXcds;
    const int slot = (k / n_blocks) * kNumXcds + b % kNumXcds;  // the pair's rank
    if (slot >= P) return false;
    nb = k % n_blocks;
    auto cost = [&](int q) {
        const int64_t vm = min<int64_t>(max(masked_m[q / m_blocks], 0), rows);
        const int64_t v = min<int64_t>(max<int64_t>(vm - (int64_t)(q % m_blocks) * T::BM, 0), T::BM);
        return (int)((v + 63) >> 6);
    };
    int count[kLevels];
#pragma unroll
    for (int L = 0; L < kLevels; ++L) count[L] = 0;
    for (int base = 0; base < P; base += 64) {
        const int q = base + lane;
        const int c = q < P ? cost(q) : -1;
#pragma unroll
        for (int L = 0; L < kLevels; ++L) count[L] += __popcll(__ballot(c == L));
    }
    int level = kLevels - 1, pos = slot;
    while (level > 0 && pos >= count[level]) pos -= count[level--];
    if (level == 0) return false;
    for (int base = 0; base < P; base += 64) {
        const int q = base + lane;
        const bool hit = q < P && cost(q) == level;
        const uint64_t m = __ballot(hit);
        const int n = __popcll(m);
        if (pos < n) {
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const int q_sel = base + __builtin_ctzll(__ballot(hit && below == pos));
            g = q_sel / m_blocks;
            mb = q_sel % m_blocks;
            return true;
        }
        pos -= n;
    }
    return false;
}

// Contiguous form: the largest valid group id below `below` among the rows
// of the 128-row block at ti.m0 and the masks of the rows carrying it; false
// when there is none.  Every wave computes this from the layout itself.
__device__ __forceinline__ bool block_group(const int32_t* __restrict__ layout, int64_t G, int below,
                                            int lane, TileInfo& ti) {
    const int id0 = layout[ti.m0 + lane], id1 = layout[ti.m0 + 64 + lane];
    auto usable = [&](int id) { return id >= 0 && id < G && id < below; };
    int gid = max(usable(id0) ? id0 : -1, usable(id1) ? id1 : -1);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) gid = max(gid, __shfl_xor(gid, d, 64));
    gid = __builtin_amdgcn_readfirstlane(gid);
    if (gid < 0) return false;
    ti.g = gid;
    ti.ok0 = __ballot(id0 == gid);
    ti.ok1 = __ballot(id1 == gid);
    return true;
}

// Decode workgroup `b`'s tile; false when it is a padding slot or the tile
// has no routed row (masked rows past masked_m, contiguous blocks of
// padding).  Contiguous: the block's first group is the largest id in
// [0, G) among its rows (the layout puts one id per 128-row block); a block
// that mixes ids is then run again for each smaller id (see gemm_kernel).
template <class T, Form kForm>
__device__ __forceinline__ bool decode_tile(int b, int m_blocks, int n_blocks, int64_t rows,
                                            int64_t G, const int32_t* __restrict__ aux,
                                            int lane, TileInfo& ti) {
    ti.ok0 = ti.ok1 = 0;
    if (kForm == Form::Masked) {
        int mb, nb;
        if (!masked_slot<T>(b, m_blocks, n_blocks, rows, (int)G, aux, lane, ti.g, mb, nb))
            return false;
        ti.m0 = mb * T::BM;
        ti.n0 = nb * T::BN;
        const int64_t vm = min<int64_t>(max(aux[ti.g], 0), rows);
        ti.valid = (int)min<int64_t>(T::BM, vm - ti.m0);
        ti.arow0 = (int64_t)ti.g * rows + ti.m0;
        return true;
    }
    int tile = xcd_tile(b, m_blocks * n_blocks);
    if (tile < 0) return false;
    ti.g = 0;
    // raster: groups of kGroupM m-blocks, m fastest inside a group
    const int span = T::kGroupM * n_blocks;
    const int first_m = (tile / span) * T::kGroupM;
    const int gm = min(m_blocks - first_m, T::kGroupM);
    const int in_span = tile % span;
    ti.m0 = (first_m + in_span % gm) * T::BM;
    ti.n0 = (in_span / gm) * T::BN;
    if (kForm == Form::Dense || kForm == Form::DenseAcc) {
        ti.valid = (int)min<int64_t>(T::BM, rows - ti.m0);
        ti.arow0 = ti.m0;
    } else {
        static_assert(kForm != Form::Contiguous || T::BM == 128, "one group per 128-row block");
        if (!block_group(aux, G, (int)G, lane, ti)) return false;
        ti.valid = T::BM;
        ti.arow0 = ti.m0;
    }
    return true;
}

// Epilogue of a tile: the lane holds tile row 16 (WAVES_M i + wm) + lr and
// columns wcol + 16j + 4lg .. +3 of acc[i][j].  DenseAcc adds the fp32 addend
// C first; then the tile is rounded to bf16, staged in LDS (which every wave
// must be done with) and stored row-predicated.
template <class T, Form kForm>
__device__ __forceinline__ void store_tile(v4f (&acc)[T::TM][T::TN], uint8_t* smem, int tid, int wm,
                                           int wcol, int lr, int lg, const TileInfo& ti,
                                           const float* __restrict__ C, uint16_t* __restrict__ D,
                                           int64_t N) {
    if constexpr (kForm == Form::DenseAcc) {
        // D = bf16(C + acc): C is read straight into the accumulators'
        // layout (one 16-byte load per sub-tile and lane), half of the
        // wave's sub-tile rows at a time with all of that half's loads in
        // flight, and added in fp32 before the single rounding below.  The
        // buffer ends with the tile's last valid row: rows past it read as
        // zero; columns past N of a valid row read C values of the next row
        // (or zero after the last one) and are never stored.
        const float* const tileC = C + ti.arow0 * N + ti.n0;
        const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(tileC), (short)0,
            (int)(uint32_t)(((int64_t)(ti.valid - 1) * N + (N - ti.n0)) * 4), 0x00020000);
        constexpr int kH = T::TM / 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4f c[kH][T::TN];
#pragma unroll
            for (int ii = 0; ii < kH; ++ii) {
                const int row = 16 * (T::WAVES_M * (h * kH + ii) + wm) + lr;
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    const uint32_t off = ((uint32_t)row * (uint32_t)N + wcol + 16 * j + 4 * lg) * 4u;
                    c[ii][j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsC, off, 0, 0));
                }
            }
#pragma unroll
            for (int ii = 0; ii < kH; ++ii)
#pragma unroll
                for (int j = 0; j < T::TN; ++j) acc[h * kH + ii][j] += c[ii][j];
        }
    }
    // Round to bf16 (v_cvt_pk_bf16_f32: nearest even), stage the whole tile
    // in LDS, then write it back in full 16-byte chunks, consecutive lanes on
    // consecutive chunks of a row.  In LDS (row pitch kPitchChunks chunks),
    // 16-byte chunk c of row r sits at c ^ (r & 15): the 16 rows a fragment
    // store touches land in distinct banks.
    constexpr int kRowBytes = T::kPitchChunks * 16;
    constexpr int kChunks = T::BN / 8;  // 16-byte chunks of an output row
    uint8_t* const sD = smem;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const int row = 16 * (T::WAVES_M * i + wm) + lr;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = wcol + 16 * j + 4 * lg;
            const v2f lo = {acc[i][j][0], acc[i][j][1]};
            const v2f hi = {acc[i][j][2], acc[i][j][3]};
            v2u packed;
            packed[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, v2bf));
            packed[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, v2bf));
            *reinterpret_cast<v2u*>(sD + row * kRowBytes + (((col >> 3) ^ (row & 15)) << 4) +
                                    ((col >> 2) & 1) * 8) = packed;
        }
    }
    __syncthreads();
    static_assert((T::BM * kChunks) % T::kThreads == 0, "whole passes over the output tile");
    // fully unrolled (the accumulators are dead by now): every pass's LDS
    // read can be in flight before the first store waits for its data
#pragma unroll
    for (int q = tid; q < T::BM * kChunks; q += T::kThreads) {
        const int row = q / kChunks, c = q % kChunks;
        const int64_t col = ti.n0 + c * 8;
        bool ok = row < ti.valid && col < N;
        if (kForm == Form::Contiguous) ok = ok && (((row < 64 ? ti.ok0 : ti.ok1) >> (row & 63)) & 1);
        const v4u v = *reinterpret_cast<const v4u*>(sD + row * kRowBytes + ((c ^ (row & 15)) << 4));
        // D is written once and not read back here: non-temporal stores keep
        // it from evicting operand slabs that later tiles still read
        if (ok) __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(D + (ti.arow0 + row) * N + col));
    }
}

// Operands are separate __restrict__ arguments so the compiler knows they
// are never written during the kernel.
//
// Pipeline (one K block = one step, two barriers per step, two stages of A
// and B in LDS): a step reads its B fragments into registers, multiplies the
// A rows [0, BM/2) (A fragments streamed from LDS one row of sub-tiles at a
// time), passes the mid barrier, multiplies the rows [BM/2, BM), and passes
// the end barrier.  Each wave loads its share of the slabs of block kb+2
// straight from memory into LDS as soon as a barrier frees their buffer, so
// every load has one and a half steps to land (see `step`).
//
// Scales (kE8 = false): fp32, [rows][K/128] and [groups][NB][K/128], each K
// block's partial promoted as acc += (sa sb) P.  With kE8: E8M0 exponent
// bytes, rows padded to a multiple of 4 bytes ([rows][SP], [groups][NB][SP]),
// applied by the scaled MFMA itself, which accumulates straight into acc.
template <class T, Form kForm, bool kE8, bool kMixed = false>
__global__ __launch_bounds__(T::kThreads, 2) void gemm_kernel(
    const uint8_t* __restrict__ A, const void* __restrict__ sa_v, const uint8_t* __restrict__ B,
    const void* __restrict__ sb_v, uint16_t* __restrict__ D, const int32_t* __restrict__ aux,
    const float* __restrict__ C, int64_t rows, int64_t N, int64_t K, int64_t G, int m_blocks,
    int n_blocks) {
    using ScaleT = typename std::conditional<kE8, uint8_t, float>::type;
    const ScaleT* __restrict__ sa = static_cast<const ScaleT*>(sa_v);
    const ScaleT* __restrict__ sb = static_cast<const ScaleT*>(sb_v);
    // Two A stages then two B stages (after the K loop: the bf16 output tile).
    // Scales come in chunks of four K blocks, two chunk buffers: row scales
    // as [row][4], column-block scales as [block][4].
    __shared__ __align__(1024) uint8_t smem[T::kSmem];
    __shared__ __align__(16) float smSA[2][T::BM * 4];
    __shared__ __align__(16) float smSB[2][64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int KB = (int)(K >> 7);
    const int NB = (int)((N + 127) >> 7);
    const int SP = kE8 ? ((KB + 3) & ~3) : KB;  // scales per scale row
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const int wcol = wn * T::WN;

    TileInfo ti;
    if constexpr (kMixed) {
        // the 128-row block blockIdx.x, from its second largest valid id on
        // (the largest one's rows are the ordinary launch's), column tile 0
        static_assert(kForm == Form::Contiguous, "mixed blocks are a contiguous-form case");
        ti.m0 = blockIdx.x * T::BM;
        ti.n0 = 0;
        ti.valid = T::BM;
        ti.arow0 = ti.m0;
        if (!block_group(aux, G, (int)G, lane, ti) || !block_group(aux, G, ti.g, lane, ti)) return;
    } else {
        if (!decode_tile<T, kForm>(blockIdx.x, m_blocks, n_blocks, rows, G, aux, lane, ti)) return;
    }

    // One pass per tile; the mixed-block launch walks every column tile of
    // its block for each of its smaller ids, each pass storing only the rows
    // of its own id.
    for (;;) {
        uint8_t* const smA = smem;
        uint8_t* const smB = smem + 2 * T::kStageA;

        // ---- slab loads.  A wave's load i fills rows [8q, 8q+8) of a stage,
        // q = wave + i * kWaves; lane l fetches the logical 16-byte chunk that
        // belongs at physical chunk l % 8 of row 8q + l / 8, i.e. chunk
        // (l % 8) ^ (row & 7) = (l % 8) ^ (l / 8).  A slab's buffer starts at the
        // K block in row 0 and ends with the tile's last valid row (A) or column
        // (B), so rows past it read as zero; blocks past the last one get an
        // empty buffer, so their loads move no data but still count towards the
        // wave's vmcnt like every other step's.
        const int sub = lane >> 3, lchunk = (lane & 7) ^ sub;
        const uint32_t offRow = (uint32_t)(wave * 8 + sub) * (uint32_t)K + lchunk * 16;
        const int nb0 = ti.n0 >> 7;
        const int vn = (int)min<int64_t>(T::BN, N - ti.n0);
        // column-scale blocks the tile touches
        const int vnb = (int)((ti.n0 + vn - 1) >> 7) - nb0 + 1;
        const uint8_t* tileA = A + ti.arow0 * K;
        const ScaleT* tileSA = sa + ti.arow0 * SP;
        const uint8_t* tileB = B + ((int64_t)ti.g * N + ti.n0) * K;
        const ScaleT* tileSB = sb + ((int64_t)ti.g * NB + nb0) * SP;
        // loads [i0, i1) of this wave's share of the A slab of block kb
        auto issue_a = [&](int kb, int st, int i0, int i1) __attribute__((always_inline)) {
            const v4u rs = buffer_rsrc(tileA + kb * 128,
                                       kb < KB ? (uint32_t)ti.valid * (uint32_t)K - kb * 128 : 0u);
#pragma unroll
            for (int i = i0; i < i1; ++i)
                load_lds_16(rs, offRow + (uint32_t)(i * T::kWaves * 8) * (uint32_t)K,
                            smA + st * T::kStageA + (wave + i * T::kWaves) * 1024);
        };
        auto issue_b = [&](int kb, int st) __attribute__((always_inline)) {
            const v4u rs = buffer_rsrc(tileB + kb * 128, kb < KB ? (uint32_t)vn * (uint32_t)K - kb * 128 : 0u);
#pragma unroll
            for (int i = 0; i < T::kLoadsB; ++i) {
                if ((T::BN / 8) % T::kWaves != 0 && wave + i * T::kWaves >= T::BN / 8) break;
                load_lds_16(rs, offRow + (uint32_t)(i * T::kWaves * 8) * (uint32_t)K,
                            smB + st * T::kStageB + (wave + i * T::kWaves) * 1024);
            }
        };

        // Scale chunk c (K blocks 4c .. 4c+3) into chunk buffer c & 1: wave
        // w < BM/64 fetches the four K blocks' row scales of rows [64w, 64w + 64)
        // (16 bytes per row, or one 4-byte word of exponents), the next wave the
        // column-block scales (fp32: lane l gets block l / 4, K block l % 4 of the
        // chunk; E8M0: lane l gets the word of block l).  The range check of a
        // buffer load is per 4-byte word, so the words of a row's last chunk past
        // K/128 (and rows past the valid ones) read as zero or as the next row's
        // scales, which no step uses.  An exponent row's padding to 4 bytes keeps
        // its chunk words aligned and in range.
        const uint32_t offSA = (uint32_t)(wave * 64 + lane) * (uint32_t)SP * (kE8 ? 1 : 4);
        const uint32_t offSB = kE8 ? (uint32_t)lane * (uint32_t)SP
                                   : ((uint32_t)(lane >> 2) * (uint32_t)KB + (lane & 3)) * 4;
        constexpr int kScaleWaves = T::BM / 64;  // waves that fetch row scales
        static_assert(kScaleWaves < T::kWaves, "one more wave fetches the column scales");
        auto issue_scales = [&](int c) __attribute__((always_inline)) {
            const int kb0 = c * 4;
            constexpr uint32_t kSz = sizeof(ScaleT);
            if (kb0 >= KB) return;
            if (wave < kScaleWaves) {
                const v4u rs = buffer_rsrc(tileSA + kb0, (uint32_t)(ti.valid * SP - kb0) * kSz);
                if (kE8)
                    load_lds_4(rs, offSA, &smSA[c & 1][wave * 64]);
                else
                    load_lds_16(rs, offSA, &smSA[c & 1][wave * 64 * 4]);
            } else if (wave == kScaleWaves) {
                load_lds_4(buffer_rsrc(tileSB + kb0, (uint32_t)(vnb * SP - kb0) * kSz),
                           lane < (kE8 ? 1 : 4) * vnb ? offSB : 0xffffff00u, &smSB[c & 1][0]);
            }
        };

        // ---- fragment reads.  Sub-tile row i of wave row wm covers tile rows
        // [16 (WAVES_M i + wm), +16): the wave rows interleave in 16-row steps, so
        // a partial tile (a masked group's last rows, a ragged M) leaves work on
        // every wave.  Every row r a lane reads is lr plus a multiple of 16, so
        // r & 7 == lr & 7 and the swizzled chunk offsets are per-lane constants;
        // sub-tile i (or j) only adds a multiple of 16 rows (an immediate).
        static_assert(T::WN % 16 == 0, "wave column offsets keep the row swizzle");
        constexpr int kRowStep = 16 * T::WAVES_M;
        const int chunk_lo = (lg ^ (lr & 7)) << 4, chunk_hi = ((lg + 4) ^ (lr & 7)) << 4;
        const int fragA = (16 * wm + lr) * 128, fragB = (wcol + lr) * 128;
        const int srow = 16 * wm + lr;
        // column-scale block of sub-tile j, relative to the tile's first one
        int sblk[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) sblk[j] = (int)((ti.n0 + wcol + 16 * j) >> 7) - nb0;
        auto frag = [&](const uint8_t* p) __attribute__((always_inline)) {
            return join(*reinterpret_cast<const v4u*>(p + chunk_lo), *reinterpret_cast<const v4u*>(p + chunk_hi));
        };

        v4f acc[T::TM][T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        v8i bf[T::TN];

        // Sub-tile rows [i0, i1) of the wave tile for the K block kb on stage st.
        // With kSkip, rows that hold no valid row of the tile are skipped.
        auto mma_rows = [&](auto skip, int kb, int st, int i0, int i1) __attribute__((always_inline)) {
            constexpr bool kSkip = decltype(skip)::value;
            const uint8_t* stA = smA + st * T::kStageA + fragA;
            if constexpr (kE8) {
                // exponent chunks: one 4-byte word per row / column block
                const uint8_t* eSA = reinterpret_cast<const uint8_t*>(smSA[(kb >> 2) & 1]) + (kb & 3);
                const uint8_t* eSB = reinterpret_cast<const uint8_t*>(smSB[(kb >> 2) & 1]) + (kb & 3);
                int e_b[T::kOneScaleB ? 1 : T::TN];
#pragma unroll
                for (int j = 0; j < (T::kOneScaleB ? 1 : T::TN); ++j) e_b[j] = eSB[sblk[j] * 4];
#pragma unroll
                for (int i = i0; i < i1; ++i) {
                    if (kSkip && 16 * wm + kRowStep * i >= ti.valid) continue;
                    const v8i af = frag(stA + i * kRowStep * 128);
                    const int e_a = eSA[(srow + kRowStep * i) * 4];
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
                        acc[i][j] = mfma_block_e8(bf[j], af, acc[i][j], e_b[T::kOneScaleB ? 0 : j], e_a);
                }
            } else {
                const float* sSA = &smSA[(kb >> 2) & 1][kb & 3];
                const float* sSB = &smSB[(kb >> 2) & 1][kb & 3];
                float s_b[T::kOneScaleB ? 1 : T::TN];
#pragma unroll
                for (int j = 0; j < (T::kOneScaleB ? 1 : T::TN); ++j) s_b[j] = sSB[sblk[j] * 4];
#pragma unroll
                for (int i = i0; i < i1; ++i) {
                    if (kSkip && 16 * wm + kRowStep * i >= ti.valid) continue;
                    const v8i af = frag(stA + i * kRowStep * 128);
                    const float s_a = sSA[(srow + kRowStep * i) * 4];
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
                        acc[i][j] += (s_a * s_b[T::kOneScaleB ? 0 : j]) * mfma_block(bf[j], af);
                }
            }
        };

        // Loads a wave issues after the ones a barrier waits for (see `step`),
        // counted for the wave that issues the fewest B loads.
        constexpr int kAfter = T::kLoadsA + T::kLoadsBMin;
        static_assert(T::kLoadsA % 2 == 0 && kAfter < 64, "A slab halves, vmcnt range");

        // One K block kb on stage st (= kb & 1), in two halves separated by a
        // barrier.  The step starts by reading its B fragments (B slab of kb);
        // the first half multiplies the A rows [0, BM/2), the second half the rows
        // [BM/2, BM).  A slab load is issued as soon as the barrier that frees its
        // buffer has passed:
        //   after the mid barrier: A rows [0, BM/2) and the B slab of block kb+2
        //     (their buffers held those of kb);
        //   after the end barrier: A rows [BM/2, BM) of block kb+2.
        // So every load has one and a half steps to land.  Loads of a wave
        // complete in issue order; a barrier publishes what it needs by waiting
        // until at most the loads issued after those (kAfter) remain.  Scale
        // chunk loads (some waves, every fourth step) only make a wait stricter.
        auto step = [&](auto skip, int kb, int st) __attribute__((always_inline)) {
            const uint8_t* stB = smB + st * T::kStageB + fragB;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) bf[j] = frag(stB + j * 16 * 128);
            mma_rows(skip, kb, st, 0, T::TM / 2);
            wait_vmcnt_lgkm0<kAfter>();  // A rows [BM/2, BM) of kb
            lds_barrier();
            issue_a(kb + 2, st, 0, T::kLoadsA / 2);
            issue_b(kb + 2, st);
            if ((kb & 3) == 0) issue_scales((kb >> 2) + 1);
            mma_rows(skip, kb, st, T::TM / 2, T::TM);
            wait_vmcnt_lgkm0<kAfter>();  // A rows [0, BM/2) and B of kb+1
            lds_barrier();
            issue_a(kb + 2, st, T::kLoadsA / 2, T::kLoadsA);
        };

        // Prologue: blocks 0 and 1 of A rows [0, BM/2) and of B, A rows
        // [BM/2, BM) of block 0 and scale chunk 0 land and are published; A rows
        // [BM/2, BM) of block 1 go last, as in the steady state, so that the
        // first waits count the same loads.
        issue_scales(0);
        issue_a(0, 0, 0, T::kLoadsA);
        issue_b(0, 0);
        issue_a(1, 1, 0, T::kLoadsA / 2);
        issue_b(1, 1);
        wait_vmcnt<0>();
        lds_barrier();
        issue_a(1, 1, T::kLoadsA / 2, T::kLoadsA);

        auto k_loop = [&](auto skip) __attribute__((always_inline)) {
            for (int kb = 0; kb < KB; kb += 2) {
                step(skip, kb, 0);
                if (kb + 1 < KB) step(skip, kb + 1, 1);
            }
        };
        // A masked tile with rows past its group's count runs a copy of the loop
        // that skips sub-tile rows without a valid row.  With fp32 scales full
        // tiles keep the branch-free loop, whose schedule is faster; with E8M0
        // scales one skipping loop serves every tile (measured faster).
        if constexpr (kForm == Form::Masked && kE8) {
            k_loop(std::true_type{});
        } else if constexpr (kForm == Form::Masked) {
            if (ti.valid < T::BM)
                k_loop(std::true_type{});
            else
                k_loop(std::false_type{});
        } else {
            k_loop(std::false_type{});
        }

        // ---- epilogue
        wait_vmcnt<0>();  // the empty loads of the last steps have retired
        lds_barrier();
        store_tile<T, kForm>(acc, smem, tid, wm, wcol, lr, lg, ti, C, D, N);
        if constexpr (!kMixed) {
            break;
        } else {
            if ((int64_t)ti.n0 + T::BN < N) {
                ti.n0 += T::BN;
            } else {
                ti.n0 = 0;
                if (!block_group(aux, G, ti.g, lane, ti)) break;
            }
            lds_barrier();  // the staged tile has been stored before the next pass loads
        }
    }
}

template <class T, Form kForm, bool kE8>
static dg_status launch_tiled(const GemmArgs& a, hipStream_t stream) {
    const int64_t m_blocks = (a.rows + T::BM - 1) / T::BM;
    const int64_t n_blocks = (a.N + T::BN - 1) / T::BN;
    int64_t grid;
    if (kForm == Form::Masked) {
        // every XCD gets ceil(pairs / 8) pairs of n_blocks tiles
        grid = (a.G * m_blocks + kNumXcds - 1) / kNumXcds * n_blocks * kNumXcds;
    } else {
        grid = (m_blocks * n_blocks + kNumXcds - 1) / kNumXcds * kNumXcds;
    }
    if (grid == 0) return DG_OK;
    if (grid > 0x7fffffff) return DG_ERR_SHAPE;
    // per-lane 32-bit offsets: a tile's rows of K bytes, its A scales
    if ((int64_t)std::max(T::BM, T::BN) * a.K >= (int64_t(1) << 32)) return DG_ERR_SHAPE;
    // and a tile's rows of fp32 C
    if (kForm == Form::DenseAcc && (int64_t)T::BM * a.N * 4 >= (int64_t(1) << 32))
        return DG_ERR_SHAPE;
    hipLaunchKernelGGL((gemm_kernel<T, kForm, kE8>), dim3((unsigned)grid), dim3(T::kThreads), 0, stream,
                       a.A, a.sa, a.B, a.sb, a.D, a.aux, a.C, a.rows, a.N, a.K, a.G, (int)m_blocks,
                       (int)n_blocks);
    if constexpr (kForm == Form::Contiguous) {
        // Blocks whose rows carry more than one valid id: one workgroup per
        // 128-row block, which exits at once unless its block is mixed.  The
        // ordinary launch above stays free of that rare case's code.
        if (launched() != DG_OK) return DG_ERR_HIP;
        hipLaunchKernelGGL((gemm_kernel<T, kForm, kE8, true>), dim3((unsigned)m_blocks), dim3(T::kThreads),
                           0, stream, a.A, a.sa, a.B, a.sb, a.D, a.aux, a.C, a.rows, a.N, a.K, a.G,
                           (int)m_blocks, (int)n_blocks);
    }
    return launched();
}

// 256x256 tiles, 8 waves of 128x64 (two per SIMD).
using TileLarge = TileConfig<256, 256, 2, 4, 4>;
// Narrower dense tiles, 8 waves of 64x112 / 64x96: fewer idle CUs in the
// last round of tiles when N is not a good multiple of 256.
using TileWide224 = TileConfig<256, 224, 4, 2, 4>;
using TileWide192 = TileConfig<256, 192, 4, 2, 4>;
using TileWide160 = TileConfig<256, 160, 4, 2, 4>;
// 128x256 tiles, 8 waves of 64x64: contiguous groups are padded to 128 rows;
// also the dense shape for few rows.
using TileRows128 = TileConfig<128, 256, 2, 4, 8>;
// Tiles for few rows (decode-sized M), 4 waves each (64x64, 64x32, 64x16):
// such a launch is bound by how many bytes of B are in flight (each tile
// keeps about 1.5 K blocks of loads outstanding), so narrower tiles, more of
// them, stream B faster.
using TileSmall = TileConfig<128, 128, 2, 2, 8>;
// 256x256 tiles, 8 waves of 64x128: each A fragment feeds eight MFMAs.  Used
// with power-of-two scales (without promotion it fits the registers: 231
// VGPRs; the fp32-scale kernel spills with it).
using TileLargeT = TileConfig<256, 256, 4, 2, 4>;
using TileNarrow64 = TileConfig<128, 64, 2, 2, 8>;
using TileNarrow32 = TileConfig<128, 32, 2, 2, 8>;
// Masked groups: 256x256 tiles.  In a tile with rows past its group's count
// a wave skips the fragment reads, MFMAs and promotion of its 16-row sub-tile
// rows that hold no valid row (a uniform branch on the count), so tiles of
// short groups finish early and stop drawing on HBM while the full slabs
// still stream; full tiles run the branch-free loop.
using TileMasked = TileConfig<256, 256, 2, 4, 4>;

// Compute units of the current device, cached per device.  Host threads may
// launch concurrently: each slot only ever receives its device's one value,
// so relaxed atomics suffice.
static int device_cus() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const bool slot = dev >= 0 && dev < 64;
    if (slot) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (slot) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// DG_FP8_DENSE_TILE=256x256|256x224|256x192|256x160|128x256|128x128|128x64|128x32|256x256t pins the dense tile
// shape (for tests and tuning; read at every call); -1 when unset or not
// one of these.
static int forced_dense_shape() {
    const char* e = getenv("DG_FP8_DENSE_TILE");
    if (!e) return -1;
    const char* names[] = {"256x256", "256x224", "256x192", "128x256", "128x128", "128x64", "128x32",
                           "256x256t", "256x160"};
    for (int i = 0; i < 9; ++i)
        if (strcmp(e, names[i]) == 0) return i;
    return -1;
}

// Dense tile shape.  The 256-row shapes and 128x256 run one workgroup per
// CU, so a launch takes about ceil(tiles / CUs) rounds of one tile's time; a
// tile's time scales with its area times a per-shape cost per output element
// (narrower tiles re-read more fragments per MFMA), and the shape with the
// least estimated time wins.  When even 256x256 tiles would leave half the
// CUs idle (few rows: decode-sized M), 128x32 tiles are used instead: such
// a launch is latency-bound on B (a lone 256x256 tile takes 60k cycles at
// K = 2048), and 128x32 tiles put the most B loads in flight (measured on
// 128 x 7168 x 2048: 13.7 us against 17.7 with 128x128 and 24 with 128x256).
template <Form kForm, bool kE8>
static dg_status launch_dense(const GemmArgs& a, hipStream_t stream) {
    struct Shape { int bm, bn; double rel; int id; };
    // per-area costs from measured loop cycles per K block (256x256: 3.43k,
    // 256x224: 3.42k, 256x192: 2.93k, 128x256: 2.08k cycles); 256x160 from
    // whole launches of 4096 x 2112 x 7168, one round of tiles each: 86.2 us
    // against 91.6 us with 256x192
    static const Shape kShapes[] = {{256, 256, 1.00, 0}, {256, 224, 1.15, 1}, {256, 192, 1.15, 2},
                                    {128, 256, 1.22, 3}, {256, 160, 1.30, 8}};
    const int64_t cus = device_cus();
    const int forced = forced_dense_shape();
    int best = forced;
    const int64_t tiles_large = ((a.rows + 255) / 256) * ((a.N + 255) / 256);
    if (best < 0 && 2 * tiles_large <= cus) best = 6;
    if (best < 0) {
        double best_cost = 0;
        for (int i = 0; i < (int)(sizeof(kShapes) / sizeof(kShapes[0])); ++i) {
            const Shape& sh = kShapes[i];
            const int64_t tiles = ((a.rows + sh.bm - 1) / sh.bm) * ((a.N + sh.bn - 1) / sh.bn);
            const double cost = (double)((tiles + cus - 1) / cus) * sh.bm * sh.bn * sh.rel;
            if (i == 0 || cost < best_cost) {
                best_cost = cost;
                best = sh.id;
            }
        }
        // with power-of-two scales the 64x128 wave layout of 256x256 is the
        // faster one (measured 2-5%)
        if (kE8 && best == 0) best = 7;
    }
    switch (best) {
        case 1: return launch_tiled<TileWide224, kForm, kE8>(a, stream);
        case 2: return launch_tiled<TileWide192, kForm, kE8>(a, stream);
        case 3: return launch_tiled<TileRows128, kForm, kE8>(a, stream);
        case 4: return launch_tiled<TileSmall, kForm, kE8>(a, stream);
        case 5: return launch_tiled<TileNarrow64, kForm, kE8>(a, stream);
        case 6: return launch_tiled<TileNarrow32, kForm, kE8>(a, stream);
        case 7: return launch_tiled<TileLargeT, kForm, kE8>(a, stream);
        case 8: return launch_tiled<TileWide160, kForm, kE8>(a, stream);
        default: return launch_tiled<TileLarge, kForm, kE8>(a, stream);
    }
}

dg_status launch_gemm(Form form, const GemmArgs& a, hipStream_t stream) {
    if (a.e8m0) {
        switch (form) {
            case Form::Dense: return launch_dense<Form::Dense, true>(a, stream);
            case Form::Contiguous: return launch_tiled<TileRows128, Form::Contiguous, true>(a, stream);
            case Form::Masked: return launch_tiled<TileLargeT, Form::Masked, true>(a, stream);
            default: return DG_ERR_UNSUPPORTED;
        }
    }
    switch (form) {
        case Form::Dense: return launch_dense<Form::Dense, false>(a, stream);
        case Form::DenseAcc: return launch_dense<Form::DenseAcc, false>(a, stream);
        case Form::Contiguous: return launch_tiled<TileRows128, Form::Contiguous, false>(a, stream);
        case Form::Masked: return launch_tiled<TileMasked, Form::Masked, false>(a, stream);
    }
    return DG_ERR_UNSUPPORTED;
}

}  // namespace dg
