// Quantize helpers: fp32 -> e4m3 codes plus scales, in the two layouts
// the GEMM reads (sa [M][K/128] per token, sb [ceil(N/128)][K/128] per
// 128x128 block).  scale = amax/448 and code = e4m3(x/scale), both divisions
// correctly rounded fp32 (x/scale through the block's reciprocal and one
// correction step, same result), e4m3 rounding to nearest even with
// saturation (the hardware conversion on inputs clamped to +-448).
// Activations may also come as bf16, converted exactly to fp32 first.
// Power-of-two variant: the scale is 2^e with e the smallest integer >= -127
// such that amax <= 448 * 2^e, stored as the E8M0 byte e + 127 in rows of
// K/128 bytes padded to a multiple of 4 (padding not written), and code =
// e4m3(x * 2^-e), an exact scaling.  These kernels are HBM-bound: 4 (fp32)
// or 2 (bf16) bytes read and 1 byte written per element.
#include "device_common.h"
#include "launch.h"

namespace dg {

// x / b rounded to nearest even, given y = RN(1/b) finite and normal: q =
// RN(x y) is within an ulp of x/b, the remainder x - b q is exact (one FMA),
// and RN(q + (x - b q) y) is the correctly rounded quotient (Markstein's
// correction step).  Three operations instead of a full IEEE division.
__device__ __forceinline__ float quotient_rn(float x, float b, float y) {
    const float q0 = x * y;
    return __builtin_fmaf(__builtin_fmaf(-q0, b, x), y, q0);
}

// The power-of-two exponent of a block: amax = 1.f * 2^u needs e = u - 8
// when 1.f <= 1.75 (448 = 1.75 * 2^8, fraction bits 0x600000) and u - 7
// otherwise; zero and fp32 subnormals (below 2^-126, far below 448 * 2^-127)
// take the least exponent, -127.
__device__ __forceinline__ int e8m0_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    const int E = (int)(b >> 23);  // biased exponent; amax >= 0
    if (E == 0) return -127;
    return max(E - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0), -127);
}

// 2^-e as an fp32 bit pattern (a normal number for e in [-127, 126]).
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Eight lanes own one 128-wide block of one row, 16 elements each: lane l
// loads columns 4l .. 4l+3 (fp32 input) or 8l .. 8l+7 (bf16 input) of each
// 32- or 64-column quarter/half, so every load instruction covers whole
// contiguous 128- or 256-byte runs of a row per 8 lanes; all of a lane's
// loads are issued before any is used.  The amax is reduced over the 8 lanes
// with shuffles.  The 128 codes of a block (one 128-byte line of q) pass
// through LDS so that each lane stores 16 contiguous bytes: one full line per
// block per store instruction.  A 256-thread workgroup covers 32 blocks.
template <class In, bool kE8>
__global__ __launch_bounds__(256) void quantize_per_token_kernel(
    const In* __restrict__ x, int64_t total_blocks, int64_t K,
    uint8_t* __restrict__ q, void* __restrict__ s) {
    __shared__ __align__(16) uint8_t codes[32][128];
    constexpr bool kBf16 = sizeof(In) == 2;
    const int64_t KB = K >> 7;
    const int grp = threadIdx.x >> 3;
    const int64_t blk = (int64_t)blockIdx.x * 32 + grp;
    const int lane = threadIdx.x & 7;
    if (blk >= total_blocks) return;  // uniform over each 8-lane group
    const int64_t m = blk / KB, kb = blk - m * KB;
    const int64_t base = m * K + kb * 128;
    float f[16];
    if (kBf16) {
        // two 16-byte loads: columns 8l .. 8l+7 and 64+8l .. 64+8l+7
        v4u raw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            raw[h] = *reinterpret_cast<const v4u*>(x + base + 64 * h + 8 * lane);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w) {  // a bf16 is the high half of its fp32
                f[8 * h + 2 * w] = __uint_as_float(raw[h][w] << 16);
                f[8 * h + 2 * w + 1] = __uint_as_float(raw[h][w] & 0xffff0000u);
            }
    } else {
        // four 16-byte loads: columns 32i + 4l .. 32i + 4l + 3
        float4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = *reinterpret_cast<const float4*>(x + base + 32 * i + 4 * lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[4 * i] = v[i].x; f[4 * i + 1] = v[i].y; f[4 * i + 2] = v[i].z; f[4 * i + 3] = v[i].w;
        }
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(f[e]));
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 8));
    const float scale = a / 448.0f;
    // x / scale through the block's reciprocal (see quotient_rn); a block
    // whose scale is below the normal range takes IEEE division instead
    const int ex = kE8 ? e8m0_exponent(a) : 0;
    const float y = kE8 ? exp2_neg(ex) : 1.0f / scale;
    const bool fast = scale >= 1.17549435e-38f && y <= 3.40282347e38f;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d[e] = kE8 ? f[4 * i + e] * y
                       : (fast ? quotient_rn(f[4 * i + e], scale, y) : f[4 * i + e] / scale);
        w[i] = (kE8 || a != 0.0f) ? e4m3x4_hw(d[0], d[1], d[2], d[3]) : 0u;
    }
    // codes to LDS in column order, back 16 bytes per lane (the group's lanes
    // are in one wave: no barrier, the LDS accesses of a wave are ordered)
    if (kBf16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v2u o;
            o[0] = w[2 * h];
            o[1] = w[2 * h + 1];
            *reinterpret_cast<v2u*>(&codes[grp][64 * h + 8 * lane]) = o;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(&codes[grp][32 * i + 4 * lane]) = w[i];
    }
    __builtin_amdgcn_wave_barrier();
    *reinterpret_cast<v4u*>(q + base + 16 * lane) = *reinterpret_cast<const v4u*>(&codes[grp][16 * lane]);
    if (lane == 0) {
        if (kE8)
            static_cast<uint8_t*>(s)[m * ((KB + 3) & ~int64_t(3)) + kb] = (uint8_t)(ex + 127);
        else
            static_cast<float*>(s)[blk] = scale;
    }
}

// One 256-thread workgroup per 128x128 block: every thread keeps 16 float4
// of the block in registers across the amax reduction, so the block is read
// from HBM once.
template <bool kE8>
__global__ __launch_bounds__(256) void quantize_per_block_kernel(
    const float* __restrict__ x, int64_t N, int64_t K,
    uint8_t* __restrict__ q, void* __restrict__ s) {
    const int64_t KB = K >> 7;
    const int64_t nb = blockIdx.y, kb = blockIdx.x;
    const int t = threadIdx.x;
    const int col = (t & 31) * 4;
    __shared__ float wave_max[4];
    float4 v[16];
    float a = 0.0f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int64_t row = nb * 128 + p * 8 + (t >> 5);
        if (row < N) {
            v[p] = *reinterpret_cast<const float4*>(x + row * K + kb * 128 + col);
        } else {
            v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v[p].x), fabsf(v[p].y)), fmaxf(fabsf(v[p].z), fabsf(v[p].w))));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 64));
    if ((t & 63) == 0) wave_max[t >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float scale = a / 448.0f;
    const int ex = kE8 ? e8m0_exponent(a) : 0;
    const float y = kE8 ? exp2_neg(ex) : 1.0f / scale;
    const bool fast = scale >= 1.17549435e-38f && y <= 3.40282347e38f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int64_t row = nb * 128 + p * 8 + (t >> 5);
        if (row < N) {
            const float xv[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
            float d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                d[e] = kE8 ? xv[e] * y : (fast ? quotient_rn(xv[e], scale, y) : xv[e] / scale);
            const uint32_t packed = (kE8 || a != 0.0f) ? e4m3x4_hw(d[0], d[1], d[2], d[3]) : 0u;
            *reinterpret_cast<uint32_t*>(q + row * K + kb * 128 + col) = packed;
        }
    }
    if (t == 0) {
        if (kE8)
            static_cast<uint8_t*>(s)[nb * ((KB + 3) & ~int64_t(3)) + kb] = (uint8_t)(ex + 127);
        else
            static_cast<float*>(s)[nb * KB + kb] = scale;
    }
}

template <class In, bool kE8>
static dg_status launch_per_token(const In* x, int64_t M, int64_t K, uint8_t* q, void* s,
                                   hipStream_t stream) {
    const int64_t total = M * (K >> 7);
    const int64_t grid = (total + 31) / 32;
    if (grid > 0x7fffffff) return DG_ERR_SHAPE;
    hipLaunchKernelGGL((quantize_per_token_kernel<In, kE8>), dim3((unsigned)grid), dim3(256), 0,
                       stream, x, total, K, q, s);
    return launched();
}

template <bool kE8>
static dg_status launch_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, void* s,
                                   hipStream_t stream) {
    const int64_t NB = (N + 127) / 128, KB = K >> 7;
    if (NB > 65535 || KB > 0x7fffffff) return DG_ERR_SHAPE;
    hipLaunchKernelGGL(quantize_per_block_kernel<kE8>, dim3((unsigned)KB, (unsigned)NB), dim3(256),
                       0, stream, x, N, K, q, s);
    return launched();
}

dg_status launch_quantize_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream) {
    return launch_per_token<float, false>(x, M, K, q, s, stream);
}

dg_status launch_quantize_per_token_bf16(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                                          float* s, hipStream_t stream) {
    return launch_per_token<uint16_t, false>(x, M, K, q, s, stream);
}

dg_status launch_quantize_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream) {
    return launch_per_block<false>(x, N, K, q, s, stream);
}

dg_status launch_quantize_per_token_e8m0(const float* x, int64_t M, int64_t K, uint8_t* q,
                                          uint8_t* s, hipStream_t stream) {
    return launch_per_token<float, true>(x, M, K, q, s, stream);
}

dg_status launch_quantize_per_block_e8m0(const float* x, int64_t N, int64_t K, uint8_t* q,
                                          uint8_t* s, hipStream_t stream) {
    return launch_per_block<true>(x, N, K, q, s, stream);
}

}  // namespace dg
