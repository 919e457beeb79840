// Quantize helpers: fp32 -> e4m3 codes plus fp32 scales, in the two layouts
// the GEMM reads (sa [M][K/128] per token, sb [ceil(N/128)][K/128] per
// 128x128 block).  scale = amax/448 and code = e4m3(x/scale), both with IEEE
// fp32 division (HIP's default correctly rounded division), round to nearest
// even with saturation.  These kernels are HBM-bound: 4 bytes read and 1 byte
// written per element.
#include "device_common.h"
#include "launch.h"

namespace dg {

// Half a wavefront (32 lanes x 4 floats) owns one 128-wide block of one row;
// a 256-thread workgroup covers 8 blocks.
__global__ __launch_bounds__(256) void quantize_per_token_kernel(
    const float* __restrict__ x, int64_t total_blocks, int64_t K,
    uint8_t* __restrict__ q, float* __restrict__ s) {
    const int64_t KB = K >> 7;
    const int64_t blk = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    if (blk >= total_blocks) return;  // uniform over each 32-lane half
    const int64_t m = blk / KB, kb = blk - m * KB;
    const int64_t off = m * K + kb * 128 + lane * 4;
    const float4 v = *reinterpret_cast<const float4*>(x + off);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 32));
    const float scale = a / 448.0f;
    uint32_t packed = 0;
    if (a != 0.0f) {
        packed = e4m3_rne_sat(v.x / scale) | (e4m3_rne_sat(v.y / scale) << 8) |
                 (e4m3_rne_sat(v.z / scale) << 16) | (e4m3_rne_sat(v.w / scale) << 24);
    }
    *reinterpret_cast<uint32_t*>(q + off) = packed;
    if (lane == 0) s[blk] = scale;
}

// One 256-thread workgroup per 128x128 block: every thread keeps 16 float4
// of the block in registers across the amax reduction, so the block is read
// from HBM once.
__global__ __launch_bounds__(256) void quantize_per_block_kernel(
    const float* __restrict__ x, int64_t N, int64_t K,
    uint8_t* __restrict__ q, float* __restrict__ s) {
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
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int64_t row = nb * 128 + p * 8 + (t >> 5);
        if (row < N) {
            uint32_t packed = 0;
            if (a != 0.0f) {
                packed = e4m3_rne_sat(v[p].x / scale) | (e4m3_rne_sat(v[p].y / scale) << 8) |
                         (e4m3_rne_sat(v[p].z / scale) << 16) | (e4m3_rne_sat(v[p].w / scale) << 24);
            }
            *reinterpret_cast<uint32_t*>(q + row * K + kb * 128 + col) = packed;
        }
    }
    if (t == 0) s[nb * KB + kb] = scale;
}

hipError_t launch_quantize_per_token(const float* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream) {
    const int64_t total = M * (K >> 7);
    const int64_t grid = (total + 7) / 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_per_token_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       x, total, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quantize_per_block(const float* x, int64_t N, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream) {
    const int64_t NB = (N + 127) / 128, KB = K >> 7;
    if (NB > 65535 || KB > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_per_block_kernel, dim3((unsigned)KB, (unsigned)NB), dim3(256), 0,
                       stream, x, N, K, q, s);
    return hipGetLastError();
}

}  // namespace dg
