// summarize.hip -- chunk summaries: the fp32 mean of each chunk's 64 keys
// (arXiv 2607.15105, gist.science technical summary 2.1, chunk selection:
// one compact summary vector per closed chunk stays resident).
//
// HBM-bound: 16 KiB of bf16 keys read and 512 B of fp32 written per
// (kv head, chunk). One 256-thread workgroup per (kv head, chunk): wave w
// reads rows 16w .. 16w+15, each 16-lane group a whole 256-byte key row per
// 16-byte load (4 loads per lane, all in flight together); lanes accumulate in
// fp32, fold their four row groups with two lane swaps, and the four waves'
// partial sums are added through LDS in wave order.
#include "hga_internal.h"

namespace hga {
namespace {

__global__ __launch_bounds__(256) void summarize_kernel(
    const uint16_t *__restrict__ K, int64_t T_cap, int64_t c_begin,
    float *__restrict__ S, int64_t n_cap)
{
    __shared__ float part[4][kD];
    const int64_t g = blockIdx.y;                   // grid (chunks, kv heads)
    const int64_t c = c_begin + blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int dseg = lane & 15;          // d = 8*dseg .. 8*dseg+7
    const int rg = lane >> 4;            // rows 16*wave + rg + 4r

    const uint16_t *base = K + ((g * T_cap + c * kC + 16 * wave + rg) * kD) + dseg * 8;
    u32x4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = *(const u32x4 *)(base + (int64_t)(4 * r) * kD);

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += bf16_lo(w[r][q]);
            acc[2 * q + 1] += bf16_hi(w[r][q]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += partner32(acc[e]);
    }
    if (rg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][dseg * 8 + e] = acc[e];
    }
    __syncthreads();
    if (threadIdx.x < kD) {
        const int d = threadIdx.x;
        const float sum = ((part[0][d] + part[1][d]) + part[2][d]) + part[3][d];
        S[(g * n_cap + c) * kD + d] = sum * (1.0f / (float)kC);   // a power of two: exact
    }
}

// Group summaries (the second routing level): the fp32 mean of each 8-token
// group of the chunk. Same loads as above; lane rows 16w + rg + {0, 4} form
// group 2w and 16w + rg + {8, 12} group 2w + 1, so two fp32 accumulators per
// lane, folded over the four row groups by the same two lane swaps, give the
// eight groups of the chunk with no LDS pass.
__global__ __launch_bounds__(256) void summarize_groups_kernel(
    const uint16_t *__restrict__ K, int64_t T_cap, int64_t c_begin,
    float *__restrict__ SG, int64_t n_gcap)
{
    const int64_t g = blockIdx.y;                   // grid (chunks, kv heads)
    const int64_t c = c_begin + blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int dseg = lane & 15;
    const int rg = lane >> 4;

    const uint16_t *base = K + ((g * T_cap + c * kC + 16 * wave + rg) * kD) + dseg * 8;
    u32x4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = *(const u32x4 *)(base + (int64_t)(4 * r) * kD);

    float acc[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[r >> 1][2 * q] += bf16_lo(w[r][q]);
            acc[r >> 1][2 * q + 1] += bf16_hi(w[r][q]);
        }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += __shfl_xor(acc[h][e], 16);
            acc[h][e] += partner32(acc[h][e]);
        }
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float *dst = SG + (g * n_gcap + c * (kC / kGroup) + 2 * wave + h) * kD + dseg * 8;
            f32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = acc[h][e] * (1.0f / (float)kGroup);        // a power of two: exact
                hi[e] = acc[h][4 + e] * (1.0f / (float)kGroup);
            }
            *(f32x4 *)dst = lo;
            *(f32x4 *)(dst + 4) = hi;
        }
    }
}

}  // namespace

hipError_t launch_summarize_groups(const uint16_t *K, int64_t Hkv, int64_t T_cap,
                                   int64_t c_begin, int64_t c_end, float *SG,
                                   int64_t n_gcap, hipStream_t stream)
{
    const int64_t n_chunks = c_end - c_begin;
    if (Hkv * n_chunks <= 0) return hipSuccess;
    if (Hkv > 65535) return hipErrorInvalidConfiguration;      // grid y limit
    hipLaunchKernelGGL(summarize_groups_kernel, dim3((unsigned)n_chunks, (unsigned)Hkv), dim3(256),
                       0, stream, K, T_cap, c_begin, SG, n_gcap);
    return hipGetLastError();
}

hipError_t launch_summarize(const uint16_t *K, int64_t Hkv, int64_t T_cap,
                            int64_t c_begin, int64_t c_end, float *S,
                            int64_t n_cap, hipStream_t stream)
{
    const int64_t n_chunks = c_end - c_begin;
    if (Hkv * n_chunks <= 0) return hipSuccess;
    if (Hkv > 65535) return hipErrorInvalidConfiguration;      // grid y limit
    hipLaunchKernelGGL(summarize_kernel, dim3((unsigned)n_chunks, (unsigned)Hkv), dim3(256), 0,
                       stream, K, T_cap, c_begin, S, n_cap);
    return hipGetLastError();
}

}  // namespace hga
