// summarize.hip -- chunk summaries: the fp32 mean of each chunk's 64 keys
// (arXiv 2607.15105, gist.science technical summary 2.1, chunk selection:
// one compact summary vector per closed chunk stays resident).
//
// HBM-bound: 16 KiB of bf16 keys read and 512 B of fp32 written per
// (kv head, chunk). One wave per (kv head, chunk): each 16-lane row group
// reads whole 256-byte key rows (coalesced 16-byte loads), lanes accumulate
// in fp32 and the four row groups are folded with two lane swaps.
#include "hga_internal.h"

namespace hga {
namespace {

__global__ __launch_bounds__(256) void summarize_kernel(
    const uint16_t *__restrict__ K, int64_t T_cap, int64_t c_begin,
    int64_t n_chunks, int64_t n_units, float *__restrict__ S, int64_t n_cap)
{
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= n_units) return;
    const int64_t g = unit / n_chunks;
    const int64_t c = c_begin + unit % n_chunks;
    const int lane = threadIdx.x & 63;
    const int dseg = lane & 15;          // d = 8*dseg .. 8*dseg+7
    const int rg = lane >> 4;            // rows rg, rg+4, ..., rg+60

    const uint16_t *base = K + ((g * T_cap + c * kC) * kD) + dseg * 8;
    u32x4 w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        w[r] = *(const u32x4 *)(base + (int64_t)(rg + 4 * r) * kD);

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
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
        const float inv = 1.0f / (float)kC;   // a power of two: exact
        f32x4 lo = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        f32x4 hi = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
        float *dst = S + (g * n_cap + c) * kD + dseg * 8;
        *(f32x4 *)dst = lo;
        *(f32x4 *)(dst + 4) = hi;
    }
}

}  // namespace

hipError_t launch_summarize(const uint16_t *K, int64_t Hkv, int64_t T_cap,
                            int64_t c_begin, int64_t c_end, float *S,
                            int64_t n_cap, hipStream_t stream)
{
    const int64_t n_chunks = c_end - c_begin;
    const int64_t n_units = Hkv * n_chunks;
    if (n_units <= 0) return hipSuccess;
    const int64_t grid = (n_units + 3) / 4;
    hipLaunchKernelGGL(summarize_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       K, T_cap, c_begin, n_chunks, n_units, S, n_cap);
    return hipGetLastError();
}

}  // namespace hga
