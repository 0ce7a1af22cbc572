// diag.hip -- gather-only diagnostic: the K/V tiles hga_attend_fwd gathers
// (the sink window, every routed chunk of the block's id row and the local
// block, per (query block, kv head)), read with the attention kernel's
// addressing and 16-byte
// loads and folded by XOR into one word per thread, with no arithmetic of the
// method. Its time is the ceiling the gather alone sets for the attention
// kernel (arXiv 2607.15105, gist.science technical summary 2.1: only the exact
// K/V of the selected chunks are read).
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv,
    int64_t T_cap, int64_t p0, const int32_t *__restrict__ ids, int k, int sink_chunks,
    uint32_t *__restrict__ sink)
{
    __shared__ int list[kChunkListMax];
    __shared__ int list_n;
    const int tid = threadIdx.x;
    const int64_t g = blockIdx.x % Hkv;
    const int64_t b = blockIdx.x / Hkv;
    const int64_t n_blocks = n_q / kC;
    const int64_t P = p0 + b * kC;
    if (tid < 64) {                         // sink chunks, routed chunks, local chunk
        const int ns = sink_units(sink_chunks, P, kC);
        write_sink_units(list, ns);
        const int n = build_unit_list(ids + (g * n_blocks + b) * k, k, sink_chunks, P / kC,
                                      list + ns);
        if (tid == 0) {
            list[ns + n] = (int)(P / kC);
            list_n = ns + n + 1;
        }
    }
    __syncthreads();
    const int n_tiles = list_n;
    const uint16_t *Kg = K + g * T_cap * kD;
    const uint16_t *Vg = V + g * T_cap * kD;
    // thread: rows tid/16 + 16*j of a tile, d = 8*(tid%16) .. +8
    const int64_t off = (int64_t)(tid >> 4) * kD + (tid & 15) * 8;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {       // two tiles (16 loads) in flight
        const int64_t r0 = (int64_t)list[t] * kC * kD + off;
        const int64_t r1 = (int64_t)list[t + 1] * kC * kD + off;
        u32x4 x[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = *(const u32x4 *)(Kg + r0 + 16 * j * kD);
            x[4 + j] = *(const u32x4 *)(Vg + r0 + 16 * j * kD);
            x[8 + j] = *(const u32x4 *)(Kg + r1 + 16 * j * kD);
            x[12 + j] = *(const u32x4 *)(Vg + r1 + 16 * j * kD);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] ^= x[j][e];
    }
    if (t < n_tiles) {
        const int64_t r0 = (int64_t)list[t] * kC * kD + off;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 xk = *(const u32x4 *)(Kg + r0 + 16 * j * kD);
            const u32x4 xv = *(const u32x4 *)(Vg + r0 + 16 * j * kD);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] ^= xk[e] ^ xv[e];
        }
    }
    sink[(int64_t)blockIdx.x * kGatherThreads + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_gather(const uint16_t *K, const uint16_t *V, int64_t Hkv, int64_t T_cap,
                         int64_t p0, int64_t n_q, const int32_t *ids, int32_t k, int32_t sink,
                         uint32_t *sink_out, hipStream_t stream)
{
    const int64_t n_units = (n_q / kC) * Hkv;
    if (n_units == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)n_units), dim3(kGatherThreads), 0, stream,
                       K, V, n_q, Hkv, T_cap, p0, ids, k, (int)sink, sink_out);
    return hipGetLastError();
}

size_t gather_sink_words(int64_t Hkv, int64_t n_q) { return (size_t)(n_q / kC) * Hkv * kGatherThreads; }

}  // namespace hga
