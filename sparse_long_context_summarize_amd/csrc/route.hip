// route.hip -- per query block top-k chunk routing, and its group-level
// variant (arXiv 2607.15105, gist.science technical summary 2.1: the current
// query block scores the resident chunk summaries and keeps the most relevant
// earlier chunks; the chosen chunks' 8-token groups are ranked the same way
// by their own summaries; no gradient flows through the choice).
//
// One 256-thread workgroup per (query block b, kv head g) runs route_block
// (route_core.h). Workgroup w serves kv head w % Hkv: with 8 kv heads the
// blocks of one head land on one XCD and share its L2 copy of that head's
// summaries.
#include "route_core.h"

namespace hga {
namespace {

template <int G, int NI, bool kGroups>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const uint16_t *__restrict__ Q, int64_t n_q, int64_t Hkv, int64_t p0,
    const float *__restrict__ S, int64_t n_cap, int k,
    const int32_t *__restrict__ chunk_ids, int kc,
    int32_t *__restrict__ ids, float *__restrict__ scores)
{
    extern __shared__ uint32_t keys[];          // [candidates of this block]
    __shared__ RouteLds sh;
    const int64_t g = blockIdx.x % Hkv;
    const int64_t b = blockIdx.x / Hkv;
    int32_t *out = ids + (g * (n_q / kC) + b) * k;
    float *sout = scores ? scores + (g * (n_q / kC) + b) * k : nullptr;
    auto q_row = [&](int row, int dseg) __attribute__((always_inline)) {
        const int64_t h = g * G + row / kC;
        const int64_t i = b * kC + row % kC;
        return *(const u32x4 *)(Q + (h * n_q + i) * kD + dseg * 8);
    };
    route_block<G, NI, kGroups, 16, kRouteWaves>(sh, keys, q_row, n_q, g, b, p0, S, n_cap, k, chunk_ids, kc,
                                    [&](int r, int id, float sc) __attribute__((always_inline)) {
                                        out[r] = id;
                                        if (sout) sout[r] = sc;
                                    });
}

template <int G, int NI, bool kGroups>
hipError_t launch_route_gn(const uint16_t *Q, int64_t Hkv, int64_t p0, int64_t n_q,
                           const float *S, int64_t n_cap, int32_t k, const int32_t *chunk_ids,
                           int32_t kc, int32_t *ids, float *scores, size_t shmem,
                           hipStream_t stream)
{
    const int64_t n_blocks = n_q / kC;
    hipLaunchKernelGGL((route_kernel<G, NI, kGroups>), dim3((unsigned)(n_blocks * Hkv)),
                       dim3(kRouteThreads), shmem, stream, Q, n_q, Hkv, p0, S, n_cap, k,
                       chunk_ids, kc, ids, scores);
    return hipGetLastError();
}

// Keys per lane of the register selection: the smallest class that holds the
// largest candidate count; beyond 2048 (chunk routing only) the LDS path
// takes over.
template <int G, bool kGroups>
hipError_t launch_route_g(const uint16_t *Q, int64_t Hkv, int64_t p0, int64_t n_q,
                          const float *S, int64_t n_cap, int32_t k, const int32_t *chunk_ids,
                          int32_t kc, int32_t *ids, float *scores, hipStream_t stream)
{
    const int64_t max_chunks = (p0 + n_q - kC) / kC;
    const int64_t max_eligible = kGroups ? (kC / kGroup) * (max_chunks < kc ? max_chunks : kc)
                                         : max_chunks;
    // chunk routing keeps the keys; group routing also sorts up to kc ids there
    int64_t slots = max_eligible > kc ? max_eligible : (kGroups ? kc : max_eligible);
    const size_t shmem = (size_t)(slots > 0 ? slots : 1) * sizeof(uint32_t);
    if (max_eligible <= 4 * 64)
        return launch_route_gn<G, 4, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids,
                                              scores, shmem, stream);
    if (max_eligible <= 8 * 64)
        return launch_route_gn<G, 8, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids,
                                              scores, shmem, stream);
    if (max_eligible <= 16 * 64)
        return launch_route_gn<G, 16, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids,
                                               scores, shmem, stream);
    return launch_route_gn<G, kMaxRegKeys, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids,
                                                    kc, ids, scores, shmem, stream);
}

template <bool kGroups>
hipError_t launch_route_any(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                            int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                            const int32_t *chunk_ids, int32_t kc, int32_t *ids, float *scores,
                            hipStream_t stream)
{
    switch (Hq / Hkv) {
    case 1: return launch_route_g<1, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids, scores, stream);
    case 2: return launch_route_g<2, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids, scores, stream);
    case 4: return launch_route_g<4, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids, scores, stream);
    case 8: return launch_route_g<8, kGroups>(Q, Hkv, p0, n_q, S, n_cap, k, chunk_ids, kc, ids, scores, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_route(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                        int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                        int32_t *ids, float *scores, hipStream_t stream)
{
    if (n_q == 0 || k == 0) return hipSuccess;
    return launch_route_any<false>(Q, Hq, Hkv, p0, n_q, S, n_cap, k, nullptr, 0, ids, scores,
                                   stream);
}

hipError_t launch_route_groups(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                               int64_t n_q, const float *SG, int64_t n_gcap,
                               const int32_t *chunk_ids, int32_t kc, int32_t m,
                               int32_t *gids, float *scores, hipStream_t stream)
{
    if (n_q == 0 || m == 0) return hipSuccess;
    return launch_route_any<true>(Q, Hq, Hkv, p0, n_q, SG, n_gcap, m, chunk_ids, kc, gids,
                                  scores, stream);
}

}  // namespace hga
