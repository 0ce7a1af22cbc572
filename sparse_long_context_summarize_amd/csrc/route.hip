// route.hip -- per query block top-k chunk routing, and its group-level
// variant (arXiv 2607.15105, gist.science technical summary 2.1: the current
// query block scores the resident chunk summaries and keeps the most relevant
// earlier chunks; the chosen chunks' 8-token groups are ranked the same way
// by their own summaries; no gradient flows through the choice).
//
// One 256-thread workgroup per (query block b, routing unit) runs route_block
// (route_core.h). A routing unit is a kv head (its G query heads share one
// id row) or, with per-query-head routing, one query head (kv_div = G query
// heads per kv head, each its own unit scored against its kv head's
// summaries). Workgroup w serves kv head w % Hkv: with 8 kv heads the blocks
// of one head land on one XCD and share its L2 copy of that head's summaries.
// kPrev: strictly causal routing, where block b scores with the queries of
// block b - 1 (Q_prev, the 64 queries before p0, for block 0).
#include "route_core.h"

namespace hga {
namespace {

template <int G, int NI, bool kGroups, bool kPrev>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Q_prev, int64_t n_q,
    int kv_div, int64_t p0, const float *__restrict__ S, int64_t n_cap, int k,
    const int32_t *__restrict__ chunk_ids, int kc, int c_lo,
    int32_t *__restrict__ ids, float *__restrict__ scores)
{
    extern __shared__ uint32_t keys[];          // [candidates of this block]
    __shared__ RouteLds sh;
    const int64_t gkv = blockIdx.x;                     // grid (Hkv, kv_div, blocks)
    const int64_t u = gkv * kv_div + blockIdx.y;        // routing unit
    const int64_t b = blockIdx.z;
    int32_t *out = ids + (u * (n_q / kC) + b) * k;
    float *sout = scores ? scores + (u * (n_q / kC) + b) * k : nullptr;
    auto q_row = [&](int row, int dseg) __attribute__((always_inline)) {
        const int64_t h = u * G + row / kC;
        if constexpr (kPrev) {
            if (b == 0) {
                // (no queries before p0 = 0: block 0 has no candidates then)
                if (!Q_prev) return u32x4{0u, 0u, 0u, 0u};
                return *(const u32x4 *)(Q_prev + (h * kC + row % kC) * kD + dseg * 8);
            }
            const int64_t i = (b - 1) * kC + row % kC;
            return *(const u32x4 *)(Q + (h * n_q + i) * kD + dseg * 8);
        } else {
            const int64_t i = b * kC + row % kC;
            return *(const u32x4 *)(Q + (h * n_q + i) * kD + dseg * 8);
        }
    };
    const int32_t *chunk_row = kGroups ? chunk_ids + (gkv * (n_q / kC) + b) * kc : nullptr;
    route_block<G, NI, kGroups, 16, kRouteWaves>(sh, keys, q_row, n_q, gkv, b, p0, S, n_cap, k,
                                                 chunk_row, kc, c_lo,
                                    [&](int r, int id, float sc) __attribute__((always_inline)) {
                                        out[r] = id;
                                        if (sout) sout[r] = sc;
                                    });
}

struct RouteArgs {
    const uint16_t *Q;
    const uint16_t *Q_prev;     // strictly causal routing only
    bool per_q_head;
    int64_t Hq, Hkv, p0, n_q;
    const float *S;             // chunk or group summaries
    int64_t n_cap;
    int32_t k;                  // chunk budget, or the group budget
    const int32_t *chunk_ids;   // group routing only
    int32_t kc;
    int32_t sink;               // sink window, chunks
    int32_t *ids;
    float *scores;
};

template <int G, int NI, bool kGroups, bool kPrev>
hipError_t launch_route_gn(const RouteArgs &a, size_t shmem, hipStream_t stream)
{
    const int64_t n_blocks = a.n_q / kC;
    const int kv_div = a.per_q_head ? (int)(a.Hq / a.Hkv) : 1;
    if (n_blocks > 65535) return hipErrorInvalidConfiguration;     // grid z limit
    hipLaunchKernelGGL((route_kernel<G, NI, kGroups, kPrev>),
                       dim3((unsigned)a.Hkv, (unsigned)kv_div, (unsigned)n_blocks),
                       dim3(kRouteThreads), shmem,
                       stream, a.Q, a.Q_prev, a.n_q, kv_div, a.p0, a.S, a.n_cap, a.k,
                       a.chunk_ids, a.kc, (int)a.sink, a.ids, a.scores);
    return hipGetLastError();
}

// Keys per lane of the register selection: the smallest class that holds the
// largest candidate count; beyond 2048 (chunk routing only) the LDS path
// takes over.
template <int G, bool kGroups, bool kPrev>
hipError_t launch_route_g(const RouteArgs &a, hipStream_t stream)
{
    int64_t max_chunks = (a.p0 + a.n_q - kC) / kC - a.sink;
    if (max_chunks < 0) max_chunks = 0;
    const int64_t max_eligible =
        kGroups ? (kC / kGroup) * (max_chunks < a.kc ? max_chunks : a.kc) : max_chunks;
    // chunk routing keeps the keys; group routing also sorts up to kc ids there
    int64_t slots = max_eligible > a.kc ? max_eligible : (kGroups ? a.kc : max_eligible);
    const size_t shmem = (size_t)(slots > 0 ? slots : 1) * sizeof(uint32_t);
    if (max_eligible <= 4 * 64) return launch_route_gn<G, 4, kGroups, kPrev>(a, shmem, stream);
    if (max_eligible <= 8 * 64) return launch_route_gn<G, 8, kGroups, kPrev>(a, shmem, stream);
    if (max_eligible <= 16 * 64) return launch_route_gn<G, 16, kGroups, kPrev>(a, shmem, stream);
    return launch_route_gn<G, kMaxRegKeys, kGroups, kPrev>(a, shmem, stream);
}

// G here is the query heads of one routing unit: 1 for per-query-head routing.
template <bool kGroups, bool kPrev>
hipError_t launch_route_any(const RouteArgs &a, hipStream_t stream)
{
    switch (a.per_q_head ? 1 : a.Hq / a.Hkv) {
    case 1: return launch_route_g<1, kGroups, kPrev>(a, stream);
    case 2: return launch_route_g<2, kGroups, kPrev>(a, stream);
    case 4: return launch_route_g<4, kGroups, kPrev>(a, stream);
    case 8: return launch_route_g<8, kGroups, kPrev>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_route(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                        int64_t n_q, const float *S, int64_t n_cap, int32_t k, int32_t sink,
                        bool per_q_head, bool prev_block, const uint16_t *Q_prev,
                        int32_t *ids, float *scores, hipStream_t stream)
{
    if (n_q == 0 || k == 0) return hipSuccess;
    const RouteArgs a{Q, Q_prev, per_q_head, Hq, Hkv, p0, n_q, S, n_cap, k, nullptr, 0, sink,
                      ids, scores};
    return prev_block ? launch_route_any<false, true>(a, stream)
                      : launch_route_any<false, false>(a, stream);
}

hipError_t launch_route_groups(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                               int64_t n_q, const float *SG, int64_t n_gcap,
                               const int32_t *chunk_ids, int32_t kc, int32_t m, int32_t sink,
                               int32_t *gids, float *scores, hipStream_t stream)
{
    if (n_q == 0 || m == 0) return hipSuccess;
    const RouteArgs a{Q, nullptr, false, Hq, Hkv, p0, n_q, SG, n_gcap, m, chunk_ids, kc, sink,
                      gids, scores};
    return launch_route_any<true, false>(a, stream);
}

}  // namespace hga
