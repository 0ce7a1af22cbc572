// hga_internal.h -- shared device helpers and launcher declarations of libhga
// (gfx950 only: wave64, bf16 MFMA with 16-deep k per instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga.h"

namespace hga {

constexpr int kD = 128;      // head dim
constexpr int kC = 64;       // chunk length == query block length
constexpr int kMaxTopK = 256;
constexpr int kGroup = 8;                  // tokens per group (second routing level)
constexpr int kMaxGroupTopK = kMaxTopK * (64 / kGroup);   // every group of kMaxTopK chunks
constexpr int kMaxSink = HGA_MAX_SINK_CHUNKS;
// tile list lengths: local + sink + routed units, chunk and group level
constexpr int kChunkListMax = 1 + kMaxSink + kMaxTopK;
constexpr int kGroupListMax = 1 + kMaxSink * (64 / kGroup) + kMaxGroupTopK;
// chunk budget up to which the two routing levels run inside the group
// attention kernel (launch_route_attend_fwd_groups)
constexpr int kFusedGroupChunks = 32;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> f32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Value of lane l ^ 32 (swap of the two half-waves).
__device__ __forceinline__ float partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0] holds lanes 0..31 of x in both halves, r[1] lanes 32..63 of x.
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Tile list of one (query block, kv head) for the attention kernels, built by
// one wave: the valid routed ids of `row` (0 <= c < local_chunk) in their
// given order with repeats dropped (the first occurrence stays: the routed
// chunks form a set), then the local chunk. Returns the list length. A
// router-made row (ascending, distinct) passes one neighbour check; only a
// row with a repeat pays the quadratic pass. `list` holds k + 1 entries and
// is read back by the same wave only.
// One wave compacts the valid units of an id row (lo <= u < hi) into list,
// in row order with repeats dropped, and returns their number. first =
// row[lane] if lane < k, else -1: a caller may load it early, so the load's
// latency overlaps the caller's other loads.
__device__ __forceinline__ int build_unit_list(const int32_t *row, int k, int64_t lo,
                                               int64_t hi, int *list, int first)
{
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int base = 0; base < k; base += 64) {
        const int r = base + lane;
        const int c = base == 0 ? first : (r < k) ? row[r] : -1;
        const bool ok = (int64_t)c >= lo && (int64_t)c < hi;
        const uint64_t m = __ballot(ok);
        if (ok) list[cnt + lanes_below(m)] = c;
        cnt += __popcll(m);
    }
    bool unsorted = false;
    for (int i = 1 + lane; i < cnt; i += 64) unsorted |= list[i] <= list[i - 1];
    if (__ballot(unsorted) != 0) {
        // Keep an entry unless an earlier one holds the same id; compact in
        // place in index order (every write lands at or below its read).
        int out = 0;
        for (int base = 0; base < cnt; base += 64) {
            const int i = base + lane;
            const int c = (i < cnt) ? list[i] : -1;
            bool keep = i < cnt;
            for (int j = 0; j < base + 64 && j < cnt; ++j)
                if (j < i && list[j] == c) keep = false;
            const uint64_t m = __ballot(keep);
            if (keep) list[out + lanes_below(m)] = c;
            out += __popcll(m);
        }
        cnt = out;
    }
    return cnt;
}

__device__ __forceinline__ int build_unit_list(const int32_t *row, int k, int64_t lo,
                                               int64_t hi, int *list)
{
    const int lane = threadIdx.x & 63;
    return build_unit_list(row, k, lo, hi, list, lane < k ? row[lane] : -1);
}

// The sink window in units of `unit` tokens for a block starting at P: the
// units of the first min(s, P/C) chunks, written as 0, 1, ... by one wave.
__device__ __forceinline__ int sink_units(int sink_chunks, int64_t P, int unit)
{
    const int64_t s = min((int64_t)sink_chunks, P / kC);
    return (int)(s * (kC / unit));
}
__device__ __forceinline__ void write_sink_units(int *list, int n)
{
    for (int i = threadIdx.x & 63; i < n; i += 64) list[i] = i;
}

// Order-preserving map of a finite float to uint32 (larger float -> larger
// key); -0 is folded onto +0 so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Launchers (argument checks are done by the caller in hga_api.cpp).
hipError_t launch_summarize(const uint16_t *K, int64_t Hkv, int64_t T_cap,
                            int64_t c_begin, int64_t c_end, float *S,
                            int64_t n_cap, hipStream_t stream);

hipError_t launch_summarize_groups(const uint16_t *K, int64_t Hkv, int64_t T_cap,
                                   int64_t c_begin, int64_t c_end, float *SG,
                                   int64_t n_gcap, hipStream_t stream);

// per_q_head: one routing unit (id row) per query head instead of per kv
// head. prev_block: strictly causal routing (block b scores with block b-1's
// queries; Q_prev [Hq][C][D] holds the C queries before p0, used by block 0,
// and may be null when p0 == 0).
hipError_t launch_route(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                        int64_t n_q, const float *S, int64_t n_cap, int32_t k, int32_t sink,
                        bool per_q_head, bool prev_block, const uint16_t *Q_prev,
                        int32_t *ids, float *scores, hipStream_t stream);

hipError_t launch_route_groups(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                               int64_t n_q, const float *SG, int64_t n_gcap,
                               const int32_t *chunk_ids, int32_t kc, int32_t m, int32_t sink,
                               int32_t *gids, float *scores, hipStream_t stream);

hipError_t launch_attend_fwd(const uint16_t *Q, const uint16_t *K,
                             const uint16_t *V, int64_t Hq, int64_t Hkv,
                             int64_t T_cap, int64_t p0, int64_t n_q,
                             const int32_t *ids, int32_t k, int32_t sink, bool per_q_head,
                             float scale, uint16_t *O, float *lse, hipStream_t stream);

hipError_t launch_attend_fwd_groups(const uint16_t *Q, const uint16_t *K,
                                    const uint16_t *V, int64_t Hq, int64_t Hkv,
                                    int64_t T_cap, int64_t p0, int64_t n_q,
                                    const int32_t *gids, int32_t m, int32_t sink, float scale,
                                    uint16_t *O, float *lse, hipStream_t stream);
// Routing and attention in one launch (ids and scores written as
// launch_route would write them). Needs (p0 + n_q - C)/C <=
// route_attend_max_candidates().
hipError_t launch_route_attend_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                   int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                   int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                                   int32_t sink, bool per_q_head, float scale, int32_t *ids,
                                   float *scores, uint16_t *O, float *lse, hipStream_t stream);
int64_t route_attend_max_candidates();
// Both routing levels and group attention in one launch (chunk ids, group ids
// and group scores written as launch_route and launch_route_groups would
// write them). Needs 0 < kc <= kFusedGroupChunks, m > 0 and (p0 + n_q - C)/C
// <= route_attend_max_candidates().
hipError_t launch_route_attend_fwd_groups(const uint16_t *Q, const uint16_t *K,
                                          const uint16_t *V, int64_t Hq, int64_t Hkv,
                                          int64_t T_cap, int64_t p0, int64_t n_q,
                                          const float *S, int64_t n_cap, int32_t kc,
                                          const float *SG, int64_t n_gcap, int32_t m,
                                          int32_t sink, float scale, int32_t *chunk_ids,
                                          int32_t *gids, float *gscores, uint16_t *O, float *lse,
                                          hipStream_t stream);
// Routed decode (decode.hip). One workspace of decode_workspace_bytes serves
// the router (the keys of up to decode_key_capacity candidates per token and
// kv head) and then the attention (the partials of decode_splits(k, sink)
// split workgroups per token and kv head).
int decode_splits(int32_t k, int32_t sink);
int64_t decode_key_capacity(int64_t p0, int64_t n_q, int32_t sink);
size_t decode_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q, int32_t k,
                              int32_t sink);
hipError_t launch_route_decode(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                               int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                               int32_t sink, int32_t *ids, float *scores, void *workspace,
                               hipStream_t stream);
hipError_t launch_attend_decode(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                int64_t n_q, const int32_t *ids, int32_t k, int32_t sink,
                                float scale, uint16_t *O, float *lse, void *workspace,
                                hipStream_t stream);
// The decode step's routing and attention in two launches (ids, scores, O and
// lse equal to launch_route_decode + launch_attend_decode); its own workspace
// size. route_attend_decode_fits: false when the survivors of the last token's
// scoring blocks exceed what the attention kernel selects among.
size_t route_attend_decode_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q,
                                           int32_t k, int32_t sink);
bool route_attend_decode_fits(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q, int32_t k,
                              int32_t sink);
hipError_t launch_route_attend_decode(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                      int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                      int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                                      int32_t sink, float scale, int32_t *ids, float *scores,
                                      uint16_t *O, float *lse, void *workspace,
                                      hipStream_t stream);
// Gather-only diagnostic (diag.hip): sink holds gather_sink_words words.
hipError_t launch_gather(const uint16_t *K, const uint16_t *V, int64_t Hkv, int64_t T_cap,
                         int64_t p0, int64_t n_q, const int32_t *ids, int32_t k, int32_t sink,
                         uint32_t *sink_out, hipStream_t stream);
size_t gather_sink_words(int64_t Hkv, int64_t n_q);
hipError_t launch_attend_bwd_groups(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                    int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                    int64_t n_q, const int32_t *gids, int32_t m, int32_t sink,
                                    float scale, const uint16_t *O, const float *lse,
                                    const uint16_t *dO, float *dQ, float *dK, float *dV,
                                    void *workspace, hipStream_t stream);

size_t bwd_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head);

// Largest active segment (queries) the backward's key-major pass can list.
int64_t bwd_max_queries();
// The dq workgroups' pass-2 flags left in a backward workspace: how many of
// the n_wg workgroups of the last call on it ran the second pass (host wait).
hipError_t bwd_second_pass_count(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head,
                                 const void *workspace, int64_t *n_second, int64_t *n_wg,
                                 hipStream_t stream);

hipError_t launch_attend_bwd(const uint16_t *Q, const uint16_t *K,
                             const uint16_t *V, int64_t Hq, int64_t Hkv,
                             int64_t T_cap, int64_t p0, int64_t n_q,
                             const int32_t *ids, int32_t k, int32_t sink, bool per_q_head,
                             float scale, const uint16_t *O, const float *lse,
                             const uint16_t *dO, float *dQ, float *dK,
                             float *dV, void *workspace, hipStream_t stream);

}  // namespace hga
