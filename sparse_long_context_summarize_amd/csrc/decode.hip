// decode.hip -- routed generation: a decode step of n_q tokens at positions
// p0 .. p0+n_q-1 (arXiv 2607.15105, gist.science technical summary 2.1 applied
// one token at a time; the pages note that the method also serves
// generation). Token p routes on its own G query heads over the closed chunks
// before its open chunk, and attends the sink window, its routed chunks and
// its open chunk up to itself.
//
//   decode_score_kernel   routing, step 1: the token's mean query (over its G
//                         heads) scored against the summaries of its candidate
//                         chunks (s <= c < Pc/C), 256 candidates per
//                         workgroup so that one token's thousands of summary
//                         rows are read by many CUs at once; order-preserving
//                         keys go to the workspace.
//   decode_select_kernel  routing, step 2: the top-k by (score desc, id asc)
//                         over those keys, with the router's selection code.
//   decode_partial_kernel split-K attention: the tiles of a (token, kv head)
//                         -- sink chunks, routed chunks, the open chunk's
//                         prefix -- are dealt kDecTiles (one) at a time to
//                         n_split workgroups; each loads its tiles into LDS at
//                         once, scores them on the vector ALUs (G query rows
//                         are too few for the matrix cores) and writes, per
//                         head, the running max (log2 units), the sum of
//                         exponentials and the unnormalised output.
//   decode_combine_kernel merges the partials of a (token, head) in split
//                         order: O (bf16) and lse.
// The same step in three launches (hga_route_attend_decode):
//   decode_route_part_kernel  the scoring workgroups of decode_score_kernel,
//                         each keeping the top k of its own 256 candidates
//                         (the exact top k of all candidates is among these
//                         survivors);
//   decode_fused_attend_kernel  one workgroup per (token, kv head, split): it
//                         selects the top k among the survivors itself (every
//                         split of a token repeats this short selection, so no
//                         workgroup waits for another) and attends its tile as
//                         decode_partial_kernel does;
//   decode_combine_kernel as above.
// The shared pieces (scoring, one tile's partial, the merge) are one device
// code each, so the two forms give equal ids, scores, O and lse bit for bit.
// (A merge inside the attention launch, by the last split workgroup of each
// (token, kv head) to finish, was measured slower than the separate merge
// launch: one workgroup then reads all G x n_split partials, and its
// device-scope loads are limited by one CU's outstanding misses.)
// At batch 1 the step reads (k + sink + 1) K/V tiles of 32 KiB per (token, kv
// head) once: HBM bound, so the split spreads those reads over many CUs.
#include <algorithm>

#include "route_core.h"

namespace hga {
namespace {

constexpr int kScoreBlock = 256;            // candidates per scoring workgroup

// Candidates of token p: chunks s .. Pc/C - 1 (none if the sink covers them).
__device__ __forceinline__ int decode_candidates(int64_t p, int sink)
{
    return (int)max((int64_t)0, p / kC - sink);
}

// Scores of candidates c0 .. c0+255 of token i, kv head g (c0 < nE), run by
// a kRouteThreads workgroup: each key goes to store(c, key). qbar is kD floats
// of LDS.
template <int G, typename Store>
__device__ __forceinline__ void score_block(const uint16_t *__restrict__ Q, int64_t n_q,
                                            int64_t g, int64_t i, const float *__restrict__ S,
                                            int64_t n_cap, int sink, int c0, int nE,
                                            float *qbar, Store store)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this lane's 16 summary rows first (they do not depend on the mean):
    // chunk c0 + 16*u + 4*wave + sub, 8 dims per lane
    const int sdseg = lane & 15, sub = lane >> 4;
    const float *Sg = S + (g * n_cap + sink) * kD + sdseg * 8;
    f32x4 slo[16], shi[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int c = min(c0 + 16 * u + 4 * wave + sub, nE - 1);   // in bounds; unused past nE
        slo[u] = *(const f32x4 *)(Sg + (int64_t)c * kD);
        shi[u] = *(const f32x4 *)(Sg + (int64_t)c * kD + 4);
    }
    if (tid < kD) {                             // mean over the G heads, in head order
        float a = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint16_t b = Q[((g * G + h) * n_q + i) * kD + tid];
            a += __uint_as_float((uint32_t)b << 16);
        }
        qbar[tid] = a * (1.0f / (float)G);      // a power of two: exact
    }
    __syncthreads();
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qbar[sdseg * 8 + e];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        float sc = qv[0] * slo[u][0];
        sc = fmaf(qv[1], slo[u][1], sc);
        sc = fmaf(qv[2], slo[u][2], sc);
        sc = fmaf(qv[3], slo[u][3], sc);
        sc = fmaf(qv[4], shi[u][0], sc);
        sc = fmaf(qv[5], shi[u][1], sc);
        sc = fmaf(qv[6], shi[u][2], sc);
        sc = fmaf(qv[7], shi[u][3], sc);
        sc = row16_sum(sc);
        const int c = c0 + 16 * u + 4 * wave + sub;
        if (sdseg == 0 && c < nE) store(c, score_key(sc));
    }
}

// Workgroup (token i, kv head g, block blk): candidates blk*256 .. +256.
template <int G>
__global__ __launch_bounds__(kRouteThreads) void decode_score_kernel(
    const uint16_t *__restrict__ Q, int64_t n_q, int64_t Hkv, int64_t p0,
    const float *__restrict__ S, int64_t n_cap, int sink, int n_blk, int64_t kcap,
    uint32_t *__restrict__ keys)
{
    __shared__ float qbar[kD];
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_blk, n_q)
    const int blk = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int nE = decode_candidates(p0 + i, sink);
    const int c0 = blk * kScoreBlock;
    if (c0 >= nE) return;                       // uniform across the workgroup
    uint32_t *kout = keys + (i * Hkv + g) * kcap;
    score_block<G>(Q, n_q, g, i, S, n_cap, sink, c0, nE, qbar,
                   [&](int c, uint32_t key) __attribute__((always_inline)) { kout[c] = key; });
}

// Workgroup (token i, kv head g, block blk) of the two-launch step: the keys
// of candidates blk*256 .. +256, then the top k of them (chunk ids ascending,
// then -1 with key 0) into the survivor rows [n_q][Hkv][n_blk][k].
template <int G>
__global__ __launch_bounds__(kRouteThreads) void decode_route_part_kernel(
    const uint16_t *__restrict__ Q, int64_t n_q, int64_t Hkv, int64_t p0,
    const float *__restrict__ S, int64_t n_cap, int k, int sink, int n_blk,
    uint32_t *__restrict__ surv_key, int32_t *__restrict__ surv_id)
{
    __shared__ float qbar[kD];
    __shared__ uint32_t keys[kScoreBlock];
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_blk, n_q)
    const int blk = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int nE = decode_candidates(p0 + i, sink);
    const int c0 = blk * kScoreBlock;
    if (k == 0 || c0 >= nE) return;             // uniform across the workgroup
    score_block<G>(Q, n_q, g, i, S, n_cap, sink, c0, nE, qbar,
                   [&](int c, uint32_t key) __attribute__((always_inline)) { keys[c - c0] = key; });
    __syncthreads();
    if ((threadIdx.x >> 6) != 0) return;
    const int64_t row = ((i * Hkv + g) * n_blk + blk) * k;
    uint32_t *sk = surv_key + row;
    int32_t *si = surv_id + row;
    auto id_of = [&](int c) __attribute__((always_inline)) { return c0 + c + sink; };
    auto emit = [&](int r, int id, float sc) __attribute__((always_inline)) {
        sk[r] = id >= 0 ? score_key(sc) : 0u;
        si[r] = id;
    };
    select_top_k_reg<4>(keys, min(kScoreBlock, nE - c0), k, id_of, emit);
}

constexpr int kSelWaves = 8;                // selection workgroup: 512 threads

// Final stage of a two-stage selection: wave 0 over the kSelWaves * k
// survivors (holes hold key 0, below every score's key), NI * 64 of them.
template <int NI, typename IdOf, typename Emit>
__device__ __forceinline__ void select_survivors(const uint32_t *cand_key, int k, IdOf id_of,
                                                 Emit emit)
{
    select_top_k_reg<NI>(cand_key, kSelWaves * k, k, id_of, emit);
}

// Workgroup (token i, kv head g): top-k of the token's keys; ids are chunk
// ids (candidate index + s), ascending, -1 padded. Up to 256 candidates one
// wave selects; beyond that each of the 8 waves selects the top k of its
// share (NI * 64 candidates at most) and wave 0 selects among the survivors,
// kept in candidate order so that ties still go to the lower id.
template <int NI>
__global__ __launch_bounds__(kSelWaves * 64) void decode_select_kernel(
    int64_t n_q, int64_t Hkv, int64_t p0, int k, int sink, int64_t kcap,
    const uint32_t *__restrict__ keys, int32_t *__restrict__ ids, float *__restrict__ scores)
{
    __shared__ uint32_t cand_key[kSelWaves * kMaxTopK];
    __shared__ int cand_pos[kSelWaves * kMaxTopK];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_q)
    const int64_t i = blockIdx.y;
    const int nE = decode_candidates(p0 + i, sink);
    const uint32_t *kin = keys + (i * Hkv + g) * kcap;
    int32_t *out = ids + (g * n_q + i) * k;
    float *sout = scores ? scores + (g * n_q + i) * k : nullptr;
    auto emit = [&](int r, int id, float sc) __attribute__((always_inline)) {
        out[r] = id;
        if (sout) sout[r] = sc;
    };
    if (nE <= 4 * 64) {
        auto id_of = [&](int c) __attribute__((always_inline)) { return c + sink; };
        if (wave == 0) select_top_k_reg<4>(kin, nE, k, id_of, emit);
        return;
    }
    const int per = (nE + kSelWaves - 1) / kSelWaves;   // <= NI * 64 (host-chosen NI)
    const int lo = min(nE, wave * per);
    const int hi = min(nE, lo + per);
    {
        auto id_of = [&](int c) __attribute__((always_inline)) { return c + lo; };
        auto keep = [&](int r, int pos, float sc) __attribute__((always_inline)) {
            cand_key[wave * k + r] = pos >= 0 ? score_key(sc) : 0u;
            cand_pos[wave * k + r] = pos;
        };
        select_top_k_reg<NI>(kin + lo, hi - lo, k, id_of, keep);
    }
    __syncthreads();
    if (wave != 0) return;
    auto id_of = [&](int c) __attribute__((always_inline)) { return cand_pos[c] + sink; };
    if (k <= 32) select_survivors<4>(cand_key, k, id_of, emit);
    else if (k <= 64) select_survivors<8>(cand_key, k, id_of, emit);
    else if (k <= 128) select_survivors<16>(cand_key, k, id_of, emit);
    else select_survivors<32>(cand_key, k, id_of, emit);
}

constexpr int kDecThreads = 256;
constexpr int kDecTiles = 1;                // tiles per split workgroup
constexpr int kDecStride = kD + 8;          // bf16 per LDS row (272 B)
constexpr int kPartFloats = 2 + kD;         // max (log2 units), sum, output
constexpr int kMaxSplits = (kMaxSink + kMaxTopK + 1 + kDecTiles - 1) / kDecTiles;

// LDS of a split workgroup: the token's tile list, its K / V tiles, the G
// query rows (fp32) and each wave's probabilities.
template <int G>
struct SplitLds {
    static constexpr int HPW = G > 4 ? 2 : 1;   // heads per wave
    int list[kChunkListMax];
    int list_n;
    __attribute__((aligned(16))) uint16_t Ks[kDecTiles][kC * kDecStride];
    __attribute__((aligned(16))) uint16_t Vs[kDecTiles][kC * kDecStride];
    float qs[G][kD];
    float ps[4][HPW][kC];
};

// The G query rows of token i, kv head g, as fp32 (all threads).
template <int G>
__device__ __forceinline__ void load_q_rows(const uint16_t *__restrict__ Q, int64_t n_q,
                                            int64_t g, int64_t i, SplitLds<G> &sh)
{
    for (int e = threadIdx.x; e < G * kD; e += kDecThreads) {
        const uint16_t b = Q[((g * G + e / kD) * n_q + i) * kD + e % kD];
        sh.qs[e / kD][e % kD] = __uint_as_float((uint32_t)b << 16);
    }
}

// Split j of token p (kv head g): tiles j*kDecTiles .. +kDecTiles of the list
// in sh (published, with sh.qs, by an earlier barrier). Wave w serves heads
// w, w + 4 (G = 8) of the group; lane l holds key l of a tile for the scores
// and output dims 2l, 2l + 1 for P.V. The partial of head h -- running max
// (log2 units), sum of exponentials, unnormalised output -- goes to
// dst + h * kPartFloats. Every thread must call it (one barrier inside).
template <int G>
__device__ __forceinline__ void split_partial(const uint16_t *__restrict__ K,
                                              const uint16_t *__restrict__ V, int64_t T_cap,
                                              int64_t g, int64_t p, int j, float scale_log2,
                                              SplitLds<G> &sh, float *__restrict__ dst)
{
    constexpr int HPW = SplitLds<G>::HPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t Pc = kC * (p / kC);           // start of the open chunk
    const int n_tiles = sh.list_n;
    const int t0 = j * kDecTiles;
    const int my_tiles = max(0, min(kDecTiles, n_tiles - t0));

    // All of this workgroup's K and V rows are loaded at once: thread t moves
    // rows t/16 + 16*r, d = 8*(t%16) .. +8; rows of the open chunk past p are
    // written as zeros (their scores are masked, and zeros keep P.V finite).
    const uint16_t *Kg = K + g * T_cap * kD;
    const uint16_t *Vg = V + g * T_cap * kD;
    for (int u = 0; u < my_tiles; ++u) {
        const int t = t0 + u;
        const int64_t c = sh.list[t];
        const int valid = (t == n_tiles - 1) ? (int)(p - Pc + 1) : kC;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (tid >> 4) + 16 * r;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (row < valid) {
                const int64_t off = (c * kC + row) * kD + (tid & 15) * 8;
                kv = *(const u32x4 *)(Kg + off);
                vv = *(const u32x4 *)(Vg + off);
            }
            *(u32x4 *)(&sh.Ks[u][row * kDecStride + (tid & 15) * 8]) = kv;
            *(u32x4 *)(&sh.Vs[u][row * kDecStride + (tid & 15) * 8]) = vv;
        }
    }
    __syncthreads();

    float m_run[HPW], l_run[HPW], o0[HPW], o1[HPW];
#pragma unroll
    for (int e = 0; e < HPW; ++e) { m_run[e] = -INFINITY; l_run[e] = 0.f; o0[e] = 0.f; o1[e] = 0.f; }
    const bool serves = wave < G;               // G < 4 leaves waves idle
    for (int u = 0; u < my_tiles && serves; ++u) {
        const int t = t0 + u;
        const int valid = (t == n_tiles - 1) ? (int)(p - Pc + 1) : kC;
        const uint16_t *kr = &sh.Ks[u][lane * kDecStride];
#pragma unroll
        for (int e = 0; e < HPW; ++e) {
            const int h = wave + 4 * e;
            float z = 0.f;
#pragma unroll 4
            for (int d = 0; d < kD; d += 8) {
                const u32x4 w = *(const u32x4 *)(kr + d);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    z = fmaf(sh.qs[h][d + 2 * q], bf16_lo(w[q]), z);
                    z = fmaf(sh.qs[h][d + 2 * q + 1], bf16_hi(w[q]), z);
                }
            }
            z = lane < valid ? z * scale_log2 : -INFINITY;
            float mt = z;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
            const float m_new = fmaxf(m_run[e], mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run[e] - m_new);
            const float pz = __builtin_amdgcn_exp2f(z - m_new);
            float sum = pz;
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
            m_run[e] = m_new;
            l_run[e] = l_run[e] * alpha + sum;
            sh.ps[wave][e][lane] = pz;
            o0[e] *= alpha;
            o1[e] *= alpha;
        }
        // (a wave reads only the probabilities it wrote: no barrier needed)
        __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
        for (int e = 0; e < HPW; ++e) {
            const uint16_t *vc = &sh.Vs[u][2 * lane];
            float a0 = 0.f, a1 = 0.f;
#pragma unroll 16
            for (int key = 0; key < kC; ++key) {
                const float pk = sh.ps[wave][e][key];
                const uint32_t w = *(const uint32_t *)(vc + key * kDecStride);
                a0 = fmaf(pk, bf16_lo(w), a0);
                a1 = fmaf(pk, bf16_hi(w), a1);
            }
            o0[e] += a0;
            o1[e] += a1;
        }
    }
    if (!serves) return;
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
        const int h = wave + 4 * e;
        float *o = dst + h * kPartFloats;
        if (lane == 0) {
            o[0] = m_run[e];
            o[1] = l_run[e];
        }
        o[2 + 2 * lane] = o0[e];
        o[3 + 2 * lane] = o1[e];
    }
}

// Partials of (token i, kv head g, split j): [n_q][Hkv][n_split][G][kPartFloats].
__device__ __forceinline__ float *split_part(float *part, int64_t Hkv, int G, int n_split,
                                             int64_t i, int64_t g, int j)
{
    return part + (((i * Hkv + g) * n_split + j) * G) * kPartFloats;
}

// Workgroup (token i, kv head g, split j): the list [sink chunks, routed
// chunks, open chunk] from the id row, then split_partial.
template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv, int64_t T_cap, int64_t p0,
    const int32_t *__restrict__ ids, int k, int sink, float scale_log2, int n_split,
    float *__restrict__ part)
{
    __shared__ SplitLds<G> sh;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_split, n_q)
    const int j = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int64_t p = p0 + i;
    const int64_t Pc = kC * (p / kC);
    if (wave == 0) {
        const int ns = sink_units(sink, Pc, kC);
        write_sink_units(sh.list, ns);
        const int n = build_unit_list(ids + (g * n_q + i) * k, k, sink, Pc / kC, sh.list + ns);
        if (lane == 0) {
            sh.list[ns + n] = (int)(Pc / kC);
            sh.list_n = ns + n + 1;
        }
    }
    load_q_rows<G>(Q, n_q, g, i, sh);
    __syncthreads();
    split_partial<G>(K, V, T_cap, g, p, j, scale_log2, sh,
                     split_part(part, Hkv, G, n_split, i, g, j));
}

// The merge weights of one head, by one wave: M = the largest split max,
// each split's weight w_j = 2^(m_j - M) written over m_j (ms[j * stride]),
// and L = sum_j l_j w_j, lane l adding splits l, l + 64, ... in order and the
// lanes then combined by a fixed butterfly. Every merge of this file uses
// this one order, so its results do not depend on which kernel merges.
__device__ __forceinline__ void merge_weights(float *ms, const float *ws, int stride,
                                              int n_split, float &M, float &L)
{
    const int lane = threadIdx.x & 63;
    float mx = -INFINITY;
    for (int j = lane; j < n_split; j += 64) mx = fmaxf(mx, ms[j * stride]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    for (int j = lane; j < n_split; j += 64) {
        const float w = __builtin_amdgcn_exp2f(ms[j * stride] - mx);   // 0 for an empty split
        sum = fmaf(ws[j * stride], w, sum);
        ms[j * stride] = w;
    }
#pragma unroll
    for (int o = 1; o <= 32; o <<= 1) sum += __shfl_xor(sum, o);
    M = mx;
    L = sum;
}

// Merge of the n_split partials of (token i, query head g*G + hh) by kD
// threads (d = output dim): merge_weights, then each output summed over the
// splits in order; O (bf16) and lse. A thread issues the loads of its output
// for the first kMergeBatch splits together with the splits' maxima and sums
// before it uses any, so up to kMergeBatch splits (k + sink < kMergeBatch)
// merge in one memory round trip. ms and ws hold kMaxSplits floats and ML
// two, in LDS.
constexpr int kMergeBatch = 34;

template <int G>
__device__ __forceinline__ void merge_head(const float *__restrict__ part, int64_t n_q,
                                           int64_t Hkv, int n_split, int64_t i, int64_t g,
                                           int hh, int d, float *ms, float *ws, float *ML,
                                           uint16_t *__restrict__ O, float *__restrict__ lse)
{
    const float *base = part + ((i * Hkv + g) * n_split * G + hh) * kPartFloats;
    const int64_t step = (int64_t)G * kPartFloats;
    float v[kMergeBatch];
    auto load_batch = [&](int j0) __attribute__((always_inline)) {
        const int last = n_split - 1;
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) v[b] = base[min(j0 + b, last) * step + 2 + d];
    };
    float acc = 0.f;
    auto fold_batch = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b)
            if (j0 + b < n_split) acc = fmaf(v[b], ms[j0 + b], acc);
    };
    load_batch(0);
    for (int j = d; j < n_split; j += kD) {
        ms[j] = base[j * step];
        ws[j] = base[j * step + 1];
    }
    __syncthreads();
    if (d < 64) {                               // one wave
        float M, L;
        merge_weights(ms, ws, 1, n_split, M, L);
        if (d == 0) {
            ML[0] = M;
            ML[1] = L;
        }
    }
    __syncthreads();
    fold_batch(0);
    for (int j0 = kMergeBatch; j0 < n_split; j0 += kMergeBatch) {
        load_batch(j0);
        fold_batch(j0);
    }
    const int64_t h = g * G + hh;
    O[(h * n_q + i) * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)(acc / ML[1]));
    if (d == 0) lse[h * n_q + i] = (ML[0] + __log2f(ML[1])) * 0.69314718055994530942f;
}

// One workgroup of kD threads per (token, query head).
template <int G>
__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float *__restrict__ part, int64_t n_q, int64_t Hkv, int n_split,
    uint16_t *__restrict__ O, float *__restrict__ lse)
{
    __shared__ float ms[kMaxSplits], ws[kMaxSplits], ML[2];
    const int64_t h = blockIdx.x;                   // grid (Hkv * G, n_q)
    const int64_t i = blockIdx.y;
    merge_head<G>(part, n_q, Hkv, n_split, i, h / G, (int)(h % G), threadIdx.x, ms, ws, ML, O,
                  lse);
}

// Waves of the fused split workgroup that share a large survivor selection.
constexpr int kFusedSelWaves = kDecThreads / 64;

// Workgroup (token i, kv head g, split j) of the fused step. The token's
// routed chunks: the top k over the survivors of its nb scoring blocks (for
// nb == 1 the survivors are the answer; up to 256 survivors one wave selects;
// beyond that each of the four waves selects among a quarter, NI * 64 at
// most, and wave 0 among their 4k survivors, all kept in id order so that
// ties still go to the lower id). Split 0 writes the id row (and scores).
// Then split_partial; decode_combine_kernel merges.
template <int G, int NI>
__global__ __launch_bounds__(kDecThreads) void decode_fused_attend_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv, int64_t T_cap, int64_t p0,
    int k, int sink, float scale_log2, int n_split, int n_blk,
    const uint32_t *__restrict__ surv_key, const int32_t *__restrict__ surv_id,
    int32_t *__restrict__ ids, float *__restrict__ scores, float *__restrict__ part)
{
    __shared__ SplitLds<G> sh;
    __shared__ uint32_t cand_key[kFusedSelWaves * kMaxTopK];
    __shared__ int cand_id[kFusedSelWaves * kMaxTopK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_split, n_q)
    const int j = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int64_t p = p0 + i;
    const int64_t Pc = kC * (p / kC);
    const int ns = sink_units(sink, Pc, kC);
    const int nE = decode_candidates(p, sink);
    const int nb = (nE + kScoreBlock - 1) / kScoreBlock;    // this token's scoring blocks
    const int64_t srow = (i * Hkv + g) * n_blk * k;
    const uint32_t *sk = surv_key + srow;
    const int32_t *si = surv_id + srow;
    int32_t *out = (j == 0 && k > 0) ? ids + (g * n_q + i) * k : nullptr;
    float *sout = (j == 0 && k > 0 && scores) ? scores + (g * n_q + i) * k : nullptr;
    auto emit = [&](int r, int id, float sc) __attribute__((always_inline)) {
        if (id >= 0) sh.list[ns + r] = id;
        if (out) out[r] = id;
        if (sout) sout[r] = sc;
    };
    const int n_surv = nb * k;
    if (k > 0 && nb > 1 && n_surv <= 4 * 64) {
        // up to 256 survivors: keys and ids to LDS by all threads at once,
        // then wave 0 selects among them
        if (tid < n_surv) {
            cand_key[tid] = sk[tid];
            cand_id[tid] = si[tid];
        }
        __syncthreads();
    } else if (k > 0 && nb > 1) {
        const int per = (n_surv + kFusedSelWaves - 1) / kFusedSelWaves;   // <= NI * 64
        const int lo = min(n_surv, wave * per);
        const int hi = min(n_surv, lo + per);
        auto id_lo = [&](int c) __attribute__((always_inline)) { return si[lo + c]; };
        auto keep = [&](int r, int id, float sc) __attribute__((always_inline)) {
            cand_key[wave * k + r] = id >= 0 ? score_key(sc) : 0u;
            cand_id[wave * k + r] = id;
        };
        select_top_k_reg<NI>(sk + lo, hi - lo, k, id_lo, keep);
        __syncthreads();
    }
    if (wave == 0) {
        write_sink_units(sh.list, ns);
        int n_sel = 0;
        if (k > 0 && nb == 1) {                 // the block's survivors are the answer
            for (int r0 = 0; r0 < k; r0 += 64) {
                const int r = r0 + lane;
                const int id = r < k ? si[r] : -1;
                if (r < k) emit(r, id, id >= 0 ? key_to_score(sk[r]) : -INFINITY);
                n_sel += __popcll(__ballot(id >= 0));
            }
        } else if (k > 0 && nb > 1) {
            auto from_cand = [&](int c) __attribute__((always_inline)) { return cand_id[c]; };
            if (n_surv <= 4 * 64) n_sel = select_top_k_reg<4>(cand_key, n_surv, k, from_cand, emit);
            else if (k <= 64) n_sel = select_top_k_reg<4>(cand_key, kFusedSelWaves * k, k, from_cand, emit);
            else n_sel = select_top_k_reg<16>(cand_key, kFusedSelWaves * k, k, from_cand, emit);
        } else if (k > 0) {                     // no candidates: an empty row
            for (int r = lane; r < k; r += 64) emit(r, -1, -INFINITY);
        }
        if (lane == 0) {
            sh.list[ns + n_sel] = (int)(Pc / kC);
            sh.list_n = ns + n_sel + 1;
        }
    }
    load_q_rows<G>(Q, n_q, g, i, sh);
    __syncthreads();
    split_partial<G>(K, V, T_cap, g, p, j, scale_log2, sh,
                     split_part(part, Hkv, G, n_split, i, g, j));
}

template <int G>
hipError_t launch_route_decode_g(const uint16_t *Q, int64_t Hkv, int64_t p0, int64_t n_q,
                                 const float *S, int64_t n_cap, int32_t k, int32_t sink,
                                 int32_t *ids, float *scores, uint32_t *keys,
                                 hipStream_t stream)
{
    const int64_t kcap = decode_key_capacity(p0, n_q, sink);
    if (n_q > 65535) return hipErrorInvalidConfiguration;      // grid y / z limit
    if (kcap > 0) {
        const int n_blk = (int)((kcap + kScoreBlock - 1) / kScoreBlock);
        hipLaunchKernelGGL((decode_score_kernel<G>),
                           dim3((unsigned)Hkv, (unsigned)n_blk, (unsigned)n_q),
                           dim3(kRouteThreads), 0, stream, Q, n_q, Hkv, p0, S, n_cap,
                           (int)sink, n_blk, kcap, keys);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)Hkv, (unsigned)n_q), block(kSelWaves * 64);
#define HGA_SELECT_DEC(NI)                                                                  \
    hipLaunchKernelGGL((decode_select_kernel<NI>), grid, block, 0, stream, n_q, Hkv, p0, k,  \
                       (int)sink, kcap, keys, ids, scores)
    // each wave's share of the most candidates any token has
    const int64_t per = (kcap + kSelWaves - 1) / kSelWaves;
    if (per <= 4 * 64) HGA_SELECT_DEC(4);
    else if (per <= 8 * 64) HGA_SELECT_DEC(8);
    else if (per <= 16 * 64) HGA_SELECT_DEC(16);
    else if (per <= 32 * 64) HGA_SELECT_DEC(32);
    else HGA_SELECT_DEC(48);
#undef HGA_SELECT_DEC
    return hipGetLastError();
}

template <int G>
hipError_t launch_attend_decode_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                  int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                                  const int32_t *ids,
                                  int32_t k, int32_t sink, float scale, uint16_t *O,
                                  float *lse, float *part, hipStream_t stream)
{
    const int n_split = decode_splits(k, sink);
    if (n_q > 65535) return hipErrorInvalidConfiguration;      // grid y / z limit
    hipLaunchKernelGGL((decode_partial_kernel<G>),
                       dim3((unsigned)Hkv, (unsigned)n_split, (unsigned)n_q),
                       dim3(kDecThreads), 0, stream, Q, K, V, n_q, Hkv, T_cap, p0, ids, k,
                       (int)sink, scale * 1.44269504088896340736f, n_split, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<G>), dim3((unsigned)(Hkv * G), (unsigned)n_q),
                       dim3(kD), 0, stream, part, n_q, Hkv, n_split, O, lse);
    return hipGetLastError();
}

// Workspace of the fused step, in order: the survivor keys and chunk ids
// [n_q][Hkv][n_blk][k], the split partials [n_q][Hkv][n_split][G][kPartFloats];
// each part 256-B aligned. ni: registers per lane of the large survivor selection (0: more
// survivors than the fused kernel takes).
struct FusedDecodeLayout {
    int n_blk, n_split, ni;
    size_t key_off, id_off, part_off, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FusedDecodeLayout fused_decode_layout(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q,
                                      int32_t k, int32_t sink)
{
    FusedDecodeLayout L;
    const int64_t kcap = decode_key_capacity(p0, n_q, sink);
    L.n_blk = (int)std::max<int64_t>(1, (kcap + kScoreBlock - 1) / kScoreBlock);
    L.n_split = (sink + k + 1 + kDecTiles - 1) / kDecTiles;
    const int64_t n_surv = (int64_t)L.n_blk * k;
    const int64_t per = (n_surv + kFusedSelWaves - 1) / kFusedSelWaves;
    L.ni = n_surv <= 4 * 64 ? 4 : per <= 4 * 64 ? 4 : per <= 16 * 64 ? 16 : per <= 48 * 64 ? 48 : 0;
    const size_t rows = (size_t)n_q * (size_t)Hkv;
    L.key_off = 0;
    L.id_off = L.key_off + align256(rows * (size_t)n_surv * sizeof(uint32_t));
    L.part_off = L.id_off + align256(rows * (size_t)n_surv * sizeof(int32_t));
    L.bytes = L.part_off + (size_t)n_q * (size_t)Hq * (size_t)L.n_split * kPartFloats *
                               sizeof(float);
    return L;
}

template <int G>
hipError_t launch_route_attend_decode_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                        int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                                        const float *S, int64_t n_cap, int32_t k, int32_t sink,
                                        float scale, int32_t *ids, float *scores, uint16_t *O,
                                        float *lse, void *workspace, hipStream_t stream)
{
    const FusedDecodeLayout L = fused_decode_layout(Hkv * G, Hkv, p0, n_q, k, sink);
    if (n_q > 65535 || L.ni == 0) return hipErrorInvalidConfiguration;
    uint8_t *ws = (uint8_t *)workspace;
    uint32_t *surv_key = (uint32_t *)(ws + L.key_off);
    int32_t *surv_id = (int32_t *)(ws + L.id_off);
    float *part = (float *)(ws + L.part_off);
    hipLaunchKernelGGL((decode_route_part_kernel<G>),
                       dim3((unsigned)Hkv, (unsigned)L.n_blk, (unsigned)n_q),
                       dim3(kRouteThreads), 0, stream, Q, n_q, Hkv, p0, S, n_cap, (int)k,
                       (int)sink, L.n_blk, surv_key, surv_id);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)Hkv, (unsigned)L.n_split, (unsigned)n_q), block(kDecThreads);
    const float sl2 = scale * 1.44269504088896340736f;
#define HGA_FUSED_DEC(NI)                                                                    \
    hipLaunchKernelGGL((decode_fused_attend_kernel<G, NI>), grid, block, 0, stream, Q, K, V,  \
                       n_q, Hkv, T_cap, p0, (int)k, (int)sink, sl2, L.n_split, L.n_blk,      \
                       surv_key, surv_id, ids, scores, part)
    if (L.ni == 4) HGA_FUSED_DEC(4);
    else if (L.ni == 16) HGA_FUSED_DEC(16);
    else HGA_FUSED_DEC(48);
#undef HGA_FUSED_DEC
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<G>), dim3((unsigned)(Hkv * G), (unsigned)n_q),
                       dim3(kD), 0, stream, part, n_q, Hkv, L.n_split, O, lse);
    return hipGetLastError();
}

}  // namespace

int decode_splits(int32_t k, int32_t sink)
{
    return (sink + k + 1 + kDecTiles - 1) / kDecTiles;
}

int64_t decode_key_capacity(int64_t p0, int64_t n_q, int32_t sink)
{
    if (n_q <= 0) return 0;
    const int64_t c = (p0 + n_q - 1) / kC - sink;   // the last token has the most candidates
    return c > 0 ? c : 0;
}

size_t decode_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q, int32_t k,
                              int32_t sink)
{
    // the router's keys and the attention's partials are used one call after
    // the other: one buffer serves both
    const size_t keys = (size_t)n_q * (size_t)Hkv * (size_t)decode_key_capacity(p0, n_q, sink) *
                        sizeof(uint32_t);
    const size_t parts = (size_t)n_q * (size_t)Hq * (size_t)decode_splits(k, sink) *
                         kPartFloats * sizeof(float);
    return keys > parts ? keys : parts;
}

size_t route_attend_decode_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q,
                                           int32_t k, int32_t sink)
{
    return fused_decode_layout(Hq, Hkv, p0, n_q, k, sink).bytes;
}

bool route_attend_decode_fits(int64_t Hq, int64_t Hkv, int64_t p0, int64_t n_q, int32_t k,
                              int32_t sink)
{
    return fused_decode_layout(Hq, Hkv, p0, n_q, k, sink).ni != 0;
}

hipError_t launch_route_attend_decode(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                      int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                      int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                                      int32_t sink, float scale, int32_t *ids, float *scores,
                                      uint16_t *O, float *lse, void *workspace,
                                      hipStream_t stream)
{
    if (n_q == 0) return hipSuccess;
    switch (Hq / Hkv) {
    case 1: return launch_route_attend_decode_g<1>(Q, K, V, Hkv, T_cap, p0, n_q, S, n_cap, k, sink, scale, ids, scores, O, lse, workspace, stream);
    case 2: return launch_route_attend_decode_g<2>(Q, K, V, Hkv, T_cap, p0, n_q, S, n_cap, k, sink, scale, ids, scores, O, lse, workspace, stream);
    case 4: return launch_route_attend_decode_g<4>(Q, K, V, Hkv, T_cap, p0, n_q, S, n_cap, k, sink, scale, ids, scores, O, lse, workspace, stream);
    case 8: return launch_route_attend_decode_g<8>(Q, K, V, Hkv, T_cap, p0, n_q, S, n_cap, k, sink, scale, ids, scores, O, lse, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_route_decode(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                               int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                               int32_t sink, int32_t *ids, float *scores, void *workspace,
                               hipStream_t stream)
{
    if (n_q == 0 || k == 0) return hipSuccess;
    uint32_t *keys = (uint32_t *)workspace;
    switch (Hq / Hkv) {
    case 1: return launch_route_decode_g<1>(Q, Hkv, p0, n_q, S, n_cap, k, sink, ids, scores, keys, stream);
    case 2: return launch_route_decode_g<2>(Q, Hkv, p0, n_q, S, n_cap, k, sink, ids, scores, keys, stream);
    case 4: return launch_route_decode_g<4>(Q, Hkv, p0, n_q, S, n_cap, k, sink, ids, scores, keys, stream);
    case 8: return launch_route_decode_g<8>(Q, Hkv, p0, n_q, S, n_cap, k, sink, ids, scores, keys, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attend_decode(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                int64_t n_q, const int32_t *ids, int32_t k, int32_t sink,
                                float scale, uint16_t *O, float *lse, void *workspace,
                                hipStream_t stream)
{
    if (n_q == 0) return hipSuccess;
    float *part = (float *)workspace;
    switch (Hq / Hkv) {
    case 1: return launch_attend_decode_g<1>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, sink, scale, O, lse, part, stream);
    case 2: return launch_attend_decode_g<2>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, sink, scale, O, lse, part, stream);
    case 4: return launch_attend_decode_g<4>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, sink, scale, O, lse, part, stream);
    case 8: return launch_attend_decode_g<8>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, sink, scale, O, lse, part, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hga
