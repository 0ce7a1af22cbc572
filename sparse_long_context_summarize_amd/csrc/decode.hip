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
// At batch 1 the step reads (k + sink + 1) K/V tiles of 32 KiB per (token, kv
// head) once: HBM bound, so the split spreads those reads over many CUs.
#include "route_core.h"

namespace hga {
namespace {

constexpr int kScoreBlock = 256;            // candidates per scoring workgroup

// Candidates of token p: chunks s .. Pc/C - 1 (none if the sink covers them).
__device__ __forceinline__ int decode_candidates(int64_t p, int sink)
{
    return (int)max((int64_t)0, p / kC - sink);
}

// Workgroup (token i, kv head g, block blk): candidates blk*256 .. +256.
template <int G>
__global__ __launch_bounds__(kRouteThreads) void decode_score_kernel(
    const uint16_t *__restrict__ Q, int64_t n_q, int64_t Hkv, int64_t p0,
    const float *__restrict__ S, int64_t n_cap, int sink, int n_blk, int64_t kcap,
    uint32_t *__restrict__ keys)
{
    __shared__ float qbar[kD];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_blk, n_q)
    const int blk = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int nE = decode_candidates(p0 + i, sink);
    const int c0 = blk * kScoreBlock;
    if (c0 >= nE) return;                       // uniform across the workgroup

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
    uint32_t *kout = keys + (i * Hkv + g) * kcap;
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
        if (sdseg == 0 && c < nE) kout[c] = score_key(sc);
    }
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

// Workgroup (token i, kv head g, split j): tiles j*kDecTiles .. +kDecTiles of
// the token's list [sink chunks, routed chunks, open chunk]. Wave w serves
// heads w, w + 4 (G = 8) of the group; lane l holds key l of a tile for the
// scores and output dims 2l, 2l + 1 for P.V.
template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv, int64_t T_cap, int64_t p0,
    const int32_t *__restrict__ ids, int k, int sink, float scale_log2, int n_split,
    float *__restrict__ part)
{
    constexpr int HPW = G > 4 ? 2 : 1;          // heads per wave
    __shared__ int list[kChunkListMax];
    __shared__ int list_n;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kDecTiles][kC * kDecStride];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kDecTiles][kC * kDecStride];
    __shared__ float qs[G][kD];
    __shared__ float ps[4][HPW][kC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t g = blockIdx.x;                   // grid (Hkv, n_split, n_q)
    const int j = (int)blockIdx.y;
    const int64_t i = blockIdx.z;
    const int64_t p = p0 + i;
    const int64_t Pc = kC * (p / kC);           // start of the open chunk
    if (wave == 0) {
        const int ns = sink_units(sink, Pc, kC);
        write_sink_units(list, ns);
        const int n = build_unit_list(ids + (g * n_q + i) * k, k, sink, Pc / kC, list + ns);
        if (lane == 0) {
            list[ns + n] = (int)(Pc / kC);
            list_n = ns + n + 1;
        }
    }
    for (int e = tid; e < G * kD; e += kDecThreads) {
        const uint16_t b = Q[((g * G + e / kD) * n_q + i) * kD + e % kD];
        qs[e / kD][e % kD] = __uint_as_float((uint32_t)b << 16);
    }
    __syncthreads();
    const int n_tiles = list_n;
    const int t0 = j * kDecTiles;
    const int my_tiles = max(0, min(kDecTiles, n_tiles - t0));

    // All of this workgroup's K and V rows are loaded at once: thread t moves
    // rows t/16 + 16*r, d = 8*(t%16) .. +8; rows of the open chunk past p are
    // written as zeros (their scores are masked, and zeros keep P.V finite).
    const uint16_t *Kg = K + g * T_cap * kD;
    const uint16_t *Vg = V + g * T_cap * kD;
    for (int u = 0; u < my_tiles; ++u) {
        const int t = t0 + u;
        const int64_t c = list[t];
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
            *(u32x4 *)(&Ks[u][row * kDecStride + (tid & 15) * 8]) = kv;
            *(u32x4 *)(&Vs[u][row * kDecStride + (tid & 15) * 8]) = vv;
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
        const uint16_t *kr = &Ks[u][lane * kDecStride];
#pragma unroll
        for (int e = 0; e < HPW; ++e) {
            const int h = wave + 4 * e;
            float z = 0.f;
#pragma unroll 4
            for (int d = 0; d < kD; d += 8) {
                const u32x4 w = *(const u32x4 *)(kr + d);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    z = fmaf(qs[h][d + 2 * q], bf16_lo(w[q]), z);
                    z = fmaf(qs[h][d + 2 * q + 1], bf16_hi(w[q]), z);
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
            ps[wave][e][lane] = pz;
            o0[e] *= alpha;
            o1[e] *= alpha;
        }
        // (a wave reads only the probabilities it wrote: no barrier needed)
        __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
        for (int e = 0; e < HPW; ++e) {
            const uint16_t *vc = &Vs[u][2 * lane];
            float a0 = 0.f, a1 = 0.f;
            for (int key = 0; key < kC; ++key) {
                const float pk = ps[wave][e][key];
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
        float *dst = part + ((((i * Hkv + g) * n_split + j) * G) + h) * kPartFloats;
        if (lane == 0) {
            dst[0] = m_run[e];
            dst[1] = l_run[e];
        }
        dst[2 + 2 * lane] = o0[e];
        dst[3 + 2 * lane] = o1[e];
    }
}

// One workgroup of kD threads per (token, query head): the splits' partials
// merged in split order (every split's max and sum loaded at once first).
constexpr int kMaxSplits = (kMaxSink + kMaxTopK + 1 + kDecTiles - 1) / kDecTiles;

template <int G>
__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float *__restrict__ part, int64_t n_q, int64_t Hkv, int n_split,
    uint16_t *__restrict__ O, float *__restrict__ lse)
{
    __shared__ float ms[kMaxSplits], ws[kMaxSplits];
    __shared__ float M_s, L_s;
    const int d = threadIdx.x;
    const int64_t h = blockIdx.x;                   // grid (Hkv * G, n_q)
    const int64_t i = blockIdx.y;
    const int64_t g = h / G, hh = h % G;
    const float *base = part + ((i * Hkv + g) * n_split * G + hh) * kPartFloats;
    const int64_t step = (int64_t)G * kPartFloats;
    for (int j = d; j < n_split; j += kD) {
        ms[j] = base[j * step];
        ws[j] = base[j * step + 1];
    }
    __syncthreads();
    if (d == 0) {
        float M = -INFINITY;
        for (int j = 0; j < n_split; ++j) M = fmaxf(M, ms[j]);
        float L = 0.f;
        for (int j = 0; j < n_split; ++j) {
            const float w = __builtin_amdgcn_exp2f(ms[j] - M);   // 0 for an empty split
            L = fmaf(ws[j], w, L);
            ms[j] = w;
        }
        M_s = M;
        L_s = L;
    }
    __syncthreads();
    float acc = 0.f;
#pragma unroll 8
    for (int j = 0; j < n_split; ++j) acc = fmaf(base[j * step + 2 + d], ms[j], acc);
    O[(h * n_q + i) * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)(acc / L_s));
    if (d == 0) lse[h * n_q + i] = (M_s + __log2f(L_s)) * 0.69314718055994530942f;
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
