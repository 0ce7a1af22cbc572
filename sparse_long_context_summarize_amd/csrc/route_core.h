// route_core.h -- the router's device code, shared by the routing kernel
// (route.hip) and the attention kernel's fused routing prologue
// (attend_fwd.hip), so both choose bit-identical ids and scores (arXiv
// 2607.15105, gist.science technical summary 2.1: the current query block
// scores the resident chunk summaries and keeps the most relevant earlier
// chunks).
//
//   1. qbar = mean of the block's G*64 query rows (fp32, LDS reduction); the
//      first batch of summary rows is loaded together with the query rows
//      (or, when the caller holds the rows in LDS, right after their sums);
//   2. score_c = qbar . S[g][c] for every candidate c: 16 lanes per chunk
//      read one 512-byte summary row with coalesced 16-byte loads, each lane
//      holding its 8-wide slice of qbar in registers; the 16 partial sums are
//      folded with four DPP row adds. Scores become order-preserving uint32
//      keys in LDS;
//   3. top-k by (score desc, id asc), for up to 2048 candidates: one wave
//      holds every key in registers (NI per lane, candidate it*64 + lane); the
//      k-th largest key is found one bit at a time from ballot/popcount counts
//      -- no barrier, no memory traffic per bit, and done as soon as exactly k
//      keys reach the threshold being built -- ties at that key go to the
//      lowest ids, and the chosen ids come out ascending from a ballot + mbcnt
//      compaction, so no sort is needed. Larger candidate sets take a
//      two-stage selection over the keys in LDS (every wave over its id range,
//      then wave 0 over the survivors).
#pragma once
#include "hga_internal.h"

#include <type_traits>

namespace hga {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxRegKeys = 32;             // keys per lane of the register selection (2048)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Max / min over the wave: within each 16-lane row by DPP (quad swaps, then
// mirrors within 8 and 16 lanes), then across row pairs and half-waves with
// the gfx950 lane-swap instructions. Every lane receives the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, dpp_u32<0xB1>(x));
    x = max(x, dpp_u32<0x4E>(x));
    x = max(x, dpp_u32<0x141>(x));
    x = max(x, dpp_u32<0x140>(x));
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)r[0], (uint32_t)r[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)q[0], (uint32_t)q[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    x = min(x, dpp_u32<0xB1>(x));
    x = min(x, dpp_u32<0x4E>(x));
    x = min(x, dpp_u32<0x141>(x));
    x = min(x, dpp_u32<0x140>(x));
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = min((uint32_t)r[0], (uint32_t)r[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return min((uint32_t)q[0], (uint32_t)q[1]);
}

// Sum over each 16-lane row, result in every lane of the row: quad swaps
// (lane ^ 1, lane ^ 2), then mirrors within 8 and within 16 lanes (DPP).
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// The selection threshold: the largest T with #{key >= T} >= k, given the
// largest and smallest key (mx, mn) and count_ge(x) = #{key >= x} over the
// candidates (n > k >= 1 of them). Bits above the highest bit in which the
// keys differ are shared by every key; below it T is built one bit at a
// time, and the search stops as soon as exactly k keys reach the candidate
// threshold (they are then the k largest, and no lower bit can change which
// keys are taken). When every key is equal, T is that key. The chosen set is
// then every key > T plus the lowest-positioned keys == T, k in all. Host and
// device code: the CPU tests run this very function.
struct SameInt {
    __host__ __device__ int operator()(int v) const { return v; }
};
// uniform(bit) marks the bit index as the same in every lane: the device
// callers pass readfirstlane, which keeps the whole step -- candidate, ballot
// counts, update -- on the scalar unit instead of crossing to vector
// registers and back every step.
template <typename CountGe, typename Uniform = SameInt>
__host__ __device__ __forceinline__ uint32_t select_threshold(uint32_t mx, uint32_t mn, int k,
                                                              CountGe count_ge,
                                                              Uniform uniform = Uniform{})
{
    const uint32_t diff = mx ^ mn;
    if (diff == 0u) return mx;
    const int top = 31 - __builtin_clz(diff);
    uint32_t T = (top == 31) ? 0u : (mx & ~((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
        bit = uniform(bit);
        const uint32_t cand = T | (1u << bit);
        const int cnt = count_ge(cand);
        if (cnt >= k) T = cand;
        if (cnt == k) break;
    }
    return T;
}

// Wave-level selection of the k largest keys[0..n) (ties: lower position
// first). Writes the chosen positions, ascending, to out_pos (LDS) and
// returns their number, min(k, n). Every lane of the wave must call it.
__device__ __forceinline__ int wave_select(const uint32_t *keys, int n, int k, int *out_pos)
{
    const int lane = threadIdx.x & 63;
    if (n <= k) {
        for (int base = 0; base < n; base += 64)
            if (base + lane < n) out_pos[base + lane] = base + lane;
        return n;
    }
    uint32_t mx = 0u, mn = 0xFFFFFFFFu;
    for (int base = 0; base < n; base += 64) {
        const int p = base + lane;
        if (p < n) { const uint32_t x = keys[p]; mx = max(mx, x); mn = min(mn, x); }
    }
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    const uint32_t T = select_threshold(mx, mn, k, [&](uint32_t cand) __attribute__((always_inline)) {
        int cnt = 0;
        for (int base = 0; base < n; base += 64) {
            const int p = base + lane;
            cnt += __popcll(__ballot(p < n && keys[p] >= cand));
        }
        return cnt;
    }, [](int v) { return __builtin_amdgcn_readfirstlane(v); });
    int n_gt = 0;
    for (int base = 0; base < n; base += 64) {
        const int p = base + lane;
        n_gt += __popcll(__ballot(p < n && keys[p] > T));
    }
    const int need = k - n_gt;   // equal keys to take, lowest positions first
    int eq_seen = 0, out = 0;
    for (int base = 0; base < n; base += 64) {
        const int p = base + lane;
        const uint32_t x = (p < n) ? keys[p] : 0u;
        const bool eq = (p < n) && x == T;
        const uint64_t em = __ballot(eq);
        const bool take = (p < n && x > T) || (eq && eq_seen + lanes_below(em) < need);
        eq_seen += __popcll(em);
        const uint64_t sm = __ballot(take);
        // (exactly k keys are taken; the bound only guards out_pos's size)
        if (take && out + lanes_below(sm) < k) out_pos[out + lanes_below(sm)] = p;
        out = min(k, out + __popcll(sm));
    }
    return out;
}

__device__ __forceinline__ float key_to_score(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Max and min over the wave, the two reductions interleaved (independent
// chains hide each other's DPP wait states); every lane receives both.
__device__ __forceinline__ void wave_max_min_u32(uint32_t &mx, uint32_t &mn) {
    mx = max(mx, dpp_u32<0xB1>(mx)); mn = min(mn, dpp_u32<0xB1>(mn));
    mx = max(mx, dpp_u32<0x4E>(mx)); mn = min(mn, dpp_u32<0x4E>(mn));
    mx = max(mx, dpp_u32<0x141>(mx)); mn = min(mn, dpp_u32<0x141>(mn));
    mx = max(mx, dpp_u32<0x140>(mx)); mn = min(mn, dpp_u32<0x140>(mn));
    const auto r = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
    const auto r2 = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
    mx = max((uint32_t)r[0], (uint32_t)r[1]);
    mn = min((uint32_t)r2[0], (uint32_t)r2[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    const auto q2 = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
    mx = max((uint32_t)q[0], (uint32_t)q[1]);
    mn = min((uint32_t)q2[0], (uint32_t)q2[1]);
}

// Wave-level top-k of keys[0..nE) (LDS), nE <= NI*64, by (key desc, candidate
// index asc): one wave holds every key in registers (candidate c = it*64 +
// lane), finds the selection threshold bit by bit from ballot counts (stopping
// as soon as exactly k keys reach the threshold being built), takes ties at
// that key from the lowest candidates, and passes id_of(c) of the chosen
// candidates in ascending candidate order (ballot + mbcnt compaction) with
// their scores to emit(r, id, score), then (r, -1, -inf) up to k; returns the
// number chosen. Empty slots
// hold key 0, below every finite score's key (>= 0x00800000) and every
// threshold tried (>= 1), so no test needs a bounds check. Every lane of the
// wave must call it.
template <int NI, typename IdOf, typename Emit>
__device__ __forceinline__ int select_top_k_reg(const uint32_t *keys, int nE, int k,
                                                IdOf id_of, Emit emit)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int c = it * 64 + lane;
        key[it] = (c < nE) ? keys[c] : 0u;
    }
    int n_sel;
    if (nE <= k) {
        n_sel = nE;
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            const int c = it * 64 + lane;
            if (c < nE) emit(c, id_of(c), key_to_score(key[it]));
        }
    } else {
        uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            mx = max(mx, key[it]);
            mn = min(mn, key[it] ? key[it] : 0xFFFFFFFFu);
        }
        wave_max_min_u32(mx, mn);
        // (every lane holds the same max and min: readfirstlane lets the
        // threshold search run in scalar registers)
        mx = (uint32_t)__builtin_amdgcn_readfirstlane((int)mx);
        mn = (uint32_t)__builtin_amdgcn_readfirstlane((int)mn);
        const uint32_t T = select_threshold(mx, mn, k, [&](uint32_t cand) __attribute__((always_inline)) {
            int cnt = 0;
#pragma unroll
            for (int it = 0; it < NI; ++it) cnt += __popcll(__ballot(key[it] >= cand));
            return cnt;
        }, [](int v) { return __builtin_amdgcn_readfirstlane(v); });
        int n_gt = 0;
#pragma unroll
        for (int it = 0; it < NI; ++it) n_gt += __popcll(__ballot(key[it] > T));
        const int need = k - n_gt;          // equal keys to take, lowest candidates first
        int eq_seen = 0, pos = 0;
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            const bool eq = key[it] == T;
            const uint64_t em = __ballot(eq);
            const bool take = key[it] > T || (eq && eq_seen + lanes_below(em) < need);
            eq_seen += __popcll(em);
            const uint64_t sm = __ballot(take);
            if (take) emit(pos + lanes_below(sm), id_of(it * 64 + lane), key_to_score(key[it]));
            pos += __popcll(sm);
        }
        n_sel = pos;
    }
    for (int r = n_sel + lane; r < k; r += 64) emit(r, -1, -INFINITY);
    return n_sel;
}


// The distinct valid chunks (lo <= c < limit) of a chunk row, ascending,
// into chl; returns their number. A router-made row (ascending, distinct)
// passes one neighbour check; any other row has its repeats dropped (first
// kept) and is rank-sorted through tmp (k entries). One wave calls it.
__device__ __forceinline__ int sorted_chunk_set(const int32_t *row, int k, int64_t lo,
                                                int64_t limit, int *chl, int *tmp)
{
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int base = 0; base < k; base += 64) {
        const int r = base + lane;
        const int c = (r < k) ? row[r] : -1;
        const bool ok = (int64_t)c >= lo && (int64_t)c < limit;
        const uint64_t m = __ballot(ok);
        if (ok) chl[cnt + lanes_below(m)] = c;
        cnt += __popcll(m);
    }
    bool unsorted = false;
    for (int i = 1 + lane; i < cnt; i += 64) unsorted |= chl[i] <= chl[i - 1];
    if (__ballot(unsorted) == 0) return cnt;
    int n = 0;
    for (int base = 0; base < cnt; base += 64) {
        const int i = base + lane;
        const int c = (i < cnt) ? chl[i] : -1;
        bool keep = i < cnt;
        for (int j = 0; j < base + 64 && j < cnt; ++j)
            if (j < i && chl[j] == c) keep = false;
        const uint64_t m = __ballot(keep);
        if (keep) tmp[n + lanes_below(m)] = c;
        n += __popcll(m);
    }
    for (int i = lane; i < n; i += 64) {
        const int v = tmp[i];
        int r = 0;
        for (int j = 0; j < n; ++j) r += tmp[j] < v;
        chl[r] = v;
    }
    return n;
}

// No extra work (route_block's default hook).
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// LDS the router uses besides the candidate keys.
struct RouteLds {
    float part[16][kD];
    float qbar[kD];
    int surv[kRouteWaves][kMaxTopK];
    int surv_n[kRouteWaves];
    uint32_t cand_key[kRouteWaves * kMaxTopK];
    int cand_pos[kRouteWaves * kMaxTopK];
    int chosen[kMaxTopK];
    int chl[kMaxTopK];
    int n_ch;
};

// The router for query block b of kv head g, run by the first kRouteThreads
// threads of a workgroup; any further threads only take part in its
// barriers, which every thread of the workgroup must reach. keys holds one
// uint32 per candidate (and kc entries for kGroups). The chosen ids reach
// emit(r, id, score) in ascending order, then (r, -1, -inf) up to k; the
// return value (their number) is meaningful in wave 0.
//
// kGroups = false: chunk routing, candidates every chunk c with c_lo <= c <
// P/C (c_lo = the sink window's chunk count), rows of S.
// kGroups = true: group routing (second level), candidates the 8 groups of
// each distinct valid chunk (c_lo <= c < P/C) of chunk_row (the block's kc
// chunk ids, in global memory or LDS), in ascending group order, rows of the
// group summaries S; k is then the group budget.
// kBatch: summary rows per lane in flight; kScoreWaves: waves that score
// (the first kScoreWaves of the workgroup). Both only distribute the
// candidates over lanes: each score's arithmetic, and so every score, is the
// same whichever lanes compute it.
// q_row(r, dseg): the 8 bf16 of query row r (0 .. G*kBq-1: head g*G +
// r/kBq, query r%kBq of the block) at d = 8*dseg .. +8, from wherever the
// caller holds them (the values, not their source, fix the result).
// kBq = 64: query blocks of 64 starting at p0 + 64*b. kBq = 1 (decode): block
// b is the single token at p0 + b, and its candidates end at the start of its
// own open chunk, P = 64*floor((p0 + b)/64).
template <int G, int NI, bool kGroups, int kBatch, int kScoreWaves, typename QRow,
          typename Emit, int kBq = kC, typename Hook = NoHook, typename QLocal = std::false_type>
__device__ __forceinline__ int route_block(
    RouteLds &sh, uint32_t *keys, QRow q_row, int64_t n_q, int64_t g,
    int64_t b, int64_t p0, const float *__restrict__ S, int64_t n_cap, int k,
    const int32_t *chunk_row, int kc, int c_lo, Emit emit,
    Hook after_loads = Hook{}, QLocal = QLocal{})
{
    // q_row reads LDS (QLocal true): the query-row sums come first and the
    // summary rows are loaded after them; reading memory, both loads go out
    // first so that their round trips overlap.
    constexpr bool kQLocal = QLocal::value;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // (uniform across the wave: readfirstlane lets every wave-level branch
    // below, and the selection inside them, run on scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool act = wave < kRouteWaves;
    const int64_t P = kBq == kC ? p0 + b * kC : kC * ((p0 + b) / kC);
    int *chl = sh.chl;
    int nE = (int)max((int64_t)0, P / kC - c_lo);
    if (kGroups) {
        // 0. the block's distinct valid routed chunks, ascending
        if (wave == 0) {
            const int n = sorted_chunk_set(chunk_row, kc, c_lo, P / kC, chl, (int *)keys);
            if (lane == 0) sh.n_ch = n;
        }
        __syncthreads();
        nE = (kC / kGroup) * sh.n_ch;
    }
    // summary row of candidate c (its chunk, or its group)
    auto row_of = [&](int c) __attribute__((always_inline)) {
        return kGroups ? chl[c >> 3] * (kC / kGroup) + (c & 7) : c + c_lo;
    };

    // Every load that does not depend on qbar is issued first: all of this
    // thread's query rows and the first batch of summary rows, so the two
    // memory round trips overlap.
    constexpr int kStride = kScoreWaves * 4 * kBatch;     // chunks per batch
    const bool scorer = wave < kScoreWaves;
    const int sdseg = lane & 15, sub = lane >> 4;
    const float *Sg = S + g * n_cap * kD + sdseg * 8;
    f32x4 slo[kBatch], shi[kBatch];
    auto load_batch = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            // past the end: re-read the last row (in bounds, result unused)
            const int c = row_of(min(base + u * kScoreWaves * 4 + sub, nE - 1));
            slo[u] = *(const f32x4 *)(Sg + (int64_t)c * kD);
            shi[u] = *(const f32x4 *)(Sg + (int64_t)c * kD + 4);
        }
    };

    // 1. qbar over the G heads x 64 queries of this block: thread (r0, dseg)
    // sums rows r0, r0 + 16, ... at d = 8*dseg .. +8.
    if (act) {
        const int dseg = tid & 15, r0 = tid >> 4;
        constexpr int kRows = G * kBq, kPer = (kRows + 15) / 16;
        u32x4 w[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            if constexpr (kRows % 16 == 0) {
                w[m] = q_row(r0 + 16 * m, dseg);
            } else {
                const u32x4 z = {0u, 0u, 0u, 0u};   // bf16 zeros
                w[m] = (r0 + 16 * m < kRows) ? q_row(r0 + 16 * m, dseg) : z;
            }
        }
        // (clamped: waves past the end re-read the last row)
        if (!kQLocal && nE > 0) load_batch(wave * 4);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo(w[m][q]);
                acc[2 * q + 1] += bf16_hi(w[m][q]);
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) sh.part[r0][dseg * 8 + e] = acc[e];
        if (kQLocal && nE > 0) load_batch(wave * 4);
    } else if (scorer) {
        if (nE > 0) load_batch(wave * 4);       // (clamped: waves past the end re-read the last row)
    }
    after_loads();      // the caller's own loads, issued behind the summary rows
    __syncthreads();
    if (tid < kD) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += sh.part[r][tid];
        sh.qbar[tid] = s * (1.0f / (float)(G * kBq));  // a power of two: exact
    }
    __syncthreads();

    // 2. scores -> keys. Each wave scores 4 chunks per step (16 lanes per
    // chunk, each holding its 8-wide slice of qbar), kBatch steps per batch.
    if (scorer) {
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = sh.qbar[sdseg * 8 + e];
        for (int base = wave * 4; base < nE; base += kStride) {
            if (base != wave * 4) load_batch(base);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                float s = qv[0] * slo[u][0];
                s = fmaf(qv[1], slo[u][1], s);
                s = fmaf(qv[2], slo[u][2], s);
                s = fmaf(qv[3], slo[u][3], s);
                s = fmaf(qv[4], shi[u][0], s);
                s = fmaf(qv[5], shi[u][1], s);
                s = fmaf(qv[6], shi[u][2], s);
                s = fmaf(qv[7], shi[u][3], s);
                s = row16_sum(s);
                const int c = base + u * kScoreWaves * 4 + sub;
                if (sdseg == 0 && c < nE) keys[c] = score_key(s);
            }
        }
    }
    __syncthreads();

    if (kGroups || NI * 64 >= nE) {
        // 3. one wave, keys in registers (group routing never has more than
        // 8 * kMaxTopK = NI * 64 candidates)
        if (wave != 0) return 0;
        return select_top_k_reg<NI>(keys, nE, k, row_of, emit);
    }

    // 3'. more than 2048 candidates: each wave selects over its contiguous id
    // range (keys in LDS), then wave 0 selects among the survivors.
    const int per = (nE + kRouteWaves - 1) / kRouteWaves;
    if (act) {
        const int lo = min(nE, wave * per);
        const int hi = min(nE, lo + per);
        const int got = wave_select(keys + lo, hi - lo, k, sh.surv[wave]);
        if (lane == 0) sh.surv_n[wave] = got;
    }
    __syncthreads();
    if (wave != 0) return 0;
    int m = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
        const int cnt = sh.surv_n[w];
        const int off = min(nE, w * per);
        for (int j = lane; j < cnt; j += 64) {
            const int pos = off + sh.surv[w][j];
            sh.cand_pos[m + j] = pos;
            sh.cand_key[m + j] = keys[pos];
        }
        m += cnt;
    }
    // cand_pos is ascending: wave ranges are in order, each list ascending.
    const int n_sel = wave_select(sh.cand_key, m, k, sh.chosen);
    for (int r = lane; r < k; r += 64) {
        if (r < n_sel)
            emit(r, row_of(sh.cand_pos[sh.chosen[r]]), key_to_score(sh.cand_key[sh.chosen[r]]));
        else
            emit(r, -1, -INFINITY);
    }
    return n_sel;
}


}  // namespace
}  // namespace hga
