// route.hip -- per query block top-k chunk routing (arXiv 2607.15105,
// gist.science technical summary 2.1: the current query block scores the
// resident chunk summaries and keeps the most relevant earlier chunks; no
// gradient flows through the choice).
//
// One 256-thread workgroup per (query block b, kv head g):
//   1. qbar = mean of the block's G*64 query rows (fp32, LDS reduction);
//   2. score_c = qbar . S[g][c] for every chunk c < P/C: 16 lanes per chunk
//      read one 512-byte summary row with coalesced 16-byte loads, each lane
//      holding its 8-wide slice of qbar in registers; the 16 partial sums are
//      folded across lanes. Scores become order-preserving uint32 keys in LDS;
//   3. top-k by (score desc, id asc): every wave selects its own contiguous
//      id range with a ballot/popcount threshold search, then wave 0 selects
//      among the survivors. Selected ids come out in ascending order from a
//      ballot + mbcnt compaction, so no sort is needed.
// Workgroup w serves kv head w % Hkv: with 8 kv heads the blocks of one head
// land on one XCD and share its L2 copy of that head's summaries.
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, s));
    return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, s));
    return x;
}

// Wave-level selection of the k largest keys[0..n) (ties: lower position
// first). Writes the chosen positions, ascending, to out_pos (LDS) and
// returns their number, min(k, n). Every lane of the wave must call it.
__device__ int wave_select(const uint32_t *keys, int n, int k, int *out_pos)
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
    // Bits above the highest bit in which the keys differ are shared by all.
    const uint32_t diff = mx ^ mn;
    int top = diff ? 31 - __builtin_clz(diff) : -1;
    uint32_t T = (top >= 31) ? 0u : (mx & ~((2u << top) - 1u));
    // Largest T with #{key >= T} >= k, one bit at a time.
    for (int bit = top; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
        for (int base = 0; base < n; base += 64) {
            const int p = base + lane;
            cnt += __popcll(__ballot(p < n && keys[p] >= cand));
        }
        if (cnt >= k) T = cand;
    }
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
        if (take) out_pos[out + lanes_below(sm)] = p;
        out += __popcll(sm);
    }
    return out;
}

__device__ __forceinline__ float key_to_score(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

template <int G>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const uint16_t *__restrict__ Q, int64_t n_q, int64_t Hkv, int64_t p0,
    const float *__restrict__ S, int64_t n_cap, int k,
    int32_t *__restrict__ ids, float *__restrict__ scores)
{
    extern __shared__ uint32_t keys[];          // [n_eligible of this block]
    __shared__ float part[16][kD];
    __shared__ float qbar[kD];
    __shared__ int surv[kRouteWaves][kMaxTopK];
    __shared__ int surv_n[kRouteWaves];
    __shared__ uint32_t cand_key[kRouteWaves * kMaxTopK];
    __shared__ int cand_pos[kRouteWaves * kMaxTopK];
    __shared__ int chosen[kMaxTopK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t n_blocks = n_q / kC;
    const int64_t g = blockIdx.x % Hkv;
    const int64_t b = blockIdx.x / Hkv;
    const int64_t P = p0 + b * kC;
    const int nE = (int)(P / kC);

    // 1. qbar over the G heads x 64 queries of this block.
    {
        const int dseg = tid & 15, r0 = tid >> 4;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int m = 0; m < G * 4; ++m) {
            const int row = r0 + 16 * m;               // 0 .. G*64-1
            const int64_t h = g * G + row / kC;
            const int64_t i = b * kC + row % kC;
            const u32x4 w = *(const u32x4 *)(Q + (h * n_q + i) * kD + dseg * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo(w[q]);
                acc[2 * q + 1] += bf16_hi(w[q]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part[r0][dseg * 8 + e] = acc[e];
    }
    __syncthreads();
    if (tid < kD) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += part[r][tid];
        qbar[tid] = s * (1.0f / (float)(G * kC));      // a power of two: exact
    }
    __syncthreads();

    // 2. scores -> keys. Each wave scores 4 chunks per step (16 lanes per
    // chunk); the loads of kBatch steps are issued before any is used so their
    // latencies overlap.
    {
        constexpr int kBatch = 16;
        const int dseg = lane & 15, sub = lane >> 4;
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qbar[dseg * 8 + e];
        const float *Sg = S + g * n_cap * kD + dseg * 8;
        for (int base = wave * 4; base < nE; base += kRouteWaves * 4 * kBatch) {
            f32x4 lo[kBatch], hi[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int c = base + u * kRouteWaves * 4 + sub;
                if (c < nE) {
                    lo[u] = *(const f32x4 *)(Sg + (int64_t)c * kD);
                    hi[u] = *(const f32x4 *)(Sg + (int64_t)c * kD + 4);
                } else {
                    lo[u] = hi[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                float s = qv[0] * lo[u][0];
                s = fmaf(qv[1], lo[u][1], s);
                s = fmaf(qv[2], lo[u][2], s);
                s = fmaf(qv[3], lo[u][3], s);
                s = fmaf(qv[4], hi[u][0], s);
                s = fmaf(qv[5], hi[u][1], s);
                s = fmaf(qv[6], hi[u][2], s);
                s = fmaf(qv[7], hi[u][3], s);
                s += __shfl_xor(s, 1);
                s += __shfl_xor(s, 2);
                s += __shfl_xor(s, 4);
                s += __shfl_xor(s, 8);
                const int c = base + u * kRouteWaves * 4 + sub;
                if (dseg == 0 && c < nE) keys[c] = score_key(s);
            }
        }
    }
    __syncthreads();

    // 3. top-k: each wave over its contiguous id range, then wave 0 merges.
    const int per = (nE + kRouteWaves - 1) / kRouteWaves;
    const int lo = min(nE, wave * per);
    const int hi = min(nE, lo + per);
    const int got = wave_select(keys + lo, hi - lo, k, surv[wave]);
    if (lane == 0) surv_n[wave] = got;
    __syncthreads();
    if (wave == 0) {
        int m = 0;
        for (int w = 0; w < kRouteWaves; ++w) {
            const int cnt = surv_n[w];
            const int off = min(nE, w * per);
            for (int j = lane; j < cnt; j += 64) {
                const int pos = off + surv[w][j];
                cand_pos[m + j] = pos;
                cand_key[m + j] = keys[pos];
            }
            m += cnt;
        }
        // cand_pos is ascending: wave ranges are in order, each list ascending.
        const int n_sel = wave_select(cand_key, m, k, chosen);
        int32_t *out = ids + (g * n_blocks + b) * k;
        float *sout = scores ? scores + (g * n_blocks + b) * k : nullptr;
        for (int r = lane; r < k; r += 64) {
            if (r < n_sel) {
                const int pos = cand_pos[chosen[r]];
                out[r] = pos;
                if (sout) sout[r] = key_to_score(cand_key[chosen[r]]);
            } else {
                out[r] = -1;
                if (sout) sout[r] = -INFINITY;
            }
        }
    }
}

template <int G>
hipError_t launch_route_g(const uint16_t *Q, int64_t Hkv, int64_t p0, int64_t n_q,
                          const float *S, int64_t n_cap, int32_t k, int32_t *ids,
                          float *scores, hipStream_t stream)
{
    const int64_t n_blocks = n_q / kC;
    const int64_t max_eligible = (p0 + n_q - kC) / kC;
    const size_t shmem = (size_t)(max_eligible > 0 ? max_eligible : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(route_kernel<G>, dim3((unsigned)(n_blocks * Hkv)), dim3(kRouteThreads),
                       shmem, stream, Q, n_q, Hkv, p0, S, n_cap, k, ids, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const uint16_t *Q, int64_t Hq, int64_t Hkv, int64_t p0,
                        int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                        int32_t *ids, float *scores, hipStream_t stream)
{
    if (n_q == 0 || k == 0) return hipSuccess;
    switch (Hq / Hkv) {
    case 1: return launch_route_g<1>(Q, Hkv, p0, n_q, S, n_cap, k, ids, scores, stream);
    case 2: return launch_route_g<2>(Q, Hkv, p0, n_q, S, n_cap, k, ids, scores, stream);
    case 4: return launch_route_g<4>(Q, Hkv, p0, n_q, S, n_cap, k, ids, scores, stream);
    case 8: return launch_route_g<8>(Q, Hkv, p0, n_q, S, n_cap, k, ids, scores, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hga
