// attend_bwd.hip -- segment-wise backward of the routed attention
// (arXiv 2607.15105, gist.science technical summary 2.2: every segment is
// back-propagated on its own and the key/value history before it is detached;
// technical summary 2.1: the routing choice carries no gradient).
//
// Two kernels; no output element is accumulated with atomics and every sum
// runs in a fixed order, so results are bitwise reproducible:
//   dq     query-major, the forward's work unit (query block x kv head), two
//          passes over the routed chunks and the causal local block:
//          pass 1: S^T = K Q^T, dP^T = V dO^T, P = exp(S - lse),
//                  Delta_i = sum_j P_ij dP_ij (fp32; written for dkdv)
//          pass 2: dS = P (dP - Delta), dQ^T += K^T dS^T.
//          Delta is not taken as dO . O: O arrives rounded to bf16, and that
//          rounding (2^-9 |O|) lands undamped on rows whose attention sits on a
//          few keys. K^T sits in LDS under the accumulator's key permutation,
//          as V^T does in the forward.
//   dkdv   key-major over the active chunks only (history is detached): the
//          workgroups of chunk a scan the routed ids for the later blocks that
//          chose a; the list (own block first) is dealt round-robin to up to
//          kSplit workgroups, each walking its blocks x the G query heads:
//          S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//          Wave w owns keys 32*(w&1).. and queries 32*(w>>1).. of each query
//          tile; the two query halves are summed through LDS. A chunk chosen
//          by one block is written directly; otherwise every workgroup stores
//          its partial sums and the last one to finish (a per-chunk counter)
//          adds the partials in workgroup order and writes the result. This
//          spreads the chunks that many blocks chose (routing concentrates on
//          high-scoring chunks) over several CUs.
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kRowStride = kD + 8;          // bf16 per row-major 128-wide row in LDS (272 B)
constexpr int kTStride = kC + 8;            // bf16 per transposed row (64 wide) in LDS (144 B)
constexpr int kRowTile = kC * kRowStride;   // elements
constexpr int kTTile = kD * kTStride;       // elements
constexpr int kMaxBlocksDkdv = 1024;        // query blocks a dkdv workgroup can list
// Above this probability a bf16 operand's rounding (2^-9 relative) is no longer
// damped by the weight: tiles holding one feed P and dS to the MFMAs as a bf16
// pair hi + lo (hi = bf16(x), lo = bf16(x - hi)), keeping them to ~2^-17.
constexpr float kPairAbove = 1.0f / 16.0f;

__device__ __forceinline__ int t_pos(int kk) {   // swap bits 2 and 3
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// 64 rows x 128 bf16 of a row-major source, thread t holds rows 4*(t/16)+r
// and d = 8*(t%16) .. +8.
struct Rows4 { u32x4 r[4]; };

__device__ __forceinline__ void load_rows(Rows4 &x, const uint16_t *src) {
    const int t = threadIdx.x;
    const uint16_t *p = src + (int64_t)(4 * (t >> 4)) * kD + (t & 15) * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) x.r[r] = *(const u32x4 *)(p + (int64_t)r * kD);
}

__device__ __forceinline__ void store_rows(const Rows4 &x, uint16_t *dst) {
    const int t = threadIdx.x;
    const int row0 = 4 * (t >> 4), dseg = t & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4 *)(dst + (row0 + r) * kRowStride + dseg * 8) = x.r[r];
}

// Transposed store: dst[d][t_pos(row)] for the thread's 4 rows and 8 d's.
__device__ __forceinline__ void store_rows_t(const Rows4 &x, uint16_t *dst) {
    const int t = threadIdx.x;
    const int row0 = 4 * (t >> 4), dseg = t & 15;
    const int pos = t_pos(row0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t a = x.r[0][q], b = x.r[1][q], c = x.r[2][q], d = x.r[3][q];
        u32x2 even, odd;
        even[0] = (a & 0xFFFFu) | (b << 16);
        even[1] = (c & 0xFFFFu) | (d << 16);
        odd[0] = (a >> 16) | (b & 0xFFFF0000u);
        odd[1] = (c >> 16) | (d & 0xFFFF0000u);
        *(u32x2 *)(dst + (dseg * 8 + 2 * q) * kTStride + pos) = even;
        *(u32x2 *)(dst + (dseg * 8 + 2 * q + 1) * kTStride + pos) = odd;
    }
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.f;
    return z;
}

// --------------------------------------------------------------------- dq

template <int G>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, float *__restrict__ delta, int *__restrict__ counters,
    int64_t n_q, int64_t Hkv, int64_t T_cap, int64_t p0, const int32_t *__restrict__ ids,
    int k, float scale_log2, float scale, float *__restrict__ dQ)
{
    constexpr int HW = G < 4 ? G : 4;
    constexpr int NHG = G / HW;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Kts[2][kTTile];
    __shared__ int list[kMaxTopK + 1];
    __shared__ int list_n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t g = blockIdx.x % Hkv;
    const int64_t rest = blockIdx.x / Hkv;
    const int hg = (int)(rest % NHG);
    const int64_t b = rest / NHG;
    const int64_t n_blocks = n_q / kC;
    const int64_t P = p0 + b * kC;
    const int64_t local_chunk = P / kC;
    const uint16_t *Kg = K + g * T_cap * kD;
    const uint16_t *Vg = V + g * T_cap * kD;

    if (wave == 0) {
        int cnt = 0;
        const int32_t *row = ids + (g * n_blocks + b) * k;
        for (int base = 0; base < k; base += 64) {
            const int r = base + lane;
            const int c = (r < k) ? row[r] : -1;
            const bool ok = c >= 0 && (int64_t)c < local_chunk;
            const uint64_t m = __ballot(ok);
            if (ok) list[cnt + lanes_below(m)] = c;
            cnt += __popcll(m);
        }
        if (lane == 0) { list[cnt] = (int)local_chunk; list_n = cnt + 1; }
    }
    // the dkdv kernel that follows counts finished workgroups per (kv head, chunk)
    if (hg == 0 && tid == 0) counters[g * n_blocks + b] = 0;
    __syncthreads();
    const int n_tiles = list_n;

    Rows4 kr, vr;
    load_rows(kr, Kg + (int64_t)list[0] * kC * kD);
    load_rows(vr, Vg + (int64_t)list[0] * kC * kD);

    const bool computes = wave < HW;
    const int64_t h = g * G + hg * HW + wave;
    const int col = lane & 31;
    const int half = lane >> 5;
    bf16x8 qf[2][8], df[2][8];
    float lse2[2], dl[2];
    if (computes) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int64_t row = h * n_q + b * kC + 32 * qt + col;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                qf[qt][ks] = *(const bf16x8 *)(Q + row * kD + 16 * ks + 8 * half);
                df[qt][ks] = *(const bf16x8 *)(dO + row * kD + 16 * ks + 8 * half);
            }
            lse2[qt] = lse[row] * 1.44269504088896340736f;
            dl[qt] = 0.f;
        }
    }
    store_rows(kr, Ks[0]);
    store_rows_t(kr, Kts[0]);
    store_rows(vr, Vs[0]);
    __syncthreads();

    // One pipeline step: prefetch the next tile (tile order: the list twice),
    // compute S^T and dP^T of the current tile, hand them to `body`.
    const int n_steps = 2 * n_tiles;
    auto step_tile = [&](int step, auto &&body) {
        const int buf = step & 1;
        const bool more = step + 1 < n_steps;
        if (more) {
            const int nxt = list[(step + 1) % n_tiles];
            load_rows(kr, Kg + (int64_t)nxt * kC * kD);
            load_rows(vr, Vg + (int64_t)nxt * kC * kD);
        }
        if (computes) {
            const uint16_t *Kb = Ks[buf];
            const uint16_t *Vb = Vs[buf];
            f32x16 s[2][2], dp[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) { s[kt][qt] = zero16(); dp[kt][qt] = zero16(); }
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const int off = (32 * kt + col) * kRowStride + 16 * ks + 8 * half;
                    const bf16x8 a = *(const bf16x8 *)(Kb + off);
                    const bf16x8 v = *(const bf16x8 *)(Vb + off);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qt][ks], s[kt][qt], 0, 0, 0);
                        dp[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, df[qt][ks], dp[kt][qt], 0, 0, 0);
                    }
                }
            }
            const int it = step < n_tiles ? step : step - n_tiles;
            const bool diag = it == n_tiles - 1;
            // P, with the causal mask on the local block (the last tile)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        float p = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][j], scale_log2, -lse2[qt]));
                        if (diag) {
                            const int key = 32 * kt + 8 * (j >> 2) + 4 * half + (j & 3);
                            if (key > 32 * qt + col) p = 0.f;
                        }
                        s[kt][qt][j] = p;
                    }
            body(s, dp, Ks[buf], Kts[buf]);
        }
        if (more) {
            store_rows(kr, Ks[buf ^ 1]);
            store_rows_t(kr, Kts[buf ^ 1]);
            store_rows(vr, Vs[buf ^ 1]);
        }
        __syncthreads();
    };

    // pass 1: Delta_i = sum_j P_ij dP_ij
    for (int step = 0; step < n_tiles; ++step)
        step_tile(step, [&](f32x16 (&p)[2][2], f32x16 (&dp)[2][2], const uint16_t *, const uint16_t *) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) dl[qt] = fmaf(p[kt][qt][j], dp[kt][qt][j], dl[qt]);
        });
    if (computes) {
        // join the two half-waves' key subsets and publish Delta for dkdv
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            dl[qt] += partner32(dl[qt]);
            if (half == 0) delta[h * n_q + b * kC + 32 * qt + col] = dl[qt];
        }
    }

    // pass 2: dS = P (dP - Delta); dQ^T += K^T dS^T
    f32x16 acc[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[qt][dt] = zero16();
    for (int step = n_tiles; step < n_steps; ++step)
        step_tile(step, [&](f32x16 (&p)[2][2], f32x16 (&dp)[2][2], const uint16_t *, const uint16_t *Ktb) {
            // dS as a bf16 pair: hi always enters the MFMA, lo only in tiles
            // holding a probability above kPairAbove (wave-uniform branch)
            bf16x8 dsh[2][4], dsl[2][4];
            bool big = false;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        big |= p[kt][qt][j] > kPairAbove;
                        const float ds = p[kt][qt][j] * (dp[kt][qt][j] - dl[qt]);
                        const __bf16 hi = (__bf16)ds;
                        dsh[qt][2 * kt + (j >> 3)][j & 7] = hi;
                        dsl[qt][2 * kt + (j >> 3)][j & 7] = (__bf16)(ds - (float)hi);
                    }
            const bool pair = __ballot(big) != 0;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 a = *(const bf16x8 *)(Ktb + (32 * dt + col) * kTStride + 16 * ks + 8 * half);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsh[qt][ks], acc[qt][dt], 0, 0, 0);
                    if (pair) {
#pragma unroll
                        for (int qt = 0; qt < 2; ++qt)
                            acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsl[qt][ks], acc[qt][dt], 0, 0, 0);
                    }
                }
        });

    if (!computes) return;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float *drow = dQ + (h * n_q + b * kC + 32 * qt + col) * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[qt][dt][4 * u + e] * scale;
                *(f32x4 *)(drow + 32 * dt + 8 * u + 4 * half) = v;
            }
    }
}

// ------------------------------------------------------------------- dkdv

// One LDS buffer of the dkdv pipeline: a 64-query tile of one head.
constexpr int kQOff = 0;
constexpr int kDOOff = kQOff + kRowTile * 2;
constexpr int kQtOff = kDOOff + kRowTile * 2;
constexpr int kDOtOff = kQtOff + kTTile * 2;
constexpr int kLseOff = kDOtOff + kTTile * 2;
constexpr int kDlOff = kLseOff + kC * 4;
constexpr int kBufBytes = kDlOff + kC * 4;
static_assert(kBufBytes % 16 == 0, "buffer alignment");
static_assert(2 * kBufBytes >= 2 * 2 * 4 * 16 * 64 * 4, "reduction scratch fits");

constexpr int kSplit = 4;                  // workgroups that share one chunk's block list

template <int G>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, int64_t n_q,
    int64_t Hkv, int64_t T_cap, int64_t p0, const int32_t *__restrict__ ids, int k,
    float scale_log2, float scale, float *__restrict__ dK, float *__restrict__ dV,
    float *__restrict__ part, int *__restrict__ counters)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];
    __shared__ int blist[kMaxBlocksDkdv];
    __shared__ int blist_n;
    __shared__ int is_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t g = blockIdx.x % Hkv;
    const int64_t rest = blockIdx.x / Hkv;
    const int split = (int)(rest % kSplit);
    const int64_t a = rest / kSplit;             // active chunk = its own query block
    const int64_t n_blocks = n_q / kC;
    const int64_t ca = p0 / kC + a;               // absolute chunk index

    // Query blocks that attend chunk a: its own (causal) and every later block
    // whose routed ids list it, in ascending block order.
    if (wave == 0) {
        int cnt = 0;
        if (lane == 0) blist[0] = (int)a;
        cnt = 1;
        for (int64_t base = a + 1; base < n_blocks; base += 64) {
            const int64_t bb = base + lane;
            bool hit = false;
            if (bb < n_blocks) {
                const int32_t *row = ids + (g * n_blocks + bb) * k;
                for (int r = 0; r < k; ++r) hit |= (row[r] == (int32_t)ca);
            }
            const uint64_t m = __ballot(hit);
            if (hit) blist[cnt + lanes_below(m)] = (int)bb;
            cnt += __popcll(m);
        }
        if (lane == 0) blist_n = cnt;
    }
    __syncthreads();
    const int n_list = blist_n;
    const int n_parts = n_list < kSplit ? n_list : kSplit;
    if (split >= n_parts) return;                 // nothing dealt to this workgroup
    const int n_mine = (n_list - split + kSplit - 1) / kSplit;   // entries split, split+kSplit, ...
    const int n_tiles = n_mine * G;

    const int col = lane & 31;
    const int half = lane >> 5;
    const int kh = wave & 1;         // keys 32*kh .. +32 of the chunk
    const int qh = wave >> 1;        // queries 32*qh .. +32 of each tile
    const int64_t key_row = ca * kC + 32 * kh + col;
    bf16x8 kb[8], vb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        kb[ks] = *(const bf16x8 *)(K + (g * T_cap + key_row) * kD + 16 * ks + 8 * half);
        vb[ks] = *(const bf16x8 *)(V + (g * T_cap + key_row) * kD + 16 * ks + 8 * half);
    }

    auto tile_src = [&](int t, int64_t &row0) {
        const int64_t bb = blist[split + kSplit * (t / G)];
        const int64_t h = g * G + t % G;
        row0 = h * n_q + bb * kC;
    };

    Rows4 qr, dr;
    float lsev = 0.f, dlv = 0.f;
    int64_t row0;
    tile_src(0, row0);
    load_rows(qr, Q + row0 * kD);
    load_rows(dr, dO + row0 * kD);
    if (tid < kC) { lsev = lse[row0 + tid]; dlv = delta[row0 + tid]; }

    auto store_buf = [&](int buf) {
        uint8_t *B = smem + buf * kBufBytes;
        store_rows(qr, (uint16_t *)(B + kQOff));
        store_rows(dr, (uint16_t *)(B + kDOOff));
        store_rows_t(qr, (uint16_t *)(B + kQtOff));
        store_rows_t(dr, (uint16_t *)(B + kDOtOff));
        if (tid < kC) {
            ((float *)(B + kLseOff))[tid] = lsev * 1.44269504088896340736f;
            ((float *)(B + kDlOff))[tid] = dlv;
        }
    };
    store_buf(0);
    __syncthreads();

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        const bool more = it + 1 < n_tiles;
        if (more) {
            tile_src(it + 1, row0);
            load_rows(qr, Q + row0 * kD);
            load_rows(dr, dO + row0 * kD);
            if (tid < kC) { lsev = lse[row0 + tid]; dlv = delta[row0 + tid]; }
        }
        const uint8_t *B = smem + buf * kBufBytes;
        const uint16_t *Qb = (const uint16_t *)(B + kQOff);
        const uint16_t *dOb = (const uint16_t *)(B + kDOOff);
        const uint16_t *Qtb = (const uint16_t *)(B + kQtOff);
        const uint16_t *dOtb = (const uint16_t *)(B + kDOtOff);
        const float *lse2s = (const float *)(B + kLseOff);
        const float *dls = (const float *)(B + kDlOff);

        // S[q][key] = Q K^T, dP[q][key] = dO V^T for this wave's 32 x 32 block.
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int off = (32 * qh + col) * kRowStride + 16 * ks + 8 * half;
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(Qb + off), kb[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(dOb + off), vb[ks], dp, 0, 0, 0);
        }
        // lane: key 32*kh + col; queries 32*qh + 8u + 4*half + e (j = 4u + e)
        const bool diag = split == 0 && (it / G) == 0;   // list entry 0 is the own block
        bf16x8 pb[2], dsb[2];
        float pf[16], dsf[16];
        bool big = false;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q0 = 32 * qh + 8 * u + 4 * half;
            const f32x4 l4 = *(const f32x4 *)(lse2s + q0);
            const f32x4 d4 = *(const f32x4 *)(dls + q0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * u + e;
                float p = __builtin_amdgcn_exp2f(fmaf(s[j], scale_log2, -l4[e]));
                if (diag && 32 * kh + col > q0 + e) p = 0.f;
                big |= p > kPairAbove;
                pf[j] = p;
                dsf[j] = p * (dp[j] - d4[e]);
                pb[j >> 3][j & 7] = (__bf16)pf[j];
                dsb[j >> 3][j & 7] = (__bf16)dsf[j];
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS (k runs over this wave's 32 queries)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = (32 * dt + col) * kTStride + 32 * qh + 16 * ks + 8 * half;
                dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(dOtb + off), pb[ks], dv[dt], 0, 0, 0);
                dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(Qtb + off), dsb[ks], dk[dt], 0, 0, 0);
            }
        if (__ballot(big) != 0) {              // wave-uniform: add the low halves
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                pb[j >> 3][j & 7] = (__bf16)(pf[j] - (float)pb[j >> 3][j & 7]);
                dsb[j >> 3][j & 7] = (__bf16)(dsf[j] - (float)dsb[j >> 3][j & 7]);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (32 * dt + col) * kTStride + 32 * qh + 16 * ks + 8 * half;
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(dOtb + off), pb[ks], dv[dt], 0, 0, 0);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8 *)(Qtb + off), dsb[ks], dk[dt], 0, 0, 0);
                }
        }
        if (more) store_buf(buf ^ 1);
        __syncthreads();
    }

    // Sum the two query halves: waves 2, 3 hand their partials to waves 0, 1.
    float *red = (float *)smem;       // [2 waves][2 tensors][4 dt][16 j][64 lanes]
    if (qh == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                red[(((kh * 2 + 0) * 4 + dt) * 16 + j) * 64 + lane] = dk[dt][j];
                red[(((kh * 2 + 1) * 4 + dt) * 16 + j) * 64 + lane] = dv[dt][j];
            }
    }
    __syncthreads();
    // lane holds key 32*kh + col, d = 32*dt + 8u + 4*half + e
    const int64_t out_row = g * n_q + a * kC + 32 * kh + col;
    if (qh == 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                dk[dt][j] += red[(((kh * 2 + 0) * 4 + dt) * 16 + j) * 64 + lane];
                dv[dt][j] += red[(((kh * 2 + 1) * 4 + dt) * 16 + j) * 64 + lane];
            }
    }
    if (n_parts == 1) {
        if (qh == 0) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 vk, vv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vk[e] = dk[dt][4 * u + e] * scale;
                        vv[e] = dv[dt][4 * u + e];
                    }
                    *(f32x4 *)(dK + out_row * kD + 32 * dt + 8 * u + 4 * half) = vk;
                    *(f32x4 *)(dV + out_row * kD + 32 * dt + 8 * u + 4 * half) = vv;
                }
        }
        return;
    }

    // Several workgroups share this chunk: store the partial, count, and let
    // the last one add the partials in workgroup order 0, 1, ... .
    const int64_t part_stride = Hkv * n_q * kD;          // floats per (split, tensor)
    if (qh == 0) {
        float *pk = part + (int64_t)(2 * split) * part_stride + out_row * kD;
        float *pv = part + (int64_t)(2 * split + 1) * part_stride + out_row * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 vk, vv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vk[e] = dk[dt][4 * u + e];
                    vv[e] = dv[dt][4 * u + e];
                }
                *(f32x4 *)(pk + 32 * dt + 8 * u + 4 * half) = vk;
                *(f32x4 *)(pv + 32 * dt + 8 * u + 4 * half) = vv;
            }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(&counters[g * n_blocks + a], 1) == n_parts - 1;
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    // 64 keys x 128 d per tensor; thread t sums float4 column (t % 32) of rows
    // t/32, t/32 + 8, ...
    const int64_t row_base = g * n_q + a * kC;
    for (int r = tid >> 5; r < kC; r += kThreads / 32) {
        const int64_t off = (row_base + r) * kD + 4 * (tid & 31);
        f32x4 sk = *(const f32x4 *)(part + off);
        f32x4 sv = *(const f32x4 *)(part + part_stride + off);
        for (int sp = 1; sp < n_parts; ++sp) {
            const f32x4 xk = *(const f32x4 *)(part + (int64_t)(2 * sp) * part_stride + off);
            const f32x4 xv = *(const f32x4 *)(part + (int64_t)(2 * sp + 1) * part_stride + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) { sk[e] += xk[e]; sv[e] += xv[e]; }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sk[e] *= scale;
        *(f32x4 *)(dK + off) = sk;
        *(f32x4 *)(dV + off) = sv;
    }
}

template <int G>
hipError_t launch_bwd_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                        int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                        const int32_t *ids, int32_t k, float scale, const float *lse,
                        const uint16_t *dO, float *dQ, float *dK, float *dV,
                        float *delta, int *counters, float *part, hipStream_t stream)
{
    constexpr int NHG = G < 4 ? 1 : G / 4;
    const int64_t n_blocks = n_q / kC;
    const float scale_log2 = scale * 1.44269504088896340736f;
    hipLaunchKernelGGL(bwd_dq_kernel<G>, dim3((unsigned)(n_blocks * Hkv * NHG)), dim3(kThreads),
                       0, stream, Q, K, V, dO, lse, delta, counters, n_q, Hkv, T_cap, p0, ids,
                       k, scale_log2, scale, dQ);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<G>, dim3((unsigned)(n_blocks * Hkv * kSplit)),
                       dim3(kThreads), 0, stream, Q, K, V, dO, lse, delta, n_q, Hkv, T_cap, p0,
                       ids, k, scale_log2, scale, dK, dV, part, counters);
    return hipGetLastError();
}

// Workspace layout: Delta [Hq][n_q] f32 | counters [Hkv][n_q/C] int32 (padded
// to 256 B) | partial sums [kSplit][dK, dV][Hkv][n_q][D] f32.
struct BwdWorkspace {
    size_t delta_off, counter_off, part_off, total;
};

BwdWorkspace bwd_layout(int64_t Hq, int64_t Hkv, int64_t n_q)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdWorkspace w;
    w.delta_off = 0;
    w.counter_off = up((size_t)(Hq * n_q) * sizeof(float));
    w.part_off = w.counter_off + up((size_t)(Hkv * (n_q / kC)) * sizeof(int));
    w.total = w.part_off + (size_t)kSplit * 2 * (size_t)(Hkv * n_q * kD) * sizeof(float);
    return w;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_q)
{
    return bwd_layout(Hq, Hkv, n_q).total;
}

int64_t bwd_max_queries() { return (int64_t)kMaxBlocksDkdv * kC; }

hipError_t launch_attend_bwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                             int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                             int64_t n_q, const int32_t *ids, int32_t k, float scale,
                             const uint16_t *O, const float *lse, const uint16_t *dO,
                             float *dQ, float *dK, float *dV, void *workspace,
                             hipStream_t stream)
{
    (void)O;    // Delta is recomputed from P and dP (see the dq kernel)
    if (n_q == 0) return hipSuccess;
    const BwdWorkspace w = bwd_layout(Hq, Hkv, n_q);
    uint8_t *ws = (uint8_t *)workspace;
    float *delta = (float *)(ws + w.delta_off);
    int *counters = (int *)(ws + w.counter_off);
    float *part = (float *)(ws + w.part_off);
    switch (Hq / Hkv) {
    case 1: return launch_bwd_g<1>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 2: return launch_bwd_g<2>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 4: return launch_bwd_g<4>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 8: return launch_bwd_g<8>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hga
