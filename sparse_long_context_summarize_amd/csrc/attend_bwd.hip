// attend_bwd.hip -- segment-wise backward of the routed attention
// (arXiv 2607.15105, gist.science technical summary 2.2: every segment is
// back-propagated on its own and the key/value history before it is detached;
// technical summary 2.1: the routing choice carries no gradient).
//
// Two kernels; no output element is accumulated with atomics and every sum
// runs in a fixed order, so results are bitwise reproducible:
//   dq     query-major, the forward's work unit (query block x kv head) and
//          wave layout (8 waves, two per SIMD, 32 queries of one head each),
//          two passes over the routed chunks and the causal local block:
//          pass 1: S^T = K Q^T, dP^T = V dO^T, P = exp(S - lse),
//                  Delta_i = sum_j P_ij dP_ij (fp32; written for dkdv)
//          pass 2: dS = P (dP - Delta), dQ^T += K^T dS^T.
//          Delta is not taken as dO . O: O arrives rounded to bf16, and that
//          rounding (2^-9 |O|) lands undamped on rows whose attention sits on a
//          few keys. K^T sits in LDS under the accumulator's key permutation,
//          as V^T does in the forward.
//   dkdv   key-major over the active chunks only (history is detached): the
//          workgroups of chunk a scan the routed ids for the later blocks that
//          chose a; the list's (block, query head) tiles, own block first,
//          are dealt round-robin to up to kSplit workgroups:
//          S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//          Wave w owns keys 32*(w&1).. and queries 32*(w>>1).. of each query
//          tile; the two query halves are summed through LDS. A chunk with
//          at most kMinTiles tiles has one workgroup, which writes the result
//          directly; a longer one is split, every workgroup stores its partial
//          sums and the last one to finish (a per-chunk counter) adds the
//          partials in workgroup order and writes the result. This spreads
//          the chunks that many blocks chose (routing concentrates on
//          high-scoring chunks) over several CUs.
// Both kernels load their tiles two steps ahead into registers (two sets
// used in a fixed order, steps run in pairs) and write them to double-buffered
// LDS one barrier before use; transposed copies are written with byte
// permutes in a lane order whose 8-byte writes fall on distinct banks.
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

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.f;
    return z;
}

// --------------------------------------------------------------------- dq

constexpr int kDqThreads = 512;
constexpr int kDqPieces = 4;       // 16-byte pieces of one tile per loader thread

// Tile loaders of the dq kernel. Waves 4-7 ("K group") move K tiles, waves
// 0-3 ("V group") V tiles; each thread holds four 16-byte pieces.
struct DqRegs { u32x4 p[kDqPieces]; };

// K group, u = thread - 256: lane takes keys 4*kg .. 4*kg+3 of the 8-wide d
// slice dp, kg = lane%16, dp = 4*(u/64) + lane/16; piece j is key 4*kg + j.
__device__ __forceinline__ void dq_load_k(DqRegs &r, const uint16_t *Kg, int64_t tok0)
{
    const int u = threadIdx.x - kDqThreads / 2, lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
    const uint16_t *src = Kg + (tok0 + 4 * kg) * kD + dp * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) r.p[j] = *(const u32x4 *)(src + j * kD);
}

// Group tiles: the same rows, 4*kg + j, lie in one 8-row group, so one
// row_tok(4*kg) call serves the thread's four pieces.
template <typename RowTok>
__device__ __forceinline__ void dq_load_k(DqRegs &r, const uint16_t *Kg, RowTok row_tok)
{
    const int u = threadIdx.x - kDqThreads / 2, lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
    const uint16_t *src = Kg + row_tok(4 * kg) * kD + dp * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) r.p[j] = *(const u32x4 *)(src + j * kD);
}

// K to LDS twice: row-major (272-B rows) for the S^T operand, and transposed,
// K^T[d][t_pos(key)], for the dQ^T operand (the 4 keys x 8 d a lane holds are
// transposed with byte permutes; with kg = lane%16 the 64 lanes' 8-byte
// writes fall on distinct banks).
__device__ __forceinline__ void dq_store_k(const DqRegs &r, uint16_t *Ks, uint16_t *Kts)
{
    const int u = threadIdx.x - kDqThreads / 2, lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j)
        *(u32x4 *)(Ks + (4 * kg + j) * kRowStride + dp * 8) = r.p[j];
    uint16_t *dst = Kts + (8 * dp) * kTStride + t_pos(4 * kg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(r.p[1][e >> 1], r.p[0][e >> 1], sel);
        w[1] = __builtin_amdgcn_perm(r.p[3][e >> 1], r.p[2][e >> 1], sel);
        *(u32x2 *)(dst + e * kTStride) = w;
    }
}

// V group, u = thread: piece j is key row 16*j + u/16, d = 8*(u%16) .. +8.
__device__ __forceinline__ void dq_load_v(DqRegs &r, const uint16_t *Vg, int64_t tok0)
{
    const int u = threadIdx.x;
    const uint16_t *src = Vg + (tok0 + (u >> 4)) * kD + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) r.p[j] = *(const u32x4 *)(src + 16 * j * kD);
}

__device__ __forceinline__ void dq_store_v(const DqRegs &r, uint16_t *Vs)
{
    const int u = threadIdx.x;
    uint16_t *dst = Vs + (u >> 4) * kRowStride + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) *(u32x4 *)(dst + 16 * j * kRowStride) = r.p[j];
}

// Group tiles, V group: thread u takes rows r0 + 2*j of one 8-row group,
// r0 = 8*(u/32) + (u/16)%2, d = 8*(u%16) .. +8 (one row_tok call per tile).
template <typename RowTok>
__device__ __forceinline__ void dq_load_v(DqRegs &r, const uint16_t *Vg, RowTok row_tok)
{
    const int u = threadIdx.x;
    const int r0 = 8 * (u >> 5) + ((u >> 4) & 1);
    const uint16_t *src = Vg + row_tok(r0) * kD + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) r.p[j] = *(const u32x4 *)(src + 2 * j * kD);
}

__device__ __forceinline__ void dq_store_v_grp(const DqRegs &r, uint16_t *Vs)
{
    const int u = threadIdx.x;
    const int r0 = 8 * (u >> 5) + ((u >> 4) & 1);
    uint16_t *dst = Vs + r0 * kRowStride + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kDqPieces; ++j) *(u32x4 *)(dst + 2 * j * kRowStride) = r.p[j];
}

// Work unit: query block b of kv head g, as in the forward. 8 waves, two per
// SIMD: wave w computes head g*G + hg*HW + w%4 for queries 32*(w/4) .. +32,
// with Q^T and dO^T in registers as MFMA B operands, in the transposed form
// S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T (each query's state in one
// lane pair). Steps walk the tile list twice (pass 1, then pass 2); tiles are
// loaded two steps ahead into registers and written to double-buffered LDS
// one barrier before use. Each 64-key tile is processed as two 32-key halves.
// kUnit = kC: ids are chunk ids. kUnit = kGroup: ids are 8-token group ids;
// each routed tile is gathered from 8 groups, and a last routed tile with
// fewer masks its missing groups' keys.
template <int G, int kUnit>
__global__ __launch_bounds__(kDqThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, float *__restrict__ delta, int *__restrict__ counters,
    int64_t n_q, int kv_div, int64_t T_cap, int64_t p0,
    const int32_t *__restrict__ ids, int k, int sink, float scale_log2, float scale,
    float *__restrict__ dQ)
{
    constexpr int HW = G < 4 ? G : 4;
    constexpr int NHG = G / HW;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Kts[2][kTTile];
    __shared__ int list[(kUnit == kC ? kChunkListMax : kGroupListMax) + 1];
    __shared__ int list_n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // grid (Hkv, kv_div * NHG, blocks): y is the query head within its kv
    // head's group (kv_div > 1) or the workgroup's share of a G = 8 unit
    const int64_t gkv = blockIdx.x;                         // kv head
    const int sub = (int)blockIdx.y;
    const int64_t g = gkv * kv_div + (kv_div > 1 ? sub : 0);  // routing unit: its id row
    const int hg = NHG > 1 ? sub : 0;
    const int64_t b = blockIdx.z;
    const int64_t n_blocks = n_q / kC;
    const int64_t P = p0 + b * kC;
    const int64_t local_chunk = P / kC;
    const uint16_t *Kg = K + gkv * T_cap * kD;
    const uint16_t *Vg = V + gkv * T_cap * kD;

    // the sink window's units, the routed units (past the sink, before P,
    // repeats dropped), then the local chunk
    if (wave == 0) {
        const int ns = sink_units(sink, P, kUnit);
        write_sink_units(list, ns);
        const int n = build_unit_list(ids + (g * n_blocks + b) * k, k,
                                      (int64_t)sink * (kC / kUnit), P / kUnit, list + ns);
        if (lane == 0) {
            list[ns + n] = (int)local_chunk;
            list_n = ns + n + 1;
        }
    }
    // the dkdv kernel that follows counts finished workgroups per (unit, chunk)
    if (hg == 0 && tid == 0) counters[g * n_blocks + b] = 0;
    __syncthreads();
    const int n_units = list_n - 1;
    const int n_tiles = (kUnit == kC ? n_units : (n_units + 7) / 8) + 1;
    // keys of the last routed tile (groups: 8 per group present; else 64)
    const int pad_keys = (kUnit != kC && (n_units & 7) != 0) ? kGroup * (n_units & 7) : kC;
    // Each pass walks the tile list once, padded to an even number of steps
    // (a padding step moves data but computes nothing), so both pass loops
    // run whole pairs with the register sets in one fixed order.
    const int n_pass = n_tiles + (n_tiles & 1);
    const int n_steps = 2 * n_pass;
    const bool kgrp = tid >= kDqThreads / 2;

    // (as in the forward: with HW < 4 the two query halves' waves sit on
    // different SIMDs)
    const int qt = wave >> 2;
    const int lane4 = wave & 3;
    const bool computes = lane4 / HW == qt % (4 / HW);
    const int hw = lane4 % HW;                   // head slot
    const int64_t h = g * G + hg * HW + hw;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t qrow = h * n_q + b * kC + 32 * qt + col;
    bf16x8 qf[8], df[8];
    float lse2 = 0.f, dl = 0.f;
    if (computes) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = *(const bf16x8 *)(Q + qrow * kD + 16 * ks + 8 * half);
            df[ks] = *(const bf16x8 *)(dO + qrow * kD + 16 * ks + 8 * half);
        }
        lse2 = lse[qrow] * 1.44269504088896340736f;
    }
    const int *lst = list;
    // first token of a chunk tile, or the token of row r of a group tile
    // (the local tile is last; padding rows repeat the tile's last group)
    auto step_tok = [&](int st) __attribute__((always_inline)) {
        const int i = min(st % n_pass, n_tiles - 1);
        if constexpr (kUnit == kC) {
            return (int64_t)lst[i] * kC;
        } else {
            const bool local = i == n_tiles - 1;
            const int64_t lbase = (int64_t)lst[n_units] * kC;
            const int g0 = 8 * i, glast = n_units - 1;
            return [=](int r) __attribute__((always_inline)) -> int64_t {
                if (local) return lbase + r;
                return (int64_t)lst[min(g0 + (r >> 3), glast)] * kGroup + (r & 7);
            };
        }
    };
    auto load = [&](DqRegs &r, int st) __attribute__((always_inline)) {
        if (kgrp) dq_load_k(r, Kg, step_tok(min(st, n_steps - 1)));
        else dq_load_v(r, Vg, step_tok(min(st, n_steps - 1)));
    };
    auto store = [&](const DqRegs &r, int buf) __attribute__((always_inline)) {
        if (kgrp) dq_store_k(r, Ks[buf], Kts[buf]);
        else if constexpr (kUnit == kC) dq_store_v(r, Vs[buf]);
        else dq_store_v_grp(r, Vs[buf]);
    };
    DqRegs r0, r1;
    load(r0, 0);
    load(r1, 1);
    store(r0, 0);
    // Q, dO and lse have landed once the first tile has (issued before it).
    __syncthreads();

    // S^T and dP^T of one 32-key half kt of the tile in buffer buf, P in place
    // of S^T. Masks: key 32*kt + 8*(j/4) + 4*half + j%4 is dropped when
    // 8*(j/4) + j%4 > thr -- on the local block above query 32*qt + col
    // (causal), on a last group tile from key pad_keys on.
    auto sdp = [&](int buf, int kt, int mode, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
        const uint16_t *Kb = Ks[buf];
        const uint16_t *Vb = Vs[buf];
        s = zero16();
        dp = zero16();
        bf16x8 ka[8], va[8];
        auto rd = [&](int ks) __attribute__((always_inline)) {
            const int off = (32 * kt + col) * kRowStride + 16 * ks + 8 * half;
            ka[ks] = *(const bf16x8 *)(Kb + off);
            va[ks] = *(const bf16x8 *)(Vb + off);
        };
        rd(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks + 1 < 8) rd(ks + 1);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], df[ks], dp, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int thr = mode == 1 ? 32 * (qt - kt) + col - 4 * half
                      : mode == 2 ? pad_keys - 32 * kt - 4 * half - 1 : 1 << 20;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[j], scale_log2, -lse2));
            s[j] = (8 * (j >> 2) + (j & 3) > thr) ? 0.f : p;
        }
    };

    // One step: prefetch step st+2 into `pre`, compute step st from LDS
    // buffer st&1 (pass 1 or pass 2 by `body`), write step st+1 (held in
    // `nxt`) to the other buffer.
    auto step = [&](int st, DqRegs &pre, const DqRegs &nxt, auto &&body) __attribute__((always_inline)) {
        const int buf = st & 1;
        load(pre, st + 2);
        const int it = st % n_pass;
        // mode: 1 = local block (causal), 2 = last routed tile of groups
        const int mode = it == n_tiles - 1 ? 1 : (it == n_tiles - 2 && pad_keys < kC) ? 2 : 0;
        if (computes && it < n_tiles) body(buf, mode);
        if (st + 1 < n_steps) store(nxt, buf ^ 1);
        __syncthreads();
    };

    // pass 1: Delta_i = sum_j P_ij dP_ij
    auto pass1 = [&](int buf, int mode) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x16 s, dp;
            sdp(buf, kt, mode, s, dp);
#pragma unroll
            for (int j = 0; j < 16; ++j) dl = fmaf(s[j], dp[j], dl);
        }
    };
    for (int st = 0; st < n_pass; st += 2) {
        step(st, r0, r1, pass1);
        step(st + 1, r1, r0, pass1);
    }
    // Delta complete: join the two half-waves' key subsets, publish for dkdv
    dl += partner32(dl);
    if (computes && half == 0) delta[qrow] = dl;

    // pass 2: dS = P (dP - Delta); dQ^T += K^T dS^T. dS enters the MFMAs as
    // bf16 hi; halves holding a probability above kPairAbove add the rounding
    // remainder lo = bf16(dS - hi) in a second round (wave-uniform branch).
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();
    auto pass2 = [&](int buf, int mode) __attribute__((always_inline)) {
        const uint16_t *Ktb = Kts[buf];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x16 s, dp;
            sdp(buf, kt, mode, s, dp);
            bf16x8 dsh[2];
            bool big = false;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                big |= s[j] > kPairAbove;
                dp[j] = s[j] * (dp[j] - dl);
                dsh[j >> 3][j & 7] = (__bf16)dp[j];
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 a = *(const bf16x8 *)(Ktb + (32 * dt + col) * kTStride + 16 * (2 * kt + kk) + 8 * half);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsh[kk], acc[dt], 0, 0, 0);
                }
            if (__ballot(big) != 0) {
                bf16x8 dsl[2];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    dsl[j >> 3][j & 7] = (__bf16)(dp[j] - (float)dsh[j >> 3][j & 7]);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8 a = *(const bf16x8 *)(Ktb + (32 * dt + col) * kTStride + 16 * (2 * kt + kk) + 8 * half);
                        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsl[kk], acc[dt], 0, 0, 0);
                    }
            }
        }
    };
    for (int st = n_pass; st < n_steps; st += 2) {
        step(st, r0, r1, pass2);
        step(st + 1, r1, r0, pass2);
    }

    if (!computes) return;
    float *drow = dQ + qrow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * u + e] * scale;
            *(f32x4 *)(drow + 32 * dt + 8 * u + 4 * half) = v;
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

// A chunk's query tiles go to one workgroup, or to kSplit of them when there
// are more than kMinTiles (more workgroups per chunk measured slower: each
// one, even one with nothing dealt, pays the scan and the set-up, and the
// dkdv workgroup holds a whole CU).
constexpr int kSplit = 2;
constexpr int kMinTiles = 8;

// kUnit = kGroup: a later block may have chosen only some of the chunk's 8
// groups; the scan records them as an 8-bit mask per listed block, and the
// keys of the other groups get P = 0 in that block's tiles.
template <int G, int kUnit>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, int64_t n_q,
    int64_t Hkv, int kv_div, int64_t T_cap, int64_t p0, const int32_t *__restrict__ ids, int k,
    int sink, float scale_log2, float scale, float *__restrict__ dK, float *__restrict__ dV,
    float *__restrict__ part, int *__restrict__ counters)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];
    __shared__ int blist[kMaxBlocksDkdv];
    __shared__ uint8_t bmask[kMaxBlocksDkdv];
    __shared__ uint8_t rmask[kMaxBlocksDkdv];   // by block: the scan's result
    __shared__ int blist_n;
    __shared__ int is_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // grid (Hkv, kv_div, blocks * kSplit)
    const int64_t gkv = blockIdx.x;                         // kv head
    const int64_t g = gkv * kv_div + blockIdx.y;            // routing unit: its id rows
    const int split = (int)(blockIdx.z % kSplit);
    const int64_t a = blockIdx.z / kSplit;       // active chunk = its own query block
    const int64_t n_blocks = n_q / kC;
    const int64_t ca = p0 / kC + a;               // absolute chunk index

    // Query blocks that attend chunk a: its own (causal) and every later block
    // whose routed ids list it (or, for group ids, any of its groups) -- every
    // later block if the chunk lies in the sink window -- in ascending block
    // order, each with the mask of the chunk's groups it attends. The four waves scan the later blocks' id rows (wave w: blocks
    // a+1+w, a+5+w, ...), each row spread over the 64 lanes and kScanRows rows
    // loaded before any is used; the masks land in LDS by block and wave 0
    // then lists the blocks in order.
    {
        constexpr int kScanRows = 4;
        const int32_t ca32 = (int32_t)ca;
        for (int64_t base = a + 1 + wave; base < n_blocks; base += 4 * kScanRows) {
            uint32_t msk[kScanRows];
#pragma unroll
            for (int rr = 0; rr < kScanRows; ++rr) msk[rr] = 0u;
            for (int c0 = 0; c0 < k; c0 += 64) {
                int32_t u[kScanRows];
#pragma unroll
                for (int rr = 0; rr < kScanRows; ++rr) {
                    const int64_t bb = base + 4 * rr;
                    u[rr] = (bb < n_blocks && c0 + lane < k)
                                ? ids[(g * n_blocks + bb) * k + c0 + lane] : -1;
                }
#pragma unroll
                for (int rr = 0; rr < kScanRows; ++rr) {
                    if constexpr (kUnit == kC) {
                        msk[rr] |= __ballot(u[rr] == ca32) != 0 ? 0xFFu : 0u;
                    } else {
                        const bool in = (u[rr] >> 3) == ca32;
#pragma unroll
                        for (int bit = 0; bit < 8; ++bit)
                            msk[rr] |= __ballot(in && (u[rr] & 7) == bit) != 0 ? 1u << bit : 0u;
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < kScanRows; ++rr) {
                const int64_t bb = base + 4 * rr;
                if (ca < sink) msk[rr] = 0xFFu;
                if (lane == 0 && bb < n_blocks) rmask[bb] = (uint8_t)msk[rr];
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        if (lane == 0) {
            blist[0] = (int)a;
            bmask[0] = 0xFF;
        }
        int cnt = 1;
        for (int64_t base = a + 1; base < n_blocks; base += 64) {
            const int64_t bb = base + lane;
            const uint32_t msk = bb < n_blocks ? rmask[bb] : 0u;
            const bool hit = msk != 0;
            const uint64_t m = __ballot(hit);
            if (hit) {
                blist[cnt + lanes_below(m)] = (int)bb;
                bmask[cnt + lanes_below(m)] = (uint8_t)msk;
            }
            cnt += __popcll(m);
        }
        if (lane == 0) blist_n = cnt;
    }
    __syncthreads();
    // The chunk's query tiles -- (listed block, query head) pairs, block-major
    // -- are dealt round-robin to n_parts workgroups: this one takes tiles
    // split, split + n_parts, ... (tile T: block blist[T / G], head T % G).
    const int n_list = blist_n;
    const int n_all = n_list * G;
    const int n_parts = min(kSplit, max(1, (n_all + kMinTiles - 1) / kMinTiles));
    if (split >= n_parts) return;                 // nothing dealt to this workgroup
    const int n_tiles = (n_all - split + n_parts - 1) / n_parts;

    const int col = lane & 31;
    const int half = lane >> 5;
    const int kh = wave & 1;         // keys 32*kh .. +32 of the chunk
    const int qh = wave >> 1;        // queries 32*qh .. +32 of each tile
    const int64_t key_row = ca * kC + 32 * kh + col;
    bf16x8 kb[8], vb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        kb[ks] = *(const bf16x8 *)(K + (gkv * T_cap + key_row) * kD + 16 * ks + 8 * half);
        vb[ks] = *(const bf16x8 *)(V + (gkv * T_cap + key_row) * kD + 16 * ks + 8 * half);
    }

    auto tile_row0 = [&](int t) __attribute__((always_inline)) -> int64_t {
        const int T = split + n_parts * min(t, n_tiles - 1);
        const int64_t bb = blist[T / G];
        const int64_t hh = g * G + T % G;
        return hh * n_q + bb * kC;
    };
    // Tile loader (all 256 threads): lane takes rows 4*kg .. 4*kg+3 of the
    // 8-wide d slice dp of the Q and dO tiles (kg = lane%16, dp = 4*wave +
    // lane/16), lse and Delta of the tile's queries on threads 0..63.
    struct TileIn { u32x4 q[4], d[4]; float l, dl; };
    const int lkg = lane & 15, ldp = 4 * wave + (lane >> 4);
    auto load = [&](TileIn &r, int t) __attribute__((always_inline)) {
        const int64_t row0 = tile_row0(t);
        const uint16_t *qs = Q + (row0 + 4 * lkg) * kD + ldp * 8;
        const uint16_t *ds = dO + (row0 + 4 * lkg) * kD + ldp * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r.q[j] = *(const u32x4 *)(qs + j * kD);
            r.d[j] = *(const u32x4 *)(ds + j * kD);
        }
        const int qi = tid & (kC - 1);
        r.l = lse[row0 + qi];
        r.dl = delta[row0 + qi];
    };
    // Q and dO to LDS row-major (S and dP operands) and transposed under the
    // accumulator's query permutation (dK and dV operands); with kg = lane%16
    // the 8-byte transposed writes of the 64 lanes fall on distinct banks.
    auto store = [&](const TileIn &r, int buf) __attribute__((always_inline)) {
        uint8_t *B = smem + buf * kBufBytes;
        uint16_t *Qs = (uint16_t *)(B + kQOff), *dOs = (uint16_t *)(B + kDOOff);
        uint16_t *Qts = (uint16_t *)(B + kQtOff), *dOts = (uint16_t *)(B + kDOtOff);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *(u32x4 *)(Qs + (4 * lkg + j) * kRowStride + ldp * 8) = r.q[j];
            *(u32x4 *)(dOs + (4 * lkg + j) * kRowStride + ldp * 8) = r.d[j];
        }
        const int pos = t_pos(4 * lkg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 wq, wd;
            wq[0] = __builtin_amdgcn_perm(r.q[1][e >> 1], r.q[0][e >> 1], sel);
            wq[1] = __builtin_amdgcn_perm(r.q[3][e >> 1], r.q[2][e >> 1], sel);
            wd[0] = __builtin_amdgcn_perm(r.d[1][e >> 1], r.d[0][e >> 1], sel);
            wd[1] = __builtin_amdgcn_perm(r.d[3][e >> 1], r.d[2][e >> 1], sel);
            *(u32x2 *)(Qts + (8 * ldp + e) * kTStride + pos) = wq;
            *(u32x2 *)(dOts + (8 * ldp + e) * kTStride + pos) = wd;
        }
        if (tid < kC) {
            ((float *)(B + kLseOff))[tid] = r.l * 1.44269504088896340736f;
            ((float *)(B + kDlOff))[tid] = r.dl;
        }
    };
    // Tiles run in pairs (register sets r0, r1 in a fixed order, loaded two
    // tiles ahead); an odd count gets one padding step that computes nothing.
    const int n_steps = n_tiles + (n_tiles & 1);
    TileIn r0, r1;
    load(r0, 0);
    load(r1, 1);
    store(r0, 0);
    __syncthreads();

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

    auto step = [&](int it, TileIn &pre, const TileIn &nxt) __attribute__((always_inline)) {
        const int buf = it & 1;
        load(pre, it + 2);
        if (it < n_tiles) {
        const uint8_t *B = smem + buf * kBufBytes;
        const uint16_t *Qb = (const uint16_t *)(B + kQOff);
        const uint16_t *dOb = (const uint16_t *)(B + kDOOff);
        const uint16_t *Qtb = (const uint16_t *)(B + kQtOff);
        const uint16_t *dOtb = (const uint16_t *)(B + kDOtOff);
        const float *lse2s = (const float *)(B + kLseOff);
        const float *dls = (const float *)(B + kDlOff);

        // S[q][key] = Q K^T, dP[q][key] = dO V^T for this wave's 32 x 32 block
        // (A operands read from LDS two k-steps ahead of their MFMAs).
        f32x16 s = zero16(), dp = zero16();
        {
            bf16x8 qa[8], da[8];
            auto rd = [&](int ks) __attribute__((always_inline)) {
                const int off = (32 * qh + col) * kRowStride + 16 * ks + 8 * half;
                qa[ks] = *(const bf16x8 *)(Qb + off);
                da[ks] = *(const bf16x8 *)(dOb + off);
            };
            rd(0);
            rd(1);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (ks + 2 < 8) rd(ks + 2);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kb[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], vb[ks], dp, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // lane: key 32*kh + col; queries 32*qh + 8u + 4*half + e (j = 4u + e).
        // P and dS stay fp32 in s and dp; their bf16 hi halves feed the MFMAs.
        const int entry = (split + n_parts * it) / G;    // list entry of this tile
        const bool diag = entry == 0;                    // entry 0 is the own block
        // (group ids: this lane's key is dropped unless its group was chosen)
        const bool kept = kUnit == kC ||
                          ((bmask[entry] >> ((32 * kh + col) >> 3)) & 1);
        bf16x8 pb[2], dsb[2];
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
                if ((diag && 32 * kh + col > q0 + e) || !kept) p = 0.f;
                big |= p > kPairAbove;
                s[j] = p;
                dp[j] = p * (dp[j] - d4[e]);
                pb[j >> 3][j & 7] = (__bf16)s[j];
                dsb[j >> 3][j & 7] = (__bf16)dp[j];
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS (k runs over this wave's 32 queries);
        // the 16 transposed operands are read before the MFMAs that use them
        // and serve the low-half round too.
        bf16x8 ta[8], tq[8];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = (32 * dt + col) * kTStride + 32 * qh + 16 * ks + 8 * half;
                ta[2 * dt + ks] = *(const bf16x8 *)(dOtb + off);
                tq[2 * dt + ks] = *(const bf16x8 *)(Qtb + off);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[2 * dt + ks], pb[ks], dv[dt], 0, 0, 0);
                dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[2 * dt + ks], dsb[ks], dk[dt], 0, 0, 0);
            }
        if (__ballot(big) != 0) {              // wave-uniform: add the low halves
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                pb[j >> 3][j & 7] = (__bf16)(s[j] - (float)pb[j >> 3][j & 7]);
                dsb[j >> 3][j & 7] = (__bf16)(dp[j] - (float)dsb[j >> 3][j & 7]);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[2 * dt + ks], pb[ks], dv[dt], 0, 0, 0);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[2 * dt + ks], dsb[ks], dk[dt], 0, 0, 0);
                }
        }
        }
        if (it + 1 < n_steps) store(nxt, buf ^ 1);
        __syncthreads();
    };
    for (int it = 0; it < n_steps; it += 2) {
        step(it, r0, r1);
        step(it + 1, r1, r0);
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
    const int64_t part_stride = Hkv * kv_div * n_q * kD;   // floats per (split, tensor)
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

// Per-query-head routing: dK, dV of kv head g are the sums over its query
// heads of each head's own contribution (dkdv ran per head into dKu, dVu
// [Hq][n_q][D]); added in head order.
__global__ __launch_bounds__(256) void sum_heads_kernel(
    const float *__restrict__ dKu, const float *__restrict__ dVu, int64_t n_vec, int G,
    int64_t per_head, float *__restrict__ dK, float *__restrict__ dV)
{
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index in dK
    if (v >= n_vec) return;
    const int64_t g = v / per_head, r = v % per_head;
    const f32x4 *sk = (const f32x4 *)dKu + g * G * per_head + r;
    const f32x4 *sv = (const f32x4 *)dVu + g * G * per_head + r;
    f32x4 ak = sk[0], av = sv[0];
    for (int hh = 1; hh < G; ++hh) {
        const f32x4 xk = sk[hh * per_head], xv = sv[hh * per_head];
#pragma unroll
        for (int e = 0; e < 4; ++e) { ak[e] += xk[e]; av[e] += xv[e]; }
    }
    ((f32x4 *)dK)[v] = ak;
    ((f32x4 *)dV)[v] = av;
}

// G: query heads per routing unit (1 with per-query-head routing, where
// kv_div = query heads per kv head and dK/dV are then the per-head buffers).
template <int G, int kUnit>
hipError_t launch_bwd_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                        int64_t Hkv, int kv_div, int64_t T_cap, int64_t p0, int64_t n_q,
                        const int32_t *ids, int32_t k, int32_t sink, float scale, const float *lse,
                        const uint16_t *dO, float *dQ, float *dK, float *dV,
                        float *delta, int *counters, float *part, hipStream_t stream)
{
    constexpr int NHG = G < 4 ? 1 : G / 4;
    const int64_t n_blocks = n_q / kC;
    const float scale_log2 = scale * 1.44269504088896340736f;
    if (n_blocks * kSplit > 65535) return hipErrorInvalidConfiguration;     // grid z limit
    hipLaunchKernelGGL((bwd_dq_kernel<G, kUnit>),
                       dim3((unsigned)Hkv, (unsigned)(kv_div * NHG), (unsigned)n_blocks),
                       dim3(kDqThreads), 0,
                       stream, Q, K, V, dO, lse, delta, counters, n_q, kv_div, T_cap, p0,
                       ids, k, (int)sink, scale_log2, scale, dQ);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<G, kUnit>),
                       dim3((unsigned)Hkv, (unsigned)kv_div, (unsigned)(n_blocks * kSplit)),
                       dim3(kThreads), 0,
                       stream, Q, K, V, dO, lse, delta, n_q, Hkv, kv_div, T_cap, p0, ids, k,
                       (int)sink, scale_log2, scale, dK, dV, part, counters);
    return hipGetLastError();
}

// Workspace layout (U routing units: Hkv, or Hq with per-query-head routing):
// Delta [Hq][n_q] f32 | counters [U][n_q/C] int32 | partial sums
// [kSplit][dK, dV][U][n_q][D] f32 | per-query-head routing only: each head's
// dK and dV, [2][Hq][n_q][D] f32. Every part starts on a 256-byte boundary.
struct BwdWorkspace {
    size_t delta_off, counter_off, part_off, head_off, total;
};

BwdWorkspace bwd_layout(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t U = per_q_head ? Hq : Hkv;
    BwdWorkspace w;
    w.delta_off = 0;
    w.counter_off = up((size_t)(Hq * n_q) * sizeof(float));
    w.part_off = w.counter_off + up((size_t)(U * (n_q / kC)) * sizeof(int));
    w.head_off = w.part_off + (size_t)kSplit * 2 * (size_t)(U * n_q * kD) * sizeof(float);
    w.total = w.head_off + (per_q_head ? 2 * (size_t)(Hq * n_q * kD) * sizeof(float) : 0);
    return w;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head)
{
    return bwd_layout(Hq, Hkv, n_q, per_q_head).total;
}

int64_t bwd_max_queries() { return (int64_t)kMaxBlocksDkdv * kC; }

namespace {

template <int kUnit>
hipError_t launch_bwd_unit(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                           int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                           const int32_t *ids, int32_t k, int32_t sink, bool per_q_head,
                           float scale, const float *lse, const uint16_t *dO, float *dQ,
                           float *dK, float *dV, void *workspace, hipStream_t stream)
{
    if (n_q == 0) return hipSuccess;
    const BwdWorkspace w = bwd_layout(Hq, Hkv, n_q, per_q_head);
    uint8_t *ws = (uint8_t *)workspace;
    float *delta = (float *)(ws + w.delta_off);
    int *counters = (int *)(ws + w.counter_off);
    float *part = (float *)(ws + w.part_off);
    const int G = (int)(Hq / Hkv);
    if (per_q_head) {
        float *dKu = (float *)(ws + w.head_off);
        float *dVu = dKu + Hq * n_q * kD;
        hipError_t e = launch_bwd_g<1, kUnit>(Q, K, V, Hkv, G, T_cap, p0, n_q, ids, k, sink,
                                              scale, lse, dO, dQ, dKu, dVu, delta, counters,
                                              part, stream);
        if (e != hipSuccess) return e;
        const int64_t per_head = n_q * kD / 4, n_vec = Hkv * per_head;
        hipLaunchKernelGGL(sum_heads_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256),
                           0, stream, dKu, dVu, n_vec, G, per_head, dK, dV);
        return hipGetLastError();
    }
    switch (G) {
    case 1: return launch_bwd_g<1, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 2: return launch_bwd_g<2, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 4: return launch_bwd_g<4, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    case 8: return launch_bwd_g<8, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, lse, dO, dQ, dK, dV, delta, counters, part, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attend_bwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                             int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                             int64_t n_q, const int32_t *ids, int32_t k, int32_t sink,
                             bool per_q_head, float scale, const uint16_t *O, const float *lse,
                             const uint16_t *dO, float *dQ, float *dK, float *dV,
                             void *workspace, hipStream_t stream)
{
    (void)O;    // Delta is recomputed from P and dP (see the dq kernel)
    return launch_bwd_unit<kC>(Q, K, V, Hq, Hkv, T_cap, p0, n_q, ids, k, sink, per_q_head,
                               scale, lse, dO, dQ, dK, dV, workspace, stream);
}

hipError_t launch_attend_bwd_groups(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                    int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                    int64_t n_q, const int32_t *gids, int32_t m, int32_t sink,
                                    float scale, const float *lse, const uint16_t *dO, float *dQ,
                                    float *dK, float *dV, void *workspace, hipStream_t stream)
{
    return launch_bwd_unit<kGroup>(Q, K, V, Hq, Hkv, T_cap, p0, n_q, gids, m, sink, false,
                                   scale, lse, dO, dQ, dK, dV, workspace, stream);
}

}  // namespace hga
