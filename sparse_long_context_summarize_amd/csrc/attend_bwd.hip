// attend_bwd.hip -- segment-wise backward of the routed attention
// (arXiv 2607.15105, gist.science technical summary 2.2: every segment is
// back-propagated on its own and the key/value history before it is detached;
// technical summary 2.1: the routing choice carries no gradient).
//
// Two kernels; no output element is accumulated with atomics and every sum
// runs in a fixed order, so results are bitwise reproducible:
//   dq     query-major, the forward's work unit (query block x kv head) and
//          wave layout (8 waves, two per SIMD, 32 queries of one head each),
//          one pass over the routed chunks and the causal local block, a
//          second one only where the first cannot be trusted:
//          pass 1: S^T = K Q^T, dP^T = V dO^T, P = exp(S - lse),
//                  Delta_i = sum_j P_ij dP_ij exactly (fp32; written for dkdv)
//                  and, against the estimate D_i = dO_i . O_i from the bf16 O,
//                  dS = P (dP - D), dQ^T += K^T dS^T, M_i = sum_j P_ij |dP_ij - D_i|.
//          The estimate's error e_i = Delta_i - D_i moves dQ_i by
//          +scale e_i sum_j P_ij K_j, at most |e_i| max_j |K_j| elementwise;
//          rounding every dS term to bf16 once (unit roundoff 2^-8) may move
//          it by up to 2^-8 M_i max_j |K_j|. A wave whose rows all have
//          |e_i| <= 2^-8 M_i keeps pass 1. The others -- attention sitting on
//          a few keys, where O's rounding lands undamped on dS, or no O
//          given -- recompute dQ in pass 2 with the exact Delta (the
//          workgroup walks its tiles again; waves that kept pass 1 only load):
//          dS = P (dP - Delta), dQ^T += K^T dS^T.
//          K^T sits in LDS under the accumulator's key permutation, as V^T
//          does in the forward.
//   dkdv   key-major over the active chunks only (history is detached): the
//          dq workgroup of block a also lists the later blocks whose ids chose
//          chunk a (the dkdv plan); the list's (block, query head) tiles, own
//          block first, are dealt round-robin to up to kSplit parts, and a
//          persistent grid (one workgroup per CU) takes (chunk, unit, part)
//          items from a work queue, largest parts first:
//          S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//          Wave w owns keys 32*(w&1).. and queries 32*(w>>1).. of each query
//          tile; the two query halves are summed through LDS. A chunk with
//          at most kMinTiles tiles is one part, which writes the result
//          directly; a longer one is split, every part stores its partial
//          sums at device scope (the first into the chunk's own dK / dV rows,
//          the others into workspace slots) and the last one to finish (a
//          per-chunk counter) adds the partials in part order and writes the
//          result. This spreads the chunks that many blocks chose (routing
//          concentrates on high-scoring chunks) over several CUs.
// Both kernels load their tiles two steps ahead into registers (two sets
// used in a fixed order, steps run in pairs) and write them to double-buffered
// LDS one barrier before use; transposed copies are written with byte
// permutes in a lane order whose 8-byte writes fall on distinct banks.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <vector>

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
// The dq kernel keeps its one-pass dQ for a row when the Delta estimate from
// the bf16 O is off by at most this fraction of sum_j P_ij |dP_ij - D_i|:
// bf16's unit roundoff, so the estimate moves dQ by no more than the
// worst-case bound of rounding every dS term to bf16 once.
constexpr float kDeltaEstTol = 1.0f / 256.0f;

__device__ __forceinline__ int t_pos(int kk) {   // swap bits 2 and 3
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = 0.f;
    return z;
}

// ----------------------------------------------------------- the dkdv plan

// The query blocks that attend active chunk a of routing unit g: its own
// block (causal) and every later block whose id row lists it (or, for group
// ids, any of its groups) -- every later block if the chunk lies in the sink
// window -- in ascending block order, each with the mask of the chunk's
// groups it attends. The dq workgroup of block a (whose unit and block the
// dkdv workgroups of chunk a share) finds them and stores them for the dkdv
// kernel: plan_n[g][a] entries of plan_blk[g][a][.] (block ids) and
// plan_msk[g][a][.] (group masks).
//
// Scan, by four waves (wave w of them: blocks a+1+w, a+5+w, ...; each id row
// spread over the 64 lanes, kScanRows rows loaded before any is used, so up
// to 32 later blocks take one memory round trip): the mask by block into
// rmask (LDS, n_blocks entries).
template <int kUnit>
__device__ __forceinline__ void plan_scan(const int32_t *__restrict__ ids, int64_t g, int64_t a,
                                          int64_t n_blocks, int k, int64_t ca, int sink,
                                          int wave4, uint8_t *rmask)
{
    constexpr int kScanRows = 8;
    const int lane = threadIdx.x & 63;
    const int32_t ca32 = (int32_t)ca;
    for (int64_t base = a + 1 + wave4; base < n_blocks; base += 4 * kScanRows) {
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

// Compaction of the scan (one wave, after a barrier): the plan entries of
// chunk a, own block first, then the hit blocks in ascending order.
__device__ __forceinline__ void plan_store(const uint8_t *rmask, int64_t a, int64_t n_blocks,
                                           int *plan_n, uint16_t *plan_blk, uint8_t *plan_msk)
{
    const int lane = threadIdx.x & 63;
    if (lane == 0) {
        plan_blk[0] = (uint16_t)a;
        plan_msk[0] = 0xFF;
    }
    int cnt = 1;
    for (int64_t base = a + 1; base < n_blocks; base += 64) {
        const int64_t bb = base + lane;
        const uint32_t msk = bb < n_blocks ? rmask[bb] : 0u;
        const bool hit = msk != 0;
        const uint64_t m = __ballot(hit);
        if (hit) {
            plan_blk[cnt + lanes_below(m)] = (uint16_t)bb;
            plan_msk[cnt + lanes_below(m)] = (uint8_t)msk;
        }
        cnt += __popcll(m);
    }
    if (lane == 0) *plan_n = cnt;
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
// lane pair). Steps walk the tile list once, or twice when a wave needs pass
// 2 (a vote by wave after pass 1; only the waves that voted compute in the
// second walk, the others load and wait at its barriers); tiles are loaded two steps ahead into
// registers and written to double-buffered LDS one barrier before use. Each
// 64-key tile is processed as two 32-key halves. O (bf16, may be NULL) only
// feeds the Delta estimate of pass 1; without it pass 1 forms Delta alone.
// kUnit = kC: ids are chunk ids. kUnit = kGroup: ids are 8-token group ids;
// each routed tile is gathered from 8 groups, and a last routed tile with
// fewer masks its missing groups' keys.
template <int G, int kUnit>
__global__ __launch_bounds__(kDqThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ O,
    const float *__restrict__ lse, float *__restrict__ delta, int *__restrict__ counters,
    int *__restrict__ next_item, int *__restrict__ plan_n, uint16_t *__restrict__ plan_blk,
    uint8_t *__restrict__ plan_msk, uint8_t *__restrict__ redo_flags,
    int64_t n_q, int kv_div, int64_t T_cap, int64_t p0,
    const int32_t *__restrict__ ids, int k, int sink, float scale_log2, float scale,
    float *__restrict__ dQ)
{
    constexpr int HW = G < 4 ? G : 4;
    constexpr int NHG = G / HW;
    // One query head per workgroup (G = 1, or per-query-head routing): the
    // two 32-key halves of each tile go to two waves on different SIMDs
    // (four computing waves instead of two), whose dQ partials are added at
    // the end.
    constexpr int KSPLIT = HW == 1 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kRowTile];
    __shared__ __attribute__((aligned(16))) uint16_t Kts[2][kTTile];
    __shared__ int list[(kUnit == kC ? kChunkListMax : kGroupListMax) + 1];
    __shared__ int list_n;
    __shared__ int redo[kDqThreads / 64];       // pass 2 votes, by wave
    __shared__ float dl_s[kDqThreads];          // Delta_i partial sums, one slot a thread
    __shared__ float mabs_s[kDqThreads];        // M_i partial sums, one slot a thread
    __shared__ uint8_t rmask[kMaxBlocksDkdv];   // the dkdv plan's scan, by block

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

    // (as in the forward: with HW < 4 the two query halves' waves sit on
    // different SIMDs)
    const int qt = wave >> 2;
    const int lane4 = wave & 3;
    // (KSPLIT = 2: waves 0, 2 take queries 0-31, waves 5, 7 queries 32-63,
    // the key half kth = lane4 / 2 each)
    const bool computes = KSPLIT == 2 ? (lane4 & 1) == qt : lane4 / HW == qt % (4 / HW);
    const int kth = KSPLIT == 2 ? lane4 >> 1 : 0;
    const int hw = lane4 % HW;                   // head slot
    const int64_t h = g * G + hg * HW + hw;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t qrow = h * n_q + b * kC + 32 * qt + col;
    bf16x8 qf[8], df[8], of[8];
    float lse2 = 0.f;
    const bool fast = O != nullptr;
    // Q^T and dO^T (MFMA operands for the whole kernel) and the O row go out
    // first, ahead of the list barrier: the plan-scan waves issue theirs after
    // their scan loads, wave 0 after its id row (loads complete in order).
    auto load_qdo = [&]() __attribute__((always_inline)) {
        if (!computes) return;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = *(const bf16x8 *)(Q + qrow * kD + 16 * ks + 8 * half);
            df[ks] = *(const bf16x8 *)(dO + qrow * kD + 16 * ks + 8 * half);
        }
        if (fast) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                of[ks] = *(const bf16x8 *)(O + qrow * kD + 16 * ks + 8 * half);
        }
        lse2 = lse[qrow] * 1.44269504088896340736f;
    };
    // the sink window's units, the routed units (past the sink, before P,
    // repeats dropped), then the local chunk
    if (wave == 0) {
        const int32_t *id_row = ids + (g * n_blocks + b) * k;
        const int id_first = lane < k ? id_row[lane] : -1;
        load_qdo();
        const int ns = sink_units(sink, P, kUnit);
        write_sink_units(list, ns);
        const int n = build_unit_list(id_row, k, (int64_t)sink * (kC / kUnit), P / kUnit,
                                      list + ns, id_first);
        if (lane == 0) {
            list[ns + n] = (int)local_chunk;
            list_n = ns + n + 1;
        }
    } else if (!(hg == 0 && wave >= 4)) {
        load_qdo();
    }
    if (lane == 0) redo[wave] = fast ? 0 : 1;
    dl_s[tid] = 0.f;
    mabs_s[tid] = 0.f;
    // the dkdv kernel that follows counts finished workgroups per (unit, chunk)
    if (hg == 0 && tid == 0) counters[g * n_blocks + b] = 0;
    if (g == 0 && b == 0 && hg == 0 && tid == 0) *next_item = 0;
    // waves 4..7 scan for the dkdv plan of chunk b (stored after the second
    // barrier below) while wave 0 lists the block's own tiles
    if (hg == 0 && wave >= 4) {
        plan_scan<kUnit>(ids, g, b, n_blocks, k, p0 / kC + b, sink, wave - 4, rmask);
        load_qdo();
    }
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
    if (hg == 0 && wave == 4) {
        const int64_t pr = g * n_blocks + b;
        plan_store(rmask, b, n_blocks, plan_n + pr, plan_blk + pr * n_blocks,
                   plan_msk + pr * n_blocks);
    }
    // the Delta estimate D_i = dO_i . O_i (this lane's 64 dims, then its
    // partner's), subtracted from dP in pass 1
    float dsub = 0.f;
    if (fast && computes) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dsub = fmaf((float)df[ks][e], (float)of[ks][e], dsub);
        dsub += partner32(dsub);
    }

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
        // (no scheduling barrier here: left to the compiler, these MFMAs mix
        // with the neighbouring work; 0.6 us a call faster than pinned)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks + 1 < 8) rd(ks + 1);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], df[ks], dp, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], scale_log2, -lse2));
        if (mode != 0) {             // (wave-uniform: one tile in 17 at the 16K layer)
            const int thr = mode == 1 ? 32 * (qt - kt) + col - 4 * half
                                      : pad_keys - 32 * kt - 4 * half - 1;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (8 * (j >> 2) + (j & 3) > thr) s[j] = 0.f;
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

    // dQ^T += K^T dS^T with dS = P (dP - dsub): dS enters the MFMAs as bf16
    // hi; halves holding a probability above kPairAbove add the rounding
    // remainder lo = bf16(dS - hi) in a second round (wave-uniform branch).
    // Pass 1 (kFirst) also sums Delta_i = sum_j P_ij dP_ij (exactly: it
    // does not lean on the estimate) and M_i = sum_j |dS_ij| =
    // sum_j P_ij |dP_ij - dsub|; without O it forms Delta only.
    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();
    // (the partial sums of Delta_i and M_i wait in LDS, one slot a thread,
    // updated once a half: two more loop-carried registers made the register
    // allocator spill, and LDS float atomics for the update took the whole
    // pass from ~2.6 to ~4.7 us a tile)
    auto pass = [&](int buf, int mode, auto first) __attribute__((always_inline)) {
        constexpr bool kFirst = decltype(first)::value;
        const uint16_t *Ktb = Kts[buf];
#pragma unroll
        for (int kk = 0; kk < 2 / KSPLIT; ++kk) {
            const int kt = KSPLIT == 2 ? kth : kk;
            f32x16 s, dp;
            sdp(buf, kt, mode, s, dp);
            float pm = s[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) pm = fmaxf(pm, s[j]);
            const bool pair = __ballot(pm > kPairAbove) != 0;
            float d = 0.f;
            if constexpr (kFirst) {
#pragma unroll
                for (int j = 0; j < 16; ++j) d = fmaf(s[j], dp[j], d);
            }
            bf16x8 dsh[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                dp[j] = s[j] * (dp[j] - dsub);
                dsh[j >> 3][j & 7] = (__bf16)dp[j];
            }
            if constexpr (kFirst) {
                float m = 0.f;                  // M_i: sum_j |dS_ij|
#pragma unroll
                for (int j = 0; j < 16; ++j) m += fabsf(dp[j]);
                dl_s[tid] += d;
                mabs_s[tid] += m;
                if (!fast) continue;
            }
            // K^T operands (dQ^T tile i&3, key step i>>2) read two MFMAs ahead,
            // the order pinned by scheduling barriers (left free, the compiler
            // placed each read behind the MFMA before it and waited on it)
            auto kt_rd = [&](int i) __attribute__((always_inline)) {
                return *(const bf16x8 *)(Ktb + (32 * (i & 3) + col) * kTStride +
                                         16 * (2 * kt + (i >> 2)) + 8 * half);
            };
            auto dq_mfmas = [&](const bf16x8 (&ds)[2]) __attribute__((always_inline)) {
                bf16x8 a[3];
                a[0] = kt_rd(0);
                a[1] = kt_rd(1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i + 2 < 8) a[(i + 2) % 3] = kt_rd(i + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % 3], ds[i >> 2], acc[i & 3], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            dq_mfmas(dsh);
            if (pair) {
                bf16x8 dsl[2];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    dsl[j >> 3][j & 7] = (__bf16)(dp[j] - (float)dsh[j >> 3][j & 7]);
                dq_mfmas(dsl);
            }
        }
    };
    auto pass1 = [&](int buf, int mode) __attribute__((always_inline)) {
        pass(buf, mode, std::true_type{});
    };
    auto pass2 = [&](int buf, int mode) __attribute__((always_inline)) {
        pass(buf, mode, std::false_type{});
    };
    for (int st = 0; st < n_pass; st += 2) {
        step(st, r0, r1, pass1);
        step(st + 1, r1, r0, pass1);
    }
    // Delta complete: join the two half-waves' key subsets, publish for dkdv;
    // a row whose estimate missed by more than kDeltaEstTol M_i (or is not
    // finite) sends its wave through pass 2
    float dl, mabs;
    if constexpr (KSPLIT == 2) {     // the two key halves' waves: tid and tid ^ 128
        const int t0 = tid & ~128;
        dl = dl_s[t0] + dl_s[t0 | 128];
        mabs = mabs_s[t0] + mabs_s[t0 | 128];
    } else {
        dl = dl_s[tid];
        mabs = mabs_s[tid];
    }
    dl += partner32(dl);
    mabs += partner32(mabs);
    if (computes && half == 0 && kth == 0) delta[qrow] = dl;
    // (an estimate or M that is not finite -- O holding Inf or NaN -- never
    // passes: inf <= inf would)
    const bool keep = __builtin_isfinite(dsub) && __builtin_isfinite(mabs) &&
                      fabsf(dl - dsub) <= kDeltaEstTol * mabs;
    if (__ballot(computes && !keep) != 0 && lane == 0) redo[wave] = 1;
    __syncthreads();
    const bool my_redo = redo[wave] != 0;
    int any_redo = 0;
#pragma unroll
    for (int w = 0; w < kDqThreads / 64; ++w) any_redo |= redo[w];
    if (tid == 0) redo_flags[(g * NHG + hg) * n_blocks + b] = (uint8_t)(any_redo != 0);
    if (any_redo) {
        if (my_redo) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();
            dsub = dl;
        }
        auto pass2w = [&](int buf, int mode) __attribute__((always_inline)) {
            if (my_redo) pass2(buf, mode);
        };
        for (int st = n_pass; st < n_steps; st += 2) {
            step(st, r0, r1, pass2w);
            step(st + 1, r1, r0, pass2w);
        }
    }

    if constexpr (KSPLIT == 2) {
        // the key-half-1 waves hand their dQ partials to the key-half-0 waves
        // through the K^T tiles (free after the last barrier), added in that order
        float *xf = (float *)&Kts[0][0] + qt * (4 * 16 * 64);
        static_assert(2 * 4 * 16 * 64 * sizeof(float) <= sizeof(Kts), "partials fit");
        if (computes && kth == 1) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * u + e];
                    *(f32x4 *)(xf + ((dt * 4 + u) * 64 + lane) * 4) = v;
                }
        }
        __syncthreads();
        if (computes && kth == 0) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x4 v = *(const f32x4 *)(xf + ((dt * 4 + u) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[dt][4 * u + e] += v[e];
                }
        }
    }
    if (!computes || kth != 0) return;
    // dQ leaves through the wave's own LDS area (the tiles are free after the
    // last barrier; waves 0-3 use Ks, 4-7 Vs), half a row at a time, so that
    // every store instruction writes four whole 256-byte row halves, as
    // non-temporal stores (nothing reads dQ again here, and no dirty lines
    // are left for the end-of-kernel write-back).
    constexpr int kStage = kD / 2 + 4;          // floats per staged half row
    float *st = (float *)(wave < 4 ? &Ks[0][0] : &Vs[0][0]) + (wave & 3) * 32 * kStage;
    const int64_t row0 = h * n_q + b * kC + 32 * qt;
    const int piece = lane & 15;
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
#pragma unroll
        for (int dt = 2 * hd; dt < 2 * hd + 2; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * u + e] * scale;
                *(f32x4 *)(st + col * kStage + 32 * (dt - 2 * hd) + 8 * u + 4 * half) = v;
            }
        // (a wave's LDS accesses complete in order: its reads see its writes)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            __builtin_nontemporal_store(*(const f32x4 *)(st + r * kStage + 4 * piece),
                                        (f32x4 *)(dQ + (row0 + r) * kD + 64 * hd + 4 * piece));
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

// A chunk's query tiles go to up to kSplit workgroups, at least kMinTiles
// tiles each. Routing concentrates on a few high-scoring chunks (at the 16K
// backward workload one chunk has 52 (block, head) tiles, the mean is 7.4,
// and 171 of the 256 (chunk, unit) pairs have only their own block's 4), so
// the kernel's time is set by how the parts are packed onto the CUs: an item
// costs about 5 us of set-up and epilogue plus 2-2.7 us per tile (measured).
constexpr int kSplit = 8;
constexpr int kMinTiles = 8;
// Work order: the items go in four size levels, largest first (parts of at
// least 9 tiles, 7-8, 5-6, then the rest), earlier chunks first within a
// level, so that small items fill in at the end instead of long ones starting
// late (a simulation of the measured item costs put this within 0.1 us of a
// full largest-first sort at the 16K backward workload). Every workgroup
// computes the same order from the plan lengths: a stable counting sort, its
// four counts packed in 16-bit fields of one 64-bit prefix sum. Up to
// kOrderUnits (chunk, unit) pairs and kOrderCap items; past that the items
// run in chunk order.
constexpr int kOrderUnits = 1024;
constexpr int kOrderCap = 4096;
constexpr int kOrderLevels = 4;
__device__ __forceinline__ int order_level(int tiles) {
    return tiles >= 9 ? 0 : tiles >= 7 ? 1 : tiles >= 5 ? 2 : 3;
}

// kUnit = kGroup: a later block may have chosen only some of the chunk's 8
// groups; the scan records them as an 8-bit mask per listed block, and the
// keys of the other groups get P = 0 in that block's tiles.
template <int G, int kUnit>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, int64_t n_q,
    int64_t Hkv, int kv_div, int64_t T_cap, int64_t p0, const int *__restrict__ plan_n,
    const uint16_t *__restrict__ plan_blk, const uint8_t *__restrict__ plan_msk,
    float scale_log2, float scale, float *__restrict__ dK, float *__restrict__ dV,
    float *__restrict__ part, int *__restrict__ counters, int *__restrict__ next_item)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kBufBytes];
    __shared__ int blist[kMaxBlocksDkdv];
    __shared__ uint8_t bmask[kMaxBlocksDkdv];
    __shared__ int is_last;
    __shared__ int item_s;
    __shared__ uint16_t order[kOrderCap];              // plan index << 4 | part
    __shared__ uint64_t o_wave[kThreads / 64];
    __shared__ uint16_t o_na[kOrderUnits];             // tiles of each (chunk, unit) pair
    __shared__ int o_total;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t n_blocks = n_q / kC;
    // Persistent: one workgroup per CU takes (chunk, unit, part) items from a
    // counter until none is left, in the size order built below (or, past
    // kOrderUnits pairs, in chunk order, earlier chunks first: more later
    // blocks can choose them, so their lists tend to be the longest).
    // (A grid of one workgroup per item left CUs idle: dispatch is in order
    // and stalls behind the busiest XCD, so the CUs freed by items with
    // nothing dealt were not refilled for tens of microseconds.)
    const int64_t n_units = Hkv * kv_div;
    const int64_t n_pairs = n_units * n_blocks;        // (unit, chunk) pairs: plan entries
    const int64_t n_items = n_pairs * kSplit;
    auto parts_of = [&](int n_all) __attribute__((always_inline)) {
        return min(kSplit, max(1, (n_all + kMinTiles - 1) / kMinTiles));
    };
    // (the first item is taken before the order is built: its round trip
    // overlaps the plan loads)
    if (tid == 0) item_s = atomicAdd(next_item, 1);
    bool sorted = n_pairs <= kOrderUnits;
    if (sorted) {
        // thread t takes pairs q = kPer t .. kPer t + kPer - 1 in chunk-major
        // order (q = a * n_units + g: plan index g * n_blocks + a); their tile
        // counts n_all wait in LDS. The parts of a pair hold ceil(n_all / np)
        // tiles (the first n_hi) or floor.
        constexpr int kPer = kOrderUnits / kThreads;
        auto plan_of = [&](int q) __attribute__((always_inline)) {
            return (int)((q % n_units) * n_blocks + q / n_units);
        };
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int q = kPer * tid + i;
            o_na[q] = q < n_pairs ? (uint16_t)(plan_n[plan_of(q)] * G) : (uint16_t)0;
        }
        auto split_of = [&](int n_all, int &np, int &n_hi, int &t_hi) __attribute__((always_inline)) {
            np = parts_of(n_all);
            t_hi = (n_all + np - 1) / np;
            n_hi = n_all % np == 0 ? np : n_all % np;
        };
        uint64_t mine = 0;                  // this thread's item counts by level
        for (int i = 0; i < kPer; ++i) {
            const int n_all = o_na[kPer * tid + i];
            if (n_all == 0) continue;
            int np, n_hi, t_hi;
            split_of(n_all, np, n_hi, t_hi);
            mine += (uint64_t)n_hi << (16 * order_level(t_hi));
            if (np > n_hi) mine += (uint64_t)(np - n_hi) << (16 * order_level(t_hi - 1));
        }
        // exclusive prefix over threads: within the wave, then across waves
        uint64_t incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t lo = __shfl_up((uint32_t)incl, o), hi = __shfl_up((uint32_t)(incl >> 32), o);
            if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
        }
        if (lane == 63) o_wave[wave] = incl;
        __syncthreads();
        uint64_t excl = incl - mine, total = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            const uint64_t v = o_wave[w];
            if (w < wave) excl += v;
            total += v;
        }
        int base[kOrderLevels];
        int start = 0;
#pragma unroll
        for (int l = 0; l < kOrderLevels; ++l) {
            base[l] = start + (int)((excl >> (16 * l)) & 0xFFFF);
            start += (int)((total >> (16 * l)) & 0xFFFF);
        }
        if (tid == 0) o_total = start;
        sorted = start <= kOrderCap;        // (the same in every thread)
        for (int i = 0; i < kPer && sorted; ++i) {
            const int q = kPer * tid + i;
            const int n_all = o_na[q];
            if (n_all == 0) continue;
            int np, n_hi, t_hi;
            split_of(n_all, np, n_hi, t_hi);
            for (int sp = 0; sp < np; ++sp) {
                const int l = order_level(sp < n_hi ? t_hi : t_hi - 1);
                int pos = 0;
#pragma unroll
                for (int m = 0; m < kOrderLevels; ++m)
                    if (m == l) pos = base[m]++;
                order[pos] = (uint16_t)((plan_of(q) << 4) | sp);
            }
        }
    }
    static_assert(kOrderLevels * 16 <= 64 && kOrderUnits * kSplit < 65536, "level counts fit 16 bits");
    static_assert(kOrderUnits * 16 <= 65536 && kSplit <= 16, "order entries fit 16 bits");
    static_assert(kOrderUnits % kThreads == 0, "whole pairs per thread");
    bool first = true;
    for (;;) {
        if (!first) {
            __syncthreads();                      // the last item is done with LDS
            if (tid == 0) item_s = atomicAdd(next_item, 1);
        }
        first = false;
        __syncthreads();
        const int64_t item = item_s;
        int split;
        int64_t g, a;
        if (sorted) {
            if (item >= o_total) break;
            const int e = order[item];
            split = e & 15;
            g = (e >> 4) / n_blocks;                    // routing unit: its id rows
            a = (e >> 4) % n_blocks;                    // active chunk = its own query block
        } else {
            if (item >= n_items) break;
            split = (int)(item % kSplit);
            g = (item / kSplit) % n_units;
            a = item / (kSplit * n_units);
        }
        const int64_t gkv = g / kv_div;                 // kv head
        const int64_t ca = p0 / kC + a;                 // absolute chunk index

        // The chunk's query tiles -- (listed block, query head) pairs, block-major
        // -- are dealt round-robin to n_parts workgroups: this one takes tiles
        // split, split + n_parts, ... (tile T: block blist[T / G], head T % G).
        // The list is the plan the dq kernel stored; a workgroup with nothing
        // dealt leaves after reading its length.
        const int64_t pr = g * n_blocks + a;
        const int n_list = plan_n[pr];
        const int n_all = n_list * G;
        const int n_parts = parts_of(n_all);
        if (split >= n_parts) continue;               // nothing dealt to this workgroup
        const int n_tiles = (n_all - split + n_parts - 1) / n_parts;
        const int col = lane & 31;
        const int half = lane >> 5;
        const int kh = wave & 1;         // keys 32*kh .. +32 of the chunk
        const int qh = wave >> 1;        // queries 32*qh .. +32 of each tile

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
        auto load_at = [&](TileIn &r, int64_t row0) __attribute__((always_inline)) {
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
        auto load = [&](TileIn &r, int t) __attribute__((always_inline)) {
            load_at(r, tile_row0(t));
        };

        // The part's first tile is its head's tile of the chunk's own block
        // (list entry 0) whenever split < G: those loads, and the chunk's
        // keys and values (MFMA operands for the whole item), go out before
        // the list is read.
        TileIn r0, r1;
        const bool first_own = split < G;
        if (first_own) load_at(r0, (g * G + split) * n_q + a * kC);
        const int64_t key_row = ca * kC + 32 * kh + col;
        bf16x8 kb[8], vb[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            kb[ks] = *(const bf16x8 *)(K + (gkv * T_cap + key_row) * kD + 16 * ks + 8 * half);
            vb[ks] = *(const bf16x8 *)(V + (gkv * T_cap + key_row) * kD + 16 * ks + 8 * half);
        }
        for (int i = tid; i < n_list; i += kThreads) {
            blist[i] = plan_blk[pr * n_blocks + i];
            bmask[i] = plan_msk[pr * n_blocks + i];
        }
        __syncthreads();                              // blist and bmask are in LDS

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
        if (!first_own) load(r0, 0);
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
        // Both paths below stage the chunk's 64 rows of dK and dV row-major in
        // LDS (the tiles are free once red has been read), so that the stores
        // write whole rows.
        const int64_t part_stride = Hkv * kv_div * n_q * kD;   // floats per (slot, tensor)
        constexpr int kStageStride = kD + 4;                   // floats per staged row
        float *stage = (float *)smem;                          // [dK, dV][64 rows][kStageStride]
        const float kscale = n_parts == 1 ? scale : 1.0f;      // partials stay unscaled
        __syncthreads();                                        // red has been read
        if (qh == 0) {
            const int row = 32 * kh + col;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 vk, vv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vk[e] = dk[dt][4 * u + e] * kscale;
                        vv[e] = dv[dt][4 * u + e];
                    }
                    *(f32x4 *)(stage + row * kStageStride + 32 * dt + 8 * u + 4 * half) = vk;
                    *(f32x4 *)(stage + (kC + row) * kStageStride + 32 * dt + 8 * u + 4 * half) = vv;
                }
        }
        __syncthreads();
        const int64_t row_base = g * n_q + a * kC;
        if (n_parts == 1) {
            // the result: non-temporal row stores (nothing here reads it again)
            for (int i = tid; i < 2 * kC * (kD / 4); i += kThreads) {
                const int t = i / (kC * (kD / 4)), w = i % (kC * (kD / 4));
                const int row = w / (kD / 4), d4 = 4 * (w % (kD / 4));
                __builtin_nontemporal_store(
                    *(const f32x4 *)(stage + (t * kC + row) * kStageStride + d4),
                    (f32x4 *)((t ? dV : dK) + (row_base + row) * kD + d4));
            }
            continue;
        }

        // Several workgroups share this chunk: store the partial (the first
        // workgroup into the chunk's own dK / dV rows, unscaled; workgroup s > 0
        // into slot s - 1), count, and let the last one add the partials in
        // workgroup order 0, 1, ... . The partials are stored at device scope
        // (written through to where every XCD reads them), 8 bytes a lane with
        // consecutive lanes on consecutive addresses (staged row-major through
        // LDS first), and the count waits for those stores to complete; only the
        // last workgroup then invalidates its L2's stale lines (an acquire)
        // before reading them. (A device-scope release fence instead writes back
        // the XCD's whole L2 in every workgroup: 7-21 us per split workgroup,
        // measured.)
        {
            float *pk = split == 0 ? dK : part + (int64_t)(2 * (split - 1)) * part_stride;
            float *pv = split == 0 ? dV : part + (int64_t)(2 * (split - 1) + 1) * part_stride;
            // pair i of tensor t: row (i / 64), dims 2 (i % 64) .. +2
            for (int i = tid; i < 2 * kC * (kD / 2); i += kThreads) {
                const int t = i / (kC * (kD / 2)), w = i % (kC * (kD / 2));
                const int row = w / (kD / 2), d2 = 2 * (w % (kD / 2));
                const float *src = stage + (t * kC + row) * kStageStride + d2;
                const uint64_t bits = (uint64_t)__float_as_uint(src[0]) |
                                      ((uint64_t)__float_as_uint(src[1]) << 32);
                uint64_t *dst = (uint64_t *)((t ? pv : pk) + (row_base + row) * kD + d2);
                __hip_atomic_store(dst, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(&counters[g * n_blocks + a], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == n_parts - 1;
        __syncthreads();
        if (!is_last) continue;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        // 64 keys x 128 d per tensor; thread t sums float4 column (t % 32) of rows
        // t/32, t/32 + 8, ... (whole rows per 32 threads: non-temporal stores).
        // This workgroup's own partial is still staged in LDS; the other
        // parts' are loaded for two rows at a time, every load issued before
        // the first add (a load-then-add chain per part would cost one memory
        // round trip each, at the end of the chunk's chain). The sum still
        // runs in part order 0, 1, ... .
        constexpr int kRowsPer = kC / (kThreads / 32);          // rows per thread
        constexpr int kRowBatch = 2;
        const int c4 = 4 * (tid & 31);
        for (int rb = 0; rb < kRowsPer; rb += kRowBatch) {
            f32x4 xk[kRowBatch][kSplit], xv[kRowBatch][kSplit];
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                const int r = (tid >> 5) + (kThreads / 32) * (rb + i);
                const int64_t off = (row_base + r) * kD + c4;
#pragma unroll
                for (int sp = 0; sp < kSplit; ++sp) {
                    xk[i][sp] = xv[i][sp] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (sp >= n_parts) continue;
                    if (sp == split) {
                        xk[i][sp] = *(const f32x4 *)(stage + r * kStageStride + c4);
                        xv[i][sp] = *(const f32x4 *)(stage + (kC + r) * kStageStride + c4);
                    } else {
                        const float *pk = sp == 0 ? dK : part + (int64_t)(2 * (sp - 1)) * part_stride;
                        const float *pv = sp == 0 ? dV : part + (int64_t)(2 * (sp - 1) + 1) * part_stride;
                        xk[i][sp] = *(const f32x4 *)(pk + off);
                        xv[i][sp] = *(const f32x4 *)(pv + off);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                const int r = (tid >> 5) + (kThreads / 32) * (rb + i);
                const int64_t off = (row_base + r) * kD + c4;
                f32x4 sk = xk[i][0], sv = xv[i][0];
#pragma unroll
                for (int sp = 1; sp < kSplit; ++sp) {
                    if (sp >= n_parts) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { sk[e] += xk[i][sp][e]; sv[e] += xv[i][sp][e]; }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sk[e] *= scale;
                __builtin_nontemporal_store(sk, (f32x4 *)(dK + off));
                __builtin_nontemporal_store(sv, (f32x4 *)(dV + off));
            }
        }
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
// Compute units of the current device (the persistent dkdv grid's size),
// asked once per device.
int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int G, int kUnit>
hipError_t launch_bwd_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                        int64_t Hkv, int kv_div, int64_t T_cap, int64_t p0, int64_t n_q,
                        const int32_t *ids, int32_t k, int32_t sink, float scale,
                        const uint16_t *O, const float *lse,
                        const uint16_t *dO, float *dQ, float *dK, float *dV,
                        float *delta, int *counters, int *plan_n, uint16_t *plan_blk,
                        uint8_t *plan_msk, uint8_t *redo_flags, float *part, hipStream_t stream)
{
    int *next_item = counters + Hkv * kv_div * (n_q / kC);
    constexpr int NHG = G < 4 ? 1 : G / 4;
    const int64_t n_blocks = n_q / kC;
    const float scale_log2 = scale * 1.44269504088896340736f;
    if (n_blocks > 65535) return hipErrorInvalidConfiguration;     // grid z limit
    hipLaunchKernelGGL((bwd_dq_kernel<G, kUnit>),
                       dim3((unsigned)Hkv, (unsigned)(kv_div * NHG), (unsigned)n_blocks),
                       dim3(kDqThreads), 0,
                       stream, Q, K, V, dO, O, lse, delta, counters, next_item, plan_n,
                       plan_blk, plan_msk, redo_flags, n_q, kv_div, T_cap, p0, ids, k, (int)sink,
                       scale_log2, scale, dQ);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_items = Hkv * kv_div * n_blocks * kSplit;
    hipLaunchKernelGGL((bwd_dkdv_kernel<G, kUnit>),
                       dim3((unsigned)std::min<int64_t>(n_items, device_cus())), dim3(kThreads),
                       0, stream, Q, K, V, dO, lse, delta, n_q, Hkv, kv_div, T_cap, p0, plan_n,
                       plan_blk, plan_msk, scale_log2, scale, dK, dV, part, counters, next_item);
    return hipGetLastError();
}

// Workspace layout (U routing units: Hkv, or Hq with per-query-head routing;
// nb = n_q/C blocks): Delta [Hq][n_q] f32 | counters [U][nb] int32 and the
// dkdv work-queue counter | the dkdv
// plan: plan_n [U][nb] int32, plan_blk [U][nb][nb] uint16, plan_msk
// [U][nb][nb] uint8 | the dq workgroups' pass-2 flags [U][2][nb] uint8 (two
// workgroups per unit when G = 8) | partial sums [kSplit - 1][dK, dV][U][n_q][D] f32 |
// per-query-head routing only: each head's dK and dV, [2][Hq][n_q][D] f32.
// Every part starts on a 256-byte boundary.
struct BwdWorkspace {
    size_t delta_off, counter_off, plan_n_off, plan_blk_off, plan_msk_off, redo_off, part_off,
        head_off, total;
};

BwdWorkspace bwd_layout(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t U = per_q_head ? Hq : Hkv;
    BwdWorkspace w;
    w.delta_off = 0;
    w.counter_off = up((size_t)(Hq * n_q) * sizeof(float));
    const size_t nb = (size_t)(n_q / kC);
    w.plan_n_off = w.counter_off + up(((size_t)U * nb + 1) * sizeof(int));
    w.plan_blk_off = w.plan_n_off + up((size_t)U * nb * sizeof(int));
    w.plan_msk_off = w.plan_blk_off + up((size_t)U * nb * nb * sizeof(uint16_t));
    w.redo_off = w.plan_msk_off + up((size_t)U * nb * nb);
    w.part_off = w.redo_off + up((size_t)U * 2 * nb);
    w.head_off = w.part_off + (size_t)(kSplit - 1) * 2 * (size_t)(U * n_q * kD) * sizeof(float);
    w.total = w.head_off + (per_q_head ? 2 * (size_t)(Hq * n_q * kD) * sizeof(float) : 0);
    return w;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head)
{
    return bwd_layout(Hq, Hkv, n_q, per_q_head).total;
}

int64_t bwd_max_queries() { return (int64_t)kMaxBlocksDkdv * kC; }

hipError_t bwd_second_pass_count(int64_t Hq, int64_t Hkv, int64_t n_q, bool per_q_head,
                                 const void *workspace, int64_t *n_second, int64_t *n_wg,
                                 hipStream_t stream)
{
    const BwdWorkspace w = bwd_layout(Hq, Hkv, n_q, per_q_head);
    const int64_t U = per_q_head ? Hq : Hkv;
    const int64_t G = per_q_head ? 1 : Hq / Hkv;
    const int64_t nhg = G < 4 ? 1 : G / 4;
    const int64_t n = U * nhg * (n_q / kC);
    std::vector<uint8_t> h((size_t)std::max<int64_t>(n, 1));
    if (n > 0) {
        hipError_t e = hipMemcpyAsync(h.data(), (const uint8_t *)workspace + w.redo_off,
                                      (size_t)n, hipMemcpyDeviceToHost, stream);
        if (e != hipSuccess) return e;
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return e;
    }
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) c += h[(size_t)i] != 0;
    *n_second = c;
    *n_wg = n;
    return hipSuccess;
}

namespace {

template <int kUnit>
hipError_t launch_bwd_unit(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                           int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                           const int32_t *ids, int32_t k, int32_t sink, bool per_q_head,
                           float scale, const uint16_t *O, const float *lse, const uint16_t *dO,
                           float *dQ, float *dK, float *dV, void *workspace, hipStream_t stream)
{
    if (n_q == 0) return hipSuccess;
    const BwdWorkspace w = bwd_layout(Hq, Hkv, n_q, per_q_head);
    uint8_t *ws = (uint8_t *)workspace;
    float *delta = (float *)(ws + w.delta_off);
    int *counters = (int *)(ws + w.counter_off);
    int *plan_n = (int *)(ws + w.plan_n_off);
    uint16_t *plan_blk = (uint16_t *)(ws + w.plan_blk_off);
    uint8_t *plan_msk = ws + w.plan_msk_off;
    uint8_t *redo = ws + w.redo_off;
    float *part = (float *)(ws + w.part_off);
    const int G = (int)(Hq / Hkv);
    if (per_q_head) {
        float *dKu = (float *)(ws + w.head_off);
        float *dVu = dKu + Hq * n_q * kD;
        hipError_t e = launch_bwd_g<1, kUnit>(Q, K, V, Hkv, G, T_cap, p0, n_q, ids, k, sink,
                                              scale, O, lse, dO, dQ, dKu, dVu, delta, counters,
                                              plan_n, plan_blk, plan_msk, redo, part, stream);
        if (e != hipSuccess) return e;
        const int64_t per_head = n_q * kD / 4, n_vec = Hkv * per_head;
        hipLaunchKernelGGL(sum_heads_kernel, dim3((unsigned)((n_vec + 255) / 256)), dim3(256),
                           0, stream, dKu, dVu, n_vec, G, per_head, dK, dV);
        return hipGetLastError();
    }
    switch (G) {
    case 1: return launch_bwd_g<1, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, O, lse, dO, dQ, dK, dV, delta, counters, plan_n, plan_blk, plan_msk, redo, part, stream);
    case 2: return launch_bwd_g<2, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, O, lse, dO, dQ, dK, dV, delta, counters, plan_n, plan_blk, plan_msk, redo, part, stream);
    case 4: return launch_bwd_g<4, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, O, lse, dO, dQ, dK, dV, delta, counters, plan_n, plan_blk, plan_msk, redo, part, stream);
    case 8: return launch_bwd_g<8, kUnit>(Q, K, V, Hkv, 1, T_cap, p0, n_q, ids, k, sink, scale, O, lse, dO, dQ, dK, dV, delta, counters, plan_n, plan_blk, plan_msk, redo, part, stream);
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
    return launch_bwd_unit<kC>(Q, K, V, Hq, Hkv, T_cap, p0, n_q, ids, k, sink, per_q_head,
                               scale, O, lse, dO, dQ, dK, dV, workspace, stream);
}

hipError_t launch_attend_bwd_groups(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                    int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                    int64_t n_q, const int32_t *gids, int32_t m, int32_t sink,
                                    float scale, const uint16_t *O, const float *lse,
                                    const uint16_t *dO, float *dQ, float *dK, float *dV,
                                    void *workspace, hipStream_t stream)
{
    return launch_bwd_unit<kGroup>(Q, K, V, Hq, Hkv, T_cap, p0, n_q, gids, m, sink, false,
                                   scale, O, lse, dO, dQ, dK, dV, workspace, stream);
}

}  // namespace hga
