// attend_fwd.hip -- exact softmax attention over the routed chunks plus the
// causal local block (arXiv 2607.15105, gist.science technical summary 2.1:
// only the exact K/V of the selected chunks enter attention; summaries are
// used for routing only).
//
// Work unit: one query block b (64 queries) of one kv head g, i.e. the G query
// heads that share g -- one gather of each routed chunk serves all of them.
// A workgroup has 8 waves (two per SIMD) and serves up to 4 query heads: wave
// w takes head g*G + 4*hg + w%4, queries 32*(w/4) .. +32 of the block. G = 8
// takes two workgroups per unit; G < 4 leaves spare waves that only load.
//
// Per chunk tile (64 keys), per wave (32 queries), v_mfma_f32_32x32x16_bf16
// with fp32 accumulation:
//   S^T[key][q] = K Q^T      A = K rows from LDS, B = Q^T held in registers
//   online softmax on S^T    each lane owns one query (lane & 31) and 16 of the
//                            32 keys of each 32-key half; lane ^ 32 holds the
//                            other 16, one lane swap joins them
//   O^T[d][q] += V^T P^T     B = P^T straight from the S^T accumulators (bf16);
//                            A = V^T, stored transposed in LDS (see store_v)
//                            so that each operand is one 16-byte read.
// The S^T accumulator's row order (8*(j/4) + 4*(lane/32) + j%4) fixes which
// keys each lane's P^T operand holds; store_v places V's keys in that order.
// The softmax needs no row maximum per tile: probabilities are taken against
// the running maximum as it stands, p = 2^(s*c - m), and only when a row's
// tile sum of p exceeds 2^16 (or is not finite) is the exact maximum taken,
// O^T and the row sum rescaled and p recomputed. Every p that enters the bf16
// operand is then at most 2^16, so O^T and the row sums keep their fp32
// relative precision; m starts at -FLT_MAX, so the first (local) tile always
// takes the exact path. This keeps the max reduction, and its wait on the
// last S^T MFMA, off the MFMA half-step.
//
// Chunk tiles (32 KiB of K and V) are loaded ahead into registers (16-byte
// coalesced loads, a 256-byte key row per 16 lanes) and written to a
// double-buffered LDS tile one barrier before use. K rows are padded to 272 B
// (conflict-free 16-byte operand reads); V^T rows to 144 B.
//
// Workgroups are dispatched with the kv head fastest (grid x), so workgroup w
// serves kv head w % Hkv: with 8 kv heads every block of one head runs on the
// same XCD, where neighbouring blocks' overlapping chunk choices hit that
// XCD's L2.
//
// Per-query-head routing (one id row per query head) runs the G = 1 kernel
// with kv_div = query heads per kv head: each query head is then its own
// unit, reading its own id row and its kv head's K and V.
#include "attend_tiles.h"
#include "route_core.h"

#include <float.h>
#include <type_traits>

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kPieces = kTilePieces;
constexpr float kSumLimit = 65536.0f;       // tile row sum that forces an exact rescale
constexpr int kLook = 6;                // MFMA operands read this many MFMAs ahead

static_assert(kPieces * 16 * kThreads / 2 == kC * kD * 2, "one loader group moves one tile");

// Tile loaders. Waves 4-7 ("K group") move K tiles, waves 0-3 ("V group")
// move V tiles; each thread holds four 16-byte pieces of one tile.
// The loaders take the first token of a chunk tile (consecutive rows), or
// row_tok(r), the token of tile row r (0..63), for a tile whose rows come 8 at
// a time from its groups.
// K group, u = thread - 256 (see load_k_rows).
__device__ __forceinline__ void load_k(TileRegs &tr, const uint16_t *Kg, int64_t tok0)
{
    load_k_rows(tr, Kg, tok0, (int)threadIdx.x - kThreads / 2);
}

// Group tiles: the K group thread takes rows r0 + 2*j of one 8-row group,
// r0 = 8*(u/32) + (u/16)%2, so a single row_tok call serves its four pieces
// (each load instruction still reads four 256-B rows).
template <typename RowTok>
__device__ __forceinline__ void load_k(TileRegs &tr, const uint16_t *Kg, RowTok row_tok)
{
    const int u = threadIdx.x - kThreads / 2;
    const int r0 = 8 * (u >> 5) + ((u >> 4) & 1);
    const uint16_t *src = Kg + row_tok(r0) * kD + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) tr.p[j] = *(const u32x4 *)(src + 2 * j * kD);
}

__device__ __forceinline__ void store_k_grp(const TileRegs &tr, uint16_t *Ks)
{
    const int u = threadIdx.x - kThreads / 2;
    const int r0 = 8 * (u >> 5) + ((u >> 4) & 1);
    uint16_t *dst = Ks + r0 * kKStride + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) *(u32x4 *)(dst + 2 * j * kKStride) = tr.p[j];
}

__device__ __forceinline__ void store_k(const TileRegs &tr, uint16_t *Ks)
{
    store_k_rows(tr, Ks, (int)threadIdx.x - kThreads / 2);
}

// V group, u = thread (see load_v_rows).
__device__ __forceinline__ void load_v(TileRegs &tr, const uint16_t *Vg, int64_t tok0)
{
    load_v_rows(tr, Vg, tok0, (int)threadIdx.x);
}

// (rows 4*kg .. 4*kg+3 lie in one 8-row group, so one row_tok call serves them)
template <typename RowTok>
__device__ __forceinline__ void load_v(TileRegs &tr, const uint16_t *Vg, RowTok row_tok)
{
    const int u = threadIdx.x, lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
    const uint16_t *src = Vg + row_tok(4 * kg) * kD + dp * 8;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) tr.p[j] = *(const u32x4 *)(src + j * kD);
}

// V goes to LDS transposed (see store_v_rows).
__device__ __forceinline__ void store_v(const TileRegs &tr, uint16_t *Vt)
{
    store_v_rows(tr, Vt, (int)threadIdx.x);
}

// kUnit = kC: ids are chunk ids, one tile per routed chunk. kUnit = kGroup:
// ids are 8-token group ids (the second routing level); each routed tile is
// gathered from 8 groups, and the last one masks the keys of its missing
// groups when their number is not a multiple of 8.
// kRouteNI = 0: ids are an input. kRouteNI > 0: the workgroup first routes
// its block itself with the router's own code (route_block, NI = kRouteNI
// keys per lane for the chunk candidates), writes ids (and scores, if not
// null) exactly as the routing kernels would, and attends over that choice;
// S / n_cap are the chunk summaries. For group tiles the routing has two
// levels: the block's kc chunks (written to chunk_ids_out), then m = k groups
// among those chunks' groups against the group summaries SG / n_gcap (at most
// kFusedGroupChunks chunks, so 4 keys per lane hold every group candidate).
template <int G, int kUnit, int kRouteNI>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attend_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int kv_div, int64_t T_cap,
    int64_t p0, int32_t *__restrict__ ids, int k, int sink, float scale_log2,
    uint16_t *__restrict__ O, float *__restrict__ lse,
    const float *__restrict__ S, int64_t n_cap, float *__restrict__ scores,
    const float *__restrict__ SG, int64_t n_gcap, int kc, int32_t *__restrict__ chunk_ids_out)
{
    static_assert(kFusedGroupChunks * (kC / kGroup) <= 4 * 64,
                  "fused group routing keeps every group candidate in 4 keys per lane");
    constexpr int HW = G < 4 ? G : 4;            // query heads per workgroup
    constexpr int NHG = G / HW;                  // workgroups per unit
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kVtTile];
    __shared__ int list[(kUnit == kC ? kChunkListMax : kGroupListMax) + 1];
    __shared__ int list_n;
    __shared__ __attribute__((aligned(16))) uint16_t Os[8][32 * kOStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Grid (Hkv, kv_div * NHG, n_blocks): linear workgroup order runs over the
    // kv heads fastest, and no index needs a division. y is the query head
    // within its kv head's group (kv_div > 1, one id row per query head) or
    // the workgroup's share of a G = 8 unit (NHG = 2); never both.
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

    // Group A = waves 0-3, group B = waves 4-7 (wave w runs on SIMD w % 4).
    // Queries 32*qt .. +32 of the block go to group qt; within a group the
    // waves of head slots 0 .. HW-1 compute (head g*G + hg*HW + slot). With
    // HW < 4 the two groups use different waves (A the first HW, B the next
    // HW), so their MFMA work lands on different SIMDs.
    const int grp = wave >> 2;
    const int qt = grp;
    const int lane4 = wave & 3;
    const bool computes = lane4 / HW == qt % (4 / HW);
    const int hw = lane4 % HW;                   // head slot
    const int64_t h = g * G + hg * HW + hw;
    const int col = lane & 31;
    const int half = lane >> 5;

    // Tile 0 is the causal local block, whose rows need no routing result:
    // its loads go out with the Q loads, and wave 0 issues the id row's load
    // before both (loads complete in order), so the list is ready early.
    int32_t *id_row = ids + (g * n_blocks + b) * k;
    const int id_first = (kRouteNI == 0 && wave == 0 && lane < k) ? id_row[lane] : -1;
    // Q^T operand: lane holds Q[q = 32*qt + lane%32][d = 16*ks + 8*(lane/32) .. +8].
    // With routing fused in and all G heads in this workgroup, the block's
    // G*64 query rows are loaded whole (each load instruction reads four
    // 256-B rows; piece p = row p/16, 16-byte segment p%16) into an LDS copy
    // that both the router and the Q^T operands read; otherwise each wave
    // loads its operand rows itself.
    constexpr bool kQInLds = kRouteNI > 0 && NHG == 1;
    constexpr int kQPieces = kQInLds ? G * kC * 16 / kThreads : 1;
    bf16x8 qf[8];
    u32x4 qraw[kQPieces];
    if constexpr (kQInLds) {
#pragma unroll
        for (int j = 0; j < kQPieces; ++j) {
            const int p = j * kThreads + tid, row = p >> 4, seg = p & 15;
            qraw[j] = *(const u32x4 *)(Q + ((g * G + row / kC) * n_q + b * kC + row % kC) * kD +
                                       seg * 8);
        }
    } else if (computes) {
        const uint16_t *qrow = Q + (h * n_q + b * kC + 32 * qt + col) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
    }
    TileRegs r0, r1;
    // (with routing fused in, the local tile is loaded behind the router's
    // first summary rows instead: the query rows come first)
    if (kRouteNI == 0) {
        if (grp == 0) load_v(r0, Vg, P); else load_k(r0, Kg, P);
    }

    // Unit list: the local chunk, the sink window's units, then the valid
    // routed ids (past the sink, before P) in order, repeats dropped.
    const int n_sink = sink_units(sink, P, kUnit);
    if constexpr (kRouteNI == 0) {
        if (wave == 0) {
            write_sink_units(list + 1, n_sink);
            const int n = build_unit_list(id_row, k, (int64_t)sink * (kC / kUnit), P / kUnit,
                                          list + 1 + n_sink, id_first);
            if (lane == 0) {
                list[0] = (int)local_chunk;
                list_n = 1 + n_sink + n;
            }
        }
    } else {
        // Route first. Its scratch lives in LDS the kernel has not used yet:
        // the V tiles (first written after the first MFMA half-step), the K
        // tiles (the local tile is stored after routing) and the output
        // staging area (used in the epilogue only). With all G heads in this
        // workgroup (G <= 4) the router reads the block's query rows from an
        // LDS copy of the Q registers rather than from memory a second time.
        // The chosen ids come out ascending and distinct: the list needs no
        // clean-up.
        static_assert(sizeof(RouteLds) <= sizeof(Vs), "router scratch must fit the V tiles");
        static_assert(NHG > 1 || G * kC * kOStride <= (int)(sizeof(Os) / sizeof(uint16_t)),
                      "the block's query rows must fit the staging area");
        RouteLds &sh = *reinterpret_cast<RouteLds *>(&Vs[0][0]);
        uint32_t *keys = reinterpret_cast<uint32_t *>(&Ks[0][0]);
        uint16_t *qcopy = &Os[0][0];                // row r = head hw*64 + query
        if constexpr (kQInLds) {
#pragma unroll
            for (int j = 0; j < kQPieces; ++j) {
                const int p = j * kThreads + tid, row = p >> 4, seg = p & 15;
                *(u32x4 *)(qcopy + row * kOStride + seg * 8) = qraw[j];
            }
            __syncthreads();
            if (computes) {
                const uint16_t *src = qcopy + (hw * kC + 32 * qt + col) * kOStride + 8 * half;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(src + 16 * ks);
            }
        }
        auto q_row = [&](int row, int dseg) __attribute__((always_inline)) {
            if constexpr (kQInLds) {
                return *(const u32x4 *)(qcopy + row * kOStride + dseg * 8);
            } else {
                const int64_t hh = g * G + row / kC;
                const int64_t i = b * kC + row % kC;
                return *(const u32x4 *)(Q + (hh * n_q + i) * kD + dseg * 8);
            }
        };
        const bool wr = hg == 0;            // one workgroup of a unit writes the ids
        float *sc_row = (scores && wr) ? scores + (g * n_blocks + b) * k : nullptr;
        constexpr int kBatchR = G >= 8 ? 4 : 8;
        auto load_local = [&]() __attribute__((always_inline)) {
            if (grp == 0) load_v(r0, Vg, P); else load_k(r0, Kg, P);
        };
        const std::integral_constant<bool, kQInLds> q_local{};
        auto emit_unit = [&](int r, int id, float sc) __attribute__((always_inline)) {
            list[1 + n_sink + r] = id;
            if (wr) {
                id_row[r] = id;
                if (sc_row) sc_row[r] = sc;
            }
        };
        int n_sel;
        if constexpr (kUnit == kC) {
            n_sel = route_block<G, kRouteNI, false, kBatchR, kThreads / 64>(
                sh, keys, q_row, n_q, gkv, b, p0, S, n_cap, k, nullptr, 0, sink, emit_unit,
                load_local, q_local);
        } else {
            // the block's chunks into chunk_sel (and the chunk id output),
            // then the groups of those chunks into the tile list
            __shared__ int chunk_sel[kFusedGroupChunks];
            int32_t *crow = (chunk_ids_out && wr) ? chunk_ids_out + (g * n_blocks + b) * kc
                                                  : nullptr;
            route_block<G, kRouteNI, false, kBatchR, kThreads / 64>(
                sh, keys, q_row, n_q, gkv, b, p0, S, n_cap, kc, nullptr, 0, sink,
                [&](int r, int id, float) __attribute__((always_inline)) {
                    chunk_sel[r] = id;
                    if (crow) crow[r] = id;
                },
                load_local, q_local);
            __syncthreads();
            n_sel = route_block<G, 4, true, kBatchR, kThreads / 64>(
                sh, keys, q_row, n_q, gkv, b, p0, SG, n_gcap, k, chunk_sel, kc, sink, emit_unit,
                NoHook{}, q_local);
        }
        if (wave == 0) {
            write_sink_units(list + 1, n_sink);
            if (lane == 0) {
                list[0] = (int)local_chunk;
                list_n = 1 + n_sink + n_sel;
            }
        }
    }
    __syncthreads();
    const int n_units = list_n - 1;                 // routed units
    const int n_tiles = (kUnit == kC ? n_units : (n_units + 7) / 8) + 1;
    // token of row r of tile t (tiles past the end repeat the last one)
    const int *lst = list;
    auto rows_of = [&](int t) __attribute__((always_inline)) {
        const int tt = min(t, n_tiles - 1);
        if constexpr (kUnit == kC) {
            return (int64_t)lst[tt] * kC;          // a chunk tile: its first token
        } else {
            const bool local = tt == 0;
            const int64_t lbase = (int64_t)lst[0] * kC;
            const int g0 = 8 * tt - 7, glast = n_units;
            return [=](int r) __attribute__((always_inline)) -> int64_t {
                if (local) return lbase + r;
                // padding rows of the last routed tile repeat its last group (masked)
                return (int64_t)lst[min(g0 + (r >> 3), glast)] * kGroup + (r & 7);
            };
        }
    };
    if (grp == 0) {
        load_v(r1, Vg, rows_of(1));
    } else {
        load_k(r1, Kg, rows_of(1));
        store_k(r0, Ks[0]);         // the local tile, loaded as consecutive rows
        load_k(r0, Kg, rows_of(2));
    }
    // The Q loads were issued first: let them land here (the eight newer tile
    // loads may stay in flight), so no wait for them is left in the loop.
    __builtin_amdgcn_s_waitcnt(kWaitVm8);
    __syncthreads();

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
    float m_run = -FLT_MAX, l_run = 0.f;
    f32x16 s[2];        // S^T of a tile, from its MFMA half-step to its softmax
    bf16x8 pb[4];       // P^T of a tile, from its softmax to the next MFMA half-step

    // MFMA half-step of tile t: PV of tile t-1 (if PV) and S^T of tile t (if
    // SC), interleaved one MFMA each, operands streamed from LDS kLook MFMAs
    // ahead of use.
    auto mf = [&](int t, auto PV, auto SC) __attribute__((always_inline)) {
        if (!computes) return;
        constexpr bool kPV = decltype(PV)::value, kSC = decltype(SC)::value;
        constexpr int NS = (kPV ? 16 : 0) + (kSC ? 16 : 0);
        const uint16_t *Kb = Ks[t & 1];
        const uint16_t *Vb = Vs[(t + 1) & 1];
        // step i -> (is_s, index within its kind)
        auto is_s = [&](int i) __attribute__((always_inline)) { return kPV && kSC ? (i & 1) == 0 : kSC; };
        auto idx = [&](int i) __attribute__((always_inline)) { return kPV && kSC ? i >> 1 : i; };
        auto read = [&](int i) __attribute__((always_inline)) -> bf16x8 {
            const int j = idx(i);
            if (is_s(i))     // j = 2*ks + kt
                return *(const bf16x8 *)(Kb + (32 * (j & 1) + col) * kKStride + 16 * (j >> 1) + 8 * half);
            return vt_operand(Vb, j & 3, j >> 2, lane);     // j = 4*kk + dt
        };
        if (kSC) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
        }
        // group tiles hold a little more addressing state: a shorter lookahead
        constexpr int kLk = kUnit == kC ? kLook : kLook - 3;
        bf16x8 op[NS];
#pragma unroll
        for (int i = 0; i < kLk; ++i) op[i] = read(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + kLk < NS) op[i + kLk] = read(i + kLk);
            const int j = idx(i);
            if (is_s(i))
                s[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], qf[j >> 1], s[j & 1], 0, 0, 0);
            else
                o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], pb[j >> 2], o[j & 3], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Softmax half-step of tile t: causal mask on the local block (tile 0),
    // online softmax in the log2 domain with a lazy rescale, P^T to bf16.
    auto va = [&](int t) __attribute__((always_inline)) {
        if (!computes) return;
        // (keeps this half-step's arithmetic behind the barrier before it)
        asm volatile("" : "+v"(s[0]), "+v"(s[1]));
        if (t == 0) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kt + 8 * (j >> 2) + 4 * half + (j & 3);
                    if (key > 32 * qt + col) s[kt][j] = -INFINITY;
                }
        } else if (kUnit != kC && t == n_tiles - 1 && (n_units & 7) != 0) {
            const int n_keys = kGroup * (n_units & 7);      // keys of the tile's groups
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kt + 8 * (j >> 2) + 4 * half + (j & 3);
                    if (key >= n_keys) s[kt][j] = -INFINITY;
                }
        }
        // Probabilities against the running maximum as it stands; the exact
        // maximum is only taken when a row's tile sum leaves [0, 2^16] (or is
        // not finite), which also covers the first tile (m_run = -FLT_MAX).
        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][j], scale_log2, -m_run));
                ps4[j & 3] += p;
                pb[2 * kt + (j >> 3)][j & 7] = (__bf16)p;
            }
        float ls = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(pb[kk]));
        const float row = ls + partner32(ls);
        if (__ballot(!(row <= kSumLimit)) != 0) {
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) m4[j & 3] = fmaxf(m4[j & 3], s[kt][j]);
            float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            mx = fmaxf(mx, partner32(mx)) * scale_log2;
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
            float qs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][j], scale_log2, -m_new));
                    qs4[j & 3] += p;
                    pb[2 * kt + (j >> 3)][j & 7] = (__bf16)p;
                }
            ls = (qs4[0] + qs4[1]) + (qs4[2] + qs4[3]);
        }
        l_run += ls;
    };

    // Loader duties, in the group's softmax half-steps. V group, tile t: V(t)
    // to LDS, prefetch V(t+2). K group, tile t: K(t+2) to LDS, prefetch K(t+4).
    auto duty_v = [&](int t, TileRegs &rr) __attribute__((always_inline)) {
        store_v(rr, Vs[t & 1]);
        load_v(rr, Vg, rows_of(t + 2));
    };
    auto duty_k = [&](int t, TileRegs &rr) __attribute__((always_inline)) {
        if (t + 2 < n_tiles) {
            if constexpr (kUnit == kC) store_k(rr, Ks[t & 1]); else store_k_grp(rr, Ks[t & 1]);
        }
        load_k(rr, Kg, rows_of(t + 4));
    };
    const std::true_type Y{};
    const std::false_type N{};

    // Half-step schedule (each ends at a workgroup barrier), tile t:
    //   slot 2t:   A: PV(t-1) + S(t)     B: softmax(t-1), K(t+1) to LDS
    //   slot 2t+1: A: softmax(t), V(t)   B: PV(t-1) + S(t)
    // so on every SIMD one wave's MFMAs overlap the other wave's softmax.
    // Buffers: K(t) is read in slots 2t, 2t+1 and rewritten with K(t+2) in
    // slot 2t+2; V(t) is written in slot 2t+1 and read in slots 2t+2, 2t+3.
    // Both groups pass 2*n_tiles barriers.
    // The loops below run whole pairs of tiles (register sets r0, r1 in a
    // fixed order) and leave an odd tile to a copy after the loop, so the
    // compiler sees one order of outstanding loads at the loop head and can
    // wait for the older prefetch set only.
    auto step_a = [&](int t, TileRegs &rr) __attribute__((always_inline)) {
        mf(t, Y, Y);
        __syncthreads();
        va(t);
        duty_v(t, rr);
        __syncthreads();
    };
    auto step_b = [&](int t, TileRegs &rr) __attribute__((always_inline)) {
        mf(t, Y, Y);
        __syncthreads();
        va(t);
        duty_k(t, rr);
        __syncthreads();
    };
    if (grp == 0) {
        mf(0, N, Y);
        __syncthreads();
        va(0);
        duty_v(0, r0);
        __syncthreads();
        int t = 1;
        for (; t + 1 < n_tiles; t += 2) {
            step_a(t, r1);
            step_a(t + 1, r0);
        }
        if (t < n_tiles) step_a(t, r1);
        mf(n_tiles, Y, N);
    } else {
        duty_k(-1, r1);
        __syncthreads();
        mf(0, N, Y);
        __syncthreads();
        int t = 0;
        if (n_tiles > 1) {
            va(0);
            duty_k(0, r0);
            __syncthreads();
            t = 1;
            for (; t + 2 < n_tiles; t += 2) {
                step_b(t, r1);
                step_b(t + 1, r0);
            }
            if (t + 1 < n_tiles) {
                step_b(t, r1);
                ++t;
            }
            // tile n_tiles-1: its softmax and the final PV need no barrier after them
            mf(t, Y, Y);
            __syncthreads();
        }
        va(t);
        mf(n_tiles, Y, N);
    }

    if (!computes) return;
    // Normalise; lane holds query 32*qt + col, d = 32*dt + 8*u + 4*half + 0..3.
    // The wave's 32 x 128 output goes through its own LDS area so that each
    // store instruction writes four whole 256-B rows (1 KiB contiguous)
    // instead of 16-B pieces of 32 rows.
    const float l_tot = l_run + partner32(l_run);
    const float inv = 1.0f / l_tot;
    uint16_t *st = Os[wave];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][4 * u + e] * inv);
            *(bf16x4 *)(st + col * kOStride + 32 * dt + 8 * u + 4 * half) = v;
        }
    const int64_t row0 = h * n_q + b * kC + 32 * qt;
    if (half == 0)
        lse[row0 + col] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
    // (a wave's LDS accesses complete in order: its reads see its writes)
    // O goes out with non-temporal stores: nothing in this kernel reads it
    // again, and written-back lines would otherwise sit dirty in L2 for the
    // end-of-kernel write-back (measured: 39.7 -> 38.4 us at the 16K layer).
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int piece = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        __builtin_nontemporal_store(*(const u32x4 *)(st + r * kOStride + 8 * piece),
                                    (u32x4 *)(O + (row0 + r) * kD + 8 * piece));
    }
}

struct FwdArgs {
    const uint16_t *Q, *K, *V;
    bool per_q_head;         // one id row per query head
    int64_t Hq, Hkv, T_cap, p0, n_q;
    int32_t *ids;
    int32_t k;
    int32_t sink;
    float scale;
    uint16_t *O;
    float *lse;
    const float *S;          // fused routing only
    int64_t n_cap;
    float *scores;
    const float *SG;         // fused group routing only
    int64_t n_gcap;
    int32_t kc;
    int32_t *chunk_ids;
};

template <int G, int kUnit, int kRouteNI>
hipError_t launch_g(const FwdArgs &a, hipStream_t stream)
{
    constexpr int NHG = G < 4 ? 1 : G / 4;
    const int64_t n_blocks = a.n_q / kC;
    const float scale_log2 = a.scale * 1.44269504088896340736f;
    const int kv_div = a.per_q_head ? (int)(a.Hq / a.Hkv) : 1;
    if (n_blocks > 65535) return hipErrorInvalidConfiguration;     // grid z limit
    hipLaunchKernelGGL((attend_fwd_kernel<G, kUnit, kRouteNI>),
                       dim3((unsigned)a.Hkv, (unsigned)(kv_div * NHG), (unsigned)n_blocks),
                       dim3(kThreads), 0,
                       stream, a.Q, a.K, a.V, a.n_q, kv_div, a.T_cap, a.p0, a.ids, a.k,
                       (int)a.sink, scale_log2, a.O, a.lse, a.S, a.n_cap, a.scores, a.SG,
                       a.n_gcap, (int)a.kc, a.chunk_ids);
    return hipGetLastError();
}

template <int kUnit, int kRouteNI>
hipError_t launch_unit(const FwdArgs &a, hipStream_t stream)
{
    if (a.n_q == 0) return hipSuccess;
    switch (a.per_q_head ? 1 : a.Hq / a.Hkv) {       // query heads per unit
    case 1: return launch_g<1, kUnit, kRouteNI>(a, stream);
    case 2: return launch_g<2, kUnit, kRouteNI>(a, stream);
    case 4: return launch_g<4, kUnit, kRouteNI>(a, stream);
    case 8: return launch_g<8, kUnit, kRouteNI>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attend_fwd(const uint16_t *Q, const uint16_t *K,
                             const uint16_t *V, int64_t Hq, int64_t Hkv,
                             int64_t T_cap, int64_t p0, int64_t n_q,
                             const int32_t *ids, int32_t k, int32_t sink, bool per_q_head,
                             float scale, uint16_t *O, float *lse, hipStream_t stream)
{
    const FwdArgs a{Q, K, V, per_q_head, Hq, Hkv, T_cap, p0, n_q, const_cast<int32_t *>(ids),
                    k, sink, scale, O, lse, nullptr, 0, nullptr};
    return launch_unit<kC, 0>(a, stream);
}

hipError_t launch_attend_fwd_groups(const uint16_t *Q, const uint16_t *K,
                                    const uint16_t *V, int64_t Hq, int64_t Hkv,
                                    int64_t T_cap, int64_t p0, int64_t n_q,
                                    const int32_t *gids, int32_t m, int32_t sink, float scale,
                                    uint16_t *O, float *lse, hipStream_t stream)
{
    const FwdArgs a{Q, K, V, false, Hq, Hkv, T_cap, p0, n_q, const_cast<int32_t *>(gids), m,
                    sink, scale, O, lse, nullptr, 0, nullptr};
    return launch_unit<kGroup, 0>(a, stream);
}

int64_t route_attend_max_candidates()
{
    return (int64_t)(sizeof(uint16_t) * 2 * kKTile / sizeof(uint32_t));   // keys in the K tiles
}

hipError_t launch_route_attend_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                   int64_t Hq, int64_t Hkv, int64_t T_cap, int64_t p0,
                                   int64_t n_q, const float *S, int64_t n_cap, int32_t k,
                                   int32_t sink, bool per_q_head, float scale, int32_t *ids,
                                   float *scores, uint16_t *O, float *lse, hipStream_t stream)
{
    const FwdArgs a{Q, K, V, per_q_head, Hq, Hkv, T_cap, p0, n_q, ids, k, sink, scale, O, lse,
                    S, n_cap, scores};
    if (k == 0) return launch_unit<kC, 0>(a, stream);
    // keys per lane of the router's register selection: the smallest class
    // that holds the largest candidate count (beyond 2048 the LDS path)
    const int64_t max_eligible = (p0 + n_q - kC) / kC - sink;
    if (max_eligible <= 4 * 64) return launch_unit<kC, 4>(a, stream);
    if (max_eligible <= 8 * 64) return launch_unit<kC, 8>(a, stream);
    if (max_eligible <= 16 * 64) return launch_unit<kC, 16>(a, stream);
    return launch_unit<kC, 32>(a, stream);
}

hipError_t launch_route_attend_fwd_groups(const uint16_t *Q, const uint16_t *K,
                                          const uint16_t *V, int64_t Hq, int64_t Hkv,
                                          int64_t T_cap, int64_t p0, int64_t n_q,
                                          const float *S, int64_t n_cap, int32_t kc,
                                          const float *SG, int64_t n_gcap, int32_t m,
                                          int32_t sink, float scale, int32_t *chunk_ids,
                                          int32_t *gids, float *gscores, uint16_t *O, float *lse,
                                          hipStream_t stream)
{
    if (kc <= 0 || kc > kFusedGroupChunks || m <= 0) return hipErrorInvalidValue;
    const FwdArgs a{Q, K, V, false, Hq, Hkv, T_cap, p0, n_q, gids, m, sink, scale, O, lse,
                    S, n_cap, gscores, SG, n_gcap, kc, chunk_ids};
    // keys per lane of the chunk router's register selection (as above)
    const int64_t max_eligible = (p0 + n_q - kC) / kC - sink;
    if (max_eligible <= 4 * 64) return launch_unit<kGroup, 4>(a, stream);
    if (max_eligible <= 8 * 64) return launch_unit<kGroup, 8>(a, stream);
    if (max_eligible <= 16 * 64) return launch_unit<kGroup, 16>(a, stream);
    return launch_unit<kGroup, 32>(a, stream);
}

}  // namespace hga
