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
//                            A = V^T read from the row-major V tile with the
//                            gfx950 transposing LDS read ds_read_b64_tr_b16
//                            (each 16-lane group turns four 4-element row
//                            pieces into four 4-key columns), two per operand.
// The S^T accumulator's row order (8*(j/4) + 4*(lane/32) + j%4) fixes which
// keys each lane's P^T operand holds; the transposing reads fetch V rows in
// exactly that order, so no data is permuted anywhere.
// The running max is rescaled lazily: O^T and the row sum are only rescaled
// when some row's max grows by more than 8 (log2 units), otherwise the stale
// max stays and probabilities up to 2^8 enter the bf16 operand unchanged.
//
// Chunk tiles (32 KiB of K and V) are loaded two tiles ahead into registers
// (16-byte coalesced loads, a 256-byte key row per 16 lanes) and written to a
// double-buffered LDS tile one barrier before use. LDS rows are padded: K to
// 272 B (conflict-free 16-byte operand reads), V to 320 B (the four rows a
// transposing read touches start 64 B apart in the banks).
//
// Workgroup w serves kv head w % Hkv: with 8 kv heads every block of one head
// runs on the same XCD, where neighbouring blocks' overlapping chunk choices
// hit that XCD's L2.
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kKStride = kD + 8;            // bf16 per K row in LDS (272 B)
constexpr int kVStride = kD + 32;           // bf16 per V row in LDS (320 B)
constexpr int kKTile = kC * kKStride;       // elements
constexpr int kVTile = kC * kVStride;       // elements
constexpr int kRowsPerThread = kC * kD * 2 / 16 / kThreads;   // 16-byte pieces per tensor
constexpr float kLazy = 8.0f;               // log2 growth that forces a rescale
// s_waitcnt immediate (gfx9 encoding): vector memory count 0, others no wait.
constexpr int kWaitVm0 = 0x0F70;

static_assert(kRowsPerThread == 2, "tile loader assumes 2 pieces per tensor per thread");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct TileRegs {
    u32x4 k[kRowsPerThread];
    u32x4 v[kRowsPerThread];
};

// Thread t loads row 32*r + t/16, d = 8*(t%16) .. +8, r = 0, 1.
__device__ __forceinline__ void load_tile(TileRegs &tr, const uint16_t *Kg,
                                          const uint16_t *Vg, int64_t tok0)
{
    const int t = threadIdx.x;
    const int row0 = t >> 4, dseg = t & 15;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
        const int64_t off = (tok0 + 32 * r + row0) * kD + dseg * 8;
        tr.k[r] = *(const u32x4 *)(Kg + off);
        tr.v[r] = *(const u32x4 *)(Vg + off);
    }
}

__device__ __forceinline__ void store_tile(const TileRegs &tr, uint16_t *Ks, uint16_t *Vs)
{
    const int t = threadIdx.x;
    const int row0 = t >> 4, dseg = t & 15;
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
        *(u32x4 *)(Ks + (32 * r + row0) * kKStride + dseg * 8) = tr.k[r];
        *(u32x4 *)(Vs + (32 * r + row0) * kVStride + dseg * 8) = tr.v[r];
    }
}

// A operand V^T[d][key] for d-tile dt, k-step ks: lane gets d = 32*dt + lane%32
// and keys 16*ks + 8*u + 4*(lane/32) + m (element 4u + m), matching the key
// order of the P^T operand taken from the S^T accumulators.
__device__ __forceinline__ bf16x8 vt_operand(const uint16_t *Vs, int dt, int ks, int lane)
{
    const int grp = lane >> 4, i = lane & 15;
    const int half = grp >> 1, dsub = grp & 1;
    const int row = 16 * ks + 4 * half + (i >> 2);
    const int col = 32 * dt + 16 * dsub + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Vs + row * kVStride + col));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Vs + (row + 8) * kVStride + col));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <int G>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attend_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv, int64_t T_cap,
    int64_t p0, const int32_t *__restrict__ ids, int k, float scale_log2,
    uint16_t *__restrict__ O, float *__restrict__ lse)
{
    constexpr int HW = G < 4 ? G : 4;            // query heads per workgroup
    constexpr int NHG = G / HW;                  // workgroups per unit
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kVTile];
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

    // Chunk list: valid routed ids (0 <= c < P/C) in order, then the local block.
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
    __syncthreads();
    const int n_tiles = list_n;

    TileRegs tr[2];
    load_tile(tr[0], Kg, Vg, (int64_t)list[0] * kC);
    load_tile(tr[1], Kg, Vg, (int64_t)list[min(1, n_tiles - 1)] * kC);

    // Q^T operand: lane holds Q[q = 32*qt + lane%32][d = 16*ks + 8*(lane/32) .. +8].
    const int hw = wave & 3, qt = wave >> 2;
    const bool computes = hw < HW;
    const int64_t h = g * G + hg * HW + hw;
    const int col = lane & 31;
    const int half = lane >> 5;
    bf16x8 qf[8];
    if (computes) {
        const uint16_t *qrow = Q + (h * n_q + b * kC + 32 * qt + col) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8 *)(qrow + 16 * ks);
    }
    store_tile(tr[0], Ks[0], Vs[0]);
    // Let the one-time Q loads land here, so no wait for them is left inside
    // the tile loop (where it would also wait for the prefetch in flight).
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // One tile step. `pre` receives tile it+2, `nxt` (holding tile it+1) is
    // written to the other LDS buffer; the caller alternates the two register
    // sets so both stay statically named.
    auto tile_step = [&](int it, TileRegs &pre, const TileRegs &nxt) {
        const int buf = it & 1;
        // Always issue the prefetch (the last tile again near the end) so the
        // wait before storing `nxt` can leave these newer loads in flight.
        load_tile(pre, Kg, Vg, (int64_t)list[min(it + 2, n_tiles - 1)] * kC);

        if (computes) {
            const uint16_t *Kb = Ks[buf];
            const uint16_t *Vb = Vs[buf];
            // S^T = K Q^T for the two 32-key halves kt: all 16 operand reads are
            // issued first (LDS answers in order, so each MFMA waits only for
            // its own operand), then the two accumulation chains interleave.
            f32x16 s[2];
            {
                bf16x8 a[2][8];
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        a[kt][ks] = *(const bf16x8 *)(Kb + (32 * kt + col) * kKStride + 16 * ks + 8 * half);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kt][ks], qf[ks], s[kt], 0, 0, 0);
            }
            // Causal mask on the local block (the last tile): key > query.
            if (it == n_tiles - 1) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = 32 * kt + 8 * (j >> 2) + 4 * half + (j & 3);
                        if (key > 32 * qt + col) s[kt][j] = -INFINITY;
                    }
            }
            // Online softmax in the log2 domain, lazily rescaled.
            // (four independent max / sum chains keep the VALU pipeline full)
            float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) m4[j & 3] = fmaxf(m4[j & 3], s[kt][j]);
            float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            mx = fmaxf(mx, partner32(mx)) * scale_log2;
            if (__ballot(mx > m_run + kLazy) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
            }
            // Per 32-key half: probabilities -> bf16 P^T operands, the half's
            // 8 V^T operands (16 transposing reads), then its 8 MFMAs.
            float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                bf16x8 pb[2];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][j], scale_log2, -m_run));
                    ps4[j & 3] += p;
                    pb[j >> 3][j & 7] = (__bf16)p;
                }
                bf16x8 va[2][4];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) va[kk][dt] = vt_operand(Vb, dt, 2 * kt + kk, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk][dt], pb[kk], o[dt], 0, 0, 0);
            }
            l_run += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
        }
        if (it + 1 < n_tiles) store_tile(nxt, Ks[buf ^ 1], Vs[buf ^ 1]);
        __syncthreads();
    };
    for (int it = 0; it < n_tiles; it += 2) {
        tile_step(it, tr[0], tr[1]);
        if (it + 1 < n_tiles) tile_step(it + 1, tr[1], tr[0]);
    }

    if (!computes) return;
    // Normalise and store: lane holds query 32*qt + col, d = 32*dt + 8*u + 4*half + 0..3.
    const float l_tot = l_run + partner32(l_run);
    const float inv = 1.0f / l_tot;
    const int64_t row = h * n_q + b * kC + 32 * qt + col;
    uint16_t *orow = O + row * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][4 * u + e] * inv);
            *(bf16x4 *)(orow + 32 * dt + 8 * u + 4 * half) = v;
        }
    if (half == 0)
        lse[row] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
}

template <int G>
hipError_t launch_g(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                    int64_t Hkv, int64_t T_cap, int64_t p0, int64_t n_q,
                    const int32_t *ids, int32_t k, float scale, uint16_t *O,
                    float *lse, hipStream_t stream)
{
    constexpr int NHG = G < 4 ? 1 : G / 4;
    const int64_t n_blocks = n_q / kC;
    const float scale_log2 = scale * 1.44269504088896340736f;
    hipLaunchKernelGGL(attend_fwd_kernel<G>, dim3((unsigned)(n_blocks * Hkv * NHG)),
                       dim3(kThreads), 0, stream, Q, K, V, n_q, Hkv, T_cap, p0, ids, k,
                       scale_log2, O, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_fwd(const uint16_t *Q, const uint16_t *K,
                             const uint16_t *V, int64_t Hq, int64_t Hkv,
                             int64_t T_cap, int64_t p0, int64_t n_q,
                             const int32_t *ids, int32_t k, float scale,
                             uint16_t *O, float *lse, hipStream_t stream)
{
    if (n_q == 0) return hipSuccess;
    switch (Hq / Hkv) {
    case 1: return launch_g<1>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, O, lse, stream);
    case 2: return launch_g<2>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, O, lse, stream);
    case 4: return launch_g<4>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, O, lse, stream);
    case 8: return launch_g<8>(Q, K, V, Hkv, T_cap, p0, n_q, ids, k, scale, O, lse, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hga
