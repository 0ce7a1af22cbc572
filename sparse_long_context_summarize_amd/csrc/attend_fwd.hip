// attend_fwd.hip -- exact softmax attention over the routed chunks plus the
// causal local block (arXiv 2607.15105, gist.science technical summary 2.1:
// only the exact K/V of the selected chunks enter attention; summaries are
// used for routing only).
//
// Work unit: one query block b (64 queries) of one kv head g, i.e. the G query
// heads that share g -- one gather of each routed chunk serves all of them.
// A workgroup has 4 waves and serves up to 4 query heads (wave w -> head
// g*G + 4*hg + w); G = 8 takes two workgroups per unit, G < 4 leaves the spare
// waves to help with the loads.
//
// Per chunk tile (64 keys), per wave (64 queries = 2 tiles of 32):
//   S^T[key][q] = K Q^T          A = K rows from LDS, B = Q^T from registers
//   online softmax on S^T        each lane owns one query (lane & 31) and 16
//                                of its 32 keys per 32-key tile; the other 16
//                                sit in lane ^ 32, one swap joins them
//   O^T[d][q] += V^T P^T         A = V^T rows from LDS, B = P^T straight from
//                                the S^T accumulators (bf16)
// using v_mfma_f32_32x32x16_bf16 (fp32 accumulate). The accumulator row order
// of a 32x32 tile (8*(j/4) + 4*(lane/32) + j%4) makes the P^T operand's k
// index a permutation of the keys; V^T is stored in LDS under the same
// permutation (bits 2 and 3 of the key index swapped), so each operand is one
// 16-byte LDS read.
//
// Chunk tiles are double buffered in LDS: the 32 KiB of K and V for tile t+1
// are loaded to registers (16-byte coalesced loads, a 256-byte key row per 16
// lanes) while tile t is computed, then written to the other buffer, one
// barrier per tile. Rows are padded (K: 272 B, V^T: 144 B) so the 16-byte
// operand reads hit distinct banks.
//
// Workgroup w serves kv head w % Hkv: with 8 kv heads every block of one head
// runs on the same XCD, where neighbouring blocks' overlapping chunk choices
// hit that XCD's L2.
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kKStride = kD + 8;            // bf16 elements per K row in LDS (272 B)
constexpr int kVtStride = kC + 8;           // bf16 elements per V^T row in LDS (144 B)
constexpr int kKTile = kC * kKStride;       // elements
constexpr int kVtTile = kD * kVtStride;     // elements
constexpr int kLoadsPerThread = kC * kD * 2 / 16 / kThreads;   // 16-byte loads of K (and of V)

static_assert(kLoadsPerThread == 4, "tile loader assumes 4 rows per thread");

// Position of key kk (0..63) inside a V^T row: swap bits 2 and 3.
__device__ __forceinline__ int vt_pos(int kk) {
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

struct TileRegs {
    u32x4 k[kLoadsPerThread];
    u32x4 v[kLoadsPerThread];
};

// Thread t loads keys 4*(t/16) + r, r = 0..3, d = 8*(t%16) .. +8.
__device__ __forceinline__ void load_tile(TileRegs &tr, const uint16_t *Kg,
                                          const uint16_t *Vg, int64_t tok0)
{
    const int t = threadIdx.x;
    const int key0 = 4 * (t >> 4);
    const int dseg = t & 15;
#pragma unroll
    for (int r = 0; r < kLoadsPerThread; ++r) {
        const int64_t off = (tok0 + key0 + r) * kD + dseg * 8;
        tr.k[r] = *(const u32x4 *)(Kg + off);
        tr.v[r] = *(const u32x4 *)(Vg + off);
    }
}

__device__ __forceinline__ void store_tile(const TileRegs &tr, uint16_t *Ks, uint16_t *Vts)
{
    const int t = threadIdx.x;
    const int key0 = 4 * (t >> 4);
    const int dseg = t & 15;
#pragma unroll
    for (int r = 0; r < kLoadsPerThread; ++r)
        *(u32x4 *)(Ks + (key0 + r) * kKStride + dseg * 8) = tr.k[r];
    // V^T: for each d of this thread's slice, the 4 keys key0..key0+3 are
    // adjacent in the permuted order -> one 8-byte write.
    const int pos = vt_pos(key0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t a = tr.v[0][q], b = tr.v[1][q], c = tr.v[2][q], d = tr.v[3][q];
        u32x2 even, odd;    // d = 8*dseg + 2q and 8*dseg + 2q + 1
        even[0] = (a & 0xFFFFu) | (b << 16);
        even[1] = (c & 0xFFFFu) | (d << 16);
        odd[0] = (a >> 16) | (b & 0xFFFF0000u);
        odd[1] = (c >> 16) | (d & 0xFFFF0000u);
        *(u32x2 *)(Vts + (dseg * 8 + 2 * q) * kVtStride + pos) = even;
        *(u32x2 *)(Vts + (dseg * 8 + 2 * q + 1) * kVtStride + pos) = odd;
    }
}

template <int G>
__global__ __launch_bounds__(kThreads, 1) void attend_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t n_q, int64_t Hkv, int64_t T_cap,
    int64_t p0, const int32_t *__restrict__ ids, int k, float scale_log2,
    uint16_t *__restrict__ O, float *__restrict__ lse)
{
    constexpr int HW = G < 4 ? G : 4;            // query heads per workgroup
    constexpr int NHG = G / HW;                  // workgroups per unit
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKTile];
    __shared__ __attribute__((aligned(16))) uint16_t Vts[2][kVtTile];
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

    TileRegs tr;
    load_tile(tr, Kg, Vg, (int64_t)list[0] * kC);

    // Q^T operands: lane holds Q[q = 32*qt + lane%32][d = 16*ks + 8*(lane/32) .. +8].
    const bool computes = wave < HW;
    const int64_t h = g * G + hg * HW + wave;
    const int col = lane & 31;
    const int half = lane >> 5;
    bf16x8 qf[2][8];
    if (computes) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                qf[qt][ks] = *(const bf16x8 *)(Q + (h * n_q + b * kC + 32 * qt + col) * kD +
                                               16 * ks + 8 * half);
    }
    store_tile(tr, Ks[0], Vts[0]);
    __syncthreads();

    f32x16 o[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[qt][dt][j] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        const bool more = it + 1 < n_tiles;
        if (more) load_tile(tr, Kg, Vg, (int64_t)list[it + 1] * kC);

        if (computes) {
            const uint16_t *Kb = Ks[buf];
            const uint16_t *Vb = Vts[buf];
            // S^T = K Q^T for key tiles kt (32 keys) x query tiles qt.
            f32x16 s[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[kt][qt][j] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8 a = *(const bf16x8 *)(Kb + (32 * kt + col) * kKStride +
                                                       16 * ks + 8 * half);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qt][ks],
                                                                            s[kt][qt], 0, 0, 0);
                }
            }
            // Causal mask on the local block (the last tile): key > query.
            if (it == n_tiles - 1) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int key = 32 * kt + 8 * (j >> 2) + 4 * half + (j & 3);
                            if (key > 32 * qt + col) s[kt][qt][j] = -INFINITY;
                        }
            }
            // Online softmax in the log2 domain.
            bf16x8 pb[2][4];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kt][qt][j]);
                mx = fmaxf(mx, partner32(mx));
                const float m_new = fmaxf(m_run[qt], mx * scale_log2);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
                m_run[qt] = m_new;
                float psum = 0.f;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][j], scale_log2, -m_new));
                        psum += p;
                        pb[qt][2 * kt + (j >> 3)][j & 7] = (__bf16)p;
                    }
                l_run[qt] = l_run[qt] * alpha + psum;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) o[qt][dt][j] *= alpha;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 a = *(const bf16x8 *)(Vb + (32 * dt + col) * kVtStride +
                                                       16 * ks + 8 * half);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qt][ks],
                                                                            o[qt][dt], 0, 0, 0);
                }
            }
        }
        if (more) store_tile(tr, Ks[buf ^ 1], Vts[buf ^ 1]);
        __syncthreads();
    }

    if (!computes) return;
    // Normalise and store: lane holds query 32*qt + col, d = 32*dt + 8*u + 4*half + 0..3.
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const float l_tot = l_run[qt] + partner32(l_run[qt]);
        const float inv = 1.0f / l_tot;
        const int64_t row = h * n_q + b * kC + 32 * qt + col;
        uint16_t *orow = O + row * kD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[qt][dt][4 * u + e] * inv);
                *(bf16x4 *)(orow + 32 * dt + 8 * u + 4 * half) = v;
            }
        if (half == 0)
            lse[row] = (m_run[qt] + __log2f(l_tot)) * 0.69314718055994530942f;
    }
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
