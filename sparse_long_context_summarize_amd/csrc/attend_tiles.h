// attend_tiles.h -- LDS layouts and tile loaders shared by the forward
// attention kernels (attend_fwd.hip).
//
// A chunk tile is 64 keys of K and V (bf16, 16 KiB each). K sits row-major
// in LDS with 272-byte rows (conflict-free 16-byte MFMA operand reads); V is
// stored transposed, V^T[d][key] with 144-byte rows, and within each 16-key
// group position 8*h + 4*u + m holds key 8*u + 4*h + m, so the 8 keys one lane
// needs for a P^T k-step (the S^T accumulator's row order) are one 16-byte
// read. Loader threads hold four 16-byte pieces of a tile in registers
// between the global load and the LDS store.
#pragma once
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kKStride = kD + 8;            // bf16 per K row in LDS (272 B)
constexpr int kVtStride = kC + 8;           // bf16 per V^T row (one d) in LDS (144 B)
constexpr int kKTile = kC * kKStride;       // elements
constexpr int kVtTile = kD * kVtStride;     // elements
constexpr int kTilePieces = 4;              // 16-byte pieces per loader thread (256 threads)
constexpr int kOStride = 136;               // output staging row: 128 bf16 + 8 pad
// s_waitcnt immediates (gfx9 encoding).
constexpr int kWaitVm8 = 0x0F78;       // vector memory count 8, others no wait
constexpr int kWaitLgkm0 = 0xC07F;     // LDS/scalar count 0, others no wait

struct TileRegs {
    u32x4 p[kTilePieces];
};

// K, loader thread u (0..255): piece j is key row 16*j + u/16, d = 8*(u%16)
// .. +8 (each load instruction reads four 256-B rows).
__device__ __forceinline__ void load_k_rows(TileRegs &tr, const uint16_t *Kg, int64_t tok0, int u)
{
    const uint16_t *src = Kg + (tok0 + (u >> 4)) * kD + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kTilePieces; ++j) tr.p[j] = *(const u32x4 *)(src + 16 * j * kD);
}

__device__ __forceinline__ void store_k_rows(const TileRegs &tr, uint16_t *Ks, int u)
{
    uint16_t *dst = Ks + (u >> 4) * kKStride + (u & 15) * 8;
#pragma unroll
    for (int j = 0; j < kTilePieces; ++j) *(u32x4 *)(dst + 16 * j * kKStride) = tr.p[j];
}

// V, loader thread u (0..255): lane takes keys 4*kg .. 4*kg+3 of the 8-wide
// d slice dp, kg = lane%16, dp = 4*(u/64) + lane/16; piece j is key 4*kg + j.
__device__ __forceinline__ void load_v_rows(TileRegs &tr, const uint16_t *Vg, int64_t tok0, int u)
{
    const int lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
    const uint16_t *src = Vg + (tok0 + 4 * kg) * kD + dp * 8;
#pragma unroll
    for (int j = 0; j < kTilePieces; ++j) tr.p[j] = *(const u32x4 *)(src + j * kD);
}

// The 4 keys x 8 d block a loader lane holds is transposed in registers
// (byte permutes) and written as 8 rows of 4 keys; with kg = lane%16 the 64
// lanes' 8-byte writes fall on distinct banks.
__device__ __forceinline__ void store_v_rows(const TileRegs &tr, uint16_t *Vt, int u)
{
    const int lane = u & 63;
    const int kg = lane & 15, dp = 4 * (u >> 6) + (lane >> 4);
    const int pos = 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
    uint16_t *dst = Vt + (8 * dp) * kVtStride + pos;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // element e of each key's 8-wide slice is the low (e even) or high
        // half of dword e/2; keys (0,1) and (2,3) pack into two dwords.
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(tr.p[1][e >> 1], tr.p[0][e >> 1], sel);
        w[1] = __builtin_amdgcn_perm(tr.p[3][e >> 1], tr.p[2][e >> 1], sel);
        *(u32x2 *)(dst + e * kVtStride) = w;
    }
}

// A operand V^T[d][key] for d-tile dt, k-step ks: lane gets d = 32*dt + lane%32
// and keys 16*ks + 8*u + 4*(lane/32) + m (element 4u + m), matching the key
// order of the P^T operand taken from the S^T accumulators.
__device__ __forceinline__ bf16x8 vt_operand(const uint16_t *Vt, int dt, int ks, int lane)
{
    return *(const bf16x8 *)(Vt + (32 * dt + (lane & 31)) * kVtStride + 16 * ks + 8 * (lane >> 5));
}

// A operand K rows for key half kt, k-step ks: lane gets key 32*kt + lane%32,
// d = 16*ks + 8*(lane/32) .. +8.
__device__ __forceinline__ bf16x8 k_operand(const uint16_t *Ks, int kt, int ks, int lane)
{
    return *(const bf16x8 *)(Ks + (32 * kt + (lane & 31)) * kKStride + 16 * ks + 8 * (lane >> 5));
}

}  // namespace
}  // namespace hga
