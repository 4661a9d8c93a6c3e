// Gathered kv tiles in LDS for the attention kernels (forward and dQ).
//
// A tile holds the kv rows of 32 consecutive index slots of one query token.
// The same rows feed two MFMA contractions with different reduction axes:
//   S^T = kv . q^T          reduces over d     -> needs rows with d contiguous
//   dq^T = kv^T . dS^T      reduces over slots -> needs columns with slots contiguous
// so the tile is written to LDS twice: row-major [32][520] (pad 8 bf16 per row:
// consecutive rows land in different bank groups) and transposed [512][40]
// (pad 8 bf16).  The transposed copy is produced in registers: every thread
// loads the same 16-byte column chunk of 8 slots, swaps 16-bit lanes with
// byte permutes, and writes 8 transposed 16-byte rows.
//
// Every wave-wide global load reads one whole 1 KiB kv row (64 lanes x 16 B).
// Masked slots (index outside [0, num_kv)) are never read; they hold zeros.
#pragma once

#include "smla_device.hpp"

namespace smla {

constexpr int kBK = 32;                                 // slots per tile
constexpr int kRowStride = kD + 8;                      // bf16 per row-major row
constexpr int kTrStride = kBK + 8;                      // bf16 per transposed row
constexpr int kRowBytes = kBK * kRowStride * 2;         // 33,280
constexpr int kTrBytes = kD * kTrStride * 2;            // 40,960
constexpr int kTileBytes = kRowBytes + kTrBytes;        // 74,240

// 16-bit element e (0..7) of an 8 x bf16 chunk
__device__ __forceinline__ uint32_t elem16(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int NW>
struct KvTile {
    static constexpr int kGroups = kBK / 8;                      // groups of 8 slots
    static constexpr int kGPT = (kGroups + NW - 1) / NW;         // groups per wave
    u32x4 r[kGPT][8];
    uint32_t mask;  // bit i: slot i of the tile addresses a kv row

    // Issue the global loads of tile `tile` (registers only, no LDS traffic).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ kv,
                                         const int32_t* __restrict__ idx_row, int K, int N,
                                         int tile, int w, int lane) {
        const int slot = tile * kBK + lane;
        const int v = (lane < kBK && slot < K) ? idx_row[slot] : -1;
        mask = (uint32_t)__ballot(lane < kBK && valid_row(v, N));
#pragma unroll
        for (int gi = 0; gi < kGPT; ++gi) {
            const int grp = w + gi * NW;
            if (grp < kGroups) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = grp * 8 + i;
                    const int row = __builtin_amdgcn_readlane(v, s);
                    if ((mask >> s) & 1u)
                        r[gi][i] = *reinterpret_cast<const u32x4*>(kv + (size_t)row * kD + lane * 8);
                    else
                        r[gi][i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    // Write the loaded rows into one LDS tile buffer (both layouts).
    __device__ __forceinline__ void store(char* buf, int w, int lane) const {
        uint16_t* rowm = reinterpret_cast<uint16_t*>(buf);
        uint16_t* tr = reinterpret_cast<uint16_t*>(buf + kRowBytes);
#pragma unroll
        for (int gi = 0; gi < kGPT; ++gi) {
            const int grp = w + gi * NW;
            if (grp < kGroups) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<u32x4*>(rowm + (grp * 8 + i) * kRowStride + lane * 8) = r[gi][i];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u32x4 o;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        o[m] = elem16(r[gi][2 * m], e) | (elem16(r[gi][2 * m + 1], e) << 16);
                    *reinterpret_cast<u32x4*>(tr + (lane * 8 + e) * kTrStride + grp * 8) = o;
                }
            }
        }
    }
};

// A operand of S^T = kv . q^T for slot sub-tile st (16 slots) and d-step ds (32 d).
// Lane (c16, g): row = slot 16*st + c16, d = 32*ds + 8*g .. +7.
__device__ __forceinline__ u32x4 tile_rows_a(const char* buf, int st, int ds, int c16, int g) {
    const uint16_t* rowm = reinterpret_cast<const uint16_t*>(buf);
    return *reinterpret_cast<const u32x4*>(rowm + (16 * st + c16) * kRowStride + 32 * ds + 8 * g);
}

// A operand of X^T = kv^T . Y^T (reduction over the 32 slots) for d-tile dt.
// Lane (c16, g): row d = 16*dt + c16; its 8 reduction elements are slots
// 4g..4g+3 then 16+4g..16+4g+3 -- the same order in which the S^T accumulator
// of sub-tiles 0 and 1 leaves them in the lane, so B = pack(acc0, acc1).
__device__ __forceinline__ u32x4 tile_cols_a(const char* buf, int dt, int c16, int g) {
    const uint16_t* tr = reinterpret_cast<const uint16_t*>(buf + kRowBytes);
    const uint16_t* p = tr + (16 * dt + c16) * kTrStride + 4 * g;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace smla
