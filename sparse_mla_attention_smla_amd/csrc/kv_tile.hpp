// Gathered kv tiles in LDS for the attention kernels (forward and dQ).
//
// Per query token, the valid index slots (index in [0, num_kv)) are first
// compacted in LDS, in increasing slot order, in chunks of up to kChunk slots:
// masked slots are never loaded or computed.  The compacted list is walked in
// tiles of 32 slots; every tile row (one kv row, 1 KiB of bf16) is copied from
// global memory straight into LDS by a buffer load with LDS destination (no
// register staging).  A ring of kNBuf tile buffers keeps kNBuf-1 tiles in
// flight while one is computed.  Tail positions past the last valid slot are
// loaded with an out-of-range offset: the buffer range check returns zeros.
// The copies are issued from inline assembly and waited for with explicit
// vmcnt counts: the compiler would otherwise drain every copy in flight before
// any LDS read, since it cannot tell the ring's buffers apart.
//
// The same LDS tile feeds two MFMA contractions with different reduction axes:
//   S^T  = kv . q^T     reduces over d     -> ds_read_b128 of 8 d of one row
//   dq^T = kv^T . dS^T  reduces over slots -> ds_read_b64_tr_b16: lane L of a
//          16-lane group names row L/4, columns 4(L%4)..+3 and receives column
//          L of those 4 consecutive rows (the transposed read of gfx950).
// Rows are kRowPitch = 1056 bytes (an odd multiple of 32) apart: measured on
// gfx950 with the LDS bank-conflict counter, such a pitch makes both patterns
// (16 rows at one 16-byte chunk; 16 consecutive rows x 8 bytes through the
// transposed read) conflict-free, while 1024, 1040 or 1072 are 2- to 8-way
// conflicted.  Every other offset is an immediate.
#pragma once

#include "smla_device.hpp"

namespace smla {

constexpr int kBK = 32;                       // slots per tile
constexpr int kRowPitch = kD * 2 + 32;        // 1056 bytes per tile row in LDS
constexpr int kTileBytes = kBK * kRowPitch;   // 33,792 bytes
constexpr int kNBuf = 4;                      // tile ring depth
constexpr int kChunk = 512;                   // slots compacted at a time

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    // a C-style cast converts the generic pointer to the LDS address space
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// 16 bytes per lane from the buffer at voffset into LDS at lds + 16*lane.
// lds must be wave-uniform; it is moved to a scalar register first.
__device__ __forceinline__ void copy_row_to_lds(i32x4 rsrc, uint32_t lds, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// The same copy with the non-temporal hint, for rows read exactly once.
__device__ __forceinline__ void copy_row_to_lds_nt(i32x4 rsrc, uint32_t lds, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voffset), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// Cache-policy operand of the buffer store builtins: non-temporal (gfx950 "nt" bit).
constexpr int kCacheNT = 2;

// Buffer resource over [p, p + bytes): loads outside the range return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = (int32_t)(uint32_t)a;
    r[1] = (int32_t)((a >> 32) & 0xFFFFu);   // stride 0
    r[2] = (int32_t)bytes;                    // num_records (bytes)
    r[3] = 0x00020000;                        // 32-bit data format, raw addressing
    return r;
}
// A row index whose byte offset (row * 1024 + lane * 16 < 2^31) lies beyond any
// kv buffer (num_kv < 2^20, so its range is below 2^30 bytes).
constexpr int kOobRow = (1 << 21) - 1;

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Compacted slot list of one chunk, in LDS.
struct SlotList {
    int32_t slot[kChunk];   // original slot index k
    int32_t row[kChunk];    // kv row idx[t, k]
    int32_t n;              // valid entries
};

// Compaction of the valid slots of [k0, min(k0 + kChunk, K)) of one index row,
// in two steps so the index loads can be issued well before the list is built.
// Run by one wave (64 lanes); the caller synchronises before others read L.
struct SlotChunk {
    int v[kChunk / 64];
};

__device__ __forceinline__ void load_slot_chunk(const int32_t* __restrict__ idx_row, int K, int k0,
                                                SlotChunk& c, int lane) {
#pragma unroll
    for (int s = 0; s < kChunk / 64; ++s) {
        const int k = k0 + 64 * s + lane;
        c.v[s] = k < K ? idx_row[k] : -1;
    }
}

__device__ __forceinline__ void build_slot_list(const SlotChunk& c, int N, int k0, SlotList* L, int lane) {
    int base = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int s = 0; s < kChunk / 64; ++s) {
        const bool ok = valid_row(c.v[s], N);
        const uint64_t m = __ballot(ok);
        if (ok) {
            const int p = base + __popcll(m & below);
            L->slot[p] = k0 + 64 * s + lane;
            L->row[p] = c.v[s];
        }
        base += __popcll(m);
    }
    if (lane == 0) L->n = base;
}

__device__ __forceinline__ void compact_slots(const int32_t* __restrict__ idx_row, int K, int N, int k0,
                                              SlotList* L, int lane) {
    SlotChunk c;
    load_slot_chunk(idx_row, K, k0, c, lane);
    build_slot_list(c, N, k0, L, lane);
}

// Issue the buffer->LDS copies of tile `ct` (compacted positions 32ct..32ct+31)
// that belong to wave w of NW: rows w, w+NW, ...  Exactly 32/NW copies per wave.
// buf is the LDS address of the ring buffer.
template <int NW>
__device__ __forceinline__ void issue_tile(i32x4 rsrc, const SlotList* L, int ct, uint32_t buf, int w,
                                           int lane) {
    static_assert(kBK % NW == 0, "rows per wave must be uniform");
    constexpr int kR = kBK / NW;
    const int n = L->n;
    // Lane i < kR fetches the kv row of copy i in one vector LDS read; tail
    // positions map to a row whose offset is past any buffer range (the range
    // check then yields zeros).  readlane hands each copy its row without
    // branches, so all copies issue back to back.
    const int lp = lane < kR ? lane : 0;
    const int pos = ct * kBK + w + NW * lp;
    const int rowv = L->row[pos < kChunk ? pos : kChunk - 1];
    const int rowsel = pos < n ? rowv : kOobRow;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int row = __builtin_amdgcn_readlane(rowsel, i);
        copy_row_to_lds(rsrc, buf + (w + NW * i) * kRowPitch, row * (kD * 2) + (lane << 4));
    }
}

// Per-lane byte offset of the S^T A operand inside a tile: lane (c16, g) reads
// row 16*st + c16, elements d = 32*ds + 8g .. +7, i.e. rows_base + st*16*pitch + ds*64.
__device__ __forceinline__ int rows_base(int c16, int g) { return c16 * kRowPitch + g * 16; }

__device__ __forceinline__ u32x4 tile_rows_a(const char* buf, int base, int st, int ds) {
    return *reinterpret_cast<const u32x4*>(buf + base + st * 16 * kRowPitch + ds * 64);
}

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ u32x2 ds_read_tr16(const char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// A operand of X^T = kv^T . Y^T (reduction over the 32 slots) for d-tile dt.
// Lane (c16, g) receives row d = 16*dt + c16 with slots 4g..4g+3 then
// 16+4g..16+4g+3: the order in which the S^T accumulators of sub-tiles 0 and 1
// leave them in the lane, so the matching B operand is pack(acc0, acc1).
// Lane L = c16 of group g names row 4g + L/4 (then 16 + 4g + L/4) and columns
// 16dt + 4(L%4) .. +3.
__device__ __forceinline__ int cols_base(int c16, int g) {
    return (4 * g + (c16 >> 2)) * kRowPitch + (c16 & 3) * 8;
}

__device__ __forceinline__ u32x4 tile_cols_a(const char* buf, int base, int dt) {
    const u32x2 lo = ds_read_tr16(buf + base + dt * 32);
    const u32x2 hi = ds_read_tr16(buf + base + 16 * kRowPitch + dt * 32);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---- positional key rows (the has_pe=True variant) ------------------------
// A head-shared positional key part of kDP = 64 bf16 (128 bytes) per kv row.
// A tile's 32 rows take 4 KiB of LDS in four 1 KiB blocks, block c holding
// tile rows 8c..8c+7 and written by one buffer->LDS copy (lane l lands at byte
// 16 l of the block).  Inside a block, 16-byte chunk k (0..7) of row r (0..7)
// sits at chunk slot pe_slot(r, k) = 16 (r % 4) + (2 r + k) % 16.  That is a
// bijection on the block's 64 slots (for each value of (2 r + k) % 16 exactly
// one of r, r + 4 has k <= 7), and it puts every byte at the same address
// modulo 256 as rows 32 bytes (mod 256) apart would, the kv tiles' pitch
// above: both operand reads below then meet the banks as the kv reads do,
// where plain back-to-back 128-byte rows are several-way conflicted.  Lane l
// of a copy fetches the chunk its slot holds; tail positions fetch from past
// the buffer's range and land as zeros.
constexpr int kDP = 64;
constexpr int kPeRow = kDP * 2;              // 128 bytes
constexpr int kPeTileBytes = kBK * kPeRow;   // 4,096 bytes

__device__ __forceinline__ int pe_slot(int r, int k) { return 16 * (r & 3) + ((2 * r + k) & 15); }

// Copies of positional tile `ct` issued by wave w of NW (NW in {1, 2, 4}):
// copies w, w + NW, ... of the four, i.e. exactly 4/NW per wave.
template <int NW>
__device__ __forceinline__ void issue_pe_tile(i32x4 rsrc, const SlotList* L, int ct, uint32_t buf, int w,
                                              int lane) {
    static_assert(NW == 1 || NW == 2 || NW == 4, "four copies split evenly over the waves");
    constexpr int kP = 4 / NW;
    const int n = L->n;
    // the (row, chunk) of the block that slot `lane` holds (inverse of pe_slot)
    const int k0 = ((lane & 15) - 2 * (lane >> 4)) & 15;
    const int r = (lane >> 4) + ((k0 >> 3) << 2), k = k0 & 7;
#pragma unroll
    for (int i = 0; i < kP; ++i) {
        const int c = w + NW * i;
        const int pos = ct * kBK + 8 * c + r;
        const int rowv = L->row[pos < kChunk ? pos : kChunk - 1];
        const int row = pos < n ? rowv : kOobRow;
        copy_row_to_lds(rsrc, buf + c * 1024, row * kPeRow + k * 16);
    }
}

// S^T A operand of the positional part: lane (c16, g) reads tile row
// 16*st + c16, positional elements 32*s + 8g .. +7 (chunk 4s + g; s = 0, 1).
__device__ __forceinline__ u32x4 pe_rows_a(const char* buf, int c16, int g, int st, int s) {
    return *reinterpret_cast<const u32x4*>(buf + (2 * st + (c16 >> 3)) * 1024 + 16 * pe_slot(c16 & 7, 4 * s + g));
}

// Transposed A operand of dq_pe^T = kpe_tile^T . dS^T for positional d-tile dt
// (dt = 0..3): the lane pattern of tile_cols_a, lane (c16, g) naming row
// 4g + c16/4 (then 16 more) and elements 16dt + 4(c16%4) .. +3, i.e. half
// c16 % 2 of chunk 2dt + (c16 % 4)/2.
__device__ __forceinline__ u32x4 pe_cols_a(const char* buf, int c16, int g, int dt) {
    const int r = 4 * g + (c16 >> 2);
    const char* p = buf + (r >> 3) * 1024 + 16 * pe_slot(r & 7, 2 * dt + ((c16 & 3) >> 1)) + 8 * (c16 & 1);
    const u32x2 lo = ds_read_tr16(p);
    const u32x2 hi = ds_read_tr16(p + 2048);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace smla
