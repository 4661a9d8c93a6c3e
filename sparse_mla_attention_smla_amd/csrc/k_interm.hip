// dKV intermediate of the sparse MLA backward, contracted over all heads.
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table,
// "dKV-interm" row (all heads contracted inside one pair of MFMA chains, q and
// dO transposed once into registers, D split across the work) and the R_CHUNK
// note (the intermediate is [T, topk, 512] bf16).
//
// For token t, with X = [q_t ; dO_t] (2H x 512) and Y_t = [scale*dS_t ; P_t]
// (2H x slots, the dsp blocks written by the dQ kernel), one product gives
// both terms of every slot's row:
//   interm^T [512 x slots] = X^T . Y_t        (reduction over r in [0, 2H))
// Work unit: one token per workgroup of 8 waves; wave w owns d in [64w, 64w+64).
// X^T fragments (MFMA A operands: one d row, 8 values of r) are built once per
// token with transposed LDS reads and stay in registers.  The token's valid
// slots are compacted exactly as in the dQ kernel, so its dsp blocks line up
// with the compacted tiles; each 32-slot block streams through a 2-deep LDS
// ring (rows padded to 96 bytes), one tile of loads in flight.  A tile's
// output rows are assembled in LDS and leave whole, one 1 KiB row per store
// instruction; q, dO, the dsp blocks and the output are each touched once, so
// every one of these streams carries the non-temporal hint (together 5% faster
// than cached accesses with each wave storing its 128-byte piece of the rows).
// Rows of masked slots are not written: the gather never reads them.
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {
constexpr int kIWaves = 8;
constexpr int kIThreads = kIWaves * 64;
constexpr int kStageRows = 64;                          // X rows staged per pass
constexpr int kStageBytes = kStageRows * kRowPitch;     // 67,584
constexpr int kYPitch = 96;                             // Y row: 32 slots (64 B) + 32 B pad
constexpr int kYRing = 2;
constexpr int kOPitch = 1040;                           // output row in LDS: 1 KiB + 16 B pad
constexpr int kOBytes = kBK * kOPitch;                  // one tile of output rows
}  // namespace

// NKS = 2H / 32 reduction steps (H = 16 * NKS).
//
// PE (the has_pe=True variant) also forms the positional intermediate
// interm_pe [T*topk, 64] = sum_h scale*dS . q_pe (bf16), from the same dS
// fragments: q_pe_t is staged in LDS (rows 160 bytes apart) and each
// MFMA-first wave 4 + e holds the transposed fragments of positional columns
// 16e .. 16e+15 over the H dS rows (the first ceil(H/32) reduction steps),
// adds one MFMA per such step, and stores its 16 columns of the tile's rows
// from a small LDS tile at the next tile, whole 128-byte rows, one store per
// wave.  With H an odd multiple of 16 the last of these steps also spans the
// first 16 P rows; the upper half of its q_pe fragment is zero, so they add
// nothing.
template <int NKS, bool PE>
__global__ __attribute__((amdgpu_flat_work_group_size(kIThreads, kIThreads), amdgpu_waves_per_eu(2, 2)))
void smla_k3_interm(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dO,
                    const uint16_t* __restrict__ dsp, const int32_t* __restrict__ idx,
                    int N, int K, uint16_t* __restrict__ interm,
                    const uint16_t* __restrict__ q_pe, uint16_t* __restrict__ interm_pe) {
    constexpr int H = NKS * 16;
    constexpr int R = 2 * H;
    constexpr int kYBytes = R * kYPitch;                 // one dsp block in LDS (padded rows)
    constexpr int kYChunks = R * kBK * 2 / 16;           // 16-B chunks of one dsp block
    constexpr int NKP = (NKS + 1) / 2;                   // reduction steps over the dS rows
    constexpr int kPeOPitch = kPeRow + 16;               // positional output row in LDS
    constexpr int kPeOBytes = kBK * kPeOPitch;
    static_assert(kYRing * kYBytes + 2 * kOBytes + (PE ? 2 * kPeOBytes : 0) <= 2 * kStageBytes,
                  "Y ring and output buffers must fit in the staging area");
    constexpr int kPasses = (R + kStageRows - 1) / kStageRows;
    constexpr int kRowsPerWave = kStageRows / kIWaves;   // row copies per wave per pass
    constexpr int kXpPitch = kPeRow + 32;                // 160 B: odd multiple of 32
    constexpr int kXpChunks = H * kDP * 2 / 16;          // 16-B chunks of q_pe_t
    constexpr int kXpPerThread = (kXpChunks + kIThreads - 1) / kIThreads;
    __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];  // two staging buffers
    __shared__ __attribute__((aligned(16))) char xpe[PE ? H * kXpPitch : 16];
    __shared__ SlotList L;

    // tokens from last to first: the late tokens (the most valid slots) go out
    // in the first rounds of workgroups, so the last round holds short ones,
    // and the first tokens taken are the ones the dQ pass touched last
    const int t = gridDim.x - 1 - blockIdx.x;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
    const size_t tok = (size_t)t * H * kD;
    const int32_t* idx_row = idx + (size_t)t * K;

    // ---- X = [q_t; dO_t] (R rows of 1 KiB) is copied straight into LDS, one
    // row per buffer->LDS copy, in passes of 64 rows through two staging
    // buffers: pass p+2 is in flight while pass p is read into registers.
    // Rows past R (a short last pass) read out of range and land as zeros.
    const i32x4 rq = make_rsrc(q + tok, (uint32_t)H * kD * 2);
    const i32x4 rd = make_rsrc(dO + tok, (uint32_t)H * kD * 2);
    const uint32_t stage0 = lds_addr(smem);
    auto issue_pass = [&](int p) {
        const uint32_t buf = stage0 + (p & 1) * kStageBytes;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = w + kIWaves * i;          // staged row within the pass
            const int row = p * kStageRows + r;     // X row
            const bool is_q = row < H;
            const int off = row < R ? (is_q ? row : row - H) * (kD * 2) + (lane << 4) : (1 << 30);
            copy_row_to_lds_nt(is_q ? rq : rd, buf + r * kRowPitch, off);
        }
    };
    // positional rows of the token, loaded first (older than every staging
    // copy, so the waits below still count only copies) and written to LDS
    // once the staging passes are through
    u32x4 xpv[kXpPerThread];
    if constexpr (PE) {
#pragma unroll
        for (int i = 0; i < kXpPerThread; ++i) {
            const int id = tid + kIThreads * i;
            if (id < kXpChunks) xpv[i] = *reinterpret_cast<const u32x4*>(q_pe + (size_t)t * H * kDP + id * 8);
        }
    }
    issue_pass(0);
    if (kPasses > 1) issue_pass(1);
    if (w == 0) compact_slots(idx_row, K, N, 0, &L, lane);

    // ---- X^T fragments: xf[dt][ks] holds column 64w + 16dt + c16 of X rows
    // 32ks + 4g .. +3, then 32ks + 16 + 4g .. +3 (the reduction order shared with
    // the Y operand).  Lane L of group g names staged row 4g + L/4 (then +16),
    // columns 64w + 16dt + 4(L%4): 16 consecutive rows per read, which with an
    // odd-multiple-of-32 pitch is free of LDS bank conflicts.
    u32x4 xf[4][NKS];
    const int xb = (4 * g + (c16 >> 2)) * kRowPitch + (64 * w + 4 * (c16 & 3)) * 2;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        // this wave's copies of pass p are done once only pass p+1's are younger
        if (p + 1 < kPasses) wait_vmcnt<kRowsPerWave>();
        else wait_vmcnt<0>();
        __syncthreads();
        const char* sbuf = smem + (p & 1) * kStageBytes;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (32 * ks >= p * kStageRows && 32 * ks < (p + 1) * kStageRows) {
                const char* ptr = sbuf + xb + (32 * ks - p * kStageRows) * kRowPitch;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const u32x2 lo = ds_read_tr16(ptr + dt * 32);
                    const u32x2 hi = ds_read_tr16(ptr + 16 * kRowPitch + dt * 32);
                    xf[dt][ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        }
        __syncthreads();
        if (p + 2 < kPasses) issue_pass(p + 2);
    }
    // xfp[ks] (waves 4-7, e = w - 4): positional column 16e + c16 of q_pe rows
    // 32ks + 4g .. +3, then 32ks + 16 + 4g .. +3 (zeros for rows past H)
    u32x4 xfp[PE ? NKP : 1];
    if constexpr (PE) {
#pragma unroll
        for (int i = 0; i < kXpPerThread; ++i) {
            const int id = tid + kIThreads * i;
            if (id < kXpChunks) *reinterpret_cast<u32x4*>(xpe + (id >> 3) * kXpPitch + (id & 7) * 16) = xpv[i];
        }
        __syncthreads();
        if (w >= kIWaves / 2) {
            const int xpb = (4 * g + (c16 >> 2)) * kXpPitch + (c16 & 3) * 8 + (w - kIWaves / 2) * 32;
#pragma unroll
            for (int ks = 0; ks < NKP; ++ks) {
                const u32x2 lo = ds_read_tr16(xpe + xpb + 32 * ks * kXpPitch);
                const u32x2 hi = 32 * ks + 16 < H ? ds_read_tr16(xpe + xpb + (32 * ks + 16) * kXpPitch)
                                                  : u32x2{0u, 0u};
                xfp[ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    }

    // ---- stream the Y tiles (one dsp block per compacted tile)
    // Waves w and w+4 share a SIMD.  After each tile's barrier, waves 4-7 go
    // straight to the next tile's MFMAs, while waves 0-3 first store the
    // previous tile's output rows and bring the next dsp block into LDS, then
    // run their MFMAs: each SIMD's MFMA pipe stays busy with one wave while the
    // other does the tile's memory work (with every wave doing both, the pair
    // did its memory work at the same time and left the pipe idle).
    const int ntk = (K + kBK - 1) / kBK;
    const uint16_t* ytok = dsp + (size_t)t * ntk * R * kBK;
    constexpr int kSWaves = kIWaves / 2;                  // waves that stage and store
    constexpr int kSThreads = kSWaves * 64;
    constexpr int kYPS = (kYChunks + kSThreads - 1) / kSThreads;
    const bool stager = w < kSWaves;
    // B operand: lane L of group g names Y row 32ks + 4g + L/4 (then +16),
    // columns 16sst + 4(L%4)
    const int yb = (4 * g + (c16 >> 2)) * kYPitch + (c16 & 3) * 8;
    u32x4 pre[kYPS];
    auto load_tile = [&](int ct) {
        const uint16_t* src = ytok + (size_t)ct * R * kBK;
#pragma unroll
        for (int i = 0; i < kYPS; ++i) {
            const int id = tid + kSThreads * i;
            if (id < kYChunks) pre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + id * 8));
        }
    };
    // piece id of the block (dsp piece layout): chunk id/64 of 16 rows, row
    // 16*(id/64) + id%16, positions 8g..8g+7 with g = (id/16)%4
    auto store_tile = [&](char* yb_lds) {
#pragma unroll
        for (int i = 0; i < kYPS; ++i) {
            const int id = tid + kSThreads * i;
            if (id < kYChunks)
                *reinterpret_cast<u32x4*>(yb_lds + ((id >> 6) * 16 + (id & 15)) * kYPitch +
                                          ((id >> 4) & 3) * 16) = pre[i];
        }
    };

    // Output rows go out as buffer stores: the slot list decides the row, and a
    // lane whose position is past the last valid slot gets an offset past the
    // token's range, which the hardware drops.
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        interm + (size_t)t * K * kD, (short)0, K * kD * 2, 0x00020000);
    // whole 1 KiB rows of tile `it` leave with one non-temporal store each
    // (staging wave w writes tile rows w, w+4, ...); row r is position r of the
    // block, i.e. slot 4(r/8) + r%4 (+16 when r%8 >= 4) of the tile
    // positional rows of tile `it`: wave 4 + e sends tile rows 8e .. 8e+7, 8
    // lanes (16 bytes each) per 128-byte row
    const __amdgpu_buffer_rsrc_t pe_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        PE ? interm_pe + (size_t)t * K * kDP : interm, (short)0, PE ? K * kPeRow : 0, 0x00020000);
    auto store_pe_rows = [&](int it, int n) {
        if constexpr (PE) {
            const char* pbuf = smem + kYRing * kYBytes + 2 * kOBytes + (it & 1) * kPeOBytes;
            const int r = 8 * (w - kIWaves / 2) + (lane >> 3);
            const int pos = it * kBK + ((r & 4) << 2) + ((r >> 3) << 2) + (r & 3);
            const u32x4 v = *reinterpret_cast<const u32x4*>(pbuf + r * kPeOPitch + (lane & 7) * 16);
            const int voff = pos < n ? L.slot[pos] * kPeRow + (lane & 7) * 16 : K * kPeRow;
            __builtin_amdgcn_raw_buffer_store_b128(v, pe_rsrc, voff, 0, kCacheNT);
        }
    };
    auto store_rows = [&](int it, int n) {
        const char* obuf = smem + kYRing * kYBytes + (it & 1) * kOBytes;
#pragma unroll
        for (int i = 0; i < kBK / kSWaves; ++i) {
            const int r = w + kSWaves * i;
            const int pos = it * kBK + ((r & 4) << 2) + ((r >> 3) << 2) + (r & 3);
            const u32x4 v = *reinterpret_cast<const u32x4*>(obuf + r * kOPitch + lane * 16);
            const int voff = pos < n ? L.slot[pos] * (kD * 2) + lane * 16 : K * kD * 2;
            __builtin_amdgcn_raw_buffer_store_b128(v, out_rsrc, voff, 0, kCacheNT);
        }
    };
    int ctg = 0;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        if (k0 > 0) {
            __syncthreads();  // the previous chunk's row stores have read L and the output buffers
            if (w == 0) compact_slots(idx_row, K, N, k0, &L, lane);
        }
        __syncthreads();
        const int n = L.n;
        const int ntile = (n + kBK - 1) / kBK;
        if (ntile > 0 && stager) {
            load_tile(ctg);
            store_tile(smem);
            if (ntile > 1) load_tile(ctg + 1);
        }
        __syncthreads();
        for (int it = 0; it < ntile; ++it) {
            if (PE && !stager && it > 0) store_pe_rows(it - 1, n);
            if (stager) {
                if (it > 0) store_rows(it - 1, n);
                // tile it+1 (loaded during the previous iteration) goes to the ring
                // slot that tile it-1 used; its loads are older than the row stores
                // just issued, so waiting for them does not wait for those
                if (it + 1 < ntile) {
                    store_tile(smem + ((it + 1) % kYRing) * kYBytes);
                    if (it + 2 < ntile) load_tile(ctg + it + 2);
                }
            }
            const char* ybuf = smem + (it % kYRing) * kYBytes;
            char* obuf = smem + kYRing * kYBytes + (it & 1) * kOBytes;
#pragma unroll
            for (int sst = 0; sst < 2; ++sst) {
                // every B fragment (32 r x 16 slots) is read once and feeds the four
                // d-blocks of this wave (four accumulation chains)
                f32x4 cacc[4], cpe = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) cacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const char* p = ybuf + yb + ks * 32 * kYPitch + sst * 32;
                    const u32x2 lo = ds_read_tr16(p);
                    const u32x2 hi = ds_read_tr16(p + 16 * kYPitch);
                    const u32x4 bfrag = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) cacc[dt] = mfma16(xf[dt][ks], bfrag, cacc[dt]);
                    if constexpr (PE) {
                        if (ks < NKP && !stager) cpe = mfma16(xfp[ks < NKP ? ks : 0], bfrag, cpe);
                    }
                }
                if constexpr (PE) {
                    // lane c16 + 16g: block position 16sst + c16, positional
                    // columns 16e + 4g .. +3
                    if (!stager) {
                        char* prow = smem + kYRing * kYBytes + 2 * kOBytes + (it & 1) * kPeOBytes +
                                     (16 * sst + c16) * kPeOPitch + ((w - kIWaves / 2) * 16 + 4 * g) * 2;
                        *reinterpret_cast<u32x2*>(prow) = u32x2{pack_bf16(cpe[0], cpe[1]), pack_bf16(cpe[2], cpe[3])};
                    }
                }
                // lane c16 + 16g holds slot it*32 + 16sst + c16, columns 64w + 16dt + 4g
                // .. +3; the tile's output rows are assembled in LDS
                char* orow = obuf + (16 * sst + c16) * kOPitch + (64 * w + 4 * g) * 2;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    *reinterpret_cast<u32x2*>(orow + dt * 32) =
                        u32x2{pack_bf16(cacc[dt][0], cacc[dt][1]), pack_bf16(cacc[dt][2], cacc[dt][3])};
            }
            __syncthreads();
        }
        if (ntile > 0 && stager) store_rows(ntile - 1, n);
        if (PE && ntile > 0 && !stager) store_pe_rows(ntile - 1, n);
        ctg += ntile;
    }
}

hipError_t launch_interm(const uint16_t* q, const uint16_t* dO, const uint16_t* dsp,
                         const int32_t* idx, int T, int H, int N, int K, uint16_t* interm,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
#define SMLA_INTERM_CASE(nks) \
    case nks: smla_k3_interm<nks, false><<<T, kIThreads, 0, s>>>(q, dO, dsp, idx, N, K, interm, nullptr, nullptr); break;
    switch (H / 16) {
        SMLA_INTERM_CASE(1)
        SMLA_INTERM_CASE(2)
        SMLA_INTERM_CASE(3)
        SMLA_INTERM_CASE(4)
        SMLA_INTERM_CASE(5)
        SMLA_INTERM_CASE(6)
        SMLA_INTERM_CASE(7)
        SMLA_INTERM_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef SMLA_INTERM_CASE
    return hipGetLastError();
}

}  // namespace smla

namespace smla {

hipError_t launch_interm_fused_pe(const uint16_t* q, const uint16_t* dO, const uint16_t* q_pe,
                                  const uint16_t* dsp, const int32_t* idx, int T, int H, int N, int K,
                                  uint16_t* interm, uint16_t* interm_pe, hipStream_t s) {
    if (T == 0) return hipSuccess;
#define SMLA_INTERM_PE_CASE(nks)                                                                   \
    case nks:                                                                                      \
        smla_k3_interm<nks, true><<<T, kIThreads, 0, s>>>(q, dO, dsp, idx, N, K, interm, q_pe, interm_pe); \
        break;
    switch (H / 16) {
        SMLA_INTERM_PE_CASE(1)
        SMLA_INTERM_PE_CASE(2)
        SMLA_INTERM_PE_CASE(3)
        SMLA_INTERM_PE_CASE(4)
        SMLA_INTERM_PE_CASE(5)
        SMLA_INTERM_PE_CASE(6)
        SMLA_INTERM_PE_CASE(7)
        SMLA_INTERM_PE_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef SMLA_INTERM_PE_CASE
    return hipGetLastError();
}

}  // namespace smla
