// dQ kernel of the sparse MLA backward (also emits scale*dS and P per slot).
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table, "dQ"
// row: the gathered kv rows are read from LDS once and feed both the S and dP
// products; the kernel also writes this pass's dS and P.
//
// Work unit: one query token t and a group of NW*16 heads (one wave = 16
// heads).  Per wave, q and dO of its heads stay in registers as MFMA B
// operands for the whole token.  The token's valid slots are compacted and
// walked in tiles of 32 kv rows copied straight into a 4-deep LDS ring:
//   S^T, dP^T [32 slots x 16 heads] = kv_tile . {q, dO}^T     (MFMA, reduce d=512)
//   P  = exp(scale*S - lse)
//   dS = P * (dP - delta)
//   dq^T [512 x 16 heads] += kv_tile^T . (scale*dS)^T           (MFMA, reduce 32 slots)
// The S^T accumulator leaves each lane with one head and 8 slots, which is
// exactly the B-operand layout of the second product: no data exchange.
//
// dsp layout (consumed by the intermediate kernel): for token t and compacted
// tile c (c < ceil(topk/32)), a [2H][32] bf16 block at ((t*ceil(topk/32) + c)*2H)*32:
// rows 0..H-1 hold scale*dS of head h, rows H..2H-1 hold P, column j is the
// j-th slot of the tile; tail columns past the last valid slot hold zeros.
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void smla_k2_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    static_assert(kNBuf == 4, "the vmcnt bounds below assume a 4-deep ring");
    constexpr int R = kBK / NW;   // DMA copies per wave per tile
    constexpr int S = 4;          // dS/P stores per wave per tile
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList L;

    const int nhg = H / (NW * 16);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int t = logical / nhg;
    const int hg = logical - t * nhg;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
    const int h = hg * NW * 16 + w * 16 + c16;
    const size_t qrow = ((size_t)t * H + h) * kD;
    const int32_t* idx_row = idx + (size_t)t * K;
    if (w == 0) compact_slots(idx_row, K, N, 0, &L, lane);

    u32x4 qf[16], dof[16];
#pragma unroll
    for (int ds = 0; ds < 16; ++ds) {
        qf[ds] = *reinterpret_cast<const u32x4*>(q + qrow + 32 * ds + 8 * g);
        dof[ds] = *reinterpret_cast<const u32x4*>(dO + qrow + 32 * ds + 8 * g);
    }
    const float lse_h = lse[(size_t)t * H + h];
    const float bias = (lse_h == -INFINITY) ? INFINITY : lse_h * kLog2e;
    const float c = scale * kLog2e;
    const float dl = delta[(size_t)t * H + h];
    const i32x4 rsrc = make_rsrc(kv, (uint32_t)N * (kD * 2));
    const uint32_t ring = lds_addr(tiles);
    const int rb = rows_base(c16, g), cb = cols_base(c16, g);
    const int ntk = (K + kBK - 1) / kBK;
    uint16_t* dsp_tok = dsp + (size_t)t * ntk * (2 * H) * kBK;

    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over the compacted tiles of a chunk.  Iteration j
    // turns tile j's S/dP accumulators into P and dS (VALU, stores), then runs
    // one unrolled block that interleaves the dq MFMAs of tile j with the S/dP
    // MFMAs of tile j+1: two independent MFMA chains hide each other's LDS read
    // latency.  Tile j+3 is copied into the ring slot tile j-1 used.
    // VMEM ops per wave: R copies per tile, 4 dS/P stores per tile; the vmcnt
    // bound when waiting for tile j+1 counts the ops issued after its copies.
    int ctg = 0;  // compacted tiles of earlier chunks
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        if (k0 > 0 && w == 0) compact_slots(idx_row, K, N, k0, &L, lane);
        __syncthreads();
        const int n = L.n;
        const int ntile = (n + kBK - 1) / kBK;
#pragma unroll
        for (int p = 0; p < kNBuf - 1; ++p) issue_tile<NW>(rsrc, &L, p, ring + p * kTileBytes, w, lane);
        if (ntile > 0) {
            f32x4 sacc[2], pacc[2];
            wait_vmcnt<(2 * R < 63 ? 2 * R : 63)>();
            __syncthreads();
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ds = 0; ds < 16; ++ds) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const u32x4 a = tile_rows_a(tiles, rb, st, ds);
                    sacc[st] = mfma16(a, qf[ds], sacc[st]);
                    pacc[st] = mfma16(a, dof[ds], pacc[st]);
                }
            }
            // P and scale*dS of tile j from its accumulators; stores; B operand of dq
            auto softmax_grad = [&](int j) -> u32x4 {
                float dss[2][4], ps[2][4];
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool v = j * kBK + 16 * st + 4 * g + i < n;
                        const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[st][i], c, -bias)) : 0.f;
                        ps[st][i] = p;
                        dss[st][i] = p * (pacc[st][i] - dl) * scale;
                    }
                uint16_t* blk = dsp_tok + (size_t)(ctg + j) * (2 * H) * kBK;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    *reinterpret_cast<u32x2*>(blk + (size_t)h * kBK + 16 * st + 4 * g) =
                        u32x2{pack_bf16(dss[st][0], dss[st][1]), pack_bf16(dss[st][2], dss[st][3])};
                    *reinterpret_cast<u32x2*>(blk + (size_t)(H + h) * kBK + 16 * st + 4 * g) =
                        u32x2{pack_bf16(ps[st][0], ps[st][1]), pack_bf16(ps[st][2], ps[st][3])};
                }
                return u32x4{pack_bf16(dss[0][0], dss[0][1]), pack_bf16(dss[0][2], dss[0][3]),
                             pack_bf16(dss[1][0], dss[1][1]), pack_bf16(dss[1][2], dss[1][3])};
            };
            for (int j = 0; j + 1 < ntile; ++j) {
                if (j == 0) wait_vmcnt<(R < 63 ? R : 63)>();
                else if (j == 1) wait_vmcnt<(R + S < 63 ? R + S : 63)>();
                else wait_vmcnt<(R + 2 * S < 63 ? R + 2 * S : 63)>();
                __syncthreads();  // tile j+1 landed everywhere; ring slot of tile j-1 is free
                issue_tile<NW>(rsrc, &L, j + kNBuf - 1, ring + ((j + kNBuf - 1) % kNBuf) * kTileBytes, w, lane);
                const u32x4 bf = softmax_grad(j);
                const char* bufa = tiles + (j % kNBuf) * kTileBytes;
                const char* bufb = tiles + ((j + 1) % kNBuf) * kTileBytes;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int ds = 0; ds < 16; ++ds) {
                    acc[2 * ds] = mfma16(tile_cols_a(bufa, cb, 2 * ds), bf, acc[2 * ds]);
                    acc[2 * ds + 1] = mfma16(tile_cols_a(bufa, cb, 2 * ds + 1), bf, acc[2 * ds + 1]);
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const u32x4 a = tile_rows_a(bufb, rb, st, ds);
                        sacc[st] = mfma16(a, qf[ds], sacc[st]);
                        pacc[st] = mfma16(a, dof[ds], pacc[st]);
                    }
                }
            }
            const int jl = ntile - 1;
            const u32x4 bf = softmax_grad(jl);
            const char* bufl = tiles + (jl % kNBuf) * kTileBytes;
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt] = mfma16(tile_cols_a(bufl, cb, dt), bf, acc[dt]);
        }
        ctg += ntile;
        wait_vmcnt<0>();   // the ring's trailing copies land before LDS is reused
        __syncthreads();
    }

    // lane holds dq^T rows d = 16*dt + 4g .. +3 of head h: 4 contiguous bf16
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
        const u32x2 v = {pack_bf16(acc[dt][0], acc[dt][1]), pack_bf16(acc[dt][2], acc[dt][3])};
        *reinterpret_cast<u32x2*>(dq + qrow + 16 * dt + 4 * g) = v;
    }
}

// Producer/consumer variant for 64-head groups (H % 64 == 0): 8 waves, two per
// SIMD, so one wave's LDS and barrier waits are covered by the other's MFMAs.
//   producers (waves 0-3): 16 heads each; q and dO in registers; S^T, dP^T of
//     a tile, then P and scale*dS (stored as dsp blocks) and the dS fragment,
//     published in LDS;
//   consumers (waves 4-7): all 64 heads x 128 d of the dq accumulator each;
//     every transposed kv read feeds four MFMAs (one per head group), which
//     halves the LDS instructions of the dq product.
// Waves w and w+4 share a SIMD (measured on gfx950 from HW_ID), so each SIMD
// runs one producer and one consumer.
// Producers run one tile ahead of consumers; one barrier per tile orders the
// kv ring, the dS fragments (double-buffered) and the ring slot reuse.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pc(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                   const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                   const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                   int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    static_assert(kNBuf == 4, "the vmcnt bounds below assume a 4-deep ring");
    constexpr int NWAVES = 8;
    constexpr int R = kBK / NWAVES;   // copies per wave per tile
    constexpr int S = 4;              // dS/P stores per producer per tile
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList L;
    __shared__ u32x4 dsfrag[2][4][64];  // dS fragments: [slot parity][producer][lane]

    const int nhg = H / 64;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int t = logical / nhg;
    const int hg = logical - t * nhg;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
    const int32_t* idx_row = idx + (size_t)t * K;
    // a consumer wave compacts the slots while the producers load q and dO
    if (w == 4) compact_slots(idx_row, K, N, 0, &L, lane);
    const i32x4 rsrc = make_rsrc(kv, (uint32_t)N * (kD * 2));
    const uint32_t ring = lds_addr(tiles);
    const int ntk = (K + kBK - 1) / kBK;

    if (w < 4) {
        // ------------------------------------------------------------ producer
        const int h = hg * 64 + w * 16 + c16;
        const size_t qrow = ((size_t)t * H + h) * kD;
        u32x4 qf[16], dof[16];
#pragma unroll
        for (int ds = 0; ds < 16; ++ds) {
            qf[ds] = *reinterpret_cast<const u32x4*>(q + qrow + 32 * ds + 8 * g);
            dof[ds] = *reinterpret_cast<const u32x4*>(dO + qrow + 32 * ds + 8 * g);
        }
        const float lse_h = lse[(size_t)t * H + h];
        const float bias = (lse_h == -INFINITY) ? INFINITY : lse_h * kLog2e;
        const float c = scale * kLog2e;
        const float dl = delta[(size_t)t * H + h];
        const int rb = rows_base(c16, g);
        uint16_t* dsp_tok = dsp + (size_t)t * ntk * (2 * H) * kBK;
        int ctg = 0;
        for (int k0 = 0; k0 < K; k0 += kChunk) {
            __syncthreads();
            const int n = L.n;
            const int ntile = (n + kBK - 1) / kBK;
#pragma unroll
            for (int p = 0; p < kNBuf - 1; ++p)
                issue_tile<NWAVES>(rsrc, &L, p, ring + p * kTileBytes, w, lane);
            // S^T, dP^T of tile j -> P, scale*dS (stored) -> dS fragment into LDS
            auto produce = [&](int j) {
                const char* buf = tiles + (j % kNBuf) * kTileBytes;
                // four independent accumulation chains (S and dP of both 16-slot halves)
                f32x4 sacc[2], pacc[2];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int ds = 0; ds < 16; ++ds) {
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const u32x4 a = tile_rows_a(buf, rb, st, ds);
                        sacc[st] = mfma16(a, qf[ds], sacc[st]);
                        pacc[st] = mfma16(a, dof[ds], pacc[st]);
                    }
                }
                float dss[2][4], ps[2][4];
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool v = j * kBK + 16 * st + 4 * g + i < n;
                        const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[st][i], c, -bias)) : 0.f;
                        ps[st][i] = p;
                        dss[st][i] = p * (pacc[st][i] - dl) * scale;
                    }
                uint16_t* blk = dsp_tok + (size_t)(ctg + j) * (2 * H) * kBK;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    *reinterpret_cast<u32x2*>(blk + (size_t)h * kBK + 16 * st + 4 * g) =
                        u32x2{pack_bf16(dss[st][0], dss[st][1]), pack_bf16(dss[st][2], dss[st][3])};
                    *reinterpret_cast<u32x2*>(blk + (size_t)(H + h) * kBK + 16 * st + 4 * g) =
                        u32x2{pack_bf16(ps[st][0], ps[st][1]), pack_bf16(ps[st][2], ps[st][3])};
                }
                dsfrag[j & 1][w][lane] =
                    u32x4{pack_bf16(dss[0][0], dss[0][1]), pack_bf16(dss[0][2], dss[0][3]),
                          pack_bf16(dss[1][0], dss[1][1]), pack_bf16(dss[1][2], dss[1][3])};
            };
            if (ntile > 0) {
                wait_vmcnt<2 * R>();
                __syncthreads();
                produce(0);
                for (int j = 0; j < ntile; ++j) {
                    if (j + 1 < ntile) {
                        if (j == 0) wait_vmcnt<R + S>();
                        else wait_vmcnt<R + 2 * S>();
                    }
                    __syncthreads();
                    issue_tile<NWAVES>(rsrc, &L, j + kNBuf - 1,
                                       ring + ((j + kNBuf - 1) % kNBuf) * kTileBytes, w, lane);
                    if (j + 1 < ntile) produce(j + 1);
                }
            }
            ctg += ntile;
            wait_vmcnt<0>();
            __syncthreads();
        }
    } else {
        // ------------------------------------------------------------ consumer
        const int dq4 = w - 4;  // d in [128 dq4, 128 dq4 + 128)
        const int cb = cols_base(c16, g);
        f32x4 acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < K; k0 += kChunk) {
            if (k0 > 0 && w == 4) compact_slots(idx_row, K, N, k0, &L, lane);
            __syncthreads();
            const int n = L.n;
            const int ntile = (n + kBK - 1) / kBK;
#pragma unroll
            for (int p = 0; p < kNBuf - 1; ++p)
                issue_tile<NWAVES>(rsrc, &L, p, ring + p * kTileBytes, w, lane);
            if (ntile > 0) {
                wait_vmcnt<2 * R>();
                __syncthreads();
                for (int j = 0; j < ntile; ++j) {
                    if (j + 1 < ntile) wait_vmcnt<R>();
                    __syncthreads();
                    issue_tile<NWAVES>(rsrc, &L, j + kNBuf - 1,
                                       ring + ((j + kNBuf - 1) % kNBuf) * kTileBytes, w, lane);
                    u32x4 b[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) b[m] = dsfrag[j & 1][m][lane];
                    const char* buf = tiles + (j % kNBuf) * kTileBytes;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const u32x4 a = tile_cols_a(buf, cb, 8 * dq4 + dt);
#pragma unroll
                        for (int m = 0; m < 4; ++m) acc[dt][m] = mfma16(a, b[m], acc[dt][m]);
                    }
                }
            }
            wait_vmcnt<0>();
            __syncthreads();
        }
        // lane holds dq^T rows d = 128dq4 + 16dt + 4g .. +3 of head 16m + c16
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int h = hg * 64 + 16 * m + c16;
            uint16_t* out = dq + ((size_t)t * H + h) * kD + 128 * dq4 + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *reinterpret_cast<u32x2*>(out + 16 * dt) =
                    u32x2{pack_bf16(acc[dt][m][0], acc[dt][m][1]), pack_bf16(acc[dt][m][2], acc[dt][m][3])};
        }
    }
}

// Heads per workgroup: 64, 32 or 16 (whichever divides H first).
int dq_waves(int H) {
    if (H % 64 == 0) return 4;
    if (H % 32 == 0) return 2;
    return 1;
}

hipError_t launch_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
                     const float* delta, const int32_t* idx, int T, int H, int N, int K, float scale,
                     uint16_t* dq, uint16_t* dsp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int nw = dq_waves(H);
    const unsigned blocks = (unsigned)T * (unsigned)(H / (nw * 16));
    switch (nw) {
        case 4: smla_k2_dq_pc<<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        case 2: smla_k2_dq<2><<<blocks, 128, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        default: smla_k2_dq<1><<<blocks, 64, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
    }
    return hipGetLastError();
}

}  // namespace smla
