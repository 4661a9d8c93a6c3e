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

// vmcnt allowed while waiting for tile `it`: DMA copies of the two tiles issued
// after it (2R) plus the dS/P stores (S per tile) of up to three iterations.
template <int R, int S>
__device__ __forceinline__ void wait_tile(int it) {
    constexpr int a0 = (2 * R) < 63 ? 2 * R : 63;
    constexpr int a1 = (2 * R + S) < 63 ? 2 * R + S : 63;
    constexpr int a2 = (2 * R + 2 * S) < 63 ? 2 * R + 2 * S : 63;
    constexpr int a3 = (2 * R + 3 * S) < 63 ? 2 * R + 3 * S : 63;
    if (it == 0) wait_vmcnt<a0>();
    else if (it == 1) wait_vmcnt<a1>();
    else if (it == 2) wait_vmcnt<a2>();
    else wait_vmcnt<a3>();
}

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void smla_k2_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    static_assert(kNBuf == 4, "wait_tile assumes a 4-deep ring");
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

    int ctg = 0;  // compacted tiles of earlier chunks
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        if (k0 > 0 && w == 0) compact_slots(idx_row, K, N, k0, &L, lane);
        __syncthreads();
        const int n = L.n;
        const int ntile = (n + kBK - 1) / kBK;
#pragma unroll
        for (int p = 0; p < kNBuf - 1; ++p) issue_tile<NW>(rsrc, &L, p, ring + p * kTileBytes, w, lane);
        for (int it = 0; it < ntile; ++it) {
            wait_tile<R, S>(it);
            __syncthreads();  // tile `it` landed for every wave; buffer (it-1)%4 is free
            issue_tile<NW>(rsrc, &L, it + kNBuf - 1, ring + ((it + kNBuf - 1) % kNBuf) * kTileBytes, w, lane);
            const char* buf = tiles + (it % kNBuf) * kTileBytes;

            f32x4 sacc[2], pacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < 16; ++ds) {
                    const u32x4 a = tile_rows_a(buf, rb, st, ds);
                    sacc[st] = mfma16(a, qf[ds], sacc[st]);
                    pacc[st] = mfma16(a, dof[ds], pacc[st]);
                }
            }
            float dss[2][4], ps[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool v = it * kBK + 16 * st + 4 * g + j < n;
                    const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[st][j], c, -bias)) : 0.f;
                    ps[st][j] = p;
                    dss[st][j] = p * (pacc[st][j] - dl) * scale;
                }
            uint16_t* blk = dsp_tok + (size_t)(ctg + it) * (2 * H) * kBK;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                *reinterpret_cast<u32x2*>(blk + (size_t)h * kBK + 16 * st + 4 * g) =
                    u32x2{pack_bf16(dss[st][0], dss[st][1]), pack_bf16(dss[st][2], dss[st][3])};
                *reinterpret_cast<u32x2*>(blk + (size_t)(H + h) * kBK + 16 * st + 4 * g) =
                    u32x2{pack_bf16(ps[st][0], ps[st][1]), pack_bf16(ps[st][2], ps[st][3])};
            }
            const u32x4 bf = {pack_bf16(dss[0][0], dss[0][1]), pack_bf16(dss[0][2], dss[0][3]),
                              pack_bf16(dss[1][0], dss[1][1]), pack_bf16(dss[1][2], dss[1][3])};
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt] = mfma16(tile_cols_a(buf, cb, dt), bf, acc[dt]);
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
        case 4: smla_k2_dq<4><<<blocks, 256, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        case 2: smla_k2_dq<2><<<blocks, 128, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        default: smla_k2_dq<1><<<blocks, 64, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
    }
    return hipGetLastError();
}

}  // namespace smla
