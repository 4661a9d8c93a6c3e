// dQ kernel of the sparse MLA backward (also emits scale*dS and P per slot).
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table, "dQ"
// row: the gathered kv rows are read from LDS once and feed both the S and dP
// products; the kernel also writes this pass's dS and P.
//
// Work unit: one query token t and a group of NW*16 heads (one wave = 16
// heads).  Per wave, q and dO of its heads stay in registers as MFMA B
// operands for the whole token; the kernel walks the token's top-k slots in
// tiles of 32 (double-buffered LDS, next tile's global loads in flight while
// the current one is computed):
//   S^T, dP^T [32 slots x 16 heads] = kv_tile . {q, dO}^T     (MFMA, reduce d=512)
//   P  = exp(scale*S - lse)   (0 on masked slots)
//   dS = P * (dP - delta)
//   dq^T [512 x 16 heads] += kv_tile^T . (scale*dS)^T           (MFMA, reduce 32 slots)
// The S^T accumulator leaves each lane with one head and 8 slots, which is
// exactly the B-operand layout of the second product: no data exchange.
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void smla_k2_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
    const int nhg = H / (NW * 16);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int t = logical / nhg;
    const int hg = logical - t * nhg;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
    const int h = hg * NW * 16 + w * 16 + c16;
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
    const int32_t* idx_row = idx + (size_t)t * K;
    const size_t dsp_tok = (size_t)t * K * (2 * H);

    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (K + kBK - 1) / kBK;
    KvTile<NW> tile;
    tile.load(kv, idx_row, K, N, 0, w, lane);
    tile.store(smem, w, lane);
    uint32_t mask = tile.mask;
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const char* buf = smem + (it & 1) * kTileBytes;
        const bool more = it + 1 < ntiles;
        if (more) tile.load(kv, idx_row, K, N, it + 1, w, lane);
        if (mask != 0u) {
            f32x4 sacc[2], pacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < 16; ++ds) {
                    const u32x4 a = tile_rows_a(buf, st, ds, c16, g);
                    sacc[st] = mfma16(a, qf[ds], sacc[st]);
                    pacc[st] = mfma16(a, dof[ds], pacc[st]);
                }
            }
            float dss[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int slot = 16 * st + 4 * g + j;
                    const bool v = (mask >> slot) & 1u;
                    const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[st][j], c, -bias)) : 0.f;
                    const float d = p * (pacc[st][j] - dl) * scale;
                    dss[st][j] = d;
                    const int k = it * kBK + slot;
                    if (k < K) {
                        const size_t o = dsp_tok + (size_t)k * (2 * H) + h;
                        dsp[o] = to_bf16(d);
                        dsp[o + H] = to_bf16(p);
                    }
                }
            }
            const u32x4 bf = {pack_bf16(dss[0][0], dss[0][1]), pack_bf16(dss[0][2], dss[0][3]),
                              pack_bf16(dss[1][0], dss[1][1]), pack_bf16(dss[1][2], dss[1][3])};
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt] = mfma16(tile_cols_a(buf, dt, c16, g), bf, acc[dt]);
        }
        if (more) {
            tile.store(smem + ((it + 1) & 1) * kTileBytes, w, lane);
            mask = tile.mask;
        }
        __syncthreads();
    }

    // lane holds dq^T rows d = 16*dt + 4g .. +3 of head h: 4 contiguous bf16
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
        const u32x2 v = {pack_bf16(acc[dt][0], acc[dt][1]), pack_bf16(acc[dt][2], acc[dt][3])};
        *reinterpret_cast<u32x2*>(dq + qrow + 16 * dt + 4 * g) = v;
    }
}

// Heads per workgroup: the largest multiple of 16 that divides H, at most 64.
static int pick_waves(int H) {
    for (int nw = 4; nw >= 1; --nw)
        if (H % (nw * 16) == 0) return nw;
    return 1;
}

hipError_t launch_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
                     const float* delta, const int32_t* idx, int T, int H, int N, int K, float scale,
                     uint16_t* dq, uint16_t* dsp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int nw = pick_waves(H);
    const unsigned blocks = (unsigned)T * (unsigned)(H / (nw * 16));
    switch (nw) {
        case 4: smla_k2_dq<4><<<blocks, 256, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        case 3: smla_k2_dq<3><<<blocks, 192, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        case 2: smla_k2_dq<2><<<blocks, 128, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
        default: smla_k2_dq<1><<<blocks, 64, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp); break;
    }
    return hipGetLastError();
}

}  // namespace smla
