// dKV intermediate of the sparse MLA backward, contracted over all heads.
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table,
// "dKV-interm" row (all heads contracted inside one pair of MFMA chains, q and
// dO transposed once into registers, D split over waves) and the R_CHUNK note
// (the intermediate is [T, topk, 512] bf16).
//
// For token t, with X = [q_t ; dO_t] (2H x 512) and Y_t[k] = [scale*dS_t[:,k] ; P_t[:,k]]
// (the dsp rows written by the dQ kernel), one product gives both terms:
//   interm^T [512 x topk] = X^T . Y_t      (reduction over r in [0, 2H))
// Work unit: one token per workgroup of 8 waves; wave w owns d in [64w, 64w+64).
// X^T fragments (MFMA A operands: one d row, 8 consecutive r) are built once
// per token through LDS and stay in registers; Y tiles of 32 slots stream
// through double-buffered LDS.  Tiles whose 32 slots are all masked are
// skipped: their interm rows are never read by the gather.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {
constexpr int kIWaves = 8;
constexpr int kIThreads = kIWaves * 64;
constexpr int kXStride = kD + 8;       // bf16 per staged X row
constexpr int kStageRows = 64;         // X rows staged per pass
constexpr int kSmemElems = kStageRows * kXStride;   // 33,280 bf16 = 66,560 B
}  // namespace

// NKS = 2H / 32 reduction steps (H = 16 * NKS)
template <int NKS>
__global__ __attribute__((amdgpu_flat_work_group_size(kIThreads, kIThreads), amdgpu_waves_per_eu(2, 2)))
void smla_k3_interm(const uint16_t* __restrict__ q, const uint16_t* __restrict__ dO,
                    const uint16_t* __restrict__ dsp, const int32_t* __restrict__ idx, int T,
                    int N, int K, uint16_t* __restrict__ interm) {
    constexpr int H = NKS * 16;
    constexpr int R = 2 * H;
    constexpr int kYStride = R + 8;                      // bf16 per Y row in LDS
    constexpr int kYChunks = 32 * (R / 8);               // 16-B chunks per tile
    constexpr int kYPT = (kYChunks + kIThreads - 1) / kIThreads;
    static_assert(2 * 32 * kYStride <= kSmemElems, "tile buffers exceed LDS staging area");
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmemElems];

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
    const size_t tok = (size_t)t * H * kD;

    // ---- X^T fragments: xf[dt][ks] = X[32ks + 8g .. +7][64w + 16dt + c16]
    u32x4 xf[4][NKS];
    for (int c0 = 0; c0 < R; c0 += kStageRows) {
#pragma unroll
        for (int i = 0; i < kStageRows * (kD / 8) / kIThreads; ++i) {
            const int id = tid + kIThreads * i;
            const int r = id >> 6, ch = id & 63;
            const int row = c0 + r;
            if (row < R) {
                const uint16_t* src = row < H ? q + tok + (size_t)row * kD
                                              : dO + tok + (size_t)(row - H) * kD;
                *reinterpret_cast<u32x4*>(smem + r * kXStride + ch * 8) =
                    *reinterpret_cast<const u32x4*>(src + ch * 8);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (32 * ks >= c0 && 32 * ks < c0 + kStageRows) {
                const int rl = 32 * ks - c0 + 8 * g;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const int d = 64 * w + 16 * dt + c16;
                    uint32_t e[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) e[k] = smem[(rl + k) * kXStride + d];
                    xf[dt][ks] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                       e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                }
            }
        }
        __syncthreads();
    }

    // ---- stream the Y tiles
    const int32_t* idx_row = idx + (size_t)t * K;
    const uint16_t* ytok = dsp + (size_t)t * K * R;
    const int ntiles = (K + 31) / 32;
    auto tile_mask = [&](int tl) -> uint32_t {
        const int slot = tl * 32 + lane;
        const int v = (lane < 32 && slot < K) ? idx_row[slot] : -1;
        return (uint32_t)__ballot(lane < 32 && valid_row(v, N));
    };
    auto next_tile = [&](int from) -> int {
        int tl = from;
        while (tl < ntiles && tile_mask(tl) == 0u) ++tl;
        return tl;
    };
    u32x4 pre[kYPT];
    auto load_tile = [&](int tl) {
#pragma unroll
        for (int i = 0; i < kYPT; ++i) {
            const int id = tid + kIThreads * i;
            const int s = id / (R / 8), ch = id - s * (R / 8);
            const int k = tl * 32 + s;
            pre[i] = (id < kYChunks && k < K)
                         ? *reinterpret_cast<const u32x4*>(ytok + (size_t)k * R + ch * 8)
                         : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](uint16_t* yb) {
#pragma unroll
        for (int i = 0; i < kYPT; ++i) {
            const int id = tid + kIThreads * i;
            const int s = id / (R / 8), ch = id - s * (R / 8);
            if (id < kYChunks) *reinterpret_cast<u32x4*>(yb + s * kYStride + ch * 8) = pre[i];
        }
    };

    int cur = next_tile(0);
    if (cur < ntiles) {
        load_tile(cur);
        store_tile(smem);
    }
    __syncthreads();
    int buf = 0;
    while (cur < ntiles) {
        const int nxt = next_tile(cur + 1);
        if (nxt < ntiles) load_tile(nxt);
        const uint16_t* yb = smem + buf * 32 * kYStride;
#pragma unroll
        for (int sst = 0; sst < 2; ++sst) {
            const int k = cur * 32 + 16 * sst + c16;
            uint16_t* orow = interm + ((size_t)t * K + k) * kD + 64 * w + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                f32x4 cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const u32x4 b =
                        *reinterpret_cast<const u32x4*>(yb + (16 * sst + c16) * kYStride + 32 * ks + 8 * g);
                    cacc = mfma16(xf[dt][ks], b, cacc);
                }
                if (k < K) {
                    const u32x2 v = {pack_bf16(cacc[0], cacc[1]), pack_bf16(cacc[2], cacc[3])};
                    *reinterpret_cast<u32x2*>(orow + 16 * dt) = v;
                }
            }
        }
        if (nxt < ntiles) store_tile(smem + (buf ^ 1) * 32 * kYStride);
        __syncthreads();
        buf ^= 1;
        cur = nxt;
    }
}

hipError_t launch_interm(const uint16_t* q, const uint16_t* dO, const uint16_t* dsp,
                         const int32_t* idx, int T, int H, int N, int K, uint16_t* interm,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
#define SMLA_INTERM_CASE(nks) \
    case nks: smla_k3_interm<nks><<<T, kIThreads, 0, s>>>(q, dO, dsp, idx, T, N, K, interm); break;
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
