// Streaming kernels of the backward: delta = rowsum(O * dO) and the sink
// gradient.  Both are HBM-bound reads with fp32 accumulation in a fixed order.
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table
// ("delta = rowsum(O*dO)" streams bf16 and accumulates fp32; "d_sink").
//
// An upstream gradient of lse enters every later phase only through delta:
// d lse / d S_k = P_k and d lse / d sink = P_sink, so dS = P (dP - delta + dlse)
// and d_sink = -sum_t P_sink (delta - dlse).  The delta kernel therefore
// stores delta - dlse when dlse is given, and nothing downstream changes.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

// One (t,h) row of O/dO is 1 KiB of bf16.  A wave covers 4 rows per step:
// 16 lanes per row, each lane loading 4 x 16 B at a 256-B stride so that every
// load instruction reads 4 contiguous 256-B runs.  The 16 partial sums of a row
// are combined by a fixed xor-butterfly.
__global__ __launch_bounds__(256) void smla_k1_delta(const uint16_t* __restrict__ O,
                                                     const uint16_t* __restrict__ dO,
                                                     const float* __restrict__ dlse,
                                                     float* __restrict__ delta, int64_t rows) {
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 4;
    const int l16 = lane & 15;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t r0 = wave * 4; r0 < rows; r0 += nwaves * 4) {
        const int64_t r = r0 + sub;
        float acc = 0.f;
        if (r < rows) {
            const u32x4* po = reinterpret_cast<const u32x4*>(O + r * kD) + l16;
            const u32x4* pd = reinterpret_cast<const u32x4*>(dO + r * kD) + l16;
            u32x4 a[4], b[4];
            // both streams are read once here (streaming loads; measured faster)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = __builtin_nontemporal_load(po + 16 * i);
                b[i] = __builtin_nontemporal_load(pd + 16 * i);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc = fmaf(bf16lo(a[i][c]), bf16lo(b[i][c]), acc);
                    acc = fmaf(bf16hi(a[i][c]), bf16hi(b[i][c]), acc);
                }
            }
        }
        acc += wave_xor(acc, 8);
        acc += wave_xor(acc, 4);
        acc += wave_xor(acc, 2);
        acc += wave_xor(acc, 1);
        if (l16 == 0 && r < rows) delta[r] = dlse != nullptr ? acc - dlse[r] : acc;
    }
}

hipError_t launch_delta(const uint16_t* o, const uint16_t* dO, const float* dlse, int64_t rows,
                        float* delta, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    int64_t want = (rows + 15) / 16;              // 16 rows per 256-thread block step
    int blocks = (int)(want < 256 * 16 ? want : 256 * 16);
    smla_k1_delta<<<blocks, 256, 0, s>>>(o, dO, dlse, delta, rows);
    return hipGetLastError();
}

// d_sink[h] = -sum_t exp(sink[h] - lse[t,h]) * delta[t,h].
// Stage 1: block b sums a fixed run of tokens per head (thread = head, reads of
// one token's [H] row are contiguous).  Stage 2: one block adds the per-run
// partials in run order.  No atomics; the order is fixed.
__global__ __launch_bounds__(128) void smla_k6_dsink_partial(const float* __restrict__ lse,
                                                             const float* __restrict__ delta,
                                                             const float* __restrict__ sink,
                                                             int T, int H,
                                                             float* __restrict__ partial) {
    const int h = threadIdx.x;
    if (h >= H) return;
    const int t0 = blockIdx.x * kDsinkTokensPerBlock;
    const int t1 = min(T, t0 + kDsinkTokensPerBlock);
    const float sk = sink[h];
    float acc = 0.f;
    for (int t = t0; t < t1; ++t) {
        const float l = lse[(int64_t)t * H + h];
        const float p = (l == -INFINITY) ? 0.f : expf(sk - l);
        acc = fmaf(p, delta[(int64_t)t * H + h], acc);
    }
    partial[(int64_t)blockIdx.x * H + h] = acc;
}

// One wave per head: lane l sums partials l, l + 64, ... in order, then a
// butterfly in a fixed pattern combines the lanes (same result every run).
__global__ __launch_bounds__(256) void smla_k6_dsink_final(const float* __restrict__ partial,
                                                           int nblocks, int H,
                                                           float* __restrict__ d_sink) {
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= H) return;  // whole wave: H is a multiple of 16, the grid covers ceil(H / 4)
    float acc = 0.f;
    for (int b = lane; b < nblocks; b += 64) acc += partial[(int64_t)b * H + h];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += wave_xor(acc, m);
    if (lane == 0) d_sink[h] = 0.f - acc;
}

hipError_t launch_dsink(const float* lse, const float* delta, const float* sink, int T, int H,
                        float* partial, float* d_sink, hipStream_t s) {
    const int nb = dsink_blocks(T);
    if (nb > 0) smla_k6_dsink_partial<<<nb, 128, 0, s>>>(lse, delta, sink, T, H, partial);
    smla_k6_dsink_final<<<(H + 3) / 4, 256, 0, s>>>(partial, nb, H, d_sink);
    return hipGetLastError();
}

}  // namespace smla
