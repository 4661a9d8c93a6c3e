// Sparse MLA forward with a sink-inclusive lse (produces the backward's O, lse).
//
// Page: aiter PR 4766 "Sparse MLA training backward", Contract section: same
// op as the forward's has_pe=False path; the forward folds the attention sink
// into its running max and running sum before taking lse = max + ln(sum), and
// the sink carries no value vector.
//
// Same work unit and kv tiles as the dQ kernel: one token, NW*16 heads, 32-slot
// tiles gathered into LDS once per tile.  Online softmax in the log2 domain:
// per tile, the 8 logits a lane holds for its head are reduced with the three
// other lanes of that head (xor 16, xor 32) to a tile max; the running sum and
// the fp32 O^T accumulator of the lane (all rows belong to one head) are
// rescaled by exp2(m_old - m_new).  The sink enters once at the end.
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void smla_k7_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                 const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                 int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
    const int nhg = H / (NW * 16);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int t = logical / nhg;
    const int hg = logical - t * nhg;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
    const int h = hg * NW * 16 + w * 16 + c16;
    const size_t qrow = ((size_t)t * H + h) * kD;

    u32x4 qf[16];
#pragma unroll
    for (int ds = 0; ds < 16; ++ds)
        qf[ds] = *reinterpret_cast<const u32x4*>(q + qrow + 32 * ds + 8 * g);
    const float c = scale * kLog2e;
    const int32_t* idx_row = idx + (size_t)t * K;

    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of the head's logits (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum, scaled to m_run

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
            f32x4 sacc[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < 16; ++ds)
                    sacc[st] = mfma16(tile_rows_a(buf, st, ds, c16, g), qf[ds], sacc[st]);
            }
            float x[2][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool v = (mask >> (16 * st + 4 * g + j)) & 1u;
                    x[st][j] = v ? sacc[st][j] * c : -INFINITY;
                    tmax = fmaxf(tmax, x[st][j]);
                }
            tmax = fmaxf(tmax, wave_xor(tmax, 16));
            tmax = fmaxf(tmax, wave_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            float p[2][4];
            if (m_new == -INFINITY) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) p[st][j] = 0.f;
            } else {
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        p[st][j] = __builtin_amdgcn_exp2f(x[st][j] - m_new);
                        l_run += p[st][j];
                    }
                m_run = m_new;
            }
            const u32x4 bf = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                              pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt] = mfma16(tile_cols_a(buf, dt, c16, g), bf, acc[dt]);
        }
        if (more) {
            tile.store(smem + ((it + 1) & 1) * kTileBytes, w, lane);
            mask = tile.mask;
        }
        __syncthreads();
    }

    float l_tot = l_run;
    l_tot += wave_xor(l_tot, 16);
    l_tot += wave_xor(l_tot, 32);
    // fold in the sink: a raw logit (not scaled) with a zero value vector
    const float xs = (sink != nullptr) ? sink[h] * kLog2e : -INFINITY;
    const float m_fin = fmaxf(m_run, xs);
    float out_scale = 0.f, lse_v = -INFINITY;
    if (m_fin != -INFINITY) {
        const float a = __builtin_amdgcn_exp2f(m_run - m_fin);
        const float z = l_tot * a + __builtin_amdgcn_exp2f(xs - m_fin);
        out_scale = a / z;
        lse_v = (m_fin + log2f(z)) * kLn2;
    }
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
        const u32x2 v = {pack_bf16(acc[dt][0] * out_scale, acc[dt][1] * out_scale),
                         pack_bf16(acc[dt][2] * out_scale, acc[dt][3] * out_scale)};
        *reinterpret_cast<u32x2*>(o + qrow + 16 * dt + 4 * g) = v;
    }
    if (g == 0) lse[(size_t)t * H + h] = lse_v;
}

static int pick_waves_fwd(int H) {
    for (int nw = 4; nw >= 1; --nw)
        if (H % (nw * 16) == 0) return nw;
    return 1;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
                      int T, int H, int N, int K, float scale, uint16_t* o, float* lse,
                      hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int nw = pick_waves_fwd(H);
    const unsigned blocks = (unsigned)T * (unsigned)(H / (nw * 16));
    switch (nw) {
        case 4: smla_k7_fwd<4><<<blocks, 256, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse); break;
        case 3: smla_k7_fwd<3><<<blocks, 192, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse); break;
        case 2: smla_k7_fwd<2><<<blocks, 128, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse); break;
        default: smla_k7_fwd<1><<<blocks, 64, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse); break;
    }
    return hipGetLastError();
}

}  // namespace smla
