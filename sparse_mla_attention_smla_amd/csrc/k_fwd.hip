// Sparse MLA forward with a sink-inclusive lse (produces the backward's O, lse).
//
// Page: aiter PR 4766 "Sparse MLA training backward", Contract section: same
// op as the forward's has_pe=False path; the forward folds the attention sink
// into its running max and running sum before taking lse = max + ln(sum), and
// the sink carries no value vector.
//
// Same work unit and kv tile ring as the dQ kernel: one token, NW*16 heads,
// compacted valid slots in 32-row tiles copied straight into LDS.  Online
// softmax in the log2 domain: per tile, the 8 logits a lane holds for its head
// are reduced with the three other lanes of that head (xor 16, xor 32) to a
// tile max; the running sum and the fp32 O^T accumulator of the lane (all its
// rows belong to one head) are rescaled by exp2(m_old - m_new).  The sink
// enters once at the end.
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

// PE adds the has_pe=True variant's positional part to the logits: q_pe
// [T,H,64] as the B operand of two more S^T steps over a 4 KiB ring of k_pe
// tiles (kv_tile.hpp); the values stay kv alone.
template <int NW, bool PE>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(1, 1)))
void smla_k7_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                 const int32_t* __restrict__ idx, const float* __restrict__ sink, int H,
                 int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse,
                 const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe) {
    constexpr int R = kBK / NW + (PE ? 4 / NW : 0);   // buffer->LDS copies per wave per tile
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[PE ? kNBuf * kPeTileBytes : 16];
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

    u32x4 qf[16], qpf[2];
#pragma unroll
    for (int ds = 0; ds < 16; ++ds)
        qf[ds] = *reinterpret_cast<const u32x4*>(q + qrow + 32 * ds + 8 * g);
    if constexpr (PE) {
        const size_t prow = ((size_t)t * H + h) * kDP;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) qpf[s2] = *reinterpret_cast<const u32x4*>(q_pe + prow + 32 * s2 + 8 * g);
    }
    const float c = scale * kLog2e;
    const i32x4 rsrc = make_rsrc(kv, (uint32_t)N * (kD * 2));
    const i32x4 rsrc_pe = make_rsrc(k_pe, PE ? (uint32_t)N * kPeRow : 0u);
    const uint32_t ring = lds_addr(tiles);
    const uint32_t pe_ring = lds_addr(pe_tiles);
    const int rb = rows_base(c16, g), cb = cols_base(c16, g);
    auto issue = [&](int ct) {
        issue_tile<NW>(rsrc, &L, ct, ring + (ct % kNBuf) * kTileBytes, w, lane);
        if constexpr (PE) issue_pe_tile<NW>(rsrc_pe, &L, ct, pe_ring + (ct % kNBuf) * kPeTileBytes, w, lane);
    };

    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of the head's logits (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum, scaled to m_run

    for (int k0 = 0; k0 < K; k0 += kChunk) {
        if (k0 > 0 && w == 0) compact_slots(idx_row, K, N, k0, &L, lane);
        __syncthreads();
        const int n = L.n;
        const int ntile = (n + kBK - 1) / kBK;
#pragma unroll
        for (int p = 0; p < kNBuf - 1; ++p) issue(p);
        for (int it = 0; it < ntile; ++it) {
            // copies issued after tile `it`: always the next two tiles (2R)
            wait_vmcnt<(2 * R < 63 ? 2 * R : 63)>();
            __syncthreads();
            issue(it + kNBuf - 1);
            const char* buf = tiles + (it % kNBuf) * kTileBytes;

            // four accumulation chains: both 16-slot halves, even and odd d-steps
            f32x4 sacc[2], sodd[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) sacc[st] = sodd[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ds = 0; ds < 16; ds += 2)
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    sacc[st] = mfma16(tile_rows_a(buf, rb, st, ds), qf[ds], sacc[st]);
                    sodd[st] = mfma16(tile_rows_a(buf, rb, st, ds + 1), qf[ds + 1], sodd[st]);
                }
            if constexpr (PE) {
                const char* pbuf = pe_tiles + (it % kNBuf) * kPeTileBytes;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    sacc[st] = mfma16(pe_rows_a(pbuf, c16, g, st, 0), qpf[0], sacc[st]);
                    sodd[st] = mfma16(pe_rows_a(pbuf, c16, g, st, 1), qpf[1], sodd[st]);
                }
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) sacc[st] += sodd[st];
            float x[2][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool v = it * kBK + 16 * st + 4 * g + j < n;
                    x[st][j] = v ? sacc[st][j] * c : -INFINITY;
                    tmax = fmaxf(tmax, x[st][j]);
                }
            tmax = max_over_rows(tmax);
            // every tile holds at least one valid slot, so m_new is finite
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] *= alpha;
            float p[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p[st][j] = __builtin_amdgcn_exp2f(x[st][j] - m_new);
                    l_run += p[st][j];
                }
            m_run = m_new;
            const u32x4 bf = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                              pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
#pragma unroll
            for (int dt = 0; dt < 32; ++dt) acc[dt] = mfma16(tile_cols_a(buf, cb, dt), bf, acc[dt]);
        }
        wait_vmcnt<0>();
        __syncthreads();
    }

    const float l_tot = sum_over_rows(l_run);
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

// Heads per workgroup of the one-wave-per-16-heads forward: 64, 32 or 16
// (whichever divides H first).
static int dq_waves(int H) {
    if (H % 64 == 0) return 4;
    if (H % 32 == 0) return 2;
    return 1;
}

hipError_t launch_fwd_pc(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
                         int T, int H, int N, int K, float scale, uint16_t* o, float* lse,
                         hipStream_t s);

hipError_t launch_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
                      int T, int H, int N, int K, float scale, uint16_t* o, float* lse,
                      hipStream_t s) {
    if (T == 0) return hipSuccess;
    // one index chunk per token: the persistent kernel (k_dq.hip) that shares
    // the dQ pass's tile stream and wave roles (64-head groups, the last one
    // padded when H is not a multiple of 64)
    if (K <= kChunk) return launch_fwd_pc(q, kv, idx, sink, T, H, N, K, scale, o, lse, s);
    const int nw = dq_waves(H);
    const unsigned blocks = (unsigned)T * (unsigned)(H / (nw * 16));
    switch (nw) {
        case 4: smla_k7_fwd<4, false><<<blocks, 256, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, nullptr, nullptr); break;
        case 2: smla_k7_fwd<2, false><<<blocks, 128, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, nullptr, nullptr); break;
        default: smla_k7_fwd<1, false><<<blocks, 64, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, nullptr, nullptr); break;
    }
    return hipGetLastError();
}

hipError_t launch_fwd_pc_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                            const int32_t* idx, const float* sink, int T, int H, int N, int K, float scale,
                            uint16_t* o, float* lse, hipStream_t s);

hipError_t launch_fwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                         const int32_t* idx, const float* sink, int T, int H, int N, int K, float scale,
                         uint16_t* o, float* lse, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (K <= kChunk) return launch_fwd_pc_pe(q, q_pe, kv, k_pe, idx, sink, T, H, N, K, scale, o, lse, s);
    const int nw = dq_waves(H);
    const unsigned blocks = (unsigned)T * (unsigned)(H / (nw * 16));
    switch (nw) {
        case 4: smla_k7_fwd<4, true><<<blocks, 256, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, q_pe, k_pe); break;
        case 2: smla_k7_fwd<2, true><<<blocks, 128, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, q_pe, k_pe); break;
        default: smla_k7_fwd<1, true><<<blocks, 64, 0, s>>>(q, kv, idx, sink, H, N, K, scale, o, lse, q_pe, k_pe); break;
    }
    return hipGetLastError();
}

}  // namespace smla
