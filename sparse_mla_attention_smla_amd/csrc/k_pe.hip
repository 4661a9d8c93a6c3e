// The has_pe=True variant's extra backward stages: the positional dKV
// intermediate and its per-kv-row gather into dk_pe.  (For H a multiple of 32
// the intermediate kernel of k_interm.hip forms the positional intermediate
// itself; the kernel here serves the other head counts.)
//
// Page: aiter PR 4766 "Sparse MLA training backward", Contract section (the
// op is the forward's has_pe=False path; has_pe=True is the forward's other
// path, whose positional part -- a q_pe on the queries and a head-shared k_pe
// on the keys, logits scale*(<q,kv> + <q_pe,k_pe>), values kv alone -- adds
// the gradient dk_pe) and Structure table ("dKV-interm" contracts over all
// heads per slot; "dKV gather" is atomic-free through the inverted index).
//
//   interm_pe[t*topk + k] = sum_h scale*dS[t,h,k] * q_pe[t,h]      (64 values)
//   dk_pe[j] = sum over the slots of kv row j of interm_pe[slot]   (CSR order)
//
// scale*dS comes from the dS/P blocks the dQ kernel wrote (rows 0..H-1 of
// each block: the first H*64 bytes, in the piece layout of include/smla.h).
#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {
constexpr int kPWaves = 4;
constexpr int kXPitch = kPeRow + 32;   // 160 B: a q_pe row plus pad (odd multiple of 32)
constexpr int kYPitch = 96;            // a dS row of one block: 32 slots (64 B) plus pad
}  // namespace

// One token per workgroup of four waves.  X = q_pe_t [H x 64] is staged in LDS
// once and its transposed MFMA fragments (one positional column x 8 heads)
// stay in registers; the token's compacted tiles are dealt to the waves in
// turn (wave w takes tiles w, w+4, ...), each wave bringing the dS rows of its
// tile's block into its own LDS area and computing
//   interm_pe^T [64 x 32 slots] = X^T . (scale*dS)      (reduction over heads)
// NKP = ceil(H/32) reduction steps; rows H..32*NKP-1 of X and of the dS area
// are zero.
template <int NKP>
__global__ __launch_bounds__(kPWaves * 64) void smla_k3_interm_pe(const uint16_t* __restrict__ q_pe,
                                                                  const uint16_t* __restrict__ dsp,
                                                                  const int32_t* __restrict__ idx, int H,
                                                                  int N, int K,
                                                                  uint16_t* __restrict__ interm_pe) {
    constexpr int kRows = 32 * NKP;
    __shared__ __attribute__((aligned(16))) char xs[kRows * kXPitch];
    __shared__ __attribute__((aligned(16))) char ys[kPWaves][kRows * kYPitch];
    __shared__ SlotList L;

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
    const int32_t* idx_row = idx + (size_t)t * K;

    // X rows (16-byte chunks), zero past H
    for (int i = tid; i < kRows * 8; i += kPWaves * 64) {
        const int r = i >> 3, ch = i & 7;
        const u32x4 v = r < H ? *reinterpret_cast<const u32x4*>(q_pe + ((size_t)t * H + r) * kDP + ch * 8)
                              : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(xs + r * kXPitch + ch * 16) = v;
    }
    // dS rows past H of every wave's area are never loaded: zero them once
    for (int i = tid; i < kPWaves * (kRows - H) * 4; i += kPWaves * 64) {
        const int ww = i / ((kRows - H) * 4), rem = i - ww * (kRows - H) * 4;
        *reinterpret_cast<u32x4*>(ys[ww] + (H + (rem >> 2)) * kYPitch + (rem & 3) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    if (w == 0) compact_slots(idx_row, K, N, 0, &L, lane);
    __syncthreads();

    // xf[dt][ks]: positional column 16dt + c16 of X rows 32ks + 4g .. +3, then
    // 32ks + 16 + 4g .. +3 (lane L of group g names row 4g + L/4, columns
    // 16dt + 4(L%4) of a transposed read)
    u32x4 xf[4][NKP];
    const int xb = (4 * g + (c16 >> 2)) * kXPitch + (c16 & 3) * 8;
#pragma unroll
    for (int ks = 0; ks < NKP; ++ks)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const char* ptr = xs + xb + 32 * ks * kXPitch + dt * 32;
            const u32x2 lo = ds_read_tr16(ptr);
            const u32x2 hi = ds_read_tr16(ptr + 16 * kXPitch);
            xf[dt][ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }

    const int ntk = (K + kBK - 1) / kBK;
    const uint16_t* ytok = dsp + (size_t)t * ntk * (2 * H) * kBK;
    char* yw = ys[w];
    const int yb = (4 * g + (c16 >> 2)) * kYPitch + (c16 & 3) * 8;
    int ctg = 0;
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        if (k0 > 0) {
            __syncthreads();   // every wave is done with the previous chunk's slot list
            if (w == 0) compact_slots(idx_row, K, N, k0, &L, lane);
            __syncthreads();
        }
        const int n = L.n;
        const int ntile = (n + kBK - 1) / kBK;
        for (int c = w; c < ntile; c += kPWaves) {
            // the block's dS rows: H*64 bytes = 4H pieces of 16 bytes; piece id goes
            // to row 16*(id/64) + id%16, byte column 16*((id/16)%4) (piece layout)
            const uint16_t* src = ytok + (size_t)(ctg + c) * (2 * H) * kBK;
            for (int id = lane; id < 4 * H; id += 64) {
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + id * 8));
                *reinterpret_cast<u32x4*>(yw + ((id >> 6) * 16 + (id & 15)) * kYPitch + ((id >> 4) & 3) * 16) = v;
            }
            // a wave's LDS operations complete in order: the reads below see the writes
#pragma unroll
            for (int sst = 0; sst < 2; ++sst) {
                f32x4 cacc[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) cacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKP; ++ks) {
                    const char* p = yw + yb + ks * 32 * kYPitch + sst * 32;
                    const u32x2 lo = ds_read_tr16(p);
                    const u32x2 hi = ds_read_tr16(p + 16 * kYPitch);
                    const u32x4 bfrag = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) cacc[dt] = mfma16(xf[dt][ks], bfrag, cacc[dt]);
                }
                // lane c16 + 16g: block position 16sst + c16, positional columns
                // 16dt + 4g .. +3; position p holds tile slot 4(p/8) + p%4 (+16 when
                // p%8 >= 4)
                const int pb = 16 * sst + c16;
                const int pos = c * kBK + 4 * (pb >> 3) + (pb & 3) + ((pb & 4) << 2);
                if (pos < n) {
                    uint16_t* dst = interm_pe + ((size_t)t * K + L.slot[pos]) * kDP + 4 * g;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
                        *reinterpret_cast<u32x2*>(dst + 16 * dt) =
                            u32x2{pack_bf16(cacc[dt][0], cacc[dt][1]), pack_bf16(cacc[dt][2], cacc[dt][3])};
                }
            }
        }
        ctg += ntile;
    }
}

hipError_t launch_interm_pe(const uint16_t* q_pe, const uint16_t* dsp, const int32_t* idx, int T, int H,
                            int N, int K, uint16_t* interm_pe, hipStream_t s) {
    if (T == 0) return hipSuccess;
    switch ((H + 31) / 32) {
        case 1: smla_k3_interm_pe<1><<<T, kPWaves * 64, 0, s>>>(q_pe, dsp, idx, H, N, K, interm_pe); break;
        case 2: smla_k3_interm_pe<2><<<T, kPWaves * 64, 0, s>>>(q_pe, dsp, idx, H, N, K, interm_pe); break;
        case 3: smla_k3_interm_pe<3><<<T, kPWaves * 64, 0, s>>>(q_pe, dsp, idx, H, N, K, interm_pe); break;
        case 4: smla_k3_interm_pe<4><<<T, kPWaves * 64, 0, s>>>(q_pe, dsp, idx, H, N, K, interm_pe); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- gather of the 64-wide positional rows ----------------------------------
// The segments of the main gather's plan (rows cut into runs of at most
// kGatherSeg contributors).  One block of 256 threads per segment: 32 groups
// of 8 lanes, group m taking contributors m, m + 32, ... of the segment and
// lane i of a group the 16-byte chunk i of each 128-byte row; the 32 group
// sums are then added in group order.  A row with one segment is rounded and
// written here; partial sums of longer rows go to `partial` for the combine.
__global__ __launch_bounds__(256) void smla_k5_gather_pe_segment(
    const uint16_t* __restrict__ interm_pe, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ seg_ptr,
    const int32_t* __restrict__ seg_row, int N, int64_t M, float* __restrict__ partial,
    uint16_t* __restrict__ dk_pe) {
    __shared__ float red[32][kDP + 4];
    const int s = gridDim.x - 1 - blockIdx.x;   // longest (pool-row) segments first, as the main gather
    if (s >= seg_ptr[N]) return;   // grid is an upper bound on the segment count
    const int j = seg_row[s];
    const int beg = row_ptr[j] + (s - seg_ptr[j]) * kGatherSeg;   // the plan checked the row's pointers
    const int end = min(beg + kGatherSeg, row_ptr[j + 1]);
    const int grp = threadIdx.x >> 3, ch = threadIdx.x & 7;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int m = beg + grp; m < end; m += 32) {
        const int sl = slots[m];
        if ((uint32_t)sl < (uint64_t)M) {
            const u32x4 v = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(interm_pe + (size_t)sl * kDP + ch * 8));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[2 * c] += bf16lo(v[c]);
                acc[2 * c + 1] += bf16hi(v[c]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp][ch * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x >= kDP) return;
    const int col = threadIdx.x;
    float sum = red[0][col];
#pragma unroll
    for (int i = 1; i < 32; ++i) sum += red[i][col];
    if (seg_ptr[j + 1] - seg_ptr[j] == 1) {
        // the row's only segment: round here, exactly as the combine would (it
        // starts from +0, which also turns a -0 sum into +0)
        dk_pe[(size_t)j * kDP + col] = to_bf16(0.f + sum);
    } else {
        partial[(size_t)s * kDP + col] = sum;
    }
}

// One wave per kv row: adds the row's segment partials in order (rows without
// contributors get zeros; single-segment rows were written by the segment kernel).
__global__ __launch_bounds__(256) void smla_k5_gather_pe_combine(const float* __restrict__ partial,
                                                                 const int32_t* __restrict__ seg_ptr, int N,
                                                                 uint16_t* __restrict__ dk_pe) {
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int col = threadIdx.x & 63;
    if (j >= N) return;
    const int s0 = seg_ptr[j], s1 = seg_ptr[j + 1];
    if (s1 - s0 == 1) return;
    float acc = 0.f;
    for (int s = s0; s < s1; ++s) acc += partial[(size_t)s * kDP + col];
    dk_pe[(size_t)j * kDP + col] = to_bf16(acc);
}

size_t gather_pe_scratch_bytes(int64_t M, int N) {
    return align_up((size_t)gather_max_segments(M, N) * kDP * 4, 256);
}

hipError_t launch_gather_pe(const uint16_t* interm_pe, const int32_t* row_ptr, const int32_t* slots,
                            int64_t M, int N, const GatherScratch& plan, float* partial, uint16_t* dk_pe,
                            hipStream_t s) {
    const int64_t ms = gather_max_segments(M, N);
    smla_k5_gather_pe_segment<<<(unsigned)ms, 256, 0, s>>>(interm_pe, row_ptr, slots, plan.seg_ptr,
                                                           plan.seg_row, N, M, partial, dk_pe);
    smla_k5_gather_pe_combine<<<(N + 3) / 4, 256, 0, s>>>(partial, plan.seg_ptr, N, dk_pe);
    return hipGetLastError();
}

}  // namespace smla
