// The has_pe=True variant's extra backward stage: the per-kv-row gather of
// the positional dKV intermediate into dk_pe.  (The intermediate itself is
// formed by the dKV intermediate kernel of k_interm.hip, from the same dS
// fragments as the main one.)
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
