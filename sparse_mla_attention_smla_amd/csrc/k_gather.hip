// dKV gather: dkv[j] = sum of interm rows of every slot that addresses kv row j.
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table, "dKV
// gather" row: atomic-free, each kv row gathers its own contributors through
// the inverted index.
//
// Rows are very uneven (a sliding-window row has <= 128 contributors, a popular
// pool row thousands), so every row is cut into segments of at most
// kGatherSeg contributors:
//   plan    -- one block: per-row segment counts, their exclusive scan (seg_ptr)
//              and the owning row of every segment (seg_row);
//   segment -- one block per segment sums its contributors in fp32 (each wave a
//              fixed residue class of contributors, waves combined in order);
//   combine -- one wave per kv row adds its segment partials in order and
//              rounds to bf16 once.  Rows without contributors get zeros; a
//              row with a single segment is rounded and written by the segment
//              kernel itself (same arithmetic, no partial round trip).
// Every index read from row_ptr / slots is range-checked, so an inconsistent
// inverted index can give wrong sums but never an out-of-bounds access.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {
constexpr int kSegWaves = 16;
static_assert(kGatherSeg % kSegWaves == 0 && kGatherSeg / kSegWaves <= 64,
              "a wave's contributor slots fit one per lane");

__device__ int block_exclusive_scan_1024_g(int v, int* lds, int* total) {
    const int tid = threadIdx.x;
    lds[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = tid >= off ? lds[tid - off] : 0;
        __syncthreads();
        lds[tid] += add;
        __syncthreads();
    }
    const int incl = lds[tid];
    *total = lds[1023];
    __syncthreads();
    return incl - v;
}
}  // namespace

// segments of row j; 0 when the row's pointers are not an increasing pair in [0, M]
__device__ __forceinline__ int row_segments(const int32_t* row_ptr, int j, int64_t M) {
    const int a = row_ptr[j], b = row_ptr[j + 1];
    if (a < 0 || b < a || (int64_t)b > M) return 0;
    return (b - a + kGatherSeg - 1) / kGatherSeg;
}

__global__ __launch_bounds__(1024) void smla_k5_gather_plan(const int32_t* __restrict__ row_ptr,
                                                            int N, int64_t M, int max_segs,
                                                            int32_t* __restrict__ seg_ptr,
                                                            int32_t* __restrict__ seg_row) {
    __shared__ int lds[1024];
    const int tid = threadIdx.x;
    const int ipt = (N + 1023) / 1024;
    const int j0 = min(N, tid * ipt), j1 = min(N, j0 + ipt);
    int local = 0;
    for (int j = j0; j < j1; ++j) local += row_segments(row_ptr, j, M);
    int all;
    int run = block_exclusive_scan_1024_g(local, lds, &all);
    for (int j = j0; j < j1; ++j) {
        seg_ptr[j] = min(run, max_segs);
        const int n = row_segments(row_ptr, j, M);
        for (int i = 0; i < n; ++i)
            if (run + i < max_segs) seg_row[run + i] = j;
        run += n;
    }
    if (tid == 0) seg_ptr[N] = min(all, max_segs);
}

__global__ __launch_bounds__(kSegWaves * 64) void smla_k5_gather_segment(
    const uint16_t* __restrict__ interm, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ seg_ptr,
    const int32_t* __restrict__ seg_row, int N, int64_t M, float* __restrict__ partial,
    uint16_t* __restrict__ dkv_single) {
    __shared__ float red[kSegWaves][kD];
    // segments from last to first: the pool rows (up to kGatherSeg contributors
    // per segment, at the end of the row order) go out first and the short
    // sliding-window segments fill the tail
    const int s = gridDim.x - 1 - blockIdx.x;
    if (s >= seg_ptr[N]) return;  // grid is an upper bound on the segment count
    const int j = seg_row[s];
    const int beg = row_ptr[j] + (s - seg_ptr[j]) * kGatherSeg;  // plan checked the row's pointers
    const int end = min(beg + kGatherSeg, row_ptr[j + 1]);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // wave w owns contributors beg + w + kSegWaves*m, m < kGatherSeg/kSegWaves (<= 64)
    const int mine = beg + w + kSegWaves * lane;
    const int my_slot = (lane < kGatherSeg / kSegWaves && mine < end) ? slots[mine] : 0;
    const int n = (end - beg - w + kSegWaves - 1) / kSegWaves;  // contributors of this wave
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    constexpr int U = 2;   // rows in flight per wave (2, 4 and 8 measured within 1%; 2 best)
    for (int m0 = 0; m0 < n; m0 += U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int m = m0 + u;
            const int sl = __builtin_amdgcn_readlane(my_slot, m < n ? m : 0);
            // each intermediate row is read once, whole (1 KiB per wave): streaming
            // (non-temporal) loads, measured 8% faster than cached ones here
            v[u] = (m < n && (uint32_t)sl < (uint64_t)M)
                       ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4*>(interm + (size_t)sl * kD + lane * 8))
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[2 * c] += bf16lo(v[u][c]);
                acc[2 * c + 1] += bf16hi(v[u][c]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = acc[e];
    __syncthreads();
    if (dkv_single != nullptr && seg_ptr[j + 1] - seg_ptr[j] == 1) {
        // the row's only segment: round to bf16 here, exactly as the combine
        // would (it starts from +0, which also turns a -0 sum into +0)
        for (int c2 = threadIdx.x; c2 < kD / 2; c2 += kSegWaves * 64) {
            float a = red[0][2 * c2], b = red[0][2 * c2 + 1];
#pragma unroll
            for (int i = 1; i < kSegWaves; ++i) {
                a += red[i][2 * c2];
                b += red[i][2 * c2 + 1];
            }
            reinterpret_cast<uint32_t*>(dkv_single + (size_t)j * kD)[c2] = pack_bf16(0.f + a, 0.f + b);
        }
        return;
    }
    for (int col = threadIdx.x; col < kD; col += kSegWaves * 64) {
        float sum = red[0][col];
#pragma unroll
        for (int i = 1; i < kSegWaves; ++i) sum += red[i][col];
        partial[(size_t)s * kD + col] = sum;
    }
}

// Rows with exactly one segment were written by the segment kernel.
__global__ __launch_bounds__(256) void smla_k5_gather_combine(const float* __restrict__ partial,
                                                              const int32_t* __restrict__ seg_ptr,
                                                              int N, uint16_t* __restrict__ dkv) {
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= N) return;
    const int s0 = seg_ptr[j], s1 = seg_ptr[j + 1];   // plan clamps both to the segment count
    if (s1 - s0 == 1) return;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s = s0; s < s1; ++s) {
        const f32x4* p = reinterpret_cast<const f32x4*>(partial + (size_t)s * kD + lane * 8);
        const f32x4 a = p[0], b = p[1];
        acc[0] += a[0]; acc[1] += a[1]; acc[2] += a[2]; acc[3] += a[3];
        acc[4] += b[0]; acc[5] += b[1]; acc[6] += b[2]; acc[7] += b[3];
    }
    u32x4 out = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                 pack_bf16(acc[6], acc[7])};
    *reinterpret_cast<u32x4*>(dkv + (size_t)j * kD + lane * 8) = out;
}

// Token-phased variant of the combine: the row's segment partials of this
// phase are added, in order, to its fp32 running sum (started at zero in the
// first phase); the last phase rounds the sum to bf16 once.  With a single
// phase this is the plain combine, operation for operation.
__global__ __launch_bounds__(256) void smla_k5_gather_combine_acc(const float* __restrict__ partial,
                                                                  const int32_t* __restrict__ seg_ptr,
                                                                  int N, int first,
                                                                  float* __restrict__ run,
                                                                  uint16_t* __restrict__ dkv) {
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (j >= N) return;
    const int s0 = seg_ptr[j], s1 = seg_ptr[j + 1];
    f32x4* r = reinterpret_cast<f32x4*>(run + (size_t)j * kD + lane * 8);
    float acc[8];
    if (first) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    } else {
        const f32x4 a = r[0], b = r[1];
        acc[0] = a[0]; acc[1] = a[1]; acc[2] = a[2]; acc[3] = a[3];
        acc[4] = b[0]; acc[5] = b[1]; acc[6] = b[2]; acc[7] = b[3];
    }
    for (int s = s0; s < s1; ++s) {
        const f32x4* p = reinterpret_cast<const f32x4*>(partial + (size_t)s * kD + lane * 8);
        const f32x4 a = p[0], b = p[1];
        acc[0] += a[0]; acc[1] += a[1]; acc[2] += a[2]; acc[3] += a[3];
        acc[4] += b[0]; acc[5] += b[1]; acc[6] += b[2]; acc[7] += b[3];
    }
    if (dkv != nullptr) {
        u32x4 out = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                     pack_bf16(acc[6], acc[7])};
        *reinterpret_cast<u32x4*>(dkv + (size_t)j * kD + lane * 8) = out;
    } else {
        r[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
        r[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

size_t gather_scratch_bytes(int64_t M, int N) {
    const int64_t ms = gather_max_segments(M, N);
    return align_up((size_t)(N + 1) * 4, 256) + align_up((size_t)ms * 4, 256) +
           align_up((size_t)ms * kD * 4, 256);
}

GatherScratch gather_carve(void* base, int64_t M, int N) {
    const int64_t ms = gather_max_segments(M, N);
    char* p = static_cast<char*>(base);
    GatherScratch w;
    w.seg_ptr = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)(N + 1) * 4, 256);
    w.seg_row = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)ms * 4, 256);
    w.partial = reinterpret_cast<float*>(p);
    return w;
}

hipError_t launch_gather_plan(const int32_t* row_ptr, int64_t M, int N, const GatherScratch& ws,
                              hipStream_t s) {
    const int64_t ms = gather_max_segments(M, N);
    smla_k5_gather_plan<<<1, 1024, 0, s>>>(row_ptr, N, M, (int)ms, ws.seg_ptr, ws.seg_row);
    return hipGetLastError();
}

hipError_t launch_gather_sum(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots,
                             int64_t M, int N, const GatherScratch& ws, uint16_t* dkv, hipStream_t s) {
    const int64_t ms = gather_max_segments(M, N);
    smla_k5_gather_segment<<<(unsigned)ms, kSegWaves * 64, 0, s>>>(interm, row_ptr, slots,
                                                                   ws.seg_ptr, ws.seg_row, N, M,
                                                                   ws.partial, dkv);
    smla_k5_gather_combine<<<(N + 3) / 4, 256, 0, s>>>(ws.partial, ws.seg_ptr, N, dkv);
    return hipGetLastError();
}

hipError_t launch_gather_sum_phase(const uint16_t* interm, const int32_t* row_ptr,
                                   const int32_t* slots, int64_t M, int N, const GatherScratch& ws,
                                   bool first, float* run, uint16_t* dkv_last, hipStream_t s) {
    const int64_t ms = gather_max_segments(M, N);
    smla_k5_gather_segment<<<(unsigned)ms, kSegWaves * 64, 0, s>>>(interm, row_ptr, slots,
                                                                   ws.seg_ptr, ws.seg_row, N, M,
                                                                   ws.partial, nullptr);
    smla_k5_gather_combine_acc<<<(N + 3) / 4, 256, 0, s>>>(ws.partial, ws.seg_ptr, N, first ? 1 : 0,
                                                           run, dkv_last);
    return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots,
                         int64_t M, int N, const GatherScratch& ws, uint16_t* dkv, hipStream_t s) {
    const hipError_t e = launch_gather_plan(row_ptr, M, N, ws, s);
    if (e != hipSuccess) return e;
    return launch_gather_sum(interm, row_ptr, slots, M, N, ws, dkv, s);
}

}  // namespace smla
