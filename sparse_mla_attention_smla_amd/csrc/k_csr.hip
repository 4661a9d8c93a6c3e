// Inverted top-k index (CSR) built on the device, deterministic and atomic-free.
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table, "CSR
// build" row: the top-k scatter is inverted so every kv row can gather its own
// contributors.  The page builds it with a library sort; here it is a counting
// sort in four passes:
//   1. sort   -- each block of 4096 slots sorts packed (row << 12 | position)
//                keys in LDS (bitonic network) and writes its per-row counts;
//   2. colscan-- per kv row, exclusive running total of the counts over blocks;
//   3. rowscan-- exclusive scan of the per-row totals -> row_ptr;
//   4. scatter-- each slot lands at row_ptr[row] + block offset + rank within
//                its block's run of equal rows.  Runs are sorted by position,
//                so every row lists its slots in increasing order.
#include "smla_device.hpp"
#include "smla_launch.hpp"

namespace smla {

namespace {
constexpr int kSortThreads = 512;
constexpr uint32_t kSentinel = 0xFFFFFFFFu;

// first position p in keys[0..n) with (keys[p] >> 12) >= row
__device__ __forceinline__ int lower_bound_row(const uint32_t* keys, int n, uint32_t row) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((keys[mid] >> 12) < row) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Exclusive scan of one int per thread across a 1024-thread block (fixed order).
__device__ int block_exclusive_scan_1024(int v, int* lds /*[1024]*/, int* total) {
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

__global__ __launch_bounds__(kSortThreads) void smla_k4_csr_sort(const int32_t* __restrict__ idx,
                                                                 int64_t M, int N,
                                                                 uint32_t* __restrict__ sorted,
                                                                 int32_t* __restrict__ cnt,
                                                                 int32_t* __restrict__ inv) {
    __shared__ uint32_t keys[kCsrBlock];
    __shared__ int wsum[kSortThreads / 64];
    const int b = blockIdx.x;
    const int64_t base = (int64_t)b * kCsrBlock;
    const int tid = threadIdx.x;
    int ninv = 0;
    for (int p = tid; p < kCsrBlock; p += kSortThreads) {
        uint32_t key = kSentinel;
        if (base + p < M) {
            const int v = idx[base + p];
            const bool ok = valid_row(v, N);
            ninv += (!ok && v != -1) ? 1 : 0;
            key = ((ok ? (uint32_t)v : (uint32_t)N) << 12) | (uint32_t)p;
        }
        keys[p] = key;
    }
    for (int m = 32; m > 0; m >>= 1) ninv += wave_xor(ninv, m);
    if ((tid & 63) == 0) wsum[tid >> 6] = ninv;
    __syncthreads();
    if (tid == 0) {
        int s = 0;
        for (int i = 0; i < kSortThreads / 64; ++i) s += wsum[i];
        inv[b] = s;
    }
    // Bitonic sorting network, ascending.  Thread T holds keys 8T .. 8T+7 in
    // registers; for partner distance j < 8 the exchange is inside the thread,
    // for 8 <= j < 512 it is with lane T ^ (j/8) of the same wave (a shuffle),
    // and only the six stages with j >= 512 go through LDS.
    static_assert(kCsrBlock == 8 * kSortThreads, "eight keys per thread");
    __syncthreads();
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = keys[8 * tid + e];
    __syncthreads();
    for (int k = 2; k <= kCsrBlock; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 512) {
#pragma unroll
                for (int e = 0; e < 8; ++e) keys[8 * tid + e] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 8 * tid + e;
                    const uint32_t o = keys[i ^ j];
                    const bool up = (i & k) == 0;
                    const bool lower = (i & j) == 0;   // i < i ^ j
                    v[e] = (lower == up) ? min(v[e], o) : max(v[e], o);
                }
                __syncthreads();
            } else if (j >= 8) {
                const int lm = j >> 3;                  // partner lane distance
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int i = 8 * tid + e;
                    const uint32_t o = (uint32_t)__shfl_xor((int)v[e], lm, 64);
                    const bool up = (i & k) == 0;
                    const bool lower = (i & j) == 0;
                    v[e] = (lower == up) ? min(v[e], o) : max(v[e], o);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int pe = e ^ j;
                    if (pe > e) {
                        const int i = 8 * tid + e;
                        const bool up = (i & k) == 0;
                        const uint32_t a = v[e], c = v[pe];
                        v[e] = up ? min(a, c) : max(a, c);
                        v[pe] = up ? max(a, c) : min(a, c);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) keys[8 * tid + e] = v[e];
    __syncthreads();
    const int nloc = (int)min((int64_t)kCsrBlock, M - base);
    for (int p = tid; p < nloc; p += kSortThreads) sorted[base + p] = keys[p];
    // Per-row counts: thread T takes rows [j0, j1), finds the first key of row
    // j0 by binary search and walks the sorted keys from there (invalid slots
    // and the sentinel sort after every valid row).
    int32_t* crow = cnt + (int64_t)b * N;
    const int rpt = (N + kSortThreads - 1) / kSortThreads;
    const int j0 = min(N, tid * rpt), j1 = min(N, j0 + rpt);
    int p = lower_bound_row(keys, kCsrBlock, (uint32_t)j0);
    for (int j = j0; j < j1; ++j) {
        int c = 0;
        while (p < kCsrBlock && (keys[p] >> 12) == (uint32_t)j) { ++p; ++c; }
        crow[j] = c;
    }
}

// Lane = kv row (64 rows per block), wave = a contiguous run of sort blocks.
__global__ __launch_bounds__(1024) void smla_k4_csr_colscan(int32_t* __restrict__ cnt, int nblk,
                                                            int N, int32_t* __restrict__ total) {
    __shared__ int part[16][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + lane;
    const int per = (nblk + 15) / 16;
    const int b0 = min(nblk, w * per), b1 = min(nblk, b0 + per);
    int s = 0;
    if (j < N)
        for (int b = b0; b < b1; ++b) s += cnt[(int64_t)b * N + j];
    part[w][lane] = s;
    __syncthreads();
    int run = 0;
    for (int i = 0; i < w; ++i) run += part[i][lane];
    if (j < N) {
        if (w == 15) total[j] = run + s;
        for (int b = b0; b < b1; ++b) {
            const int64_t o = (int64_t)b * N + j;
            const int c = cnt[o];
            cnt[o] = run;
            run += c;
        }
    }
}

__global__ __launch_bounds__(1024) void smla_k4_csr_rowscan(const int32_t* __restrict__ total,
                                                            int N, const int32_t* __restrict__ inv,
                                                            int nblk, int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ n_invalid) {
    __shared__ int lds[1024];
    const int tid = threadIdx.x;
    const int ipt = (N + 1023) / 1024;
    const int j0 = min(N, tid * ipt), j1 = min(N, j0 + ipt);
    int local = 0;
    for (int j = j0; j < j1; ++j) local += total[j];
    int grand;
    int run = block_exclusive_scan_1024(local, lds, &grand);
    for (int j = j0; j < j1; ++j) {
        row_ptr[j] = run;
        run += total[j];
    }
    if (tid == 0) row_ptr[N] = grand;
    if (n_invalid != nullptr) {
        int s = 0;
        for (int b = tid; b < nblk; b += 1024) s += inv[b];
        int all;
        block_exclusive_scan_1024(s, lds, &all);
        if (tid == 0) *n_invalid = all;
    }
}

__global__ __launch_bounds__(kSortThreads) void smla_k4_csr_scatter(
    const uint32_t* __restrict__ sorted, int64_t M, int N, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ slots) {
    __shared__ uint32_t keys[kCsrBlock];
    const int b = blockIdx.x;
    const int64_t base = (int64_t)b * kCsrBlock;
    const int nloc = (int)min((int64_t)kCsrBlock, M - base);
    for (int p = threadIdx.x; p < kCsrBlock; p += kSortThreads)
        keys[p] = p < nloc ? sorted[base + p] : kSentinel;
    __syncthreads();
    const int32_t* crow = cnt + (int64_t)b * N;
    for (int p = threadIdx.x; p < nloc; p += kSortThreads) {
        const uint32_t key = keys[p];
        const uint32_t row = key >> 12;
        if (row < (uint32_t)N) {
            const int first = lower_bound_row(keys, kCsrBlock, row);
            const int64_t out = (int64_t)row_ptr[row] + crow[row] + (p - first);
            if (out >= 0 && out < M) slots[out] = (int32_t)(base + (key & 0xFFFu));
        }
    }
}

// out = sum of n per-call counts, in index order (one wave)
__global__ __launch_bounds__(64) void smla_k4_sum_counts(const int32_t* __restrict__ c, int n,
                                                         int32_t* __restrict__ out) {
    int s = 0;
    for (int i = threadIdx.x; i < n; i += 64) s += c[i];
    for (int m = 32; m > 0; m >>= 1) s += wave_xor(s, m);
    if (threadIdx.x == 0) *out = s;
}

hipError_t launch_sum_counts(const int32_t* counts, int n, int32_t* out, hipStream_t s) {
    smla_k4_sum_counts<<<1, 64, 0, s>>>(counts, n, out);
    return hipGetLastError();
}

size_t csr_scratch_bytes(int64_t M, int N) {
    const int64_t nblk = csr_blocks(M);
    return align_up((size_t)M * 4, 256) + align_up((size_t)nblk * N * 4, 256) +
           align_up((size_t)N * 4, 256) + align_up((size_t)(nblk > 0 ? nblk : 1) * 4, 256);
}

CsrScratch csr_carve(void* base, int64_t M, int N) {
    const int64_t nblk = csr_blocks(M);
    char* p = static_cast<char*>(base);
    CsrScratch w;
    w.sorted = reinterpret_cast<uint32_t*>(p);
    p += align_up((size_t)M * 4, 256);
    w.cnt = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)nblk * N * 4, 256);
    w.total = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)N * 4, 256);
    w.inv = reinterpret_cast<int32_t*>(p);
    return w;
}

hipError_t launch_csr(const int32_t* idx, int64_t M, int N, const CsrScratch& ws, int32_t* row_ptr,
                      int32_t* slots, int32_t* n_invalid, hipStream_t s) {
    const int nblk = (int)csr_blocks(M);
    if (nblk > 0) {
        smla_k4_csr_sort<<<nblk, kSortThreads, 0, s>>>(idx, M, N, ws.sorted, ws.cnt, ws.inv);
        smla_k4_csr_colscan<<<(N + 63) / 64, 1024, 0, s>>>(ws.cnt, nblk, N, ws.total);
    } else {
        // no slots: every row is empty
        smla_k4_csr_colscan<<<(N + 63) / 64, 1024, 0, s>>>(ws.cnt, 0, N, ws.total);
    }
    smla_k4_csr_rowscan<<<1, 1024, 0, s>>>(ws.total, N, ws.inv, nblk, row_ptr, n_invalid);
    if (nblk > 0)
        smla_k4_csr_scatter<<<nblk, kSortThreads, 0, s>>>(ws.sorted, M, N, ws.cnt, row_ptr, slots);
    return hipGetLastError();
}

}  // namespace smla
