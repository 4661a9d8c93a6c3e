// Host-side launchers of the gfx950 kernels (one per kernel family).  Every
// launcher only enqueues on `stream`; shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smla {

// Compute units of the current device (cached per device).
hipError_t compute_units(int* n);

// ---- streaming ------------------------------------------------------------
// delta[r] = sum_d o[r,d] * dO[r,d], minus dlse[r] when dlse is not null
hipError_t launch_delta(const uint16_t* o, const uint16_t* dO, const float* dlse, int64_t rows,
                        float* delta, hipStream_t s);
constexpr int kDsinkTokensPerBlock = 32;
inline int dsink_blocks(int T) { return (T + kDsinkTokensPerBlock - 1) / kDsinkTokensPerBlock; }
hipError_t launch_dsink(const float* lse, const float* delta, const float* sink, int T, int H,
                        float* partial, float* d_sink, hipStream_t s);

// ---- CSR ------------------------------------------------------------------
constexpr int kCsrBlock = 4096;  // keys per sort block (12-bit in-block position)
inline int64_t csr_blocks(int64_t M) { return (M + kCsrBlock - 1) / kCsrBlock; }
struct CsrScratch {
    uint32_t* sorted;   // [M]        block-sorted packed (row << 12 | position)
    int32_t* cnt;       // [nblk * N] per-block row counts, then per-block row offsets
    int32_t* total;     // [N]        per-row totals
    int32_t* inv;       // [nblk]     per-block count of out-of-range indices
};
size_t csr_scratch_bytes(int64_t M, int N);
CsrScratch csr_carve(void* base, int64_t M, int N);
hipError_t launch_csr(const int32_t* idx, int64_t M, int N, const CsrScratch& ws, int32_t* row_ptr,
                      int32_t* slots, int32_t* n_invalid, hipStream_t s);
// *out = counts[0] + ... + counts[n-1]
hipError_t launch_sum_counts(const int32_t* counts, int n, int32_t* out, hipStream_t s);

// ---- gather ---------------------------------------------------------------
constexpr int kGatherSeg = 1024;  // contributors per gather segment (64 per wave of 16)
inline int64_t gather_max_segments(int64_t M, int N) { return N + (M + kGatherSeg - 1) / kGatherSeg; }
struct GatherScratch {
    int32_t* seg_ptr;   // [N + 1]
    int32_t* seg_row;   // [max segments]
    float* partial;     // [max segments * 512]
};
size_t gather_scratch_bytes(int64_t M, int N);
GatherScratch gather_carve(void* base, int64_t M, int N);
// plan (needs only row_ptr) and the sums (need the intermediate) can be
// enqueued on different streams; launch_gather does both in order
hipError_t launch_gather_plan(const int32_t* row_ptr, int64_t M, int N, const GatherScratch& ws,
                              hipStream_t s);
hipError_t launch_gather_sum(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots,
                             int64_t M, int N, const GatherScratch& ws, uint16_t* dkv, hipStream_t s);
hipError_t launch_gather(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots,
                         int64_t M, int N, const GatherScratch& ws, uint16_t* dkv, hipStream_t s);
// one token phase of a phased backward: adds the phase's sums to the fp32
// running sums `run` [N, 512] (set, when first); dkv_last (non-null on the
// last phase only) receives the bf16 rounding of the final sums instead
hipError_t launch_gather_sum_phase(const uint16_t* interm, const int32_t* row_ptr,
                                   const int32_t* slots, int64_t M, int N, const GatherScratch& ws,
                                   bool first, float* run, uint16_t* dkv_last, hipStream_t s);

// ---- attention tiles (MFMA) -----------------------------------------------
hipError_t launch_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
                     const float* delta, const int32_t* idx, int T, int H, int N, int K, float scale,
                     uint16_t* dq, uint16_t* dsp, hipStream_t s);
hipError_t launch_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
                      int T, int H, int N, int K, float scale, uint16_t* o, float* lse,
                      hipStream_t s);
hipError_t launch_interm(const uint16_t* q, const uint16_t* dO, const uint16_t* dsp,
                         const int32_t* idx, int T, int H, int N, int K, uint16_t* interm,
                         hipStream_t s);

// ---- the has_pe=True variant (positional part of width 64) -----------------
hipError_t launch_dq_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                        const uint16_t* dO, const float* lse, const float* delta, const int32_t* idx, int T,
                        int H, int N, int K, float scale, uint16_t* dq, uint16_t* dq_pe, uint16_t* dsp,
                        hipStream_t s);
hipError_t launch_fwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                         const int32_t* idx, const float* sink, int T, int H, int N, int K, float scale,
                         uint16_t* o, float* lse, hipStream_t s);
// both intermediates of the has_pe=True variant in one pass
hipError_t launch_interm_fused_pe(const uint16_t* q, const uint16_t* dO, const uint16_t* q_pe,
                                  const uint16_t* dsp, const int32_t* idx, int T, int H, int N, int K,
                                  uint16_t* interm, uint16_t* interm_pe, hipStream_t s);
size_t gather_pe_scratch_bytes(int64_t M, int N);
// sums of the positional intermediate per kv row, over the segments of an
// existing gather plan (launch_gather_plan on the same row_ptr)
hipError_t launch_gather_pe(const uint16_t* interm_pe, const int32_t* row_ptr, const int32_t* slots,
                            int64_t M, int N, const GatherScratch& plan, float* partial, uint16_t* dk_pe,
                            hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace smla
