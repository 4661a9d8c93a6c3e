/*
 * smla.h -- C ABI of the MI355X (gfx950) sparse MLA attention library.
 *
 * The op is the DeepSeek-V4 sparse MLA attention of ROCm/aiter PR 4766
 * ("[DSV4] Sparse MLA training backward"), Contract section: every query head
 * of token t attends to its own top-k rows of ONE shared kv tensor of width
 * 512 (K == V == kv), index -1 means "masked", the logits are scaled by
 * `scale` (1/sqrt(512) in the page), and an optional per-head attention sink
 * enters only the softmax denominator.  The forward's lse includes the sink.
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *    row-major memory on the current HIP device.  bf16 tensors are passed as
 *    uint16_t bit patterns.  Nothing is allocated by the library; nothing is
 *    freed.  Inputs are read only; outputs are fully overwritten (never
 *    accumulated into).
 *  - D (head dimension) is fixed at 512.  Shapes: T query tokens, H heads,
 *    num_kv kv rows, topk index slots per token.  Limits (else SMLA_ERR_SHAPE):
 *    T >= 0, 16 <= H <= 128 with H % 16 == 0, 1 <= topk <= 2^20, T*topk < 2^31,
 *    num_kv >= max(T, 1) (the Contract section allows num_kv > T: rows past T
 *    are a compressed pool) and num_kv < 2^20.
 *  - Index values outside [0, num_kv) are masked like -1 (never read); values
 *    other than -1 are counted into *n_invalid when that pointer is given.
 *  - 16-byte alignment is required for bf16 tensors and the workspace, 4-byte
 *    for float/int32 tensors (else SMLA_ERR_ALIGN).  Output and workspace
 *    ranges must not overlap any other argument (else SMLA_ERR_INVALID_ARG).
 *  - Every pointer must be device (or managed) memory of the current device;
 *    host memory, pinned or not, and other devices' memory are refused with
 *    SMLA_ERR_INVALID_ARG before anything is enqueued.  The first and last
 *    byte of each argument's range are checked, so a buffer shorter than its
 *    range is also refused when the bytes past its end are not this device's
 *    memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work: they return without synchronising; results are ready when the
 *    stream reaches that point.  A smla_bwd / smla_bwd_phased / smla_bwd_pe
 *    call also uses a library-owned helper stream (default priority): it forks
 *    there with an event recorded on `stream` and joins back with an event
 *    that `stream` waits on, so all of its results are still ordered on
 *    `stream`.  Eager calls share one helper stream per device.  A call on a
 *    stream that is being captured into a HIP graph uses a helper of that
 *    capture's own (one of four per device, created by the first eager call):
 *    the fork and join are captured with it, so eager calls of other threads
 *    never enter the graph and two open captures never share a helper.  With
 *    no such helper free, the captured call enqueues every stage on `stream`
 *    itself (same kernels, same results bit for bit).  No hipMemset is
 *    enqueued (every output cell is written by a kernel).  Calls from several
 *    host threads are safe, also while other threads capture: the library's
 *    enqueues are serialised by one mutex, and eager calls on different
 *    streams share only the eager helper stream (their work there runs in
 *    enqueue order; each call's buffers are its own).
 *  - Argument errors are reported synchronously before anything is enqueued.
 *    SMLA_ERR_ARCH is returned when the current device is not gfx950 (the
 *    page's wrapper likewise refuses other architectures).  A failed launch
 *    returns SMLA_ERR_HIP.  The library never prints, aborts or exits.
 *  - Results are bitwise deterministic run to run: no atomics anywhere, every
 *    reduction has a fixed order.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_INVALID_ARG = 1, /* null pointer, overlap, memory not on the current device,
                                 non-finite scale, sink/d_sink mismatch */
    SMLA_ERR_SHAPE = 2,       /* a size outside the limits above */
    SMLA_ERR_ALIGN = 3,       /* a pointer not aligned as required */
    SMLA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the query function says */
    SMLA_ERR_ARCH = 5,        /* current device is not gfx950 */
    SMLA_ERR_HIP = 6          /* a HIP call or kernel launch failed */
} smla_status;

#define SMLA_D 512

/* Human-readable name of a status code (static string, never NULL). */
const char* smla_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Forward (produces the backward's O and lse)                              */
/* ------------------------------------------------------------------------ */

/*
 * smla_fwd -- sparse MLA forward with a sink-inclusive lse.
 * Page: aiter PR 4766, Contract section (the op; the forward's lse folds the
 * sink into the running max and sum, lse = max + ln(sum)).
 *   q    bf16 [T, H, 512]      kv   bf16 [num_kv, 512]
 *   idx  int32 [T, topk]       sink float [H] or NULL (no sink)
 *   o    bf16 [T, H, 512] out  lse  float [T, H] out
 * For each (t, h): S_k = scale * <q[t,h], kv[idx[t,k]]> over valid slots,
 * lse = ln(sum_k exp(S_k) + exp(sink[h])), o = sum_k exp(S_k - lse) kv[idx[t,k]].
 * A row with no valid slot gets o = 0 and lse = -inf (no sink) or sink[h].
 */
int smla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
             int T, int H, int num_kv, int topk, float scale,
             uint16_t* o, float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* Backward                                                                 */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace smla_bwd needs for this shape (0 on a shape error or
 * flags != 0). */
size_t smla_bwd_workspace_bytes(int T, int H, int num_kv, int topk, uint32_t flags);

/*
 * smla_bwd -- training backward: (dq, dkv, d_sink) from (q, kv, dO, O, lse, idx, sink).
 * Page: aiter PR 4766, Contract section (op and lse convention) and Structure
 * table (phases delta, dQ, dKV-interm, CSR build, dKV gather, d_sink).
 *   q, dO, o  bf16 [T, H, 512]   kv bf16 [num_kv, 512]   lse float [T, H]
 *   idx int32 [T, topk]          sink float [H] or NULL
 *   dlse float [T, H] or NULL: upstream gradient of lse, for callers that use
 *             lse downstream (the page's op takes none; NULL means zero).  It
 *             must be finite.  Derived: d lse / d S_k = P_k and
 *             d lse / d sink = P_sink, so it enters as delta -> delta - dlse.
 *   dq  bf16 [T, H, 512] out     dkv bf16 [num_kv, 512] out
 *   d_sink float [H] out; must be non-NULL exactly when sink is non-NULL
 *   flags     reserved for variants of the op; must be 0 (else
 *             SMLA_ERR_INVALID_ARG, before anything is enqueued)
 *   n_invalid int32 [1] out or NULL: count of index values that are neither
 *             -1 nor in [0, num_kv)
 *   workspace device scratch of at least smla_bwd_workspace_bytes() bytes,
 *             owned by the caller; its contents on entry do not matter.
 * Math (per token t, head h, valid slot k): P = exp(scale*<q,kv_k> - lse),
 * dP = <dO, kv_k>, delta = <O, dO> - dlse, dS = P*(dP - delta);
 * dq = scale * sum_k dS kv_k;  dkv[j] = sum over slots (t,k) with idx = j of
 * sum_h (scale*dS q[t,h] + P dO[t,h]);  d_sink[h] = -sum_t exp(sink - lse)*delta.
 * Rows with lse = -inf contribute nothing.  dq/dkv accumulate in fp32.
 */
int smla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
             const float* lse, const int32_t* idx, const float* sink, const float* dlse,
             int T, int H, int num_kv, int topk, float scale, uint32_t flags,
             uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * smla_bwd_timed -- smla_bwd (same arguments, same kernels, same results) that
 * also records five caller-owned events on `stream`, so that a caller can time
 * each stage inside a real call: events[0] before delta, [1] after delta,
 * [2] after dQ, [3] after the intermediate, [4] after the gather (including its
 * wait for the helper stream's CSR build).  Page: aiter PR 4766, Structure table
 * (the per-phase split the events follow).
 *   events  array of 5 hipEvent_t created by the caller on the current device
 *           (timing enabled); the library only records them.
 * Errors: as smla_bwd; a NULL array or NULL event is SMLA_ERR_INVALID_ARG
 * (before any launch); a failed record is SMLA_ERR_HIP.
 */
int smla_bwd_timed(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                   const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                   int T, int H, int num_kv, int topk, float scale, uint32_t flags,
                   uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid,
                   void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/* Bytes of workspace smla_bwd_phased needs (0 on a shape error, phase_tokens < 1
 * or flags != 0). */
size_t smla_bwd_phased_workspace_bytes(int T, int H, int num_kv, int topk, int phase_tokens,
                                       uint32_t flags);

/*
 * smla_bwd_phased -- the same backward with a workspace bounded by a token
 * phase instead of T.  The page notes that the intermediate grows as
 * T * topk * 512 bf16 (its R_CHUNK note, Structure section); here the dS/P
 * blocks, the intermediate, the inverted index and the gather scratch hold
 * phase_tokens tokens at a time, and dkv is carried across phases as an fp32
 * running sum (num_kv * 2 KiB of workspace) that is rounded to bf16 once.
 *   phase_tokens >= 1 (else SMLA_ERR_SHAPE); all other arguments (flags
 *   included) as smla_bwd.
 * Phases run in token order; each phase's inverted index is built on the
 * helper stream while dQ and the intermediate of that phase run (the same
 * fork/join pattern as smla_bwd).  With
 * phase_tokens >= T the results equal smla_bwd's bit for bit; otherwise dkv
 * differs from it only by the fp32 summation order across phases.
 */
int smla_bwd_phased(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                    const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                    int T, int H, int num_kv, int topk, float scale, uint32_t flags, int phase_tokens,
                    uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * smla_bwd_noalloc -- the backward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it takes no workspace and allocates nothing.  Its
 * workspace is a fixed 256 MiB device array inside the library (one copy per
 * GPU, held from the library's first use on that GPU until the process ends).
 *   Arguments as smla_bwd, without workspace/workspace_bytes.
 * It runs smla_bwd_phased with the largest token phase whose workspace fits
 * the array, every stage on `stream` (no helper stream), so its results equal
 * smla_bwd_phased's at that phase: dq and d_sink as smla_bwd's bit for bit,
 * dkv up to the fp32 summation order across phases.
 * Errors: as smla_bwd; SMLA_ERR_WORKSPACE (before anything is enqueued) when
 * even a one-token phase does not fit the array (its fixed part is about
 * 4*T*H + 2 KiB*num_kv bytes); SMLA_ERR_HIP if the array's device address
 * cannot be obtained.
 * Every call on one GPU uses that GPU's one array, and nothing in it needs to
 * be cleared between calls (every cell is written before it is read).  Calls
 * that may run at the same time on one GPU (on different streams) race on the
 * array and give wrong results: order them on one stream.
 */
int smla_bwd_noalloc(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                     const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                     int T, int H, int num_kv, int topk, float scale, uint32_t flags,
                     uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid, void* stream);

/* ------------------------------------------------------------------------ */
/* The backward's stages, exported individually (same conventions)          */
/* ------------------------------------------------------------------------ */

/*
 * smla_delta -- delta[t,h] = sum_d O[t,h,d] * dO[t,h,d] (bf16 in, fp32 accumulation),
 * minus dlse[t,h] when dlse is given (the shift smla_bwd applies for it).
 * Page: aiter PR 4766, Structure table, "delta = rowsum(O*dO)" row.
 *   o, dO bf16 [T, H, 512]   dlse float [T, H] or NULL   delta float [T, H] out
 */
int smla_delta(const uint16_t* o, const uint16_t* dO, const float* dlse, int T, int H,
               float* delta, void* stream);

/*
 * smla_dq -- dq and the per-slot probabilities/gradients of the logits.
 * Page: aiter PR 4766, Structure table, "dQ" row (one LDS copy of the gathered
 * kv feeds both the S and dP products; the kernel also emits dS and P).
 *   q, dO bf16 [T,H,512]  kv bf16 [num_kv,512]  lse, delta float [T,H]  idx int32 [T,topk]
 *   dq  bf16 [T, H, 512] out
 *   dsp bf16 out, smla_dsp_bytes() bytes: per token t, the valid slots of its
 *       index row (in increasing slot order, taken in runs of 512 slots) are
 *       grouped in tiles of 32; tile c of token t is the block of 2H*32 values
 *       at dsp + (t*ceil(topk/32) + c) * 2H*32, holding for rows r < 2H (r = h:
 *       scale*dS[t,h,.], r = H + h: P[t,h,.]) and tile slots j < 32 the value
 *       of (r, j) at block offset (r/16)*512 + ((j%16)/4*16 + r%16)*8 + (j/16)*4
 *       + j%4 (the "piece layout": 16-row chunks of 64 pieces of 8 values, piece
 *       g*16 + r%16 holding slots 4g..4g+3 and 16+4g..16+4g+3 of row r, the order
 *       in which the MFMA lanes hold them); slots past the last valid slot of a
 *       run hold 0, and blocks past the token's last tile are left unwritten.
 */
int smla_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
            const float* delta, const int32_t* idx, int T, int H, int num_kv, int topk,
            float scale, uint16_t* dq, uint16_t* dsp, void* stream);

/* Bytes of the dsp buffer of smla_dq / smla_interm (0 on a shape error). */
size_t smla_dsp_bytes(int T, int H, int topk);

/*
 * smla_interm -- per-slot dKV intermediate, contracted over all heads.
 * Page: aiter PR 4766, Structure table, "dKV-interm" row, and the R_CHUNK note
 * (the intermediate is [T, topk, 512] bf16).
 *   q, dO bf16 [T,H,512]  dsp (from smla_dq, same idx)  idx int32 [T,topk]
 *   interm bf16 [T*topk, 512] out: for every valid slot (t,k),
 *       interm[t*topk+k] = sum_h scale*dS[t,h,k] q[t,h] + P[t,h,k] dO[t,h];
 *       rows of masked slots are left unwritten (the gather never reads them).
 */
int smla_interm(const uint16_t* q, const uint16_t* dO, const uint16_t* dsp, const int32_t* idx,
                int T, int H, int num_kv, int topk, uint16_t* interm, void* stream);

/* Bytes of workspace smla_build_csr needs (0 on a shape error). */
size_t smla_csr_workspace_bytes(int T, int topk, int num_kv);

/*
 * smla_build_csr -- inverted top-k index, built on the device without atomics.
 * Page: aiter PR 4766, Structure table, "CSR build" row (the top-k scatter is
 * inverted so each kv row can gather its contributors).
 *   idx int32 [T, topk]
 *   row_ptr int32 [num_kv+1] out: row_ptr[0] = 0, row_ptr[j+1]-row_ptr[j] = number
 *           of valid slots addressing row j
 *   slots   int32 [T*topk] out (capacity): slots[row_ptr[j] .. row_ptr[j+1]) are the
 *           slots s = t*topk + k with idx[t,k] == j, strictly increasing; entries
 *           past row_ptr[num_kv] are left unwritten
 *   n_invalid int32 [1] out or NULL
 */
int smla_build_csr(const int32_t* idx, int T, int topk, int num_kv,
                   int32_t* row_ptr, int32_t* slots, int32_t* n_invalid,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace smla_gather needs (0 on a shape error). */
size_t smla_gather_workspace_bytes(int T, int topk, int num_kv);

/*
 * smla_gather -- dkv[j] = bf16( sum over s in slots[row_ptr[j]..row_ptr[j+1]) of interm[s] ),
 * fp32 accumulation in a fixed order; rows with no contributor get 0.
 * Page: aiter PR 4766, Structure table, "dKV gather" row (atomic-free: each kv
 * row gathers its own contributors).
 *   interm bf16 [T*topk, 512]  row_ptr int32 [num_kv+1]  slots int32 [row_ptr[num_kv]]
 *   dkv bf16 [num_kv, 512] out
 */
int smla_gather(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots,
                int T, int topk, int num_kv, uint16_t* dkv,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace smla_dsink needs (0 on a shape error). */
size_t smla_dsink_workspace_bytes(int T, int H);

/*
 * smla_dsink -- d_sink[h] = -sum_t exp(sink[h] - lse[t,h]) * delta[t,h] (fixed-order sum).
 * Page: aiter PR 4766, Structure table, "d_sink" row.  The formula is the
 * derivative of O with respect to the sink logit: dO/dsink = -P_sink * O.
 *   lse, delta float [T, H]  sink float [H]  d_sink float [H] out
 */
int smla_dsink(const float* lse, const float* delta, const float* sink, int T, int H,
               float* d_sink, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The has_pe=True variant                                                   */
/* ------------------------------------------------------------------------ */
/*
 * Page: aiter PR 4766, Contract section -- the backward is "the forward's
 * has_pe=False path"; has_pe=True is the forward's other path, which the page
 * names without describing.  Reading used here (DeepSeek's decoupled RoPE):
 * the queries carry an extra positional part q_pe [T, H, 64] and the keys an
 * extra head-shared part k_pe [num_kv, 64]; the logit of slot k is
 * scale * (<q, kv_k> + <q_pe, k_pe_k>); the values are kv alone (512 wide),
 * so O, lse, delta and dkv keep their has_pe=False definitions, and the extra
 * gradients are dq_pe = scale * sum_k dS k_pe_k and, per kv row j,
 * dk_pe[j] = sum over the slots (t, k) with idx = j of sum_h scale*dS q_pe[t,h].
 * The scale is the caller's (1/sqrt(512 + 64) is the natural choice).
 * All conventions (masking, sink, alignment, overlap, streams, determinism)
 * are those of smla_fwd / smla_bwd; q_pe, k_pe, dq_pe, dk_pe are bf16 and
 * need 16-byte alignment.
 */
#define SMLA_DPE 64

/* smla_fwd with the positional part: o bf16 [T,H,512], lse float [T,H] (sink-inclusive). */
int smla_fwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                const int32_t* idx, const float* sink, int T, int H, int num_kv, int topk, float scale,
                uint16_t* o, float* lse, void* stream);

/* Bytes of workspace smla_bwd_pe needs (0 on a shape error or flags != 0). */
size_t smla_bwd_pe_workspace_bytes(int T, int H, int num_kv, int topk, uint32_t flags);

/*
 * smla_bwd_pe -- smla_bwd with the positional part: additionally reads q_pe
 * [T,H,64] and k_pe [num_kv,64] and writes dq_pe bf16 [T,H,64] and dk_pe bf16
 * [num_kv,64] (rows no slot addresses get zeros).  The stages are smla_bwd's
 * (the dS/P blocks now come from the logits with the positional term), plus a
 * positional intermediate [T*topk, 64] contracted over the heads and its
 * gather through the same inverted index.  flags must be 0.
 */
int smla_bwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                const uint16_t* dO, const uint16_t* o, const float* lse, const int32_t* idx,
                const float* sink, const float* dlse, int T, int H, int num_kv, int topk, float scale,
                uint32_t flags, uint16_t* dq, uint16_t* dq_pe, uint16_t* dkv, uint16_t* dk_pe,
                float* d_sink, int32_t* n_invalid, void* workspace, size_t workspace_bytes,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
