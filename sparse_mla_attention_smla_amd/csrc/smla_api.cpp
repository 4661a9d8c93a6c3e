// Host side of the C ABI declared in include/smla.h: argument validation, the
// gfx950 gate, workspace carving and the launch order of the backward.
//
// Page: aiter PR 4766 "Sparse MLA training backward" -- the public wrapper of
// the page checks head_dim == 512, kv/dO/O shapes, num_kv >= T and
// contiguity, defaults the scale to 1/sqrt(D) and refuses non-gfx950 devices;
// its review asks for dtype and lse/sink shape checks too.  Here the same
// checks are made on raw sizes and pointers before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "smla.h"
#include "kv_tile.hpp"
#include "smla_launch.hpp"
#include "smla_device.hpp"

using namespace smla;

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxTopk = 1 << 20;  // index slots per token
int g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::mutex g_arch_mu;

smla_status check_arch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SMLA_ERR_ARCH;
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SMLA_ERR_HIP;
        g_arch_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return g_arch_state[dev] == 1 ? SMLA_OK : SMLA_ERR_ARCH;
}

}  // namespace

// Compute units of the current device (cached per device).
hipError_t smla::compute_units(int* n) {
    static int cache[kMaxDevices] = {};
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cache[dev] = v > 0 ? v : 1;
    }
    *n = cache[dev];
    return hipSuccess;
}

namespace {

// A helper stream per device (default priority, non-blocking) with fork, join
// and after-delta events: smla_bwd runs the CSR build, the gather plan and
// (once delta is done) d_sink there, concurrently with delta, dQ and the
// intermediate, and joins before the gather sums (smla_bwd_phased does the
// same per token phase).  One mutex covers a whole enqueue so calls from
// several host threads cannot interleave records of the shared events.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, after_delta = nullptr;
    hipEvent_t gather_done = nullptr;   // phased backward: the phase's gather has read the CSR
    int state = 0;  // 0 not tried, 1 ready, 2 unavailable
};
SideStream g_side[kMaxDevices];
// helper streams for calls under graph capture: each serves one open capture
// at a time (it joins that capture through the fork event and leaves it when
// the capture ends)
constexpr int kCapSlots = 4;
SideStream g_cap[kMaxDevices][kCapSlots];
std::mutex g_side_mu;

bool make_side(SideStream& d) {
    if (d.state == 0) {
        d.state = 2;
        if (hipStreamCreateWithFlags(&d.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&d.join, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&d.after_delta, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&d.gather_done, hipEventDisableTiming) == hipSuccess)
            d.state = 1;
    }
    return d.state == 1;
}

// The eager helper stream of `dev`; its first use also creates the capture
// helpers, so that no stream is ever created while a capture is open.
SideStream* side_stream(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    for (int i = 0; i < kCapSlots; ++i) (void)make_side(g_cap[dev][i]);
    return make_side(g_side[dev]) ? &g_side[dev] : nullptr;
}

// The helper stream for a call on `s`, or nullptr to enqueue every stage on
// `s` itself.  Eager calls share the device's helper stream.  A call on a
// stream being captured into a graph gets a capture helper of its own: the
// one already joined to that capture (same capture id), else one that is in
// no capture; so the eager helper never joins a capture, eager calls of other
// threads never land in a graph, and two open captures never share a helper.
// With no capture helper free (or none created yet: they are made by the first
// eager call, never during a capture), the call runs in line on `s`.  *err is
// set when the capture state cannot be read.
SideStream* side_for(hipStream_t s, int dev, bool* err) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    *err = hipStreamGetCaptureInfo(s, &cs, &id) != hipSuccess;
    if (*err) return nullptr;
    if (cs == hipStreamCaptureStatusNone) return side_stream(dev);
    if (cs != hipStreamCaptureStatusActive || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream* free_slot = nullptr;
    for (int i = 0; i < kCapSlots; ++i) {
        SideStream& c = g_cap[dev][i];
        if (c.state != 1) continue;
        hipStreamCaptureStatus cs2 = hipStreamCaptureStatusNone;
        unsigned long long id2 = 0;
        if (hipStreamGetCaptureInfo(c.s, &cs2, &id2) != hipSuccess) continue;
        if (cs2 == hipStreamCaptureStatusActive && id2 == id) return &c;
        if (cs2 == hipStreamCaptureStatusNone && free_slot == nullptr) free_slot = &c;
    }
    return free_slot;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    const void* p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// all[first_out..nall) are outputs: each must be disjoint from every other range
bool outputs_disjoint(const Range* all, int nall, int first_out) {
    for (int i = first_out; i < nall; ++i)
        for (int j = 0; j < nall; ++j)
            if (i != j && overlap(all[i], all[j])) return false;
    return true;
}

// Every argument range must lie in device (or managed) memory of the current
// device: a host pointer, or another device's buffer, reaching a kernel would
// fault the GPU.  The first and the last byte of each range are looked up
// (about 0.1 us each, no stream work, so also legal under graph capture); a
// buffer that ends before its range does is caught as well whenever the bytes
// past its end are not this device's memory.
smla_status device_ranges(const Range* all, int nall) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    for (int i = 0; i < nall; ++i) {
        if (all[i].p == nullptr || all[i].n == 0) continue;
        const char* first = static_cast<const char*>(all[i].p);
        const char* ends[2] = {first, first + (all[i].n - 1)};
        for (const char* p : ends) {
            hipPointerAttribute_t a{};
            if (hipPointerGetAttributes(&a, p) != hipSuccess) {
                (void)hipGetLastError();   // leave no error behind for the caller's next call
                return SMLA_ERR_INVALID_ARG;
            }
            if ((a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) || a.device != dev)
                return SMLA_ERR_INVALID_ARG;
        }
    }
    return SMLA_OK;
}

// Outputs disjoint from everything else, and every range on this device.
smla_status check_ranges(const Range* all, int nall, int first_out) {
    if (!outputs_disjoint(all, nall, first_out)) return SMLA_ERR_INVALID_ARG;
    return device_ranges(all, nall);
}

smla_status check_shape(int T, int H, int num_kv, int topk) {
    if (T < 0 || H < 16 || H > 128 || H % 16 != 0 || topk < 1) return SMLA_ERR_SHAPE;
    if (num_kv < 1 || num_kv < T || num_kv >= (1 << 20)) return SMLA_ERR_SHAPE;
    if ((int64_t)T * topk >= (int64_t)1 << 31) return SMLA_ERR_SHAPE;
    // a token's intermediate block (topk rows of 1 KiB) is addressed with
    // 32-bit buffer offsets
    if (topk > kMaxTopk) return SMLA_ERR_SHAPE;
    return SMLA_OK;
}

smla_status hip_status(hipError_t e) { return e == hipSuccess ? SMLA_OK : SMLA_ERR_HIP; }

// dS/P blocks: per token ceil(topk/32) blocks of 2H*32 bf16 (the piece layout of smla.h)
size_t dsp_bytes(int T, int H, int topk) {
    return (size_t)T * (size_t)((topk + 31) / 32) * 2 * H * 32 * 2;
}

constexpr size_t kWsAlign = 256;

struct BwdLayout {
    size_t delta, dsp, interm, row_ptr, slots, csr, gather, dsink, total;
};

BwdLayout bwd_layout(int T, int H, int num_kv, int topk) {
    const int64_t M = (int64_t)T * topk;
    BwdLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes, kWsAlign);
        return at;
    };
    L.delta = take((size_t)T * H * 4);
    L.dsp = take(dsp_bytes(T, H, topk));
    L.interm = take((size_t)M * kD * 2);
    L.row_ptr = take((size_t)(num_kv + 1) * 4);
    L.slots = take((size_t)(M > 0 ? M : 1) * 4);
    L.csr = take(csr_scratch_bytes(M, num_kv));
    L.gather = take(gather_scratch_bytes(M, num_kv));
    L.dsink = take((size_t)(dsink_blocks(T) > 0 ? dsink_blocks(T) : 1) * H * 4);
    L.total = off;
    return L;
}

// The has_pe=True backward: the plain layout plus the positional intermediate
// [T*topk, 64] bf16 and the positional gather partials.
struct PeLayout {
    BwdLayout base;
    size_t interm_pe, gather_pe, total;
};

PeLayout pe_layout(int T, int H, int num_kv, int topk) {
    PeLayout L;
    L.base = bwd_layout(T, H, num_kv, topk);
    const int64_t M = (int64_t)T * topk;
    size_t off = L.base.total;
    L.interm_pe = off;
    off += align_up((size_t)M * kDP * 2, kWsAlign);
    L.gather_pe = off;
    off += gather_pe_scratch_bytes(M, num_kv);
    L.total = off;
    return L;
}

// Token-phased backward: phases of Tp = min(phase_tokens, T) tokens (at least
// one phase); the dS/P blocks, the intermediate, the CSR and the gather scratch
// are sized for one phase, plus an fp32 running dkv and one invalid-index count
// per phase.
struct PhasedLayout {
    int Tp, nphase;
    size_t delta, dsp, interm, row_ptr, slots, csr, gather, dsink, run, inv, total;
};

PhasedLayout phased_layout(int T, int H, int num_kv, int topk, int phase_tokens) {
    PhasedLayout L;
    L.Tp = T < phase_tokens ? T : phase_tokens;
    if (L.Tp < 1) L.Tp = 1;
    L.nphase = T > 0 ? (T + L.Tp - 1) / L.Tp : 1;
    const int64_t Mp = (int64_t)L.Tp * topk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align_up(bytes, kWsAlign);
        return at;
    };
    L.delta = take((size_t)T * H * 4);
    L.dsp = take(dsp_bytes(L.Tp, H, topk));
    L.interm = take((size_t)Mp * kD * 2);
    L.row_ptr = take((size_t)(num_kv + 1) * 4);
    L.slots = take((size_t)Mp * 4);
    L.csr = take(csr_scratch_bytes(Mp, num_kv));
    L.gather = take(gather_scratch_bytes(Mp, num_kv));
    L.dsink = take((size_t)(dsink_blocks(T) > 0 ? dsink_blocks(T) : 1) * H * 4);
    L.run = take((size_t)num_kv * kD * 4);
    L.inv = take((size_t)L.nphase * 4);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

const char* smla_status_string(int status) {
    switch (status) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_INVALID_ARG: return "invalid argument";
        case SMLA_ERR_SHAPE: return "unsupported shape";
        case SMLA_ERR_ALIGN: return "misaligned pointer";
        case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
        case SMLA_ERR_ARCH: return "device is not gfx950";
        case SMLA_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

size_t smla_bwd_workspace_bytes(int T, int H, int num_kv, int topk, uint32_t flags) {
    if (flags != 0 || check_shape(T, H, num_kv, topk) != SMLA_OK) return 0;
    return bwd_layout(T, H, num_kv, topk).total;
}

size_t smla_bwd_phased_workspace_bytes(int T, int H, int num_kv, int topk, int phase_tokens,
                                       uint32_t flags) {
    if (flags != 0 || check_shape(T, H, num_kv, topk) != SMLA_OK || phase_tokens < 1) return 0;
    return phased_layout(T, H, num_kv, topk, phase_tokens).total;
}

size_t smla_csr_workspace_bytes(int T, int topk, int num_kv) {
    if (check_shape(T, 16, num_kv, topk) != SMLA_OK) return 0;
    return csr_scratch_bytes((int64_t)T * topk, num_kv);
}

size_t smla_gather_workspace_bytes(int T, int topk, int num_kv) {
    if (check_shape(T, 16, num_kv, topk) != SMLA_OK) return 0;
    return gather_scratch_bytes((int64_t)T * topk, num_kv);
}

size_t smla_dsp_bytes(int T, int H, int topk) {
    if (check_shape(T, H, T > 0 ? T : 1, topk) != SMLA_OK) return 0;
    return dsp_bytes(T, H, topk);
}

size_t smla_dsink_workspace_bytes(int T, int H) {
    if (check_shape(T, H, T > 0 ? T : 1, 1) != SMLA_OK) return 0;
    return (size_t)(dsink_blocks(T) > 0 ? dsink_blocks(T) : 1) * H * 4;
}

int smla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
             int T, int H, int num_kv, int topk, float scale, uint16_t* o, float* lse,
             void* stream) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (!std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !idx || !o || !lse)) return SMLA_ERR_INVALID_ARG;
    if (!kv) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(o, 16) || !aligned(idx, 4) ||
        !aligned(lse, 4) || !aligned(sink, 4))
        return SMLA_ERR_ALIGN;
    const size_t qb = (size_t)T * H * kD * 2;
    const Range all[] = {{q, qb}, {kv, (size_t)num_kv * kD * 2}, {idx, (size_t)T * topk * 4},
                         {sink, sink ? (size_t)H * 4 : 0}, {o, qb}, {lse, (size_t)T * H * 4}};
    if ((st = check_ranges(all, 6, 4)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_fwd(q, kv, idx, sink, T, H, num_kv, topk, scale, o, lse,
                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
// The whole backward; when `ev` is given, its five events are recorded on the
// caller's stream before delta and after delta, dQ, the intermediate and the gather.
int bwd_impl(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
             const float* lse, const int32_t* idx, const float* sink, const float* dlse, int T,
             int H, int num_kv, int topk, float scale, uint32_t flags, uint16_t* dq, uint16_t* dkv,
             float* d_sink, int32_t* n_invalid, void* workspace, size_t workspace_bytes,
             void* stream, void* const* ev) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (flags != 0 || !std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (!kv || !dkv) return SMLA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !dO || !o || !lse || !idx || !dq)) return SMLA_ERR_INVALID_ARG;
    if ((sink == nullptr) != (d_sink == nullptr)) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(dO, 16) || !aligned(o, 16) ||
        !aligned(dq, 16) || !aligned(dkv, 16) || !aligned(lse, 4) || !aligned(idx, 4) ||
        !aligned(sink, 4) || !aligned(dlse, 4) || !aligned(d_sink, 4) ||
        !aligned(n_invalid, 4) || !aligned(workspace, 16))
        return SMLA_ERR_ALIGN;
    const BwdLayout L = bwd_layout(T, H, num_kv, topk);
    if (workspace == nullptr || workspace_bytes < L.total) return SMLA_ERR_WORKSPACE;
    const size_t qb = (size_t)T * H * kD * 2;
    const size_t hb = (size_t)H * 4;
    const Range all[] = {{q, qb},
                         {kv, (size_t)num_kv * kD * 2},
                         {dO, qb},
                         {o, qb},
                         {lse, (size_t)T * H * 4},
                         {idx, (size_t)T * topk * 4},
                         {sink, sink ? hb : 0},
                         {dlse, dlse ? (size_t)T * H * 4 : 0},
                         {dq, qb},
                         {dkv, (size_t)num_kv * kD * 2},
                         {d_sink, d_sink ? hb : 0},
                         {n_invalid, n_invalid ? 4u : 0u},
                         {workspace, L.total}};
    if ((st = check_ranges(all, 13, 8)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(ws + L.delta);
    uint16_t* dsp = reinterpret_cast<uint16_t*>(ws + L.dsp);
    uint16_t* interm = reinterpret_cast<uint16_t*>(ws + L.interm);
    int32_t* row_ptr = reinterpret_cast<int32_t*>(ws + L.row_ptr);
    int32_t* slots = reinterpret_cast<int32_t*>(ws + L.slots);
    const int64_t M = (int64_t)T * topk;
    const CsrScratch cs = csr_carve(ws + L.csr, M, num_kv);
    const GatherScratch gs = gather_carve(ws + L.gather, M, num_kv);
    float* dsink_part = reinterpret_cast<float*>(ws + L.dsink);

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_side_mu);
    bool cap_err = false;
    SideStream* side = side_for(s, dev, &cap_err);
    if (cap_err) return SMLA_ERR_HIP;
    // The CSR and the gather plan depend only on the indices, d_sink only on
    // lse and delta: they run on the helper stream while dQ and the
    // intermediate run on the caller's stream (all in one order on the
    // caller's stream under graph capture, or when no helper stream could be
    // made).
    hipStream_t aux = side != nullptr ? side->s : s;
    if (side != nullptr) {
        if (hipEventRecord(side->fork, s) != hipSuccess ||
            hipStreamWaitEvent(aux, side->fork, 0) != hipSuccess)
            return SMLA_ERR_HIP;
    }
    if (launch_csr(idx, M, num_kv, cs, row_ptr, slots, n_invalid, aux) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_gather_plan(row_ptr, M, num_kv, gs, aux) != hipSuccess) return SMLA_ERR_HIP;
    auto mark = [&](int i) {
        return ev == nullptr || hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) == hipSuccess;
    };
    if (!mark(0)) return SMLA_ERR_HIP;
    if (launch_delta(o, dO, dlse, (int64_t)T * H, delta, s) != hipSuccess) return SMLA_ERR_HIP;
    if (!mark(1)) return SMLA_ERR_HIP;
    if (sink != nullptr) {
        if (side != nullptr && (hipEventRecord(side->after_delta, s) != hipSuccess ||
                                hipStreamWaitEvent(aux, side->after_delta, 0) != hipSuccess))
            return SMLA_ERR_HIP;
        if (launch_dsink(lse, delta, sink, T, H, dsink_part, d_sink, aux) != hipSuccess)
            return SMLA_ERR_HIP;
    }
    if (side != nullptr && hipEventRecord(side->join, aux) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_dq(q, kv, dO, lse, delta, idx, T, H, num_kv, topk, scale, dq, dsp, s) != hipSuccess)
        return SMLA_ERR_HIP;
    if (!mark(2)) return SMLA_ERR_HIP;
    if (launch_interm(q, dO, dsp, idx, T, H, num_kv, topk, interm, s) != hipSuccess)
        return SMLA_ERR_HIP;
    if (!mark(3)) return SMLA_ERR_HIP;
    if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_gather_sum(interm, row_ptr, slots, M, num_kv, gs, dkv, s) != hipSuccess)
        return SMLA_ERR_HIP;
    if (!mark(4)) return SMLA_ERR_HIP;
    return SMLA_OK;
}
}  // namespace

extern "C" {

int smla_bwd(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
             const float* lse, const int32_t* idx, const float* sink, const float* dlse, int T,
             int H, int num_kv, int topk, float scale, uint32_t flags, uint16_t* dq, uint16_t* dkv,
             float* d_sink, int32_t* n_invalid, void* workspace, size_t workspace_bytes,
             void* stream) {
    return bwd_impl(q, kv, dO, o, lse, idx, sink, dlse, T, H, num_kv, topk, scale, flags, dq, dkv,
                    d_sink, n_invalid, workspace, workspace_bytes, stream, nullptr);
}

int smla_bwd_timed(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                   const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                   int T, int H, int num_kv, int topk, float scale, uint32_t flags, uint16_t* dq,
                   uint16_t* dkv, float* d_sink, int32_t* n_invalid, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* events) {
    if (events == nullptr) return SMLA_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (events[i] == nullptr) return SMLA_ERR_INVALID_ARG;
    return bwd_impl(q, kv, dO, o, lse, idx, sink, dlse, T, H, num_kv, topk, scale, flags, dq, dkv,
                    d_sink, n_invalid, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

namespace {

// ---- scratch of the no-allocation backward ---------------------------------
// A fixed device array holds the workspace of smla_bwd_noalloc.  Host code
// never uses the array's name as a device address: once per device, with that
// device current, hipGetSymbolAddress yields the device's own copy, and that
// pointer is what the kernels receive.
constexpr size_t kScratchBytes = (size_t)256 << 20;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

smla_status scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SMLA_ERR_ARCH;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SMLA_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SMLA_OK;
}

// Largest token phase whose phased workspace fits the scratch (0 if even one
// token does not).
int noalloc_phase_tokens(int T, int H, int num_kv, int topk) {
    auto fits = [&](int tp) { return phased_layout(T, H, num_kv, topk, tp).total <= kScratchBytes; };
    if (!fits(1)) return 0;
    int lo = 1, hi = T > 1 ? T : 1;
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (fits(mid)) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The token-phased backward.  With use_helper false, every stage stays on the
// caller's stream (no library-owned stream or event is created or used).  With
// use_scratch, `workspace` is ignored and the phase must fit the scratch; its
// address is taken only after every argument check has passed.
int phased_impl(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                const float* lse, const int32_t* idx, const float* sink, const float* dlse, int T,
                int H, int num_kv, int topk, float scale, uint32_t flags, int phase_tokens,
                uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid, void* workspace,
                size_t workspace_bytes, void* stream, bool use_helper, bool use_scratch = false) {
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = kScratchBytes;
    }
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (phase_tokens < 1) return SMLA_ERR_SHAPE;
    if (flags != 0 || !std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (!kv || !dkv) return SMLA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !dO || !o || !lse || !idx || !dq)) return SMLA_ERR_INVALID_ARG;
    if ((sink == nullptr) != (d_sink == nullptr)) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(dO, 16) || !aligned(o, 16) ||
        !aligned(dq, 16) || !aligned(dkv, 16) || !aligned(lse, 4) || !aligned(idx, 4) ||
        !aligned(sink, 4) || !aligned(dlse, 4) || !aligned(d_sink, 4) ||
        !aligned(n_invalid, 4) || !aligned(workspace, 16))
        return SMLA_ERR_ALIGN;
    const PhasedLayout L = phased_layout(T, H, num_kv, topk, phase_tokens);
    if ((!use_scratch && workspace == nullptr) || workspace_bytes < L.total) return SMLA_ERR_WORKSPACE;
    const size_t qb = (size_t)T * H * kD * 2;
    const size_t hb = (size_t)H * 4;
    const Range all[] = {{q, qb},
                         {kv, (size_t)num_kv * kD * 2},
                         {dO, qb},
                         {o, qb},
                         {lse, (size_t)T * H * 4},
                         {idx, (size_t)T * topk * 4},
                         {sink, sink ? hb : 0},
                         {dlse, dlse ? (size_t)T * H * 4 : 0},
                         {dq, qb},
                         {dkv, (size_t)num_kv * kD * 2},
                         {d_sink, d_sink ? hb : 0},
                         {n_invalid, n_invalid ? 4u : 0u},
                         {workspace, L.total}};
    if ((st = check_ranges(all, 13, 8)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    if (use_scratch && (st = scratch_of_current_device(&workspace)) != SMLA_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(ws + L.delta);
    uint16_t* dsp = reinterpret_cast<uint16_t*>(ws + L.dsp);
    uint16_t* interm = reinterpret_cast<uint16_t*>(ws + L.interm);
    int32_t* row_ptr = reinterpret_cast<int32_t*>(ws + L.row_ptr);
    int32_t* slots = reinterpret_cast<int32_t*>(ws + L.slots);
    const int64_t Mp = (int64_t)L.Tp * topk;
    const CsrScratch cs = csr_carve(ws + L.csr, Mp, num_kv);
    const GatherScratch gs = gather_carve(ws + L.gather, Mp, num_kv);
    float* dsink_part = reinterpret_cast<float*>(ws + L.dsink);
    float* run = reinterpret_cast<float*>(ws + L.run);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);

    // delta and d_sink cover all tokens at once; every later stage runs per
    // phase on token-range views, in phase order.  As in smla_bwd, the inverted
    // index and gather plan of a phase are built on the helper stream while dQ
    // and the intermediate of that phase run on the caller's stream; the next
    // phase's build waits until this phase's gather has read them.
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideStream* side = nullptr;
    if (use_helper) {
        bool cap_err = false;
        side = side_for(s, dev, &cap_err);
        if (cap_err) return SMLA_ERR_HIP;
    }
    hipStream_t aux = side != nullptr ? side->s : s;
    auto rec_wait = [&](hipEvent_t e, hipStream_t from, hipStream_t to) {
        return side == nullptr ||
               (hipEventRecord(e, from) == hipSuccess && hipStreamWaitEvent(to, e, 0) == hipSuccess);
    };
    if (!rec_wait(side ? side->fork : nullptr, s, aux)) return SMLA_ERR_HIP;
    if (launch_delta(o, dO, dlse, (int64_t)T * H, delta, s) != hipSuccess) return SMLA_ERR_HIP;
    for (int p = 0; p < L.nphase; ++p) {
        const int t0 = p * L.Tp;
        const int tp = T - t0 < L.Tp ? T - t0 : L.Tp;
        const size_t tok = (size_t)t0 * H * kD;
        const size_t row = (size_t)t0 * H;
        const int32_t* idx_p = idx + (size_t)t0 * topk;
        const int64_t M = (int64_t)tp * topk;
        if (p > 0 && !rec_wait(side ? side->gather_done : nullptr, s, aux)) return SMLA_ERR_HIP;
        if (launch_csr(idx_p, M, num_kv, cs, row_ptr, slots, n_invalid ? inv + p : nullptr, aux) !=
            hipSuccess)
            return SMLA_ERR_HIP;
        if (launch_gather_plan(row_ptr, M, num_kv, gs, aux) != hipSuccess) return SMLA_ERR_HIP;
        if (side != nullptr && hipEventRecord(side->join, aux) != hipSuccess) return SMLA_ERR_HIP;
        if (p == 0 && sink != nullptr) {
            if (!rec_wait(side ? side->after_delta : nullptr, s, aux)) return SMLA_ERR_HIP;
            if (launch_dsink(lse, delta, sink, T, H, dsink_part, d_sink, aux) != hipSuccess)
                return SMLA_ERR_HIP;
        }
        if (launch_dq(q + tok, kv, dO + tok, lse + row, delta + row, idx_p, tp, H, num_kv, topk, scale,
                      dq + tok, dsp, s) != hipSuccess)
            return SMLA_ERR_HIP;
        if (launch_interm(q + tok, dO + tok, dsp, idx_p, tp, H, num_kv, topk, interm, s) != hipSuccess)
            return SMLA_ERR_HIP;
        if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return SMLA_ERR_HIP;
        if (launch_gather_sum_phase(interm, row_ptr, slots, M, num_kv, gs, p == 0, run,
                                    p + 1 == L.nphase ? dkv : nullptr, s) != hipSuccess)
            return SMLA_ERR_HIP;
    }
    // everything enqueued on the helper stream (d_sink included) joins here
    if (!rec_wait(side ? side->join : nullptr, aux, s)) return SMLA_ERR_HIP;
    if (n_invalid != nullptr && launch_sum_counts(inv, L.nphase, n_invalid, s) != hipSuccess)
        return SMLA_ERR_HIP;
    return SMLA_OK;
}
}  // namespace

extern "C" {

int smla_bwd_phased(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                    const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                    int T, int H, int num_kv, int topk, float scale, uint32_t flags, int phase_tokens,
                    uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return phased_impl(q, kv, dO, o, lse, idx, sink, dlse, T, H, num_kv, topk, scale, flags,
                       phase_tokens, dq, dkv, d_sink, n_invalid, workspace, workspace_bytes, stream,
                       true);
}

int smla_bwd_noalloc(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const uint16_t* o,
                     const float* lse, const int32_t* idx, const float* sink, const float* dlse,
                     int T, int H, int num_kv, int topk, float scale, uint32_t flags,
                     uint16_t* dq, uint16_t* dkv, float* d_sink, int32_t* n_invalid, void* stream) {
    const smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    const int tp = noalloc_phase_tokens(T, H, num_kv, topk);
    if (tp == 0) return SMLA_ERR_WORKSPACE;
    return phased_impl(q, kv, dO, o, lse, idx, sink, dlse, T, H, num_kv, topk, scale, flags, tp, dq,
                       dkv, d_sink, n_invalid, nullptr, 0, stream, false, true);
}

int smla_delta(const uint16_t* o, const uint16_t* dO, const float* dlse, int T, int H,
               float* delta, void* stream) {
    smla_status st = check_shape(T, H, T > 0 ? T : 1, 1);
    if (st != SMLA_OK) return st;
    if (T > 0 && (!o || !dO || !delta)) return SMLA_ERR_INVALID_ARG;
    if (!aligned(o, 16) || !aligned(dO, 16) || !aligned(dlse, 4) || !aligned(delta, 4))
        return SMLA_ERR_ALIGN;
    const size_t qb = (size_t)T * H * kD * 2;
    const size_t rb = (size_t)T * H * 4;
    const Range all[] = {{o, qb}, {dO, qb}, {dlse, dlse ? rb : 0}, {delta, rb}};
    if ((st = check_ranges(all, 4, 3)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(
        launch_delta(o, dO, dlse, (int64_t)T * H, delta, static_cast<hipStream_t>(stream)));
}

int smla_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
            const float* delta, const int32_t* idx, int T, int H, int num_kv, int topk,
            float scale, uint16_t* dq, uint16_t* dsp, void* stream) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (!std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (!kv || (T > 0 && (!q || !dO || !lse || !delta || !idx || !dq || !dsp)))
        return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(dO, 16) || !aligned(dq, 16) ||
        !aligned(dsp, 16) || !aligned(lse, 4) || !aligned(delta, 4) || !aligned(idx, 4))
        return SMLA_ERR_ALIGN;
    const size_t qb = (size_t)T * H * kD * 2;
    const Range all[] = {{q, qb},          {kv, (size_t)num_kv * kD * 2},
                         {dO, qb},         {lse, (size_t)T * H * 4},
                         {delta, (size_t)T * H * 4}, {idx, (size_t)T * topk * 4},
                         {dq, qb},         {dsp, dsp_bytes(T, H, topk)}};
    if ((st = check_ranges(all, 8, 6)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_dq(q, kv, dO, lse, delta, idx, T, H, num_kv, topk, scale, dq, dsp,
                                static_cast<hipStream_t>(stream)));
}

int smla_interm(const uint16_t* q, const uint16_t* dO, const uint16_t* dsp, const int32_t* idx,
                int T, int H, int num_kv, int topk, uint16_t* interm, void* stream) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (T > 0 && (!q || !dO || !dsp || !idx || !interm)) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(dO, 16) || !aligned(dsp, 16) || !aligned(interm, 16) ||
        !aligned(idx, 4))
        return SMLA_ERR_ALIGN;
    const size_t qb = (size_t)T * H * kD * 2;
    const Range all[] = {{q, qb},
                         {dO, qb},
                         {dsp, dsp_bytes(T, H, topk)},
                         {idx, (size_t)T * topk * 4},
                         {interm, (size_t)T * topk * kD * 2}};
    if ((st = check_ranges(all, 5, 4)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_interm(q, dO, dsp, idx, T, H, num_kv, topk, interm,
                                    static_cast<hipStream_t>(stream)));
}

int smla_build_csr(const int32_t* idx, int T, int topk, int num_kv, int32_t* row_ptr,
                   int32_t* slots, int32_t* n_invalid, void* workspace, size_t workspace_bytes,
                   void* stream) {
    smla_status st = check_shape(T, 16, num_kv, topk);
    if (st != SMLA_OK) return st;
    const int64_t M = (int64_t)T * topk;
    if (!row_ptr || (M > 0 && (!idx || !slots))) return SMLA_ERR_INVALID_ARG;
    if (!aligned(idx, 4) || !aligned(row_ptr, 4) || !aligned(slots, 4) || !aligned(n_invalid, 4) ||
        !aligned(workspace, 16))
        return SMLA_ERR_ALIGN;
    const size_t need = csr_scratch_bytes(M, num_kv);
    if (workspace == nullptr || workspace_bytes < need) return SMLA_ERR_WORKSPACE;
    const Range all[] = {{idx, (size_t)M * 4},
                         {row_ptr, (size_t)(num_kv + 1) * 4},
                         {slots, (size_t)M * 4},
                         {n_invalid, n_invalid ? 4u : 0u},
                         {workspace, need}};
    if ((st = check_ranges(all, 5, 1)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_csr(idx, M, num_kv, csr_carve(workspace, M, num_kv), row_ptr, slots,
                                 n_invalid, static_cast<hipStream_t>(stream)));
}

int smla_gather(const uint16_t* interm, const int32_t* row_ptr, const int32_t* slots, int T,
                int topk, int num_kv, uint16_t* dkv, void* workspace, size_t workspace_bytes,
                void* stream) {
    smla_status st = check_shape(T, 16, num_kv, topk);
    if (st != SMLA_OK) return st;
    const int64_t M = (int64_t)T * topk;
    if (!row_ptr || !dkv || (M > 0 && (!interm || !slots))) return SMLA_ERR_INVALID_ARG;
    if (!aligned(interm, 16) || !aligned(dkv, 16) || !aligned(row_ptr, 4) || !aligned(slots, 4) ||
        !aligned(workspace, 16))
        return SMLA_ERR_ALIGN;
    const size_t need = gather_scratch_bytes(M, num_kv);
    if (workspace == nullptr || workspace_bytes < need) return SMLA_ERR_WORKSPACE;
    // slots holds row_ptr[num_kv] entries, a device-side count: only its first entry is checked
    const Range all[] = {{interm, (size_t)M * kD * 2},
                         {row_ptr, (size_t)(num_kv + 1) * 4},
                         {slots, 4},
                         {dkv, (size_t)num_kv * kD * 2},
                         {workspace, need}};
    if ((st = check_ranges(all, 5, 3)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_gather(interm, row_ptr, slots, M, num_kv,
                                    gather_carve(workspace, M, num_kv), dkv,
                                    static_cast<hipStream_t>(stream)));
}

int smla_dsink(const float* lse, const float* delta, const float* sink, int T, int H,
               float* d_sink, void* workspace, size_t workspace_bytes, void* stream) {
    smla_status st = check_shape(T, H, T > 0 ? T : 1, 1);
    if (st != SMLA_OK) return st;
    if (!sink || !d_sink || (T > 0 && (!lse || !delta))) return SMLA_ERR_INVALID_ARG;
    if (!aligned(lse, 4) || !aligned(delta, 4) || !aligned(sink, 4) || !aligned(d_sink, 4) ||
        !aligned(workspace, 4))
        return SMLA_ERR_ALIGN;
    const size_t need = smla_dsink_workspace_bytes(T, H);
    if (workspace == nullptr || workspace_bytes < need) return SMLA_ERR_WORKSPACE;
    const Range all[] = {{lse, (size_t)T * H * 4},
                         {delta, (size_t)T * H * 4},
                         {sink, (size_t)H * 4},
                         {d_sink, (size_t)H * 4},
                         {workspace, need}};
    if ((st = check_ranges(all, 5, 3)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_dsink(lse, delta, sink, T, H, static_cast<float*>(workspace), d_sink,
                                   static_cast<hipStream_t>(stream)));
}

// ---- the has_pe=True variant -------------------------------------------------

size_t smla_bwd_pe_workspace_bytes(int T, int H, int num_kv, int topk, uint32_t flags) {
    if (flags != 0 || check_shape(T, H, num_kv, topk) != SMLA_OK) return 0;
    return pe_layout(T, H, num_kv, topk).total;
}

int smla_fwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                const int32_t* idx, const float* sink, int T, int H, int num_kv, int topk, float scale,
                uint16_t* o, float* lse, void* stream) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (!std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !q_pe || !idx || !o || !lse)) return SMLA_ERR_INVALID_ARG;
    if (!kv || !k_pe) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(q_pe, 16) || !aligned(kv, 16) || !aligned(k_pe, 16) ||
        !aligned(o, 16) || !aligned(idx, 4) || !aligned(lse, 4) || !aligned(sink, 4))
        return SMLA_ERR_ALIGN;
    const size_t qb = (size_t)T * H * kD * 2;
    const Range all[] = {{q, qb},
                         {q_pe, (size_t)T * H * kDP * 2},
                         {kv, (size_t)num_kv * kD * 2},
                         {k_pe, (size_t)num_kv * kDP * 2},
                         {idx, (size_t)T * topk * 4},
                         {sink, sink ? (size_t)H * 4 : 0},
                         {o, qb},
                         {lse, (size_t)T * H * 4}};
    if ((st = check_ranges(all, 8, 6)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;
    return hip_status(launch_fwd_pe(q, q_pe, kv, k_pe, idx, sink, T, H, num_kv, topk, scale, o, lse,
                                    static_cast<hipStream_t>(stream)));
}

int smla_bwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                const uint16_t* dO, const uint16_t* o, const float* lse, const int32_t* idx,
                const float* sink, const float* dlse, int T, int H, int num_kv, int topk, float scale,
                uint32_t flags, uint16_t* dq, uint16_t* dq_pe, uint16_t* dkv, uint16_t* dk_pe,
                float* d_sink, int32_t* n_invalid, void* workspace, size_t workspace_bytes,
                void* stream) {
    smla_status st = check_shape(T, H, num_kv, topk);
    if (st != SMLA_OK) return st;
    if (flags != 0 || !std::isfinite(scale)) return SMLA_ERR_INVALID_ARG;
    if (!kv || !k_pe || !dkv || !dk_pe) return SMLA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !q_pe || !dO || !o || !lse || !idx || !dq || !dq_pe)) return SMLA_ERR_INVALID_ARG;
    if ((sink == nullptr) != (d_sink == nullptr)) return SMLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(q_pe, 16) || !aligned(kv, 16) || !aligned(k_pe, 16) ||
        !aligned(dO, 16) || !aligned(o, 16) || !aligned(dq, 16) || !aligned(dq_pe, 16) ||
        !aligned(dkv, 16) || !aligned(dk_pe, 16) || !aligned(lse, 4) || !aligned(idx, 4) ||
        !aligned(sink, 4) || !aligned(dlse, 4) || !aligned(d_sink, 4) || !aligned(n_invalid, 4) ||
        !aligned(workspace, 16))
        return SMLA_ERR_ALIGN;
    const PeLayout L = pe_layout(T, H, num_kv, topk);
    if (workspace == nullptr || workspace_bytes < L.total) return SMLA_ERR_WORKSPACE;
    const size_t qb = (size_t)T * H * kD * 2, pb = (size_t)T * H * kDP * 2;
    const size_t hb = (size_t)H * 4;
    const Range all[] = {{q, qb},
                         {q_pe, pb},
                         {kv, (size_t)num_kv * kD * 2},
                         {k_pe, (size_t)num_kv * kDP * 2},
                         {dO, qb},
                         {o, qb},
                         {lse, (size_t)T * H * 4},
                         {idx, (size_t)T * topk * 4},
                         {sink, sink ? hb : 0},
                         {dlse, dlse ? (size_t)T * H * 4 : 0},
                         {dq, qb},
                         {dq_pe, pb},
                         {dkv, (size_t)num_kv * kD * 2},
                         {dk_pe, (size_t)num_kv * kDP * 2},
                         {d_sink, d_sink ? hb : 0},
                         {n_invalid, n_invalid ? 4u : 0u},
                         {workspace, L.total}};
    if ((st = check_ranges(all, 17, 10)) != SMLA_OK) return st;
    if ((st = check_arch()) != SMLA_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const BwdLayout& B = L.base;
    float* delta = reinterpret_cast<float*>(ws + B.delta);
    uint16_t* dsp = reinterpret_cast<uint16_t*>(ws + B.dsp);
    uint16_t* interm = reinterpret_cast<uint16_t*>(ws + B.interm);
    uint16_t* interm_pe = reinterpret_cast<uint16_t*>(ws + L.interm_pe);
    int32_t* row_ptr = reinterpret_cast<int32_t*>(ws + B.row_ptr);
    int32_t* slots = reinterpret_cast<int32_t*>(ws + B.slots);
    const int64_t M = (int64_t)T * topk;
    const CsrScratch cs = csr_carve(ws + B.csr, M, num_kv);
    const GatherScratch gs = gather_carve(ws + B.gather, M, num_kv);
    float* dsink_part = reinterpret_cast<float*>(ws + B.dsink);
    float* pe_partial = reinterpret_cast<float*>(ws + L.gather_pe);

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_side_mu);
    bool cap_err = false;
    SideStream* side = side_for(s, dev, &cap_err);
    if (cap_err) return SMLA_ERR_HIP;
    // the same stage order and helper-stream use as smla_bwd, plus the
    // positional intermediate and its gather
    hipStream_t aux = side != nullptr ? side->s : s;
    if (side != nullptr) {
        if (hipEventRecord(side->fork, s) != hipSuccess ||
            hipStreamWaitEvent(aux, side->fork, 0) != hipSuccess)
            return SMLA_ERR_HIP;
    }
    if (launch_csr(idx, M, num_kv, cs, row_ptr, slots, n_invalid, aux) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_gather_plan(row_ptr, M, num_kv, gs, aux) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_delta(o, dO, dlse, (int64_t)T * H, delta, s) != hipSuccess) return SMLA_ERR_HIP;
    if (sink != nullptr) {
        if (side != nullptr && (hipEventRecord(side->after_delta, s) != hipSuccess ||
                                hipStreamWaitEvent(aux, side->after_delta, 0) != hipSuccess))
            return SMLA_ERR_HIP;
        if (launch_dsink(lse, delta, sink, T, H, dsink_part, d_sink, aux) != hipSuccess)
            return SMLA_ERR_HIP;
    }
    if (side != nullptr && hipEventRecord(side->join, aux) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_dq_pe(q, q_pe, kv, k_pe, dO, lse, delta, idx, T, H, num_kv, topk, scale, dq, dq_pe, dsp, s) !=
        hipSuccess)
        return SMLA_ERR_HIP;
    // one pass over the dS/P blocks forms both intermediates
    if (launch_interm_fused_pe(q, dO, q_pe, dsp, idx, T, H, num_kv, topk, interm, interm_pe, s) != hipSuccess)
        return SMLA_ERR_HIP;
    if (side != nullptr && hipStreamWaitEvent(s, side->join, 0) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_gather_sum(interm, row_ptr, slots, M, num_kv, gs, dkv, s) != hipSuccess) return SMLA_ERR_HIP;
    if (launch_gather_pe(interm_pe, row_ptr, slots, M, num_kv, gs, pe_partial, dk_pe, s) != hipSuccess)
        return SMLA_ERR_HIP;
    return SMLA_OK;
}

}  // extern "C"
