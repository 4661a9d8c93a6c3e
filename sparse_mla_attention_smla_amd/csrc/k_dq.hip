// dQ kernel of the sparse MLA backward (also emits scale*dS and P per slot).
//
// Page: aiter PR 4766 "Sparse MLA training backward", Structure table, "dQ"
// row: the gathered kv rows are read from LDS once and feed both the S and dP
// products; the kernel also writes this pass's dS and P.
//
// Work unit: one query token t and a group of 64 heads (the last group of a
// token padded when H is not a multiple of 64), walked by persistent
// workgroups of producer and consumer waves (below).  The token's valid slots
// are compacted and streamed in tiles of 32 kv rows copied straight into an
// LDS ring:
//   S^T, dP^T [32 slots x 16 heads] = kv_tile . {q, dO}^T     (MFMA, reduce d=512)
//   P  = exp(scale*S - lse)
//   dS = P * (dP - delta)
//   dq^T [512 x 16 heads] += kv_tile^T . (scale*dS)^T           (MFMA, reduce 32 slots)
// The S^T accumulator leaves each lane with one head and 8 slots, which is
// exactly the B-operand layout of the second product: no data exchange.
//
// The same stream and roles also run the forward (smla_k7_fwd_pc*), with an
// online softmax in place of the gradient.  Page, Contract section: the
// forward's lse is sink-inclusive (the sink enters the running max and sum
// once, before lse = max + ln(sum)) and the sink carries no value vector.
//
// dsp layout (consumed by the intermediate kernel): for token t and compacted
// tile c (c < ceil(topk/32)), a block of 2H x 32 bf16 values at
// ((t*ceil(topk/32) + c)*2H)*32: rows 0..H-1 hold scale*dS of head h, rows
// H..2H-1 hold P, for the 32 slots of the tile (zeros past the last valid
// slot).  Each 16-row chunk is 64 pieces of 8 values in MFMA lane order:
// piece g*16 + r%16 holds slots 4g..4g+3 and 16+4g..16+4g+3 of row r.
#include <type_traits>

#include "kv_tile.hpp"
#include "smla_launch.hpp"

namespace smla {

// Items of one persistent workgroup: ids lo + r * G below n_items, r < count.
// The items are dealt in rounds of G consecutive ids.  With a grid that is a
// multiple of 8, workgroup b runs on XCD b % 8 (blocks are dealt to the XCDs
// in turn) and gets id (b % 8) * G/8 + b / 8 of every round: each XCD works on
// neighbouring items (their tokens share kv rows in that XCD's L2), and every
// XCD sees every part of the token range (balanced work).  All workgroups walk
// the rounds in the same order, so the whole grid stays on one stretch of
// tokens at a time (starting workgroups at staggered rounds, to spread their
// item switches, was measured about 1% slower: it spreads the kv rows in use).
struct ItemSeq {
    int lo, step, n;
    __device__ ItemSeq(int b, int G, int n_items) {
        const bool xcd = (G & 7) == 0;
        lo = xcd ? (b & 7) * (G >> 3) + (b >> 3) : b;
        step = G;
        n = lo < n_items ? (n_items - lo + G - 1) / G : 0;
    }
    __device__ int count() const { return n; }
    __device__ int item(int r) const { return lo + r * step; }
};

// Persistent producer/consumer kernels over 64-head groups: one 512-thread
// workgroup per CU walks its items (token, 64 heads; when H is not a multiple
// of 64, the last group of each token is padded, see PAD below); an item is
// cut into segments of up to 512 index slots.  Waves w and w+4 share a SIMD
// (measured on gfx950 from HW_ID), so each SIMD runs one wave of each role:
//   producers (waves 0-3): 16 heads each, q and dO in registers; per tile the
//     S^T, dP^T products, then P and scale*dS (stored as dsp blocks) and the dS
//     fragment, published in LDS;
//   consumers (waves 4-7): all 64 heads x 128 d of the dq accumulator each
//     (every transposed kv read feeds four MFMAs); they also issue every kv
//     row copy, so each explicit vmcnt wait counts only that wave's own copies,
//     warming copies and dq stores.
// Producers run one tile ahead of consumers; one barrier per tile.  The tiles
// of consecutive segments form one stream over the ring (4 tiles deep; 3 in
// the has_pe=True variant, whose positional ring takes the room): while segment
// s ends, the first tiles of segment s+1 are already copied, its slot list
// (double-buffered, built by producer 0 during segment s) is ready, its first tile
// is produced, and for a new item the producers reload q and dO during their
// last tile of the old one.  Segments shorter than kMinStream tiles end with a
// drain and restart instead.
// Both roles run the same segment/tile control flow (same barrier sequence);
// each role is its own instantiation so that only its state occupies registers.
struct DqShared {
    char* tiles;        // ring slots of kTileBytes (kNBuf, or 3 with PE)
    SlotList* Lb;       // [2] slot lists, segment s uses Lb[s & 1]
    u32x4 (*dsfrag)[4][64];  // [2][4][64] dS (forward: P) fragments: [position parity][producer][lane]
    char* touch;             // 1 KiB landing area of the cache-warming copies (never read)
    // forward only, [position parity][producer]: whether the producer moved the
    // reference max of any of its heads at that tile, the factors by which the
    // output accumulators of its 16 heads are rescaled, and at an item's last
    // tile the output scale 1/sum of each head
    int (*resc)[4];
    float (*alpha)[4][16];
    float (*oscale)[4][16];
    char* pe_tiles;     // has_pe=True: ring slots of kPeTileBytes (positional key rows)
    // forward over several index chunks per item, [position parity][producer][lane]:
    // the producer lane's running softmax state after that tile (reference max,
    // its share of the sum); the consumers finish each head from it
    float (*mst)[4][64][2] = nullptr;
};

constexpr int kMinStream = 5;  // segments this long hand over to the next without a drain

// q/dO B fragments.  In the MFMA B layout lane c16 + 16g holds head c16,
// d-chunk g, so the four lanes of a quad name four different rows and the L1
// splits each load into four times as many partial-line accesses (measured on
// gfx950: about 15 B/clk per CU, from L2 too).  The fragments are therefore
// loaded with lane 4*c16 + p holding head c16 (each quad reads 64 contiguous
// bytes of one row: about 50 B/clk) and moved to lane c16 + 16g with one fixed
// lane permutation per register.  Heads 8..15 take their chunks rotated by two
// within the quad (lane 4*c16 + p holds chunk (p + 2) % 4), so that each half
// wave of the permutation reads 32 source lanes that are distinct modulo 32:
// free of LDS bank conflicts (the plain order gives two-way conflicts, about
// 2 extra cycles per permutation, measured).  Reading the registers there
// also makes the compiler complete their loads at that point: registers still
// in flight at a loop's back edge would make it wait, with a vmcnt that also
// covers every earlier store, at the start of each later iteration.
__device__ __forceinline__ int frag_load_lane_row(int lane) { return lane >> 2; }
__device__ __forceinline__ int frag_load_lane_chunk(int lane) { return ((lane & 3) + ((lane >> 4) & 2)) & 3; }

template <int N>
__device__ __forceinline__ void frag_to_mfma_lanes(u32x4 (&r)[N], int lane) {
    // destination lane l = c16 + 16g takes source lane 4*c16 + (g + 2*(c16 >= 8)) % 4
    const int addr = 4 * (4 * (lane & 15) + (((lane >> 4) + ((lane >> 2) & 2)) & 3));
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[i][e] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)r[i][e]);
}

__device__ __forceinline__ void settle_scalars(float a, float b) {
    asm volatile("" : : "v"(a), "v"(b));
}

// FWD selects the forward pass on the same stream: the producers compute only
// S^T and keep an online softmax per head (lse, written at the item's last
// tile); the consumers accumulate O^T = kv^T . P^T and scale it by 1/sum in
// their epilogue.  Then dO, delta and dsp are unused, lse is written (not
// read), dq receives O, and the forward needs one segment per item (topk <= 512).
//
// PE adds the has_pe=True variant's positional part: the producers add
// q_pe . k_pe^T to S^T (two more d-steps per 16-slot half, q_pe fragments in
// registers), the consumers copy each tile's positional key rows into a second
// ring and, in the backward, accumulate dq_pe^T = k_pe^T . (scale*dS)^T (16 of
// its 64 columns each).  The ring is then 3 tiles deep instead of 4 so that
// both rings fit in LDS: the stream only ever holds the consumers' tile, the
// producers' tile and the one being copied.
template <bool PROD, bool FWD, bool PE = false, bool PAD = false, int SPLIT = 0, bool MULTI = false>
__device__ __forceinline__ void dq_pc_role(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                           const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                                           const float* __restrict__ delta, const int32_t* __restrict__ idx,
                                           int T, int H, int N, int K, float scale, uint16_t* __restrict__ dq,
                                           uint16_t* __restrict__ dsp, const DqShared sh, int w, int lane,
                                           const float* __restrict__ sink = nullptr,
                                           float* __restrict__ lse_out = nullptr,
                                           const uint16_t* __restrict__ q_pe = nullptr,
                                           const uint16_t* __restrict__ k_pe = nullptr,
                                           uint16_t* __restrict__ dq_pe = nullptr) {
    constexpr int NB = PE ? 3 : kNBuf;           // ring depth
    constexpr int kAhead = 2;                    // tiles copied ahead of the consumers
    static_assert(NB > kAhead, "the ring holds the consumers', the producers' and the copied tile");
    constexpr int R = kBK / 4 + (PE ? 1 : 0);    // copies per consumer wave per tile
    // MULTI (forward, topk > 512): an item streams through several segments, so
    // no tile is known to be its last when produced; the producers publish their
    // softmax state every tile and the consumers finish each head (output scale,
    // lse) in their epilogue, from the state of the item's last consumed tile
    static_assert(!MULTI || FWD, "several segments per forward item");
    // global stores of one consumer epilogue (4 heads x 8 d-blocks, + 4 of dq_pe,
    // or + 4 of lse)
    constexpr int kEpiStores = 32 + (PE && !FWD ? 4 : 0) + (MULTI ? 4 : 0);
    constexpr int kWarmTiles = 8;   // tiles over which the next item's q/dO are warmed (32 chunks)
    const int c16 = lane & 15, g = lane >> 4;
    auto ring_slot = [](int pos) { return NB == 4 ? (pos & 3) : pos % NB; };
    // PAD: H a multiple of 16 but not of 64; the last group of each token holds
    // H % 64 heads, and the producers whose 16 heads lie past H run on head H-1
    // and store nothing
    const int nhg = PAD ? (H + 63) / 64 : H / 64;
    const ItemSeq seq(blockIdx.x, gridDim.x, T * nhg);
    const int spi = (K + kChunk - 1) / kChunk;   // segments per item
    const int nseg = seq.count() * spi;
    if (nseg == 0) return;  // uniform: the whole workgroup has no item
    const int ntk = (K + kBK - 1) / kBK;
    const uint32_t ring = lds_addr(sh.tiles);
    SlotList* const Lb = sh.Lb;
    auto seg_item = [&](int s) { return seq.item(s / spi); };
    auto seg_k0 = [&](int s) { return (s % spi) * kChunk; };

    // ---------------------------------------------------------------- producer
    u32x4 qf[16], dof[16];
    u32x4 qpf[2];                   // PE: q_pe B fragments (lane c16 + 16g: head c16, chunk g)
    float bias = 0.f, dl = 0.f;     // of the item being produced
    float nbias = 0.f, ndl = 0.f;   // of the next item, loaded with its q/dO
    // forward: bias/nbias hold the head's sink logit in log2 units (-inf: none);
    // online softmax state of this lane's head, in log2 units
    constexpr float kLazy = 8.f;    // the reference max moves only when exceeded by this
    float m_use = -INFINITY;        // reference max the exponents are taken against
    float l_run = 0.f;              // this lane's share of the sum, relative to m_use
    int p_n = 0;                    // valid slots of the segment being produced
    int p_ctg = 0;                  // compacted tiles of the item before that segment
    int p_h = 0;                    // head of this lane
    size_t p_item_row = 0;          // forward: row of lse_out of the wave's first head
    uint16_t* p_blk = dsp;          // dsp block of the item's compacted tile 0
    const float c = scale * kLog2e;
    // PAD: the 16-head blocks of an item's group (1 to 4).  SPLIT (backward,
    // H = 16 * SPLIT, one group of one or two blocks per token): each block gets
    // two producers, each taking one 16-slot half of every tile (the backward's
    // softmax needs no reduction over slots), so all four SIMDs share the work.
    static_assert(SPLIT == 0 || (PAD && !FWD && SPLIT <= 2), "split groups: backward, 16 or 32 heads");
    auto blocks_of = [&](int item) { return min(4, (H - (item % nhg) * 64) >> 4); };
    // the producer's head block of `item` (SPLIT: w / 2)
    auto head_block = [&](int item) { return SPLIT > 0 ? (w >> 1) : w; };
    auto item_rows = [&](int item, int& h, size_t& lrow) {
        const int t = item / nhg, hg = item - t * nhg;
        if constexpr (PAD) {
            h = hg * 64 + head_block(item) * 16 + c16;
            h = h < H ? h : H - 1;
        } else {
            h = hg * 64 + w * 16 + c16;
        }
        lrow = (size_t)t * H + h;
    };
    // PAD: whether this producer's 16 heads of `item` exist (wave-uniform)
    auto wave_active = [&](int item) { return head_block(item) < blocks_of(item); };
    bool p_act = true;              // PAD: of the item being produced
    auto bias_of = [](float l) { return (l == -INFINITY) ? INFINITY : l * kLog2e; };
    auto sink_of = [&](int h) { return sink != nullptr ? sink[h] * kLog2e : -INFINITY; };
    // first element of this lane's load row (lane 4*c16 + g: head c16, chunk g)
    auto frag_src = [&](int item) {
        const int t = item / nhg, hg = item - t * nhg;
        if constexpr (PAD) {
            const int hrow = hg * 64 + head_block(item) * 16 + frag_load_lane_row(lane);
            return ((size_t)t * H + (hrow < H ? hrow : H - 1)) * kD + 8 * frag_load_lane_chunk(lane);
        } else {
            return ((size_t)t * H + hg * 64 + w * 16 + frag_load_lane_row(lane)) * kD +
                   8 * frag_load_lane_chunk(lane);
        }
    };
    // PE: first element of this lane's q_pe fragment (loaded in MFMA order: 2 loads)
    auto pe_src = [&](int item) {
        int h; size_t lrow;
        item_rows(item, h, lrow);
        return lrow * kDP + 8 * g;
    };
    auto load_item = [&](int item) {
        int h; size_t lrow;
        item_rows(item, h, lrow);
        const size_t src = frag_src(item);
#pragma unroll
        for (int ds = 0; ds < 16; ++ds) {
            qf[ds] = *reinterpret_cast<const u32x4*>(q + src + 32 * ds);
            if constexpr (!FWD) dof[ds] = *reinterpret_cast<const u32x4*>(dO + src + 32 * ds);
        }
        if constexpr (PE) {
            const size_t ps = pe_src(item);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) qpf[s2] = *reinterpret_cast<const u32x4*>(q_pe + ps + 32 * s2);
        }
        if constexpr (FWD) {
            nbias = sink_of(h);
        } else {
            nbias = bias_of(lse[lrow]);
            ndl = delta[lrow];
        }
    };
    auto finish_load = [&]() {
        // keep the lane permutation (and the wait for the loads it implies) after
        // everything before it: hoisted into a reload tile's MFMA loop it would
        // stall that loop on the loads' latency
        __builtin_amdgcn_sched_barrier(0);
        frag_to_mfma_lanes(qf, lane);
        if constexpr (!FWD) frag_to_mfma_lanes(dof, lane);
        settle_scalars(nbias, ndl);
        if constexpr (PE) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) asm volatile("" : : "v"(qpf[s2]));
        }
    };
    // forward: lse of the item whose last tile was just produced (or that has no
    // valid slot), with the sink folded in; returns the output scale a/z of the head
    auto finish_softmax = [&]() -> float {
        const float l_tot = sum_over_rows(l_run);
        const float m_fin = fmaxf(m_use, bias);
        float osc = 0.f, lse_v = -INFINITY;
        if (m_fin != -INFINITY) {
            const float a = __builtin_amdgcn_exp2f(m_use - m_fin);
            const float z = l_tot * a + __builtin_amdgcn_exp2f(bias - m_fin);
            osc = a / z;
            lse_v = (m_fin + log2f(z)) * kLn2;
        }
        if (g == 0 && (!PAD || p_act)) lse_out[p_item_row + c16] = lse_v;
        m_use = -INFINITY;
        l_run = 0.f;
        return osc;
    };
    // point the producer at segment s (its slot list must be visible)
    auto enter_segment = [&](int s, bool new_item) {
        const int item = seg_item(s);
        size_t lrow;
        item_rows(item, p_h, lrow);
        if constexpr (PAD) p_act = wave_active(item);
        if (new_item) { bias = nbias; dl = ndl; p_ctg = 0; }
        p_n = Lb[s & 1].n;
        if constexpr (FWD) {
            p_item_row = lrow - c16;
            if constexpr (MULTI) {
                if (new_item) {
                    m_use = -INFINITY;
                    l_run = 0.f;
                }
            } else {
                if (p_n == 0) (void)finish_softmax();   // no valid slot: only lse is written
            }
        } else {
            p_blk = dsp + (size_t)(item / nhg) * ntk * (2 * H) * kBK;
        }
    };
    // S^T, dP^T of tile jt of the producer's segment (ring position pos) -> P,
    // scale*dS (stored) -> dS fragment into LDS.  With RELOAD, each d-chunk of
    // q/dO is replaced by the next item's right after its MFMAs.
    auto produce = [&](int pos, int jt, auto reload, const uint16_t* nq, const uint16_t* nd,
                       const uint16_t* nqp) {
        const char* buf = sh.tiles + ring_slot(pos) * kTileBytes;
        const int rb = rows_base(c16, g);
        f32x4 sacc[2], pacc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            sacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
            pacc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // kv fragments are read two d-chunks ahead of their MFMAs (the schedule
        // is pinned: the compiler's own keeps about one chunk ahead)
        constexpr int PF = 2;
        u32x4 ab[16][2];
#pragma unroll
        for (int ds = 0; ds < PF; ++ds)
#pragma unroll
            for (int st = 0; st < 2; ++st) ab[ds][st] = tile_rows_a(buf, rb, st, ds);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int ds = 0; ds < 16; ++ds) {
            if (ds + PF < 16) {
#pragma unroll
                for (int st = 0; st < 2; ++st) ab[ds + PF][st] = tile_rows_a(buf, rb, st, ds + PF);
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                sacc[st] = mfma16(ab[ds][st], qf[ds], sacc[st]);
                if constexpr (!FWD) pacc[st] = mfma16(ab[ds][st], dof[ds], pacc[st]);
            }
            if (ds + PF < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, FWD ? 2 : 4, 0);
            if constexpr (decltype(reload)::value) {
                qf[ds] = *reinterpret_cast<const u32x4*>(nq + 32 * ds);
                if constexpr (!FWD) dof[ds] = *reinterpret_cast<const u32x4*>(nd + 32 * ds);
            }
        }
        if constexpr (PE) {
            // positional part of S^T, then (reload) the next item's q_pe fragments
            const char* pbuf = sh.pe_tiles + ring_slot(pos) * kPeTileBytes;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int st = 0; st < 2; ++st) sacc[st] = mfma16(pe_rows_a(pbuf, c16, g, st, s2), qpf[s2], sacc[st]);
            if constexpr (decltype(reload)::value) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) qpf[s2] = *reinterpret_cast<const u32x4*>(nqp + 32 * s2);
            }
        }
        if constexpr (FWD) {
            // Online softmax with a lazily moved reference max: exponents are
            // taken against m_use, which moves only when a logit of the head
            // exceeds it by more than kLazy, so P <= 2^kLazy and the consumers
            // rescale their accumulators only at such moves (rare after the first
            // tile).  The lane's 8 logits belong to head c16; the other three
            // lanes of that head are lane ^ 16 and lane ^ 32.
            float x[2][4];
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool v = jt * kBK + 16 * st + 4 * g + i < p_n;
                    x[st][i] = v ? sacc[st][i] * c : -INFINITY;
                    tmax = fmaxf(tmax, x[st][i]);
                }
            tmax = max_over_rows(tmax);
            // every tile holds a valid slot, so tmax is finite and the first tile moves
            const bool move = tmax > m_use + kLazy;
            const float m_new = move ? tmax : m_use;
            const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);   // 1, or 0 from -inf
            const bool rescale = move && m_use != -INFINITY;            // accumulators hold data
            l_run *= alpha;
            m_use = m_new;
            float ps[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ps[st][i] = __builtin_amdgcn_exp2f(x[st][i] - m_use);
                    l_run += ps[st][i];
                }
            const int par = pos & 1;
            const bool any = __ballot(rescale) != 0ull;
            if (any && g == 0) sh.alpha[par][w][c16] = alpha;
            if (lane == 0) sh.resc[par][w] = any ? 1 : 0;
            sh.dsfrag[par][w][lane] =
                u32x4{pack_bf16(ps[0][0], ps[0][1]), pack_bf16(ps[0][2], ps[0][3]),
                      pack_bf16(ps[1][0], ps[1][1]), pack_bf16(ps[1][2], ps[1][3])};
            if constexpr (MULTI) {
                *reinterpret_cast<float2*>(sh.mst[par][w][lane]) = make_float2(m_use, l_run);
            } else if (jt == (p_n + kBK - 1) / kBK - 1) {
                const float osc = finish_softmax();
                if (g == 0) sh.oscale[par][w][c16] = osc;
            }
        } else {
            float dss[2][4], ps[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool v = jt * kBK + 16 * st + 4 * g + i < p_n;
                    const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[st][i], c, -bias)) : 0.f;
                    ps[st][i] = p;
                    dss[st][i] = p * (pacc[st][i] - dl) * scale;
                }
            // dsp pieces of this wave's 16 heads: lane l = c16 + 16g holds the 8
            // slots 4g..4g+3 and 16+4g..16+4g+3 of head c16, which is piece l of
            // the heads' 1 KiB chunk (dsp piece layout), so each store writes
            // 1 KiB contiguously from the MFMA lanes as they are (no permutation)
            uint16_t* blk = p_blk + (size_t)(p_ctg + jt) * (2 * H) * kBK + (size_t)(p_h - c16) * kBK + lane * 8;
            const u32x4 dsv = {pack_bf16(dss[0][0], dss[0][1]), pack_bf16(dss[0][2], dss[0][3]),
                               pack_bf16(dss[1][0], dss[1][1]), pack_bf16(dss[1][2], dss[1][3])};
            if (!PAD || p_act) {
                *reinterpret_cast<u32x4*>(blk) = dsv;
                *reinterpret_cast<u32x4*>(blk + (size_t)H * kBK) =
                    u32x4{pack_bf16(ps[0][0], ps[0][1]), pack_bf16(ps[0][2], ps[0][3]),
                          pack_bf16(ps[1][0], ps[1][1]), pack_bf16(ps[1][2], ps[1][3])};
            }
            sh.dsfrag[pos & 1][w][lane] = dsv;
        }
    };
    // SPLIT: the 16-slot half st = w % 2 of tile jt for the
    // block's 16 heads (the same steps as produce on one half); the dsp pieces and
    // the dS fragment get this half's 8 bytes, the block's other producer the rest
    auto produce_half = [&](int pos, int jt, auto reload, const uint16_t* nq, const uint16_t* nd,
                            const uint16_t* nqp) {
        const int st = w & 1;
        const char* buf = sh.tiles + ring_slot(pos) * kTileBytes;
        const int rb = rows_base(c16, g);
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
        constexpr int PF = 2;
        u32x4 ab[16];
#pragma unroll
        for (int ds = 0; ds < PF; ++ds) ab[ds] = tile_rows_a(buf, rb, st, ds);
        __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
        for (int ds = 0; ds < 16; ++ds) {
            if (ds + PF < 16) ab[ds + PF] = tile_rows_a(buf, rb, st, ds + PF);
            sacc = mfma16(ab[ds], qf[ds], sacc);
            pacc = mfma16(ab[ds], dof[ds], pacc);
            if (ds + PF < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if constexpr (decltype(reload)::value) {
                qf[ds] = *reinterpret_cast<const u32x4*>(nq + 32 * ds);
                dof[ds] = *reinterpret_cast<const u32x4*>(nd + 32 * ds);
            }
        }
        if constexpr (PE) {
            const char* pbuf = sh.pe_tiles + ring_slot(pos) * kPeTileBytes;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) sacc = mfma16(pe_rows_a(pbuf, c16, g, st, s2), qpf[s2], sacc);
            if constexpr (decltype(reload)::value) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) qpf[s2] = *reinterpret_cast<const u32x4*>(nqp + 32 * s2);
            }
        }
        float dss[4], ps[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool v = jt * kBK + 16 * st + 4 * g + i < p_n;
            const float p = v ? __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -bias)) : 0.f;
            ps[i] = p;
            dss[i] = p * (pacc[i] - dl) * scale;
        }
        if (p_act) {
            uint16_t* blk =
                p_blk + (size_t)(p_ctg + jt) * (2 * H) * kBK + (size_t)(p_h - c16) * kBK + lane * 8 + 4 * st;
            const u32x2 dsv = {pack_bf16(dss[0], dss[1]), pack_bf16(dss[2], dss[3])};
            *reinterpret_cast<u32x2*>(blk) = dsv;
            *reinterpret_cast<u32x2*>(blk + (size_t)H * kBK) = u32x2{pack_bf16(ps[0], ps[1]), pack_bf16(ps[2], ps[3])};
            reinterpret_cast<u32x2*>(&sh.dsfrag[pos & 1][w >> 1][lane])[st] = dsv;
        }
    };
    // the tile's producer work
    auto produce_tile = [&](int pos, int jt, auto reload, const uint16_t* nq, const uint16_t* nd,
                            const uint16_t* nqp) {
        if constexpr (SPLIT > 0) produce_half(pos, jt, reload, nq, nd, nqp);
        else produce(pos, jt, reload, nq, nd, nqp);
    };
    using NoReload = std::integral_constant<bool, false>;
    using Reload = std::integral_constant<bool, true>;

    // ---------------------------------------------------------------- consumer
    const int dq4 = w - 4;  // d in [128 dq4, 128 dq4 + 128) (dq_pe: [16 dq4, 16 dq4 + 16))
    const i32x4 rsrc = make_rsrc(kv, (uint32_t)N * (kD * 2));
    const i32x4 rsrc_pe = make_rsrc(k_pe, PE ? (uint32_t)N * kPeRow : 0u);
    const uint32_t pe_ring = lds_addr(PE ? sh.pe_tiles : sh.tiles);
    f32x4 acc[8][4], acc_pe[4];
    if constexpr (!PROD) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) acc_pe[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // consumer wave dq4 copies rows dq4, dq4 + 4, ... of tile ct of a slot list
    // (PE: then positional copy dq4 of the four)
    auto issue = [&](const SlotList* L, int ct, int pos) {
        issue_tile<4>(rsrc, L, ct, ring + ring_slot(pos) * kTileBytes, dq4, lane);
        if constexpr (PE) issue_pe_tile<4>(rsrc_pe, L, ct, pe_ring + ring_slot(pos) * kPeTileBytes, dq4, lane);
    };
    // Cache warming: during a segment's last tiles the consumers read the next
    // item's q and dO rows (64 KiB each, in 4 KiB chunks of 64 lines) into a
    // scratch LDS area, so that the producers' reload of them hits L2/MALL.
    // Every iteration issues exactly one such copy per consumer (a zero-length
    // one when there is nothing to warm), which keeps the vmcnt bounds exact.
    const uint32_t touch_lds = lds_addr(sh.touch);
    auto touch = [&](int item_next, int k) {
        const bool real = item_next >= 0 && k >= 0 && k < (FWD ? 16 : 32);   // forward: q only
        const int it = real ? item_next : 0;
        const int t = it / nhg, hg = it - t * nhg;
        const uint16_t* rows = (k < 16 ? q : dO) + ((size_t)t * H + hg * 64) * kD;
        // PAD: a short last group reads only its own heads (past them: nothing)
        const uint32_t span = PAD ? (uint32_t)min(64, H - hg * 64) * (kD * 2) : 65536u;
        copy_row_to_lds(make_rsrc(rows, real ? span : 0u), touch_lds, (k & 15) * 4096 + lane * 64);
    };
    auto consume = [&](int pos) {
        const int cb = cols_base(c16, g);
        u32x4 b[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) b[m] = sh.dsfrag[pos & 1][m][lane];
        const char* buf = sh.tiles + ring_slot(pos) * kTileBytes;
        // transposed kv reads two d-blocks ahead of their four MFMAs (pinned)
        u32x4 ca[8];
        ca[0] = tile_cols_a(buf, cb, 8 * dq4);
        ca[1] = tile_cols_a(buf, cb, 8 * dq4 + 1);
        if constexpr (FWD) {
            // lane c16 + 16g of acc[.][m] belongs to head 16m + c16: apply the
            // producers' rescale factors before this tile's P is added.  The
            // four flags are one 16-byte read issued with the operand reads
            // above, so the check adds no LDS round trip of its own (reading
            // them first and branching per flag cost the forward 9%).
            const u32x4 rf = *reinterpret_cast<const u32x4*>(sh.resc[pos & 1]);
            if (__builtin_amdgcn_readfirstlane(rf[0] | rf[1] | rf[2] | rf[3])) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (__builtin_amdgcn_readfirstlane(rf[m])) {
                        const float a = sh.alpha[pos & 1][m][c16];
#pragma unroll
                        for (int dt = 0; dt < 8; ++dt) acc[dt][m] *= a;
                    }
                }
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4 + 4, 0);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            if (dt + 2 < 8) ca[dt + 2] = tile_cols_a(buf, cb, 8 * dq4 + dt + 2);
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[dt][m] = mfma16(ca[dt], b[m], acc[dt][m]);
            if (dt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        if constexpr (PE && !FWD) {
            const u32x4 pa = pe_cols_a(sh.pe_tiles + ring_slot(pos) * kPeTileBytes, c16, g, dq4);
#pragma unroll
            for (int m = 0; m < 4; ++m) acc_pe[m] = mfma16(pa, b[m], acc_pe[m]);
        }
    };
    // SPLIT: only the group's head blocks are multiplied
    auto consume_nb = [&](int pos, auto nb_c) {
        constexpr int NBK = decltype(nb_c)::value;   // head blocks of the item
        const int cb = cols_base(c16, g);
        u32x4 b[4];
#pragma unroll
        for (int m = 0; m < NBK; ++m) b[m] = sh.dsfrag[pos & 1][m][lane];
        const char* buf = sh.tiles + ring_slot(pos) * kTileBytes;
        // transposed kv reads two d-blocks ahead of their four MFMAs (pinned)
        u32x4 ca[8];
        ca[0] = tile_cols_a(buf, cb, 8 * dq4);
        ca[1] = tile_cols_a(buf, cb, 8 * dq4 + 1);
        if constexpr (FWD) {
            // lane c16 + 16g of acc[.][m] belongs to head 16m + c16: apply the
            // producers' rescale factors before this tile's P is added.  The
            // four flags are one 16-byte read issued with the operand reads
            // above, so the check adds no LDS round trip of its own (reading
            // them first and branching per flag cost the forward 9%).
            const u32x4 rf = *reinterpret_cast<const u32x4*>(sh.resc[pos & 1]);
            if (__builtin_amdgcn_readfirstlane(rf[0] | rf[1] | rf[2] | rf[3])) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (__builtin_amdgcn_readfirstlane(rf[m])) {
                        const float a = sh.alpha[pos & 1][m][c16];
#pragma unroll
                        for (int dt = 0; dt < 8; ++dt) acc[dt][m] *= a;
                    }
                }
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NBK + 4, 0);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            if (dt + 2 < 8) ca[dt + 2] = tile_cols_a(buf, cb, 8 * dq4 + dt + 2);
#pragma unroll
            for (int m = 0; m < NBK; ++m) acc[dt][m] = mfma16(ca[dt], b[m], acc[dt][m]);
            if (dt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NBK, 0);
        }
        if constexpr (PE && !FWD) {
            const u32x4 pa = pe_cols_a(sh.pe_tiles + ring_slot(pos) * kPeTileBytes, c16, g, dq4);
#pragma unroll
            for (int m = 0; m < NBK; ++m) acc_pe[m] = mfma16(pa, b[m], acc_pe[m]);
        }
    };
    auto consume_any = [&](int pos) {
        if constexpr (SPLIT > 0) consume_nb(pos, std::integral_constant<int, SPLIT>{});
        else consume(pos);
    };
    // lane c16 + 16g holds dq^T rows d = 128dq4 + 16dt + 4g .. +3 of head 16m + c16;
    // stored quad-contiguous (lane 4*c + g writes head 16m + c)
    // Forward: the output is scaled by the producers' 1/sum of the head, published
    // with the item's last tile at position pos_last (-1: the item has no tile).
    auto epilogue = [&](int item, int pos_last) {
        const int t = item / nhg, hg = item - t * nhg;
        // PAD: the stores go through buffer ranges that end at the group's last
        // head, so those of heads past H are dropped by the hardware; they are
        // still issued, which keeps the vmcnt bounds above exact
        __amdgpu_buffer_rsrc_t out_rsrc, pe_rsrc, lse_rsrc;
        if constexpr (MULTI) {
            // the group's lse row; lanes that do not write it store past its end
            const int nh = PAD ? min(64, H - hg * 64) : 64;
            lse_rsrc = __builtin_amdgcn_make_buffer_rsrc(lse_out + (size_t)t * H + hg * 64, (short)0, nh * 4,
                                                         0x00020000);
        }
        if constexpr (PAD) {
            const int nh = min(64, H - hg * 64);
            out_rsrc = __builtin_amdgcn_make_buffer_rsrc(dq + ((size_t)t * H + hg * 64) * kD, (short)0,
                                                         nh * kD * 2, 0x00020000);
            if constexpr (PE && !FWD)
                pe_rsrc = __builtin_amdgcn_make_buffer_rsrc(dq_pe + ((size_t)t * H + hg * 64) * kDP, (short)0,
                                                            nh * kDP * 2, 0x00020000);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int hl = 16 * m + (lane >> 2);   // PAD: head within the group
            const int h = hg * 64 + 16 * m + (lane >> 2);
            uint16_t* out = dq + ((size_t)t * H + h) * kD + 128 * dq4 + 4 * (lane & 3);
            float sc = 0.f;
            if constexpr (FWD && MULTI) {
                // head 16m + c16 of the group: its softmax as the producers left it
                // at the item's last tile (none: empty), with the sink folded in
                float mu = -INFINITY, lt = 0.f;
                if (pos_last >= 0) {
                    const float (*st)[2] = sh.mst[pos_last & 1][m];
                    mu = st[c16][0];
                    lt = (st[c16][1] + st[c16 + 16][1]) + (st[c16 + 32][1] + st[c16 + 48][1]);
                }
                const int hh = hg * 64 + 16 * m + c16;
                const float b = sink != nullptr ? sink[hh < H ? hh : H - 1] * kLog2e : -INFINITY;
                const float m_fin = fmaxf(mu, b);
                float lse_v = -INFINITY;
                if (m_fin != -INFINITY) {
                    const float a = __builtin_amdgcn_exp2f(mu - m_fin);
                    const float z = lt * a + __builtin_amdgcn_exp2f(b - m_fin);
                    sc = a / z;
                    lse_v = (m_fin + log2f(z)) * kLn2;
                }
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), lse_rsrc,
                                                      (dq4 == 0 && g == 0) ? (16 * m + c16) * 4 : 256, 0, 0);
            } else if constexpr (FWD) {
                sc = pos_last >= 0 ? sh.oscale[pos_last & 1][m][c16] : 0.f;
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                f32x4 v = acc[dt][m];
                if constexpr (FWD) v *= sc;
                if constexpr (PAD)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        to_quad_rows(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, lane), out_rsrc,
                        (hl * kD + 128 * dq4 + 4 * (lane & 3) + 16 * dt) * 2, 0, 0);
                else
                    *reinterpret_cast<u32x2*>(out + 16 * dt) =
                        to_quad_rows(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, lane);
                acc[dt][m] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if constexpr (PE && !FWD) {
                // dq_pe^T rows 16dq4 + 4g .. +3 of head 16m + c16, stored quad-contiguous
                uint16_t* op = dq_pe + ((size_t)t * H + h) * kDP + 16 * dq4 + 4 * (lane & 3);
                const f32x4 v = acc_pe[m];
                if constexpr (PAD)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        to_quad_rows(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, lane), pe_rsrc,
                        (hl * kDP + 16 * dq4 + 4 * (lane & 3)) * 2, 0, 0);
                else
                    *reinterpret_cast<u32x2*>(op) =
                        to_quad_rows(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, lane);
                acc_pe[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    // ---------------------------------------------------------------- prologue
    if constexpr (PROD) {
        load_item(seg_item(0));
        finish_load();
    } else {
        if (w == 4) compact_slots(idx + (size_t)(seg_item(0) / nhg) * K, K, N, seg_k0(0), &Lb[0], lane);
    }
    __syncthreads();

    SlotChunk nxt;     // producer 0: index slots of the next segment, loaded early
    int c_last = -1;   // consumer: position of the current item's last consumed tile
    int base = 0;      // stream position of tile 0 of segment s
    bool primed = false;
    int post_epi = 0;  // consumer: iterations whose wait must skip the last epilogue's stores
    int since = 0;     // consumer: iterations since the last restart
    for (int s = 0; s < nseg; ++s) {
        const int n = Lb[s & 1].n;
        const int ntile = (n + kBK - 1) / kBK;
        const bool first_of_item = (s % spi) == 0;
        const bool last_of_item = (s % spi) == spi - 1;
        const bool has_next = s + 1 < nseg;
        const bool next_new_item = has_next && last_of_item;
        const bool cont = has_next && ntile >= kMinStream;
        const int item = seg_item(s);
        if (first_of_item) c_last = -1;
        const int32_t* idx_next = has_next ? idx + (size_t)(seg_item(s + 1) / nhg) * K : idx;
        const int k0_next = has_next ? seg_k0(s + 1) : 0;
        if (!primed) {
            // restart: copy tiles 0 and 1 of s, then produce tile 0
            if constexpr (PROD) {
                enter_segment(s, first_of_item);
            } else {
#pragma unroll
                for (int p = 0; p < kAhead; ++p) issue(&Lb[s & 1], p, base + p);
                wait_vmcnt<R>();
                since = 0;
            }
            __syncthreads();
            if constexpr (PROD) {
                if (ntile > 0) produce_tile(base, 0, NoReload{}, nullptr, nullptr, nullptr);
            }
        }
        for (int j = 0; j < ntile; ++j) {
            const int pos = base + j;
            if constexpr (!PROD) {
                // Tile pos+1 is produced in this iteration unless the stream ends.
                // Its copies were issued in the previous iteration (two tiles ahead
                // of the consumer, one ahead of the producer; a deeper lookahead
                // was measured no faster).  Vector memory ops complete in issue
                // order, so the bound is the count of ops issued after them: that
                // iteration's warming copy (none right after a restart) and, if it
                // ran an epilogue, its dq stores.
                if (j + 1 < ntile || cont) {
                    if (since == 0) wait_vmcnt<0>();
                    else if (post_epi > 0) wait_vmcnt<1 + kEpiStores>();
                    else wait_vmcnt<1>();
                }
            }
            __syncthreads();
            if constexpr (PROD) {
                // producer 0 builds the next segment's slot list: its index loads,
                // issued a tile early, are waited for by compiler-counted stores only
                if (w == 0 && has_next && ntile >= 2) {
                    if (j == 0) load_slot_chunk(idx_next, K, k0_next, nxt, lane);
                    else if (j == 1) build_slot_list(nxt, N, k0_next, &Lb[(s + 1) & 1], lane);
                }
                if (j + 1 < ntile) {
                    if (j + 2 == ntile && cont && next_new_item) {
                        int h; size_t lrow;
                        const int nitem = seg_item(s + 1);
                        item_rows(nitem, h, lrow);
                        const size_t src = frag_src(nitem);
                        produce_tile(pos + 1, j + 1, Reload{}, q + src, dO + src, PE ? q_pe + pe_src(nitem) : nullptr);
                        if constexpr (FWD) {
                            nbias = sink_of(h);
                        } else {
                            nbias = bias_of(lse[lrow]);
                            ndl = delta[lrow];
                        }
                        finish_load();
                    } else {
                        produce_tile(pos + 1, j + 1, NoReload{}, nullptr, nullptr, nullptr);
                    }
                } else if (cont) {
                    if (!next_new_item) p_ctg += ntile;
                    enter_segment(s + 1, next_new_item);
                    if (p_n > 0) produce_tile(pos + 1, 0, NoReload{}, nullptr, nullptr, nullptr);
                }
            } else {
                const int ahead = j + kAhead;
                if (ahead < ntile || !cont) issue(&Lb[s & 1], ahead, pos + kAhead);
                else issue(&Lb[(s + 1) & 1], ahead - ntile, pos + kAhead);
                {
                    const int first = ntile > kWarmTiles + 2 ? ntile - kWarmTiles - 2 : 0;
                    const bool warm = next_new_item && j >= first && j + 2 < ntile;
                    touch(warm ? seg_item(s + 1) : -1, (j - first) * 4 + dq4);
                }
                consume_any(pos);
                c_last = pos;
                if (post_epi > 0) --post_epi;
                ++since;
                if (j + 1 == ntile && last_of_item) {
                    epilogue(item, pos);
                    post_epi = 1;   // the next iteration's wait skips these stores
                }
            }
        }
        if (!cont) {
            // drain, then restart with segment s+1
            if constexpr (PROD) {
                if (next_new_item) {
                    load_item(seg_item(s + 1));
                    finish_load();
                } else if (has_next) {
                    p_ctg += ntile;
                }
            } else {
                if (w == 4 && has_next && ntile < 2) compact_slots(idx_next, K, N, k0_next, &Lb[(s + 1) & 1], lane);
                if (ntile == 0 && last_of_item) epilogue(item, MULTI ? c_last : -1);
                wait_vmcnt<0>();
                post_epi = 0;
            }
            __syncthreads();
            primed = false;
        } else {
            primed = true;
        }
        base += ntile;
    }
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pc(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                   const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                   const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                   int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    static_assert(kNBuf == 4, "the stream assumes a 4-deep ring");
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4) dq_pc_role<true, false>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane);
    else dq_pc_role<false, false>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane);
}

// Forward on the same persistent stream (64-head groups with H % 64 == 0,
// topk <= 512): o and lse for every (token, head).
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pc(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                    int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse) {
    static_assert(kNBuf == 4, "the stream assumes a 4-deep ring");
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    __shared__ __attribute__((aligned(16))) int resc[2][4];
    __shared__ float alpha[2][4][16];
    __shared__ float oscale[2][4][16];
    const DqShared sh{tiles, Lb, dsfrag, touch, resc, alpha, oscale};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                               lane, sink, lse);
    else
        dq_pc_role<false, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                                lane, sink, lse);
}

// has_pe=True variants of the two persistent kernels: 3-deep kv ring plus the
// positional ring (about 131 KiB of LDS).
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pc_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                      const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                      const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                      int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp,
                      const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe,
                      uint16_t* __restrict__ dq_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr, pe_tiles};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, false, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane,
                                      nullptr, nullptr, q_pe, k_pe, dq_pe);
    else
        dq_pc_role<false, false, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane,
                                       nullptr, nullptr, q_pe, k_pe, dq_pe);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pc_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                       int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse,
                       const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    __shared__ __attribute__((aligned(16))) int resc[2][4];
    __shared__ float alpha[2][4][16];
    __shared__ float oscale[2][4][16];
    const DqShared sh{tiles, Lb, dsfrag, touch, resc, alpha, oscale, pe_tiles};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, true, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                                     lane, sink, lse, q_pe, k_pe, nullptr);
    else
        dq_pc_role<false, true, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                                      lane, sink, lse, q_pe, k_pe, nullptr);
}

// The four persistent kernels for head counts that are a multiple of 16 but
// not of 64 (the last group of each token padded to 64 heads, see PAD above):
// the same streams, the same LDS.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pcx(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                    const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                    int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4) dq_pc_role<true, false, false, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane);
    else dq_pc_role<false, false, false, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pcx(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                     const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                     int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    __shared__ __attribute__((aligned(16))) int resc[2][4];
    __shared__ float alpha[2][4][16];
    __shared__ float oscale[2][4][16];
    const DqShared sh{tiles, Lb, dsfrag, touch, resc, alpha, oscale};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, true, false, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh,
                                            w, lane, sink, lse);
    else
        dq_pc_role<false, true, false, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh,
                                             w, lane, sink, lse);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pcx_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                       const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                       int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp,
                       const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe,
                       uint16_t* __restrict__ dq_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr, pe_tiles};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, false, true, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane,
                                            nullptr, nullptr, q_pe, k_pe, dq_pe);
    else
        dq_pc_role<false, false, true, true>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w, lane,
                                             nullptr, nullptr, q_pe, k_pe, dq_pe);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pcx_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                        const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                        int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse,
                        const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    __shared__ __attribute__((aligned(16))) int resc[2][4];
    __shared__ float alpha[2][4][16];
    __shared__ float oscale[2][4][16];
    const DqShared sh{tiles, Lb, dsfrag, touch, resc, alpha, oscale, pe_tiles};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, true, true, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                                           lane, sink, lse, q_pe, k_pe, nullptr);
    else
        dq_pc_role<false, true, true, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh, w,
                                            lane, sink, lse, q_pe, k_pe, nullptr);
}

// Backward for 16 or 32 heads (SPLIT = H / 16): one group per token whose
// head blocks each get two producers, one per 16-slot half of every tile.
template <int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pcs(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                    const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                    const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                    int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp) {
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, false, false, true, SPLIT>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh,
                                                    w, lane);
    else
        dq_pc_role<false, false, false, true, SPLIT>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh,
                                                     w, lane);
}

template <int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k2_dq_pcs_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                       const float* __restrict__ delta, const int32_t* __restrict__ idx, int T, int H,
                       int N, int K, float scale, uint16_t* __restrict__ dq, uint16_t* __restrict__ dsp,
                       const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe,
                       uint16_t* __restrict__ dq_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    const DqShared sh{tiles, Lb, dsfrag, touch, nullptr, nullptr, nullptr, pe_tiles};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, false, true, true, SPLIT>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w,
                                                   lane, nullptr, nullptr, q_pe, k_pe, dq_pe);
    else
        dq_pc_role<false, false, true, true, SPLIT>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, sh, w,
                                                    lane, nullptr, nullptr, q_pe, k_pe, dq_pe);
}

// Forward with topk above one index chunk (several segments per item, MULTI):
// plain and has_pe, with 64-head groups or a padded last group.
template <bool PE, bool PAD>
__device__ __forceinline__ void fwd_pcm_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                                             const int32_t* __restrict__ idx, const float* __restrict__ sink,
                                             int T, int H, int N, int K, float scale, uint16_t* __restrict__ o,
                                             float* __restrict__ lse, const uint16_t* __restrict__ q_pe,
                                             const uint16_t* __restrict__ k_pe, char* tiles, char* pe_tiles) {
    __shared__ SlotList Lb[2];
    __shared__ u32x4 dsfrag[2][4][64];
    __shared__ __attribute__((aligned(16))) char touch[1024];
    __shared__ __attribute__((aligned(16))) int resc[2][4];
    __shared__ float alpha[2][4][16];
    __shared__ float oscale[2][4][16];
    __shared__ __attribute__((aligned(16))) float mst[2][4][64][2];
    const DqShared sh{tiles, Lb, dsfrag, touch, resc, alpha, oscale, pe_tiles, mst};
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < 4)
        dq_pc_role<true, true, PE, PAD, 0, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh,
                                                 w, lane, sink, lse, q_pe, k_pe, nullptr);
    else
        dq_pc_role<false, true, PE, PAD, 0, true>(q, kv, q, nullptr, nullptr, idx, T, H, N, K, scale, o, nullptr, sh,
                                                  w, lane, sink, lse, q_pe, k_pe, nullptr);
}

template <bool PAD>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pcm(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                     const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                     int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) char tiles[kNBuf * kTileBytes];
    fwd_pcm_body<false, PAD>(q, kv, idx, sink, T, H, N, K, scale, o, lse, nullptr, nullptr, tiles, nullptr);
}

template <bool PAD>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void smla_k7_fwd_pcm_pe(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                        const int32_t* __restrict__ idx, const float* __restrict__ sink, int T, int H,
                        int N, int K, float scale, uint16_t* __restrict__ o, float* __restrict__ lse,
                        const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe) {
    __shared__ __attribute__((aligned(16))) char tiles[3 * kTileBytes];
    __shared__ __attribute__((aligned(16))) char pe_tiles[3 * kPeTileBytes];
    fwd_pcm_body<true, PAD>(q, kv, idx, sink, T, H, N, K, scale, o, lse, q_pe, k_pe, tiles, pe_tiles);
}

// Persistent grid: one workgroup per compute unit (its LDS use admits one),
// never more than there are items (token, 64-head group).
static hipError_t persistent_blocks(int T, int H, unsigned* blocks) {
    const int items = T * ((H + 63) / 64);
    int cus = 0;
    const hipError_t e = compute_units(&cus);
    if (e != hipSuccess) return e;
    *blocks = (unsigned)(items < cus ? items : cus);
    return hipSuccess;
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* sink,
                      int T, int H, int N, int K, float scale, uint16_t* o, float* lse,
                      hipStream_t s) {
    if (T == 0) return hipSuccess;
    unsigned blocks = 0;
    const hipError_t e = persistent_blocks(T, H, &blocks);
    if (e != hipSuccess) return e;
    if (K > kChunk) {
        if (H % 64 == 0)
            smla_k7_fwd_pcm<false><<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse);
        else
            smla_k7_fwd_pcm<true><<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse);
    } else if (H % 64 == 0) {
        smla_k7_fwd_pc<<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse);
    } else {
        smla_k7_fwd_pcx<<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse);
    }
    return hipGetLastError();
}


hipError_t launch_dq(const uint16_t* q, const uint16_t* kv, const uint16_t* dO, const float* lse,
                     const float* delta, const int32_t* idx, int T, int H, int N, int K, float scale,
                     uint16_t* dq, uint16_t* dsp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    unsigned blocks = 0;
    const hipError_t e = persistent_blocks(T, H, &blocks);
    if (e != hipSuccess) return e;
    if (H % 64 == 0)
        smla_k2_dq_pc<<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp);
    else if (H == 16)
        smla_k2_dq_pcs<1><<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp);
    else if (H == 32)
        smla_k2_dq_pcs<2><<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp);
    else
        smla_k2_dq_pcx<<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp);
    return hipGetLastError();
}

hipError_t launch_fwd_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                         const int32_t* idx, const float* sink, int T, int H, int N, int K, float scale,
                         uint16_t* o, float* lse, hipStream_t s) {
    if (T == 0) return hipSuccess;
    unsigned blocks = 0;
    const hipError_t e = persistent_blocks(T, H, &blocks);
    if (e != hipSuccess) return e;
    if (K > kChunk) {
        if (H % 64 == 0)
            smla_k7_fwd_pcm_pe<false><<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse, q_pe, k_pe);
        else
            smla_k7_fwd_pcm_pe<true><<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse, q_pe, k_pe);
    } else if (H % 64 == 0) {
        smla_k7_fwd_pc_pe<<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse, q_pe, k_pe);
    } else {
        smla_k7_fwd_pcx_pe<<<blocks, 512, 0, s>>>(q, kv, idx, sink, T, H, N, K, scale, o, lse, q_pe, k_pe);
    }
    return hipGetLastError();
}

hipError_t launch_dq_pe(const uint16_t* q, const uint16_t* q_pe, const uint16_t* kv, const uint16_t* k_pe,
                        const uint16_t* dO, const float* lse, const float* delta, const int32_t* idx, int T,
                        int H, int N, int K, float scale, uint16_t* dq, uint16_t* dq_pe, uint16_t* dsp,
                        hipStream_t s) {
    if (T == 0) return hipSuccess;
    unsigned blocks = 0;
    const hipError_t e = persistent_blocks(T, H, &blocks);
    if (e != hipSuccess) return e;
    if (H % 64 == 0)
        smla_k2_dq_pc_pe<<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, q_pe,
                                                k_pe, dq_pe);
    else if (H == 16)
        smla_k2_dq_pcs_pe<1><<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, q_pe,
                                                    k_pe, dq_pe);
    else if (H == 32)
        smla_k2_dq_pcs_pe<2><<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, q_pe,
                                                    k_pe, dq_pe);
    else
        smla_k2_dq_pcx_pe<<<blocks, 512, 0, s>>>(q, kv, dO, lse, delta, idx, T, H, N, K, scale, dq, dsp, q_pe,
                                                 k_pe, dq_pe);
    return hipGetLastError();
}

}  // namespace smla
