// Balanced single pass: the streaming kernel over equal tile ranges and the
// kernel that merges contexts split between waves.
#pragma once

#include "decode_core.h"
#include "decode_mfma.h"
#include "decode_valu.h"

namespace {

using namespace pkv::dev;

// ---------------------------------------------------------------------------
// Balanced single pass.
//
// Context lengths in a batch vary widely (16 to 8192 tokens in a log-normal
// batch), so one workgroup per sequence, or per fixed-size partition, leaves
// the GPU waiting on the longest items or paying a start-up per item. Here the
// grid is exactly the waves the GPU holds at once. The kv heads are taken in
// groups of hg (as many as a workgroup has waves, 8 or 4, when the head count
// allows, else the largest power of two that divides it), and the units of
// the whole batch, ordered (sequence, head group, block), are cut into R equal
// contiguous ranges, one per group of hg waves of a workgroup: wave i of the
// group reads head i of the head group of each unit, so the group's waves
// stream the same blocks in step and their loads at any moment fall on hg
// adjacent head tiles of one block (runs of hg x 4 KiB instead of scattered
// 4 KiB tiles, which the HBM serves faster). A wave streams its range through
// its tile ring without a break: the ring runs across (sequence, head)
// boundaries. Each run of tiles of one (sequence, kv head) inside a range is a
// segment. A segment
// that covers its whole context writes the output directly; a context split
// over several waves leaves one partial (o / l, m, l) per wave in the
// workspace, and a second, small kernel on the same stream merges them with
// the log-sum-exp rule (the kernel boundary makes the partials visible; a
// merge inside the streaming kernel would need device-wide cache maintenance
// per split, which costs more than the launch).
//
// After a shared-prefix pass (decode_prefix.h), a group member's tiles start
// at the first block after the shared run, a member's context written whole
// by one wave goes to its own partial slot instead of the output, and the
// merge folds the prefix partial in as one more piece.

// Issue-side walker over one wave's tiles, in (sequence, head group, block)
// order with the wave's own head of each group, holding the block ids of the current sequence's table row: the first
// 128 blocks from the window's start stay in registers for the row's other
// heads, later blocks rotate through a second pair of 64-id chunks. A
// sequence's tiles are its blocks jlo .. nblk-1: jlo is 0, or a sliding
// window's first block, or the first block after those a shared-prefix pass
// covers; with kFold, the new token's tile (index nblk) follows them.
struct TileWalk {
    int s, g, j, nblk;   // current tile: sequence, kv head, block; blocks end at nblk
    int jlo, lo;         // first block read, first token attended (sliding window)
    int L;               // tokens of sequence s read from its blocks (kFold: without
                         // the new token's position)
    int has_pre;         // sequence s has a shared-prefix partial
    int64_t a_sg;        // global index of unit (s, g / hg, jlo)
    int chunk;           // sequences 64*chunk .. +63 have their lengths in lens
    int lens;            // per lane: tokens of sequence 64*chunk + lane
    int pres;            // per lane: its leading blocks covered by the prefix pass
    int keeps;           // per lane: its leading shared blocks read through the L2
    int keep;            // sequence s: blocks below this are read with the caching policy
    int news;            // per lane: 1 when its new token is a tile of its own (kFold)
    int nend;            // tiles end at nend: nblk, plus the new token's tile
    int last_id;         // kFold: id of the last block issued (the new token's block)
    int rbase;           // jlo rounded down to 64: row0_* start there
    int row0_a, row0_b;  // ids of blocks rbase .. +63 and +64 .. +127 of row s (per lane)
    int ids_a, ids_b;    // ids of blocks base .. base+127 (per lane, two chunks)
    int base;
};

__device__ __forceinline__ void walk_set_seq(const DecodeParams& p, TileWalk& t, int L, int pre) {
    t.L = L;
    t.nblk = (L + 15) >> 4;
    t.nend = t.nblk;
    t.lo = window_lo(p, L);
    t.jlo = first_block(p, L, pre);
    t.has_pre = pre > 0;
}

__device__ __forceinline__ int walk_row_ids(const DecodeParams& p, const TileWalk& t, int j0,
                                            int lane) {
    const int jj = j0 + lane;
    return jj < t.nblk ? p.block_tables[static_cast<size_t>(t.s) * p.max_blocks + jj] : -1;
}

__device__ __forceinline__ void walk_enter_row(const DecodeParams& p, TileWalk& t, int lane) {
    t.rbase = t.jlo & ~63;
    t.row0_a = walk_row_ids(p, t, t.rbase, lane);
    t.row0_b = walk_row_ids(p, t, t.rbase + 64, lane);
    t.base = t.j & ~63;
    t.ids_a = t.base == t.rbase ? t.row0_a : walk_row_ids(p, t, t.base, lane);
    t.ids_b = t.base == t.rbase ? t.row0_b : walk_row_ids(p, t, t.base + 64, lane);
}

// Block id of the current tile.
__device__ __forceinline__ int walk_id(const DecodeParams& p, TileWalk& t, int lane) {
    if (t.j >= t.base + 64) {  // blocks of a segment are walked in increasing order
        t.base += 64;
        t.ids_a = t.ids_b;
        t.ids_b = walk_row_ids(p, t, t.base + 64, lane);
    }
    return __builtin_amdgcn_readlane(t.ids_a, t.j - t.base);
}

// Step to the next tile. kPre: sequences may begin after shared-prefix blocks;
// kKeep: sequences have leading shared blocks read through the L2; kFold: a
// sequence's new token is one more tile after its blocks.
template <bool kPre, bool kKeep, bool kFold>
__device__ __forceinline__ void walk_advance(const DecodeParams& p, TileWalk& t, int lane) {
    if (++t.j < t.nend) return;
    t.j = t.jlo;
    t.a_sg += t.nend - t.jlo;
    // same row, the wave's head of the next group: its first 128 blocks are at hand
    if ((t.g += p.head_group) < p.num_kv_heads) {
        t.base = t.rbase;
        t.ids_a = t.row0_a;
        t.ids_b = t.row0_b;
        return;
    }
    t.g &= p.head_group - 1;  // the wave's head of the first group (hg is a power of 2)
    // Next sequence with tokens. A wave's range ends at or before the batch's
    // last tile, so a later non-empty sequence exists; the bound only keeps s
    // inside the batch should the lengths change under a running kernel.
    do {
        ++t.s;
        if ((t.s >> 6) != t.chunk) {
            t.chunk = t.s >> 6;
            const int jj = t.chunk * 64 + lane;
            t.lens = jj < p.num_seqs ? seq_tokens(p, jj) : 0;
            t.pres = kPre && jj < p.num_seqs ? pre_of(p, jj) : 0;
            if constexpr (kKeep) t.keeps = jj < p.num_seqs ? keep_of(p, jj) : 0;
            if constexpr (kFold) t.news = jj < p.num_seqs ? new_of(p, jj) : 0;
        }
        walk_set_seq(p, t, __builtin_amdgcn_readlane(t.lens, t.s & 63),
                     __builtin_amdgcn_readlane(t.pres, t.s & 63));
        if constexpr (kKeep) t.keep = __builtin_amdgcn_readlane(t.keeps, t.s & 63);
        if constexpr (kFold) {
            const int nt = __builtin_amdgcn_readlane(t.news, t.s & 63);
            t.nend = t.nblk + nt;
            t.L -= nt;
        }
    } while (t.jlo >= t.nblk && t.s + 1 < p.num_seqs);
    t.j = t.jlo;
    walk_enter_row(p, t, lane);
}

// Ring-slot description of an issued tile (all wave-uniform, packed: a ring
// of them lives in scalar registers beside the kernel's pointers).
struct SlotInfo {
    // The tile's attended tokens [nlo, nvalid) (nvalid 0 past the range) in
    // bits 0-4 and 5-9, then the flags below.
    int bits;
    int s, g;   // its segment's sequence and kv head
    int vslot;  // a new token's tile: its slot, block id * 16 + position
                // (-1: another tile, or no slot to store to)
    static constexpr int kFirst = 1 << 10;   // first tile of a segment
    static constexpr int kLast = 1 << 11;    // last tile of a segment
    static constexpr int kHasPre = 1 << 12;  // its sequence has a shared-prefix partial
    static constexpr int kWhole = 1 << 13;   // the segment is its context's every tile
    static constexpr int kSlot1 = 1 << 14;   // a split context's piece that began in this range
    __device__ int nvalid() const { return bits & 31; }
    __device__ int nlo() const { return (bits >> 5) & 31; }
};

template <int D>
struct SlotGeoB {
    static constexpr int kStride = D + 4;  // floats per (wave, slot, head): o[D], m, l, pad
};

// Vector-ALU math for one query head per kv head (16-bit caches).
template <int KV, int D>
struct ValuMath {
    using Gm = Geo<KV, D>;
    static constexpr int kG = 1;
    static constexpr bool kPrefetchQ = true;  // q is small: ride in the ring with its tile
    static constexpr bool kSplit = false;     // the tile math is one piece (consume)
    static constexpr bool kLds = false;       // the ring is NBUF tiles of registers
    static constexpr int kEpl = Gm::kEpl, kLpt = Gm::kLpt, kNld = Gm::kNld, kTB = Gm::kTileBytes;
    using TileT = Tile<KV, D>;
    using QT = QSlice<KV, D>;
    struct State {
        SoftmaxState<KV, D, 1> st;
    };

    __device__ static void fetch_q(const DecodeParams& p, QT& q, int s, int g, int lane) {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                               (static_cast<size_t>(s) * p.num_q_heads + g) * D;
        load_q<KV, KV, D>(q, qrow, lane % kLpt);
    }
    __device__ static void fetch_q_lds(const DecodeParams&, State&, int, int, int) {}
    // kept: the tile is shared with other sequences of the batch; load it with
    // the caching policy so that their reads of it can hit the L2.
    __device__ static void issue(TileT& t, const TileRef& r, int lane, bool kept = false) {
        if (kept) {
#pragma unroll
            for (int i = 0; i < kNld; ++i) t.k[i] = rsrc_load16_kept(r.k, lane * 16 + i * 1024);
#pragma unroll
            for (int i = 0; i < kNld; ++i) t.v[i] = rsrc_load16_kept(r.v, lane * 16 + i * 1024);
            return;
        }
#pragma unroll
        for (int i = 0; i < kNld; ++i) t.k[i] = rsrc_load16(r.k, lane * 16 + i * 1024);
#pragma unroll
        for (int i = 0; i < kNld; ++i) t.v[i] = rsrc_load16(r.v, lane * 16 + i * 1024);
    }
    // A new token's tile holds the token in row 0 (lanes 0 .. D/8 - 1 of load
    // 0, 16 bytes each, for K and for V): store it to the slot row at dst.
    __device__ static void store_new(const DecodeParams& p, const TileT& t, int64_t dst,
                                     int lane) {
        if (lane >= 2 * D / 16) return;
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.k_plane) + dst + lane * 16) = t.k[0];
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.v_plane) + dst + lane * 16) = t.v[0];
    }
    __device__ static void reset(State& x) {
        x.st.m[0] = -INFINITY;
        x.st.l[0] = 0.0f;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) x.st.o[0][e] = 0.0f;
    }
    template <bool kPartial>
    __device__ static void consume(State& x, const TileT& t, int nvalid, int nlo, const QT& q,
                                   float sscale, int lane) {
        const QT qs[1] = {q};
        consume_tile<KV, D, 1, kPartial>(x.st, t, nvalid, nlo, qs, sscale, lane / kLpt);
    }
    // Merge the rows of the wave; afterwards lanes of row 0 hold dims
    // col*EPL .. +EPL, and every lane holds m and l.
    __device__ static void finish(State& x) {
#pragma unroll
        for (int off = kLpt; off < 64; off <<= 1) {
            const float m2 = __shfl_xor(x.st.m[0], off);
            const float l2 = __shfl_xor(x.st.l[0], off);
            const float mx = fmaxf(x.st.m[0], m2);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            const float a = fast_exp2(x.st.m[0] - ms), b = fast_exp2(m2 - ms);
            x.st.l[0] = x.st.l[0] * a + l2 * b;
#pragma unroll
            for (int e = 0; e < kEpl; ++e) {
                const float o2 = __shfl_xor(x.st.o[0][e], off);
                x.st.o[0][e] = x.st.o[0][e] * a + o2 * b;
            }
            x.st.m[0] = mx;
        }
    }
    __device__ static void store_out(const DecodeParams& p, const State& x, int s, int g, int lane) {
        if (lane >= kLpt) return;
        const float inv = x.st.l[0] > 0.0f ? 1.0f / x.st.l[0] : 0.0f;
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) +
                                              (static_cast<size_t>(s) * p.num_q_heads + g) * D +
                                              lane * kEpl);
#pragma unroll
        for (int e = 0; e < kEpl / 8; ++e) {
            uint32_t wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wv[i] = pack2<KV>(x.st.o[0][8 * e + 2 * i] * inv, x.st.o[0][8 * e + 2 * i + 1] * inv);
            dst[e] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
    __device__ static void store_partial(float* slot, const State& x, int lane) {
        if (lane >= kLpt) return;
        const float inv = x.st.l[0] > 0.0f ? 1.0f / x.st.l[0] : 0.0f;
        float4* dst = reinterpret_cast<float4*>(slot + lane * kEpl);
#pragma unroll
        for (int e = 0; e < kEpl / 4; ++e)
            dst[e] = make_float4(x.st.o[0][4 * e] * inv, x.st.o[0][4 * e + 1] * inv,
                                 x.st.o[0][4 * e + 2] * inv, x.st.o[0][4 * e + 3] * inv);
        if (lane == 0) {
            slot[D] = x.st.m[0];
            slot[D + 1] = x.st.l[0];
        }
    }
};

// The same math with the tile ring in LDS: two slots per wave, filled by
// direct buffer-to-LDS loads (no registers held for tiles in flight) and read
// into one register tile when consumed.
template <int KV, int D>
struct ValuLdsMath : ValuMath<KV, D> {
    using Base = ValuMath<KV, D>;
    static constexpr bool kLds = true;
    static constexpr int kNld = Base::kNld, kTB = Base::kTB;
    static constexpr int kSlotBytes = 2 * kTB;  // K, then V
    // Loads of one tile into a slot: 2 * kNld, the count the waits below rely on.
    __device__ static void issue_lds(uint8_t* slot, const TileRef& r, int lane, bool kept) {
        typedef __attribute__((address_space(3))) void* lds_ptr;
        // The slot's earlier reads must have completed: the refill's LDS writes
        // do not queue behind this wave's own LDS reads.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        if (kept) {
#pragma unroll
            for (int i = 0; i < kNld; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k, (lds_ptr)(slot + i * 1024), 16,
                                                         lane * 16 + i * 1024, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < kNld; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r.v, (lds_ptr)(slot + kTB + i * 1024), 16,
                                                         lane * 16 + i * 1024, 0, 0, 0);
            return;
        }
#pragma unroll
        for (int i = 0; i < kNld; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k, (lds_ptr)(slot + i * 1024), 16,
                                                     lane * 16 + i * 1024, 0, 0, kStreamPolicy);
#pragma unroll
        for (int i = 0; i < kNld; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r.v, (lds_ptr)(slot + kTB + i * 1024), 16,
                                                     lane * 16 + i * 1024, 0, 0, kStreamPolicy);
    }
    // The slot's tile into registers. The other slot's 2 * kNld loads were
    // issued after this slot's, and a wave's loads complete in order: once at
    // most 2 * kNld operations are outstanding, this slot's loads have landed
    // (stores and other loads issued in between only make the wait longer).
    __device__ static void read_slot(typename Base::TileT& t, const uint8_t* slot, int lane) {
        static_assert(2 * kNld < 16, "vmcnt field");
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kNld));  // vmcnt(2 * kNld)
#pragma unroll
        for (int i = 0; i < kNld; ++i)
            t.k[i] = *reinterpret_cast<const uint4*>(slot + i * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < kNld; ++i)
            t.v[i] = *reinterpret_cast<const uint4*>(slot + kTB + i * 1024 + lane * 16);
    }
};

// Matrix-core math for G grouped query heads (16-bit caches).
template <int KV, int D, int G>
struct MfmaMath {
    using Gm = MfmaGeo<D>;
    static constexpr int kG = G;
    static constexpr bool kPrefetchQ = false;  // fetched into LDS at segment start
    // The tile math comes in two halves (front reads the tile's registers,
    // back does the softmax and PV from LDS), so the ring slot is refilled
    // between them.
    static constexpr bool kSplit = true;
    static constexpr bool kLds = false;
    static constexpr int kNk = Gm::kNk, kNv = Gm::kNv, kNd = Gm::kNd, kTB = Gm::kTileBytes;
    static constexpr int kQBytes = kNk * 1024;  // Q^T operand of one wave in LDS
    using TileT = MfmaTile<D>;
    struct QT {  // the operand lives in LDS (QLds); nothing rides in the ring
    };
    struct State {
        f32x4_t o[Gm::kNd];
        float m, lsum;
        uint8_t* stage;
        uint8_t* qlds;
        uint8_t* kst;  // K stage: tiles are loaded in their natural layout
    };

    __device__ static void fetch_q(const DecodeParams&, QT&, int, int, int) {}
    // Q^T operand of (s, g) into the wave's LDS: head hl (zeros for the
    // padding heads; they read head G-1, always inside q), dims 32c + 8*kg.
    __device__ static void fetch_q_lds(const DecodeParams& p, State& x, int s, int g, int lane) {
        const int hl = lane & 15, kg = lane >> 4;
        const int hq = g * G + min(hl, G - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(p.q) + (static_cast<size_t>(s) * p.num_q_heads + hq) * D;
        uint4 v[kNk];
#pragma unroll
        for (int c = 0; c < kNk; ++c) v[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * kg);
#pragma unroll
        for (int c = 0; c < kNk; ++c)
            *reinterpret_cast<uint4*>(x.qlds + c * 1024 + lane * 16) =
                hl < G ? v[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    // K and V in their natural layout: each load is 1 KiB of the tile.
    __device__ static void issue(TileT& t, const TileRef& r, int lane, bool kept = false) {
        if (kept) {  // shared with other sequences: the caching policy (see ValuMath)
#pragma unroll
            for (int c = 0; c < kNk; ++c) t.k[c] = rsrc_load16_kept(r.k, lane * 16 + 1024 * c);
#pragma unroll
            for (int i = 0; i < kNv; ++i) t.v[i] = rsrc_load16_kept(r.v, lane * 16 + 1024 * i);
            return;
        }
#pragma unroll
        for (int c = 0; c < kNk; ++c) t.k[c] = rsrc_load16(r.k, lane * 16 + 1024 * c);
#pragma unroll
        for (int i = 0; i < kNv; ++i) t.v[i] = rsrc_load16(r.v, lane * 16 + 1024 * i);
    }
    // A new token's tile holds the token in row 0: lanes 0 .. D/8 - 1 of load
    // 0, 16 bytes each, for K and for V. Store it to the slot row at dst.
    __device__ static void store_new(const DecodeParams& p, const TileT& t, int64_t dst,
                                     int lane) {
        if (lane >= Gm::kRowBytes / 16) return;
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.k_plane) + dst + lane * 16) = t.k[0];
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.v_plane) + dst + lane * 16) = t.v[0];
    }
    __device__ static void reset(State& x) {
#pragma unroll
        for (int j = 0; j < kNd; ++j) x.o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        x.m = -INFINITY;
        x.lsum = 0.0f;
    }
    template <bool kPartial>
    __device__ static void consume(State& x, const TileT& t, int nvalid, int nlo, const QT&,
                                   float sscale, int lane) {
        mfma_consume<KV, D, kPartial>(t, nvalid, nlo, QLds<D>{x.qlds}, x.o, x.m, x.lsum, sscale,
                                      x.stage, lane, x.kst);
    }
    template <bool kPartial>
    __device__ static f32x4_t front(State& x, const TileT& t, int nvalid, int nlo, int lane) {
        return mfma_front<KV, D, kPartial>(t, nvalid, nlo, QLds<D>{x.qlds}, x.stage, lane, x.kst);
    }
    template <bool kPartial>
    __device__ static void back(State& x, f32x4_t sacc, int nvalid, int nlo, float sscale,
                                int lane) {
        mfma_back<KV, D, kPartial>(sacc, nvalid, nlo, x.o, x.m, x.lsum, sscale, x.stage, lane);
    }
    __device__ static void finish(State& x) {
        x.lsum += __shfl_xor(x.lsum, 16);
        x.lsum += __shfl_xor(x.lsum, 32);
    }
    __device__ static void store_out(const DecodeParams& p, const State& x, int s, int g, int lane) {
        const int hl = lane & 15, kg = lane >> 4;
        if (hl >= G) return;
        const float inv = x.lsum > 0.0f ? 1.0f / x.lsum : 0.0f;
        uint16_t* dst = static_cast<uint16_t*>(p.out) +
                        (static_cast<size_t>(s) * p.num_q_heads + g * G + hl) * D + 4 * kg;
#pragma unroll
        for (int j = 0; j < kNd; ++j)
            *reinterpret_cast<uint2*>(dst + 16 * j) =
                make_uint2(pack2<KV>(x.o[j][0] * inv, x.o[j][1] * inv),
                           pack2<KV>(x.o[j][2] * inv, x.o[j][3] * inv));
    }
    __device__ static void store_partial(float* slot, const State& x, int lane) {
        const int hl = lane & 15, kg = lane >> 4;
        if (hl >= G) return;
        float* hs = slot + hl * SlotGeoB<D>::kStride;
        const float inv = x.lsum > 0.0f ? 1.0f / x.lsum : 0.0f;
#pragma unroll
        for (int j = 0; j < kNd; ++j)
            *reinterpret_cast<float4*>(hs + 16 * j + 4 * kg) =
                make_float4(x.o[j][0] * inv, x.o[j][1] * inv, x.o[j][2] * inv, x.o[j][3] * inv);
        if (kg == 0) {
            hs[D] = x.m;
            hs[D + 1] = x.lsum;
        }
    }
};

// kPre: a shared-prefix pass covered the leading blocks of some sequences
// (pre_blocks); without it that bookkeeping is compiled out, so its registers
// cost the other forms nothing.
// kKeep: some sequences begin with blocks that others of the batch share
// (keep_blocks); those are loaded with the caching policy. kFold (fold_new):
// a sequence's new token is one more tile of its context, read from the
// source rows (16 bytes per lane of row 0; the other rows lie past the end of
// the row's buffer descriptor and read as zeros), attended with weight like
// any token and stored to its slot by the wave that reads it. The context's
// blocks are read without that position (another wave may be storing it).
// Waves per workgroup of the streaming kernel, and so its largest head group:
// eight for the vector math (7B layer, 32 heads: 325.5 against 326.7 us per
// call with four), four for the matrix cores (GQA batch, 8 kv heads: 139.7
// against 140.7 us with eight).
template <class M>
constexpr int balanced_wpg() {
    return M::kG == 1 ? 8 : 4;
}

template <class M, int KV, int D, int NBUF, bool kPre = false, bool kKeep = false,
          bool kFold = false>
__global__ __launch_bounds__(balanced_wpg<M>() * 64, 8 / balanced_wpg<M>()) void
decode_balanced_kernel(const DecodeParams p) {
    constexpr int WPG = balanced_wpg<M>();
    static_assert(!(kPre && kKeep), "one shared-prefix form at a time");
    constexpr int G = M::kG;
    constexpr int SS = SlotGeoB<D>::kStride;
    const int lane = threadIdx.x & 63;
    const int wv_in = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x * WPG + wv_in;
    const int hg = p.head_group, hs = __builtin_ctz(hg);  // hg is 1, 2, 4 or 8
    const int rk = w >> hs, gi = w & (hg - 1);  // the wave's range, its head in each group
    const int W = p.num_waves >> hs;            // ranges the launch can hold

    // Total units (tiles of a head group) of the batch, then this group's range [t0, t1).
    int64_t total = 0;
    for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {
        const int jj = c0 + lane;
        total += wave_sum(jj < p.num_seqs ? pass_tiles(p, seq_tokens(p, jj),
                                                      kPre ? pre_of(p, jj) : 0) +
                                                (kFold ? new_of(p, jj) : 0)
                                          : 0);
    }
    total *= p.num_kv_heads >> hs;
    // R non-empty ranges: with fewer units than ranges the surplus waves idle,
    // so every wave of a split context really holds a piece of it.
    const int R = static_cast<int>(total < W ? total : W);
    if (rk >= R) return;
    const int64_t t0 = range_start(total, rk, R);
    const int64_t t1 = range_start(total, rk + 1, R);
    const int n = static_cast<int>(t1 - t0);

    // Locate unit t0: the sequence holding it, then its head group and block.
    TileWalk tw;
    bool found = false;
    {
        int64_t carry = 0;
        for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {  // t0 < total: some chunk holds it
            const int jj = c0 + lane;
            const int len = jj < p.num_seqs ? seq_tokens(p, jj) : 0;
            const int pre = kPre && jj < p.num_seqs ? pre_of(p, jj) : 0;
            const int news = kFold && jj < p.num_seqs ? new_of(p, jj) : 0;
            const int tiles = (pass_tiles(p, len, pre) + news) * (p.num_kv_heads >> hs);
            const int incl = wave_incl_scan(tiles, lane);
            const uint64_t hit = __ballot(jj < p.num_seqs && carry + incl > t0);
            if (hit) {
                const int ln = __builtin_ffsll(static_cast<long long>(hit)) - 1;
                tw.s = c0 + ln;
                tw.chunk = c0 >> 6;
                tw.lens = len;
                tw.pres = pre;
                walk_set_seq(p, tw, __builtin_amdgcn_readlane(len, ln),
                             __builtin_amdgcn_readlane(pre, ln));
                if constexpr (kKeep) {
                    tw.keeps = jj < p.num_seqs ? keep_of(p, jj) : 0;
                    tw.keep = __builtin_amdgcn_readlane(tw.keeps, ln);
                }
                if constexpr (kFold) {
                    tw.news = news;
                    const int nt = __builtin_amdgcn_readlane(news, ln);
                    tw.nend = tw.nblk + nt;
                    tw.L -= nt;
                }
                const int nt = tw.nend - tw.jlo;  // tiles per head
                const int64_t a_s = carry + __builtin_amdgcn_readlane(incl - tiles, ln);
                const int64_t off = t0 - a_s;
                const int grp = static_cast<int>(off / nt);
                tw.g = grp * hg + gi;
                tw.j = tw.jlo + static_cast<int>(off % nt);
                tw.a_sg = a_s + static_cast<int64_t>(grp) * nt;
                found = true;
                break;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
    }
    if (!found) return;  // lengths changed between the two passes
    walk_enter_row(p, tw, lane);

    __shared__ __attribute__((aligned(16))) uint8_t stage_all[WPG][G > 1 ? MfmaGeo<D>::kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t q_all[WPG][G > 1 ? MfmaGeo<D>::kNk * 1024 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t kst_all[WPG][G > 1 ? MfmaGeo<D>::kStage : 16];
    typename M::State st;
    if constexpr (G > 1) {
        st.stage = stage_all[wv_in];
        st.qlds = q_all[wv_in];
        st.kst = kst_all[wv_in];
    }
    M::reset(st);
    typename M::QT q;
    typename M::QT qring[M::kPrefetchQ ? NBUF : 1];

    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * M::kTB;
    // The ring: NBUF tiles of registers, or (M::kLds) two LDS slots per wave,
    // one array per slot, and one register tile the consumed slot is read into.
    static_assert(!M::kLds || NBUF == 2, "LDS ring: two slots");
    constexpr int kRingBytes = M::kLds ? 2 * M::kTB : 16;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[M::kLds ? WPG : 1][kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[M::kLds ? WPG : 1][kRingBytes];
    typename M::TileT tr[M::kLds ? 1 : NBUF];
    SlotInfo si[NBUF];
    auto load_tile = [&](typename M::TileT& tt, const TileRef& r, int x, bool kept) {
        if constexpr (M::kLds)
            M::issue_lds(x == 0 ? ring0[wv_in] : ring1[wv_in], r, lane, kept);
        else
            M::issue(tt, r, lane, kept);
    };

    // Issue tile kn of the range into ring slot x (and the q of a segment
    // that starts there).
    auto issue = [&](typename M::TileT& tt, SlotInfo& info, typename M::QT& qq, int kn, int x) {
        if (kn >= n) {
            info.bits = 0;
            info.s = info.g = 0;
            info.vslot = -1;
            const TileRef r = tile_ref(p, p.k_plane, p.v_plane, bstride, M::kTB, -1, 0, 0, 0);
            load_tile(tt, r, x, false);
            return;
        }
        if (kn > 0) walk_advance<kPre, kKeep, kFold>(p, tw, lane);
        const bool first = kn == 0 || tw.j == tw.jlo;
        const bool last = kn == n - 1 || tw.j == tw.nend - 1;
        // Where the segment's result goes: its context lies wholly in this
        // range, or it is a piece (slot 1 if it began in this range).
        const bool whole = tw.a_sg >= t0 && tw.a_sg + (tw.nend - tw.jlo) <= t1;
        const int flags = (first ? SlotInfo::kFirst : 0) | (last ? SlotInfo::kLast : 0) |
                          (kPre && tw.has_pre ? SlotInfo::kHasPre : 0) |
                          (whole ? SlotInfo::kWhole : 0) | (tw.a_sg > t0 ? SlotInfo::kSlot1 : 0);
        info.s = tw.s;
        info.g = tw.g;
        info.vslot = -1;
        if constexpr (M::kPrefetchQ) {
            if (first) M::fetch_q(p, qq, tw.s, tw.g, lane);
        }
        if (kFold && tw.j == tw.nblk) {
            // The new token's tile. Its slot is in the last block, whose id the
            // wave issued just before, unless its range starts here (then
            // nothing is in flight yet to wait behind).
            const int id = kn > 0 ? tw.last_id
                                  : __builtin_amdgcn_readfirstlane(
                                        p.block_tables[static_cast<size_t>(tw.s) * p.max_blocks +
                                                       tw.nblk - 1]);
            const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks);
            const size_t row = (static_cast<size_t>(tw.s) * p.num_kv_heads + tw.g) * (D * 2);
            TileRef r;
            r.k = tile_rsrc(p.new_k + row, ok ? D * 2 : 0);
            r.v = tile_rsrc(p.new_v + row, ok ? D * 2 : 0);
            info.bits = flags | (ok ? 1 : 0);  // no slot: the token is not in the context
            info.vslot = ok ? id * 16 + (tw.L & 15) : -1;  // position L - 1 of the context
            load_tile(tt, r, x, false);
            return;
        }
        const uint8_t* kpl = p.k_plane + static_cast<size_t>(tw.g) * M::kTB;
        const uint8_t* vpl = p.v_plane + static_cast<size_t>(tw.g) * M::kTB;
        const int id = walk_id(p, tw, lane);
        if constexpr (kFold) tw.last_id = id;
        const TileRef r = tile_ref(p, kpl, vpl, bstride, M::kTB, id, tw.j * 16, tw.L, tw.lo);
        info.bits = flags | r.nvalid | (r.nlo << 5);
        load_tile(tt, r, x, kKeep && tw.j < tw.keep);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x)
        issue(tr[M::kLds ? 0 : x], si[x], qring[M::kPrefetchQ ? x : 0], x, x);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            typename M::TileT& tx = tr[M::kLds ? 0 : x];
            const SlotInfo cur = si[x];
            const int cnv = cur.nvalid(), cnl = cur.nlo();
            if (cur.bits & SlotInfo::kFirst) {
                if constexpr (M::kPrefetchQ)
                    q = qring[x];
                else
                    M::fetch_q_lds(p, st, cur.s, cur.g, lane);
            }
            if constexpr (M::kLds) M::read_slot(tx, x == 0 ? ring0[wv_in] : ring1[wv_in], lane);
            if (kFold && cur.vslot >= 0)
                M::store_new(p, tx,
                             static_cast<int64_t>(cur.vslot >> 4) * bstride +
                                 static_cast<int64_t>(cur.g) * M::kTB + (cur.vslot & 15) * (D * 2),
                             lane);
            const bool full = cnv == 16 && cnl == 0;
            if constexpr (M::kSplit) {
                // First half, then the slot's refill, then the second half.
                f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
                if (full)
                    sacc = M::template front<false>(st, tx, 16, 0, lane);
                else if (cnv > 0)
                    sacc = M::template front<true>(st, tx, cnv, cnl, lane);
                issue(tx, si[x], qring[M::kPrefetchQ ? x : 0], k0 + x + NBUF, x);
                if (full)
                    M::template back<false>(st, sacc, 16, 0, p.scale_log2, lane);
                else if (cnv > 0)
                    M::template back<true>(st, sacc, cnv, cnl, p.scale_log2, lane);
            } else {
                // LDS ring: the tile is in registers now, so the slot is
                // refilled before the math (the other slot stays in flight).
                if constexpr (M::kLds) issue(tx, si[x], qring[M::kPrefetchQ ? x : 0], k0 + x + NBUF, x);
                if (full)
                    M::template consume<false>(st, tx, 16, 0, q, p.scale_log2, lane);
                else if (cnv > 0)
                    M::template consume<true>(st, tx, cnv, cnl, q, p.scale_log2, lane);
            }
            if (cur.bits & SlotInfo::kLast) {
                // End of a segment: write the output, or the partial of a split context.
                M::finish(st);
                if (cur.bits & SlotInfo::kWhole) {
                    if (kPre && (cur.bits & SlotInfo::kHasPre))  // the merge folds that in
                        M::store_partial(p.suf + static_cast<size_t>(cur.s * p.num_kv_heads + cur.g) *
                                                     G * SS,
                                         st, lane);
                    else
                        M::store_out(p, st, cur.s, cur.g, lane);
                } else {  // split context: slot 0 if it began before this range, else 1
                    const int slot = (cur.bits & SlotInfo::kSlot1) ? 1 : 0;
                    M::store_partial(p.slots + static_cast<size_t>(w * 2 + slot) * G * SS, st, lane);
                }
                M::reset(st);
            }
            if constexpr (!M::kSplit && !M::kLds)
                issue(tx, si[x], qring[M::kPrefetchQ ? x : 0], k0 + x + NBUF, x);
        }
    }
}

// Second kernel of the balanced single pass: one workgroup per (kv head,
// sequence). It recomputes the split of the batch into R ranges, and for a
// context that was split merges the partials its waves left in their slots;
// contexts written whole by one wave were stored by the streaming kernel and
// are left alone. With a shared-prefix pass, a member's prefix partial joins
// the merge, and so does its suffix partial when one wave read the whole
// suffix. A thread owns 4 dims of one head and merges the partials online,
// eight at a time: the loads of a group are all issued before any is used,
// and the running (max, sum, output) is rescaled when a group raises the
// maximum, so a context split over up to eight waves costs one round trip to
// memory after the lengths.
// Threads per (kv head, sequence): one per 4 output dims of the G heads,
// rounded up to whole waves. When that is one wave, a workgroup takes four kv
// heads of the sequence, a wave each.
template <int D, int G>
constexpr int merge_threads() {
    return (G * D / 4 + 63) / 64 * 64 < 256 ? (G * D / 4 + 63) / 64 * 64 : 256;
}
template <int D, int G>
constexpr int merge_heads_per_wg() {
    return merge_threads<D, G>() == 64 ? 4 : 1;
}

template <int KV, int D, int G>
__global__ __launch_bounds__((merge_threads<D, G>() * merge_heads_per_wg<D, G>())) void
balanced_merge_kernel(const DecodeParams p) {
    constexpr int NT = merge_threads<D, G>();
    constexpr int HPW = merge_heads_per_wg<D, G>();
    constexpr int SS = SlotGeoB<D>::kStride;
    constexpr int kGroup = 8;
    const int g = blockIdx.x * HPW + (HPW > 1 ? static_cast<int>(threadIdx.x >> 6) : 0);
    const int s = blockIdx.y, lane = threadIdx.x & 63;
    if (g >= p.num_kv_heads) return;  // a whole wave: the last workgroup's spare heads
    int64_t total = 0, before = 0;  // tiles per head of the batch, and of sequences < s
    for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {
        const int jj = c0 + lane;
        const int nb = jj < p.num_seqs ? pass_tiles(p, seq_tokens(p, jj), pre_of(p, jj)) +
                                             (p.fold_new ? new_of(p, jj) : 0)
                                       : 0;
        total += wave_sum(nb);
        before += wave_sum(jj < s ? nb : 0);
    }
    const int pre = pre_of(p, s);
    const bool has_pre = pre > 0;
    const int nblk = pass_tiles(p, seq_tokens(p, s), pre) + (p.fold_new ? new_of(p, s) : 0);
    uint16_t* out = static_cast<uint16_t*>(p.out) +
                    (static_cast<size_t>(s) * p.num_q_heads + g * G) * D;
    const int t = HPW > 1 ? lane : static_cast<int>(threadIdx.x);
    if (nblk == 0 && !has_pre) {
        for (int idx = t; idx < G * D; idx += NT) out[idx] = 0;
        return;
    }
    // Ranges wa .. wb hold pieces of this context, each read by wave gi of its
    // range's head group (none when the prefix pass covered all of it); whole:
    // one wave read it all and left its partial in suf.
    const int hg = p.head_group, hs = __builtin_ctz(hg);  // hg is 1, 2, 4 or 8
    const int grp = g >> hs, gi = g & (hg - 1);
    int wa = 0, wb = -1, slot_a = 0;
    bool whole = false;
    if (nblk > 0) {
        total *= p.num_kv_heads >> hs;
        const int Wr = p.num_waves >> hs;
        const int R = static_cast<int>(total < Wr ? total : Wr);
        const int64_t a_sg = before * (p.num_kv_heads >> hs) + static_cast<int64_t>(grp) * nblk;
        wa = wave_of(a_sg, total, R);
        wb = wave_of(a_sg + nblk - 1, total, R);
        if (wa == wb) {
            if (!has_pre) return;  // written whole by its wave
            whole = true;
        }
        // A context that begins inside range wa (past its first unit) has its
        // piece there in slot 1; every other piece is in slot 0.
        slot_a = (a_sg <= range_start(total, wa, R)) ? 0 : 1;
    }
    for (int idx = t; idx < G * D / 4; idx += NT) {
        const int h = idx / (D / 4), d = (idx % (D / 4)) * 4;
        const float* base = p.slots + static_cast<size_t>(h) * SS;
        float run_m = -INFINITY, run_l = 0.0f;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        // Fold one partial (o normalised, m in log2 units, l).
        auto fold = [&](const float* src) {
            const float4 ov = *reinterpret_cast<const float4*>(src + d);
            const float mv = src[D], lv = src[D + 1];
            const float mx = fmaxf(run_m, mv);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            const float a = fast_exp2(run_m - ms);
            const float wv = lv * fast_exp2(mv - ms);
            run_l = run_l * a + wv;
            acc = make_float4(fmaf(wv, ov.x, acc.x * a), fmaf(wv, ov.y, acc.y * a),
                              fmaf(wv, ov.z, acc.z * a), fmaf(wv, ov.w, acc.w * a));
            run_m = mx;
        };
        const size_t row = (static_cast<size_t>(s) * p.num_q_heads + g * G + h) * SS;
        if (has_pre) fold(p.pre + row);
        if (whole) fold(p.suf + row);
        for (int v0 = wa; !whole && v0 <= wb; v0 += kGroup) {
            float mv[kGroup], lv[kGroup];
            float4 ov[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int v = v0 + i;
                if (v <= wb) {
                    const int slot = v == wa ? slot_a : 0;
                    const float* ps = base + static_cast<size_t>((v * hg + gi) * 2 + slot) * G * SS;
                    ov[i] = *reinterpret_cast<const float4*>(ps + d);
                    mv[i] = ps[D];
                    lv[i] = ps[D + 1];
                } else {
                    ov[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    mv[i] = -INFINITY;
                    lv[i] = 0.0f;
                }
            }
            float mx = run_m;
#pragma unroll
            for (int i = 0; i < kGroup; ++i) mx = fmaxf(mx, mv[i]);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            const float a = fast_exp2(run_m - ms);  // 0 while nothing has been merged
            run_l *= a;
            acc = make_float4(acc.x * a, acc.y * a, acc.z * a, acc.w * a);
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const float wv = lv[i] * fast_exp2(mv[i] - ms);
                run_l += wv;
                acc = make_float4(fmaf(wv, ov[i].x, acc.x), fmaf(wv, ov[i].y, acc.y),
                                  fmaf(wv, ov[i].z, acc.z), fmaf(wv, ov[i].w, acc.w));
            }
            run_m = mx;
        }
        const float inv = run_l > 0.0f ? 1.0f / run_l : 0.0f;
        *reinterpret_cast<uint2*>(out + h * D + d) =
            make_uint2(pack2<KV>(acc.x * inv, acc.y * inv), pack2<KV>(acc.z * inv, acc.w * inv));
    }
}

}  // namespace
