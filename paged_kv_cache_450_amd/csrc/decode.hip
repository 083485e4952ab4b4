// paged_attn_decode: single-query attention over a paged KV cache.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", section
// "PagedAttention：把操作系统的虚拟内存搬进 GPU": the attention kernel must read
// K/V correctly from non-contiguous physical blocks through the page table
// without giving up speed; the page names block prefetching and regrouping KV
// in on-chip memory as the CUDA techniques used (prior art here, not a plan).
// [P3] "突破大模型推理瓶颈：...", section 2.4: accumulate in FP32.
//
// gfx950 design (decode is HBM-bound: about 1 flop per KV byte for MHA):
//  * one workgroup of NW wave64s per (sequence, kv head, partition); the NW
//    waves take the partition's blocks round robin;
//  * a (block, kv head) tile of 16 tokens x D is contiguous, so wave load i of
//    a tile is the 1 KiB at tile + i*1024, 16 bytes per lane: every global
//    load is a fully coalesced dwordx4. A token row spans LPT = D*esize/16
//    lanes; a wave load covers TPI = 64/LPT tokens;
//  * QK: each lane dots its 16-byte slice with its slice of every query head
//    of the group (packed dot2 for fp16/bf16, hardware FP8->fp32 for e4m3),
//    then a DPP butterfly inside the LPT-lane group finishes the dot product;
//  * GQA: the G query heads that share a kv head live in one workgroup, so
//    each K/V tile is read from HBM once for all G heads;
//  * softmax: every lane runs an online (max, sum) update over the tokens of
//    its row, in base-2 with log2(e) folded into the scale; V is
//    accumulated in fp32. At the end the TPI rows of a wave and the NW waves
//    are merged with the log-sum-exp rule (shuffles, then LDS);
//  * each wave streams its tiles through a ring of NBUF tiles in registers:
//    as soon as a tile is folded into the softmax state, its registers are
//    refilled with the tile NBUF positions ahead, so the wave has NBUF tiles
//    of loads in flight from its first tile to its last (there is no
//    load-wait-compute cadence per batch);
//  * tiles are read with raw buffer loads whose descriptor is built per tile
//    from the (wave-uniform) block id; a tile past the end of the range, or
//    with an id outside the pool, gets a descriptor of size 0, so its loads
//    return zeros and move no bytes;
//  * block ids for a wave's next 64 tiles are fetched with one vector load
//    and broadcast with readlane; the following 64 are always in flight;
//  * split-K: with partition_size > 0 each workgroup covers one partition and
//    writes (m, l, o) to the workspace; paged_attn_reduce merges them.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "common.h"
#include "device.h"

namespace {

using namespace pkv::dev;

struct DecodeParams {
    const uint8_t* k_plane;  // this layer's K plane: [num_blocks][Hkv][16][D]
    const uint8_t* v_plane;
    const void* q;           // [B][Hq][D]
    void* out;               // [B][Hq][D] (unpartitioned)
    float* ws_ml;            // [B][Hq][P][2] (partitioned)
    float* ws_o;             // [B][Hq][P][D]
    const int32_t* block_tables;
    const int32_t* context_lens;
    const float* k_scale;
    const float* v_scale;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t max_ctx;
    int32_t blocks_per_part;  // 0: one workgroup covers the whole context
    int32_t num_parts;        // P of the workspace
    int32_t longest_first;    // single pass over <= 256 sequences: longest first
    float scale_log2;         // scale * log2(e)
};

template <int KV, int D>
struct Geo {
    static constexpr int kEsz = (KV == PKV_FP8_E4M3) ? 1 : 2;
    static constexpr int kEpl = 16 / kEsz;     // elements per lane per load
    static constexpr int kLpt = D / kEpl;      // lanes per token row
    static constexpr int kTpi = 64 / kLpt;     // tokens per wave load
    static constexpr int kNld = 16 / kTpi;     // wave loads per tile
    static constexpr int kTileBytes = 16 * D * kEsz;
    static_assert(kLpt >= 2 && kLpt <= 16 && kNld >= 1, "geometry");
};

// Query slice of one head for one lane: raw 16-bit pairs for 16-bit caches,
// fp32 values for FP8 caches.
template <int KV, int D>
struct QSlice {
    static constexpr int kEpl = Geo<KV, D>::kEpl;
    static constexpr int kWords = (KV == PKV_FP8_E4M3) ? kEpl : kEpl / 2;
    float f[(KV == PKV_FP8_E4M3) ? kEpl : 1];
    uint32_t w[(KV == PKV_FP8_E4M3) ? 1 : kEpl / 2];
};

template <int QD>
__device__ __forceinline__ void to_f32x2(uint32_t w, float& a, float& b) {
    if constexpr (QD == PKV_F16) {
        a = f16_lo(w);
        b = f16_hi(w);
    } else {
        a = bf16_lo(w);
        b = bf16_hi(w);
    }
}

template <int KV, int QD, int D>
__device__ __forceinline__ void load_q(QSlice<KV, D>& qs, const uint16_t* qrow, int col) {
    constexpr int kEpl = Geo<KV, D>::kEpl;
    const uint4* p = reinterpret_cast<const uint4*>(qrow + col * kEpl);
    if constexpr (KV != PKV_FP8_E4M3) {
        const uint4 x = p[0];
        qs.w[0] = x.x; qs.w[1] = x.y; qs.w[2] = x.z; qs.w[3] = x.w;
    } else {
#pragma unroll
        for (int c = 0; c < kEpl / 8; ++c) {
            const uint4 x = p[c];
            const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) to_f32x2<QD>(ws[i], qs.f[c * 8 + 2 * i], qs.f[c * 8 + 2 * i + 1]);
        }
    }
}

// Partial dot product of one lane's 16-byte K slice with its query slice.
template <int KV, int D>
__device__ __forceinline__ float qk_partial(const uint4& k, const QSlice<KV, D>& qs) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    float acc = 0.0f;
    if constexpr (KV == PKV_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kw[i]),
                                         __builtin_bit_cast(half2_t, qs.w[i]), acc, false);
    } else if constexpr (KV == PKV_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, kw[i]),
                                                  __builtin_bit_cast(bf162_t, qs.w[i]), acc,
                                                  false);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2_t lo = e4m3x2_lo(kw[i]);
            const float2_t hi = e4m3x2_hi(kw[i]);
            acc = fmaf(lo.x, qs.f[4 * i + 0], acc);
            acc = fmaf(lo.y, qs.f[4 * i + 1], acc);
            acc = fmaf(hi.x, qs.f[4 * i + 2], acc);
            acc = fmaf(hi.y, qs.f[4 * i + 3], acc);
        }
    }
    return acc;
}

// One lane's 16-byte V slice as fp32.
template <int KV, int D>
__device__ __forceinline__ void v_to_f32(const uint4& v, float (&out)[Geo<KV, D>::kEpl]) {
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (KV == PKV_F16) {
            out[2 * i] = f16_lo(vw[i]);
            out[2 * i + 1] = f16_hi(vw[i]);
        } else if constexpr (KV == PKV_BF16) {
            out[2 * i] = bf16_lo(vw[i]);
            out[2 * i + 1] = bf16_hi(vw[i]);
        } else {
            const float2_t lo = e4m3x2_lo(vw[i]);
            const float2_t hi = e4m3x2_hi(vw[i]);
            out[4 * i + 0] = lo.x;
            out[4 * i + 1] = lo.y;
            out[4 * i + 2] = hi.x;
            out[4 * i + 3] = hi.y;
        }
    }
}

template <int KV, int D>
struct Tile {
    uint4 k[Geo<KV, D>::kNld];
    uint4 v[Geo<KV, D>::kNld];
};

template <int KV, int D, int G>
struct SoftmaxState {
    float m[G];                       // running max, base-2 units
    float l[G];                       // running sum of exp2(s - m)
    float o[G][Geo<KV, D>::kEpl];     // running sum of exp2(s - m) * v, this lane's dims
};

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros without touching memory, so a tile that is not part of the
// context (past the end of the wave's range, or a block id outside the pool)
// is "loaded" with bytes = 0 and costs no HBM traffic. The base is
// wave-uniform (one block id), so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                             bytes, 0x00020000);
}

// KV bytes are read once per decode step, so the tile loads carry the
// non-temporal policy (cache-policy bit 1, "nt" on gfx950): they stream
// through the caches instead of displacing lines that are reused. Measured
// on MI355X it lifts the decode's KV read rate by about 10%.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint4 rsrc_load16(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(uint4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kStreamPolicy));
}

// Longest-first order of the sequences of a single-pass decode: returns the
// index of the r-th longest sequence (ties: lower index first) and its
// clamped length. Workgroups are dispatched roughly in index order, so
// handing the longest contexts to the first workgroups keeps a long sequence
// from starting last and running alone at the end of the kernel.
// Every wave computes it redundantly from one load of all lengths: a radix
// select, most significant bit first, over the unique keys
// (blocks << 8) | (255 - index), counting candidates with ballots.
// Needs num_seqs <= 256.
__device__ __forceinline__ int longest_first(const DecodeParams& p, int num_seqs, int r,
                                             int& L_out) {
    const int lane = threadIdx.x & 63;
    const int max_tokens = min(p.max_ctx, p.max_blocks * 16);
    uint32_t key[4];
    int len[4];
    bool in[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = c * 64 + lane;
        in[c] = j < num_seqs;
        len[c] = in[c] ? min(max(p.context_lens[j], 0), max_tokens) : 0;
        key[c] = (static_cast<uint32_t>((len[c] + 15) >> 4) << 8) | static_cast<uint32_t>(255 - j);
    }
    const uint32_t max_blk = static_cast<uint32_t>((max_tokens + 15) >> 4);
    const int nbits = 8 + (max_blk ? 32 - __builtin_clz(max_blk) : 0);
    uint32_t prefix = 0, mask = 0;
    int rem = r;
    for (int b = nbits - 1; b >= 0; --b) {
        const uint32_t bit = 1u << b;
        int cnt = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            cnt += __popcll(__ballot(in[c] && (key[c] & mask) == prefix && (key[c] & bit)));
        if (rem < cnt)
            prefix |= bit;
        else
            rem -= cnt;
        mask |= bit;
    }
    const int s = 255 - static_cast<int>(prefix & 255u);
    L_out = __shfl(len[s >> 6], s & 63);
    return s;
}

// Fold one tile into the lane's online-softmax state. nvalid = number of
// leading tokens of the tile that belong to the context (0..16). kPartial
// selects the masked form, needed only when nvalid < 16 (the last block of a
// context, or a tile outside the context): tokens past nvalid get score -inf
// and their V bytes, which may be stale or NaN, are replaced by zeros.
template <int KV, int D, int G, bool kPartial>
__device__ __forceinline__ void consume_tile(SoftmaxState<KV, D, G>& st, const Tile<KV, D>& t,
                                             int nvalid, const QSlice<KV, D> (&qs)[G],
                                             float sscale, int row) {
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, TPI = Gm::kTpi, NLD = Gm::kNld;
    float sc[G][NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = qk_partial<KV, D>(t.k[i], qs[h]);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = group_sum<LPT>(sc[h][i]) * sscale;
    bool valid[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) valid[i] = !kPartial || (i * TPI + row) < nvalid;
    if constexpr (kPartial) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) sc[h][i] = valid[i] ? sc[h][i] : -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mx = st.m[h];
#pragma unroll
        for (int i = 0; i < NLD; ++i) mx = fmaxf(mx, sc[h][i]);
        const float ms = (mx == -INFINITY) ? 0.0f : mx;
        const float alpha = fast_exp2(st.m[h] - ms);
        st.m[h] = mx;
        float lsum = st.l[h] * alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.o[h][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            sc[h][i] = fast_exp2(sc[h][i] - ms);
            lsum += sc[h][i];
        }
        st.l[h] = lsum;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        float vf[EPL];
        v_to_f32<KV, D>(t.v[i], vf);
        if constexpr (kPartial) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vf[e] = valid[i] ? vf[e] : 0.0f;  // stale bytes never enter
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) st.o[h][e] = fmaf(sc[h][i], vf[e], st.o[h][e]);
    }
}

// Store one lane's EPL consecutive results of query head qh (dims
// [d0, d0 + EPL)): fp32 into the workspace, or rounded to the q dtype into out.
template <int QD, int D, int EPL>
__device__ __forceinline__ void store_result(const DecodeParams& p, int s, int qh, int part,
                                             int d0, const float (&r)[EPL]) {
    if (p.blocks_per_part > 0) {
        const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
        float4* dst = reinterpret_cast<float4*>(p.ws_o + slot * D + d0);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e)
            dst[e] = make_float4(r[4 * e], r[4 * e + 1], r[4 * e + 2], r[4 * e + 3]);
    } else {
        const size_t o_idx = (static_cast<size_t>(s) * p.num_q_heads + qh) * D + d0;
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o_idx);
#pragma unroll
        for (int e = 0; e < EPL / 8; ++e) {
            uint32_t wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = r[8 * e + 2 * i], b = r[8 * e + 2 * i + 1];
                const uint32_t lo = (QD == PKV_F16) ? f32_to_f16_bits(a) : f32_to_bf16_bits(a);
                const uint32_t hi = (QD == PKV_F16) ? f32_to_f16_bits(b) : f32_to_bf16_bits(b);
                wv[i] = lo | (hi << 16);
            }
            dst[e] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
}

__device__ __forceinline__ void store_ml(const DecodeParams& p, int s, int qh, int part,
                                         float m_log2, float l) {
    const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
    p.ws_ml[slot * 2] = (m_log2 == -INFINITY) ? -INFINITY : m_log2 * kLn2;
    p.ws_ml[slot * 2 + 1] = l;
}

// One workgroup of NW wave64s per (partition, kv head, sequence). The
// partition's blocks are dealt to the waves round robin; each wave streams its
// tiles through a ring of NBUF tiles held in registers: after a tile is folded
// into the softmax state its registers are refilled with the tile NBUF
// positions ahead, so every wave keeps NBUF tiles of loads in flight from its
// first tile to its last.
template <int KV, int QD, int D, int G, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, NLD = Gm::kNld, TB = Gm::kTileBytes;

    // Grid (kv head, sequence, partition), kv head fastest. Workgroups are
    // dealt to the 8 XCDs round robin in linear order, so consecutive indices
    // must carry comparable work: the heads of one sequence do (same length),
    // while partitions do not (short sequences have no late partitions).
    const int g = blockIdx.x;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;

    // Lr: the context as the reduce sees it (clamped to max_ctx); L: the
    // tokens this kernel can reach through a table row of max_blocks ids.
    int s, Lr, L;
    if (p.longest_first) {
        s = longest_first(p, gridDim.y, blockIdx.y, L);
        Lr = L;  // single pass: no reduce reads this sequence's partitions
    } else {
        s = blockIdx.y;
        Lr = max(0, min(p.context_lens[s], p.max_ctx));
        L = min(Lr, p.max_blocks * 16);
    }
    const int nblk = (L + 15) >> 4;
    int b0 = 0, b1 = nblk;
    if (p.blocks_per_part > 0) {
        b0 = part * p.blocks_per_part;
        b1 = min(b0 + p.blocks_per_part, nblk);
        if (b0 >= nblk) {
            // No tokens in this partition. If the reduce will still read it
            // (a table row narrower than the context), leave an empty partial.
            const int ps = p.blocks_per_part * 16;
            if (part < (Lr + ps - 1) / ps) {
                for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
                    const int h = idx / D, d = idx % D;
                    const size_t slot =
                        (static_cast<size_t>(s) * p.num_q_heads + g * G + h) * p.num_parts + part;
                    p.ws_o[slot * D + d] = 0.0f;
                    if (d == 0) store_ml(p, s, g * G + h, part, -INFINITY, 0.0f);
                }
            }
            return;
        }
    }

    // This wave's tiles: logical blocks b0 + w + k*NW for k < n.
    const int span = b1 - b0;
    const int n = span > w ? (span - w + NW - 1) / NW : 0;
    const int32_t* bt = p.block_tables + static_cast<size_t>(s) * p.max_blocks + b0 + w;
    auto load_ids = [&](int k0) -> int {  // ids of tiles k0 .. k0+63, one per lane
        const int k = k0 + lane;
        return k < n ? bt[k * NW] : -1;
    };
    int ids_a = load_ids(0);
    int ids_b = load_ids(64);

    // Query slices of the G heads of this group.
    QSlice<KV, D> qs[G];
    const uint16_t* qbase = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t qrow = (static_cast<size_t>(s) * p.num_q_heads + g * G + h) * D;
        load_q<KV, QD, D>(qs[h], qbase + qrow, col);
    }
    float sscale = p.scale_log2;
    if constexpr (KV == PKV_FP8_E4M3) sscale *= p.k_scale[g];

    SoftmaxState<KV, D, G> st;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.o[h][e] = 0.0f;
    }

    const uint8_t* kpl = p.k_plane + static_cast<size_t>(g) * TB;
    const uint8_t* vpl = p.v_plane + static_cast<size_t>(g) * TB;
    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * TB;
    const int voff = lane * 16;

    Tile<KV, D> t[NBUF];
    int nv[NBUF];
    // Issue the loads of tile kn into ring slot x. Tiles are issued in
    // increasing kn, so the id chunks rotate exactly once per 64 tiles; the
    // chunk after the current one is always already in flight.
    auto issue = [&](Tile<KV, D>& tt, int& nvalid, int kn) {
        if (kn >= 64 && (kn & 63) == 0) {
            ids_a = ids_b;
            ids_b = load_ids(kn + 64);
        }
        int id = -1;
        if (kn < n) id = __builtin_amdgcn_readlane(ids_a, kn & 63);
        const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks);
        nvalid = ok ? min(L - (b0 + w + kn * NW) * 16, 16) : 0;
        const size_t off = static_cast<size_t>(ok ? id : 0) * bstride;
        const int bytes = ok ? TB : 0;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpl + off, bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpl + off, bytes);
#pragma unroll
        for (int i = 0; i < NLD; ++i) tt.k[i] = rsrc_load16(rk, voff + i * 1024);
#pragma unroll
        for (int i = 0; i < NLD; ++i) tt.v[i] = rsrc_load16(rv, voff + i * 1024);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(t[x], nv[x], x);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            if (nv[x] == 16)
                consume_tile<KV, D, G, false>(st, t[x], 16, qs, sscale, row);
            else
                consume_tile<KV, D, G, true>(st, t[x], nv[x], qs, sscale, row);
            issue(t[x], nv[x], k0 + x + NBUF);
        }
    }

    // Merge the rows of this wave: lanes lane ^ off (off = LPT, 2*LPT, ...)
    // hold the same dims for other tokens.
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(st.m[h], off);
            const float l2 = __shfl_xor(st.l[h], off);
            const float mx = fmaxf(st.m[h], m2);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            const float a = fast_exp2(st.m[h] - ms), b = fast_exp2(m2 - ms);
            st.l[h] = st.l[h] * a + l2 * b;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float o2 = __shfl_xor(st.o[h][e], off);
                st.o[h][e] = st.o[h][e] * a + o2 * b;
            }
            st.m[h] = mx;
        }
    }

    float vscale = 1.0f;
    if constexpr (KV == PKV_FP8_E4M3) vscale = p.v_scale[g];

    if constexpr (NW == 1) {
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = st.l[h] > 0.0f ? vscale / st.l[h] : 0.0f;
                float r[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) r[e] = st.o[h][e] * inv;
                store_result<QD, D, EPL>(p, s, g * G + h, part, col * EPL, r);
                if (p.blocks_per_part > 0 && col == 0) store_ml(p, s, g * G + h, part, st.m[h], st.l[h]);
            }
        }
    } else {
        // Merge the NW waves through LDS.
        __shared__ float lds_o[NW][G][D];
        __shared__ float lds_m[NW][G];
        __shared__ float lds_l[NW][G];
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) lds_o[w][h][col * EPL + e] = st.o[h][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                lds_m[w][h] = st.m[h];
                lds_l[w][h] = st.l[h];
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
            const int h = idx / D, d = idx % D;
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < NW; ++x) mx = fmaxf(mx, lds_m[x][h]);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            float lsum = 0.0f, acc = 0.0f;
#pragma unroll
            for (int x = 0; x < NW; ++x) {
                const float a = fast_exp2(lds_m[x][h] - ms);
                lsum = fmaf(lds_l[x][h], a, lsum);
                acc = fmaf(lds_o[x][h][d], a, acc);
            }
            const float res = lsum > 0.0f ? (acc / lsum) * vscale : 0.0f;
            const int qh = g * G + h;
            if (p.blocks_per_part > 0) {
                const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
                p.ws_o[slot * D + d] = res;
                if (d == 0) store_ml(p, s, qh, part, mx, lsum);
            } else {
                const size_t o_idx = (static_cast<size_t>(s) * p.num_q_heads + qh) * D + d;
                const uint16_t bits = (QD == PKV_F16) ? f32_to_f16_bits(res) : f32_to_bf16_bits(res);
                static_cast<uint16_t*>(p.out)[o_idx] = bits;
            }
        }
    }
}

// Tiles kept in flight per wave: the ring must fit beside the softmax state
// of the G heads.
template <int KV, int D, int G>
constexpr int ring_depth() {
    return (G <= 2) ? 4 : (G == 4 ? 2 : 1);
}

template <int KV, int QD, int D, int G, int NW>
hipError_t launch(const DecodeParams& prm, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, ring_depth<KV, D, G>()>), grid,
                       dim3(NW * 64), 0, stream, prm);
    return hipGetLastError();
}

// Waves per workgroup: a partition of up to 16 blocks is one wave's stream;
// longer ranges (big partitions, or the whole context when unpartitioned) are
// shared by four waves and merged through LDS.
template <int KV, int QD, int D, int G>
hipError_t by_waves(const DecodeParams& prm, dim3 grid, hipStream_t st) {
    if (prm.blocks_per_part > 0 && prm.blocks_per_part <= 16)
        return launch<KV, QD, D, G, 1>(prm, grid, st);
    if (prm.blocks_per_part > 0 && prm.blocks_per_part <= 32)
        return launch<KV, QD, D, G, 2>(prm, grid, st);
    return launch<KV, QD, D, G, 4>(prm, grid, st);
}

template <int KV, int QD, int D>
hipError_t by_group(int G, const DecodeParams& prm, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: return by_waves<KV, QD, D, 1>(prm, grid, st);
        case 2: return by_waves<KV, QD, D, 2>(prm, grid, st);
        case 4: return by_waves<KV, QD, D, 4>(prm, grid, st);
        default: return by_waves<KV, QD, D, 8>(prm, grid, st);
    }
}

template <int KV, int QD>
hipError_t by_dim(int D, int G, const DecodeParams& prm, dim3 grid, hipStream_t st) {
    if (D == 64) return by_group<KV, QD, 64>(G, prm, grid, st);
    return by_group<KV, QD, 128>(G, prm, grid, st);
}

}  // namespace

extern "C" size_t paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
    if (partition_size <= 0 || num_seqs < 0 || num_q_heads < 0 || head_dim <= 0 ||
        max_context_len < 0)
        return 0;
    const size_t parts = (static_cast<size_t>(max_context_len) + partition_size - 1) / partition_size;
    return pkv::ws_o_offset(num_seqs, num_q_heads, parts) +
           static_cast<size_t>(num_seqs) * num_q_heads * parts * static_cast<size_t>(head_dim) *
               sizeof(float);
}

extern "C" pkv_status paged_attn_decode(const pkv_pool* pool, int32_t layer, const void* q,
                                        int32_t q_dtype, void* out, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads, float scale,
                                        const float* k_scale, const float* v_scale,
                                        int32_t max_context_len, int32_t partition_size,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    using pkv::fail;
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "paged_attn_decode: pool is NULL");
    const pkv_pool_desc& d = pool->desc;
    if (pool->base == nullptr)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: pool has no device memory");
    if (layer < 0 || layer >= d.num_layers)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: layer %d out of range", layer);
    if (!pkv::is_16bit(q_dtype))
        return fail(PKV_ERR_INVALID, "paged_attn_decode: q dtype must be F16 or BF16");
    if (pkv::is_16bit(d.kv_dtype) && q_dtype != d.kv_dtype)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: q dtype must equal the 16-bit cache dtype");
    if (num_seqs < 0 || num_seqs > 65535)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: num_seqs %d outside [0, 65535]", num_seqs);
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads != 0)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: %d query heads for %d kv heads",
                    num_q_heads, d.num_kv_heads);
    const int G = num_q_heads / d.num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: group size %d not in {1,2,4,8}", G);
    if (max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: negative table width or context");
    if (partition_size < 0 || partition_size % 16 != 0)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: partition_size %d not a multiple of 16",
                    partition_size);
    if (!std::isfinite(scale))
        return fail(PKV_ERR_INVALID, "paged_attn_decode: scale is not finite");
    if (max_blocks_per_seq > (1 << 26))
        return fail(PKV_ERR_INVALID, "paged_attn_decode: max_blocks_per_seq too large");
    if (num_seqs == 0) return PKV_OK;
    if (d.num_blocks == 0)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: the pool has no blocks");
    if (q == nullptr || block_tables == nullptr || context_lens == nullptr)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: NULL q, block_tables or context_lens");
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: q must be 16-byte aligned");
    if (d.kv_dtype == PKV_FP8_E4M3 && (k_scale == nullptr || v_scale == nullptr))
        return fail(PKV_ERR_INVALID, "paged_attn_decode: an FP8 cache needs k_scale and v_scale");

    DecodeParams prm{};
    const uint8_t* base = static_cast<const uint8_t*>(pool->base);
    prm.k_plane = base + pkv::layer_plane_offset(d, layer, 0);
    prm.v_plane = base + pkv::layer_plane_offset(d, layer, 1);
    prm.q = q;
    prm.out = out;
    prm.block_tables = block_tables;
    prm.context_lens = context_lens;
    prm.k_scale = k_scale;
    prm.v_scale = v_scale;
    prm.max_blocks = max_blocks_per_seq;
    prm.num_blocks = d.num_blocks;
    prm.num_kv_heads = d.num_kv_heads;
    prm.num_q_heads = num_q_heads;
    prm.max_ctx = max_context_len;
    prm.scale_log2 = scale * pkv::dev::kLog2e;

    uint32_t parts = 1;
    if (partition_size > 0) {
        const size_t need = paged_attn_workspace_bytes(num_seqs, num_q_heads, d.head_dim,
                                                       max_context_len, partition_size);
        if (workspace == nullptr || workspace_bytes < need)
            return fail(PKV_ERR_INVALID, "paged_attn_decode: workspace of %zu bytes, %zu needed",
                        workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return fail(PKV_ERR_INVALID, "paged_attn_decode: workspace must be 16-byte aligned");
        const int64_t P = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
        if (P == 0) return PKV_OK;  // no tokens anywhere; the reduce writes zeros
        if (P > 65535)
            return fail(PKV_ERR_INVALID, "paged_attn_decode: %lld partitions (at most 65535)",
                        static_cast<long long>(P));
        parts = static_cast<uint32_t>(P);
        prm.blocks_per_part = partition_size / 16;
        prm.num_parts = static_cast<int32_t>(P);
        prm.ws_ml = static_cast<float*>(workspace);
        prm.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                            pkv::ws_o_offset(num_seqs, num_q_heads, P));
    } else {
        if (out == nullptr) return fail(PKV_ERR_INVALID, "paged_attn_decode: out is NULL");
        if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
            return fail(PKV_ERR_INVALID, "paged_attn_decode: out must be 16-byte aligned");
        prm.blocks_per_part = 0;
        prm.num_parts = 1;
        // The ordering keys hold the block count in 23 bits.
        const int64_t max_tokens =
            std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * 16);
        prm.longest_first = (num_seqs <= 256 && (max_tokens + 15) / 16 < (1 << 23)) ? 1 : 0;
    }

    const dim3 grid(static_cast<uint32_t>(d.num_kv_heads), static_cast<uint32_t>(num_seqs), parts);
    hipError_t e;
    if (d.kv_dtype == PKV_F16)
        e = by_dim<PKV_F16, PKV_F16>(d.head_dim, G, prm, grid, stream);
    else if (d.kv_dtype == PKV_BF16)
        e = by_dim<PKV_BF16, PKV_BF16>(d.head_dim, G, prm, grid, stream);
    else if (q_dtype == PKV_F16)
        e = by_dim<PKV_FP8_E4M3, PKV_F16>(d.head_dim, G, prm, grid, stream);
    else
        e = by_dim<PKV_FP8_E4M3, PKV_BF16>(d.head_dim, G, prm, grid, stream);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "paged_attn_decode: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}
