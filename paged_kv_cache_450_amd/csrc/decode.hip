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
    // Balanced single pass (see decode_balanced_kernel).
    float* slots;             // [waves][2][G][D + 4] partials of split contexts
    int32_t num_waves;        // waves of the balanced launch
    int32_t num_seqs;
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
    // Uniform by construction; readfirstlane tells the compiler so (otherwise
    // every value derived from it, down to the tile descriptors, is treated as
    // per-lane and each buffer load becomes a loop over distinct descriptors).
    L_out = __builtin_amdgcn_readfirstlane(__shfl(len[s >> 6], s & 63));
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

// Merge the (m, l, o) partials that the NW waves of a workgroup left in LDS
// for the G heads, and store the result: the workspace partial of this
// partition, or the normalised output. o is unnormalised (scaled by
// exp2(s - m)); vscale multiplies the result (the FP8 V scale, else 1).
template <int QD, int D, int G, int NW>
__device__ __forceinline__ void combine_waves(const DecodeParams& p, int s, int g, int part,
                                              const float (*lds_o)[G][D],
                                              const float (*lds_m)[G],
                                              const float (*lds_l)[G], float vscale) {
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

// The work of one wave: sequence s, its length L as this kernel reads it, and
// its tiles, the logical blocks b0 + w + k*NW for k < n (the partition's
// blocks dealt round robin to the NW waves of the workgroup).
struct WaveWork {
    int s, L, b0, n;
};

// Grid (kv head, sequence, partition), kv head fastest. Workgroups are dealt
// to the 8 XCDs round robin in linear order, so consecutive indices must carry
// comparable work: the heads of one sequence do (same length), while
// partitions do not (short sequences have no late partitions).
// Returns false when the workgroup has no tokens; every wave of the
// workgroup takes the same branch.
template <int G, int D, int NW>
__device__ __forceinline__ bool locate_work(const DecodeParams& p, int g, int part, int w,
                                            WaveWork& ww) {
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
            return false;
        }
    }
    const int span = b1 - b0;
    ww.s = s;
    ww.L = L;
    ww.b0 = b0 + w;
    ww.n = span > w ? (span - w + NW - 1) / NW : 0;
    return true;
}

// Block ids of a wave's tiles, 64 per vector load, broadcast with readlane.
// Tiles are requested in increasing order, so the chunks rotate exactly once
// per 64 tiles, and the chunk after the current one is always in flight.
template <int NW>
struct BlockIds {
    const int32_t* row;  // table row of the sequence, from the wave's first block
    int n, lane, a, b;

    __device__ __forceinline__ int load(int k0) const {  // ids of tiles k0 .. k0+63
        const int k = k0 + lane;
        return k < n ? row[k * NW] : -1;
    }
    __device__ __forceinline__ void init(const int32_t* r, int count, int ln) {
        row = r;
        n = count;
        lane = ln;
        a = load(0);
        b = load(64);
    }
    // Id of tile kn, or -1 past the end of the wave's tiles.
    __device__ __forceinline__ int next(int kn) {
        if (kn >= 64 && (kn & 63) == 0) {
            a = b;
            b = load(kn + 64);
        }
        return kn < n ? __builtin_amdgcn_readlane(a, kn & 63) : -1;
    }
};

// Descriptors of the K and V tiles of block `id` for kv head g, and the number
// of context tokens in it. An id outside the pool, or past the end (-1), gives
// size-0 descriptors and no tokens.
struct TileRef {
    __amdgpu_buffer_rsrc_t k, v;
    int nvalid;
};

__device__ __forceinline__ TileRef tile_ref(const DecodeParams& p, const uint8_t* kpl,
                                            const uint8_t* vpl, size_t bstride, int tile_bytes,
                                            int id, int first_token, int L) {
    const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks);
    const size_t off = static_cast<size_t>(ok ? id : 0) * bstride;
    const int bytes = ok ? tile_bytes : 0;
    TileRef t;
    t.k = tile_rsrc(kpl + off, bytes);
    t.v = tile_rsrc(vpl + off, bytes);
    t.nvalid = ok ? min(L - first_token, 16) : 0;
    return t;
}

// Vector-ALU decode: one workgroup of NW wave64s per (kv head, sequence,
// partition). Each wave streams its tiles through a ring of NBUF tiles held in
// registers: after a tile is folded into the softmax state its registers are
// refilled with the tile NBUF positions ahead, so every wave keeps NBUF tiles
// of loads in flight from its first tile to its last. Used for FP8 caches and
// for one query head per kv head.
template <int KV, int QD, int D, int G, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, NLD = Gm::kNld, TB = Gm::kTileBytes;

    const int g = blockIdx.x;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;

    WaveWork ww;
    if (!locate_work<G, D, NW>(p, g, part, w, ww)) return;
    const int s = ww.s, L = ww.L, n = ww.n;
    BlockIds<NW> ids;
    ids.init(p.block_tables + static_cast<size_t>(s) * p.max_blocks + ww.b0, n, lane);

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
    // Issue the loads of tile kn into a ring slot.
    auto issue = [&](Tile<KV, D>& tt, int& nvalid, int kn) {
        const TileRef r = tile_ref(p, kpl, vpl, bstride, TB, ids.next(kn), (ww.b0 + kn * NW) * 16, L);
        nvalid = r.nvalid;
#pragma unroll
        for (int i = 0; i < NLD; ++i) tt.k[i] = rsrc_load16(r.k, voff + i * 1024);
#pragma unroll
        for (int i = 0; i < NLD; ++i) tt.v[i] = rsrc_load16(r.v, voff + i * 1024);
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
        combine_waves<QD, D, G, NW>(p, s, g, part, lds_o, lds_m, lds_l, vscale);
    }
}

// ---------------------------------------------------------------------------
// Matrix-core decode for 16-bit caches with grouped query heads.
//
// With G query heads per kv head a tile costs G times the multiply-adds of one
// head (8 flop per KV byte at G = 8), which the vector ALU cannot sustain at
// HBM rate. Here both products run on MFMA, with the G heads padded to 16:
//   S^T = K Q^T    (v_mfma 16x16x32: rows = the 16 tokens of a tile,
//                   columns = heads, contraction over 32 dims per step)
//   O^T += V^T P^T (v_mfma 16x16x16: rows = 16 dims, columns = heads,
//                   contraction over the 16 tokens of the tile)
// Lane l works for head l % 16. After the QK product it holds that head's
// scores for tokens 4*(l/16) .. +3, which is exactly the B operand P^T of the
// PV product, so the probabilities never move between lanes; the running max
// is shared by the four lanes of a head with two xor-shuffles, and the O^T
// accumulator of a lane belongs to its own head, so rescaling is lane-local.
// K is loaded straight into the A-operand layout (token l % 16, 8 dims).
// V^T, the A operand of the PV product, needs each lane to hold 4 tokens of
// one dim: V goes through a per-wave LDS tile in its natural layout, and
// ds_read_tr16_b64 returns the transposed 4 x 16-bit groups (one read per 16
// dims). Row pitches 2D + 48 (D = 128) and 2D + 16 (D = 64) bytes keep both
// the row writes and the transposed reads free of bank conflicts.
// P is rounded to the cache dtype for the PV product; both products
// accumulate in fp32.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <int KV>
__device__ __forceinline__ f32x4_t mfma_qk(const uint4& a, const uint4& b, f32x4_t c) {
    if constexpr (KV == PKV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int KV>
__device__ __forceinline__ f32x4_t mfma_pv(s16x4_t a, s16x4_t b, f32x4_t c) {
    if constexpr (KV == PKV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two fp32 values rounded to nearest even into the 16-bit type, packed
// (hardware conversions; v_cvt_pk_bf16_f32 on gfx950). Not for NaN inputs.
template <int KV>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (KV == PKV_F16) {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(a))) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(b))) << 16);
    } else {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
    }
}

template <int D>
struct MfmaGeo {
    static constexpr int kTileBytes = 16 * D * 2;
    static constexpr int kNk = D / 32;                 // QK steps = K loads per tile
    static constexpr int kNv = D / 32;                 // 1 KiB V loads per tile
    static constexpr int kNd = D / 16;                 // PV steps per tile
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kPitch = 2 * D + (D == 128 ? 48 : 16);
    static constexpr int kStage = 16 * kPitch;         // LDS bytes of one staged V tile
};

template <int D>
struct MfmaTile {
    uint4 k[MfmaGeo<D>::kNk];
    uint4 v[MfmaGeo<D>::kNv];
};

// The Q^T operand of a wave lives in its LDS (leaving the registers to a
// deeper tile ring), chunk-major so that each per-tile read of one 32-dim
// chunk is a contiguous, conflict-free 1 KiB.
template <int D>
struct QLds {
    const uint8_t* base;  // kNk x 1 KiB
    __device__ __forceinline__ uint4 get(int c, int lane) const {
        return *reinterpret_cast<const uint4*>(base + c * 1024 + lane * 16);
    }
};

template <int KV, int D, bool kPartial, class QSrc>
__device__ __forceinline__ void mfma_consume(const MfmaTile<D>& t, int nvalid, const QSrc& qsrc,
                                             f32x4_t (&o)[MfmaGeo<D>::kNd], float& m, float& lsum,
                                             float sscale, uint8_t* stage, int lane) {
    using Gm = MfmaGeo<D>;
    const int kg = lane >> 4;   // this lane's tokens: 4*kg .. 4*kg + 3
    const int hl = lane & 15;
    // Scores of head hl for tokens 4*kg + r.
    f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < Gm::kNk; ++c) sacc = mfma_qk<KV>(t.k[c], qsrc.get(c, lane), sacc);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        sc[r] = sacc[r] * sscale;
        if constexpr (kPartial) sc[r] = (4 * kg + r < nvalid) ? sc[r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // m is the reference of the exponentials. It is raised, and the sums
    // rescaled, only when a score passes it by more than kSlack (log2 units),
    // so probabilities stay below 2^kSlack and rescaling is rare: the O^T
    // accumulators live in AGPRs, where a rescale costs three instructions
    // per element.
    constexpr float kSlack = 8.0f;
    if (__ballot(mx > m + kSlack)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mnew);  // m = -inf: 0 (o and lsum are still 0)
        lsum *= alpha;
#pragma unroll
        for (int j = 0; j < Gm::kNd; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[j][r] *= alpha;
        m = mnew;
    }
    const float ms = (m == -INFINITY) ? 0.0f : m;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - ms);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const s16x4_t pb = __builtin_bit_cast(
        s16x4_t, make_uint2(pack2<KV>(pr[0], pr[1]), pack2<KV>(pr[2], pr[3])));

    // Stage V in LDS (natural layout, padded rows); tokens past nvalid become
    // zeros so that stale or NaN bytes never meet a zero probability.
    constexpr int kLanesPerRow = Gm::kRowBytes / 16;
#pragma unroll
    for (int i = 0; i < Gm::kNv; ++i) {
        const int tok = i * (64 / kLanesPerRow) + lane / kLanesPerRow;
        uint4 v = t.v[i];
        if constexpr (kPartial) {
            if (tok >= nvalid) v = make_uint4(0u, 0u, 0u, 0u);
        }
        *reinterpret_cast<uint4*>(stage + tok * Gm::kPitch + (lane % kLanesPerRow) * 16) = v;
    }
    // Transposed reads: lane (within its group of 16) j' supplies row
    // 4*kg + j'/4, dims 16*jd + 4*(j'%4); it receives dims 16*jd + j' of
    // tokens 4*kg .. 4*kg + 3.
    const uint8_t* rd = stage + (4 * kg + (hl >> 2)) * Gm::kPitch + 8 * (hl & 3);
#pragma unroll
    for (int jd = 0; jd < Gm::kNd; ++jd) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(rd + 32 * jd));
        o[jd] = mfma_pv<KV>(__builtin_bit_cast(s16x4_t, va), pb, o[jd]);
    }
}

template <int KV, int D, int G, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeParams p) {
    using Gm = MfmaGeo<D>;
    constexpr int NK = Gm::kNk, NV = Gm::kNv, ND = Gm::kNd, TB = Gm::kTileBytes;
    static_assert(G >= 1 && G <= 16, "heads padded to 16");

    const int g = blockIdx.x;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 15;
    const int kg = lane >> 4;

    WaveWork ww;
    if (!locate_work<G, D, NW>(p, g, part, w, ww)) return;
    const int s = ww.s, L = ww.L, n = ww.n;
    BlockIds<NW> ids;
    ids.init(p.block_tables + static_cast<size_t>(s) * p.max_blocks + ww.b0, n, lane);

    // Q^T operand in the wave's LDS: head hl (zeros for the padding heads),
    // dims 32c + 8*kg .. +8. Padding lanes read head G-1 (always inside q) and
    // discard it.
    __shared__ __attribute__((aligned(16))) uint8_t q_all[NW][NK * 1024];
    const QLds<D> qr{q_all[w]};
    {
        const int hq = g * G + min(hl, G - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(p.q) + (static_cast<size_t>(s) * p.num_q_heads + hq) * D;
        uint4 qv[NK];
#pragma unroll
        for (int c = 0; c < NK; ++c) qv[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * kg);
#pragma unroll
        for (int c = 0; c < NK; ++c)
            *reinterpret_cast<uint4*>(q_all[w] + c * 1024 + lane * 16) =
                hl < G ? qv[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    const float sscale = p.scale_log2;
    f32x4_t o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f;

    __shared__ __attribute__((aligned(16))) uint8_t stage_all[NW][Gm::kStage];
    uint8_t* stage = stage_all[w];

    const uint8_t* kpl = p.k_plane + static_cast<size_t>(g) * TB;
    const uint8_t* vpl = p.v_plane + static_cast<size_t>(g) * TB;
    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * TB;
    const int koff = hl * Gm::kRowBytes + 16 * kg;  // + 64*c: token hl, dims 32c + 8*kg
    const int voff = lane * 16;                     // + 1024*i: natural rows

    MfmaTile<D> t[NBUF];
    int nv[NBUF];
    auto issue = [&](MfmaTile<D>& tt, int& nvalid, int kn) {
        const TileRef r = tile_ref(p, kpl, vpl, bstride, TB, ids.next(kn), (ww.b0 + kn * NW) * 16, L);
        nvalid = r.nvalid;
#pragma unroll
        for (int c = 0; c < NK; ++c) tt.k[c] = rsrc_load16(r.k, koff + 64 * c);
#pragma unroll
        for (int i = 0; i < NV; ++i) tt.v[i] = rsrc_load16(r.v, voff + 1024 * i);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(t[x], nv[x], x);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            if (nv[x] == 16)
                mfma_consume<KV, D, false>(t[x], 16, qr, o, m, lsum, sscale, stage, lane);
            else
                mfma_consume<KV, D, true>(t[x], nv[x], qr, o, m, lsum, sscale, stage, lane);
            issue(t[x], nv[x], k0 + x + NBUF);
        }
    }

    // The four lanes of a head share m; their partial sums add up to l.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    if constexpr (NW == 1) {
        if (hl < G) {
            const int qh = g * G + hl;
            const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
            if (p.blocks_per_part > 0) {
                const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
                float* dst = p.ws_o + slot * D + 4 * kg;
#pragma unroll
                for (int j = 0; j < ND; ++j)
                    *reinterpret_cast<float4*>(dst + 16 * j) =
                        make_float4(o[j][0] * inv, o[j][1] * inv, o[j][2] * inv, o[j][3] * inv);
                if (kg == 0) store_ml(p, s, qh, part, m, lsum);
            } else {
                uint16_t* dst = static_cast<uint16_t*>(p.out) +
                                (static_cast<size_t>(s) * p.num_q_heads + qh) * D + 4 * kg;
#pragma unroll
                for (int j = 0; j < ND; ++j)
                    *reinterpret_cast<uint2*>(dst + 16 * j) =
                        make_uint2(pack2<KV>(o[j][0] * inv, o[j][1] * inv),
                                   pack2<KV>(o[j][2] * inv, o[j][3] * inv));
            }
        }
    } else {
        __shared__ float lds_o[NW][G][D];
        __shared__ float lds_m[NW][G];
        __shared__ float lds_l[NW][G];
        if (hl < G) {
#pragma unroll
            for (int j = 0; j < ND; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) lds_o[w][hl][16 * j + 4 * kg + r] = o[j][r];
            if (kg == 0) {
                lds_m[w][hl] = m;
                lds_l[w][hl] = lsum;
            }
        }
        __syncthreads();
        combine_waves<KV, D, G, NW>(p, s, g, part, lds_o, lds_m, lds_l, 1.0f);
    }
}

// ---------------------------------------------------------------------------
// Balanced single pass.
//
// Context lengths in a batch vary widely (16 to 8192 tokens in a log-normal
// batch), so one workgroup per sequence, or per fixed-size partition, leaves
// the GPU waiting on the longest items or paying a start-up per item. Here the
// grid is exactly the waves the GPU holds at once, and the tiles of the whole
// batch, ordered (sequence, kv head, block), are cut into R equal contiguous
// ranges, one per wave. A wave streams its range through its tile ring
// without a break: the ring runs across (sequence, head) boundaries. Each run
// of tiles of one (sequence, kv head) inside a range is a segment. A segment
// that covers its whole context writes the output directly; a context split
// over several waves leaves one partial (o / l, m, l) per wave in the
// workspace, and a second, small kernel on the same stream merges them with
// the log-sum-exp rule (the kernel boundary makes the partials visible; a
// merge inside the streaming kernel would need device-wide cache maintenance
// per split, which costs more than the launch).

// Tokens of sequence j as this kernel reads them (clamped like the other paths).
__device__ __forceinline__ int seq_tokens(const DecodeParams& p, int j) {
    return min(max(p.context_lens[j], 0), min(p.max_ctx, p.max_blocks * 16));
}

__device__ __forceinline__ int64_t range_start(int64_t total, int w, int W) {
    return total * w / W;
}
// The wave whose range holds tile t (ranges [range_start(w), range_start(w+1)),
// all non-empty).
__device__ __forceinline__ int wave_of(int64_t t, int64_t total, int W) {
    return static_cast<int>(((t + 1) * W - 1) / total);
}

// Sum over the wave, as a wave-uniform value.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Issue-side walker over the tiles of the batch in (sequence, kv head, block)
// order, holding the block ids of the current sequence's table row: blocks
// 0..127 of the row stay in registers for the row's other heads, later blocks
// rotate through a second pair of 64-id chunks.
struct TileWalk {
    int s, g, j, nblk;   // current tile: sequence, kv head, block
    int L;               // tokens of sequence s as read here
    int64_t a_sg;        // global index of tile (s, g, 0)
    int chunk;           // sequences 64*chunk .. +63 have their lengths in lens
    int lens;            // per lane: tokens of sequence 64*chunk + lane
    int row0_a, row0_b;  // ids of blocks 0..63 and 64..127 of row s (per lane)
    int ids_a, ids_b;    // ids of blocks base .. base+127 (per lane, two chunks)
    int base;
};

__device__ __forceinline__ int walk_row_ids(const DecodeParams& p, const TileWalk& t, int j0,
                                            int lane) {
    const int jj = j0 + lane;
    return jj < t.nblk ? p.block_tables[static_cast<size_t>(t.s) * p.max_blocks + jj] : -1;
}

__device__ __forceinline__ void walk_enter_row(const DecodeParams& p, TileWalk& t, int lane) {
    t.row0_a = walk_row_ids(p, t, 0, lane);
    t.row0_b = walk_row_ids(p, t, 64, lane);
    t.base = t.j & ~63;
    t.ids_a = t.base == 0 ? t.row0_a : walk_row_ids(p, t, t.base, lane);
    t.ids_b = t.base == 0 ? t.row0_b : walk_row_ids(p, t, t.base + 64, lane);
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

// Step to the next tile. Returns true when it starts a new segment.
__device__ __forceinline__ void walk_advance(const DecodeParams& p, TileWalk& t, int lane) {
    if (++t.j < t.nblk) return;
    t.j = 0;
    t.a_sg += t.nblk;
    if (++t.g < p.num_kv_heads) {  // same row, next head: blocks 0..127 are at hand
        t.base = 0;
        t.ids_a = t.row0_a;
        t.ids_b = t.row0_b;
        return;
    }
    t.g = 0;
    // Next sequence with tokens. A wave's range ends at or before the batch's
    // last tile, so a later non-empty sequence exists; the bound only keeps s
    // inside the batch should the lengths change under a running kernel.
    do {
        ++t.s;
        if ((t.s >> 6) != t.chunk) {
            t.chunk = t.s >> 6;
            const int jj = t.chunk * 64 + lane;
            t.lens = jj < p.num_seqs ? seq_tokens(p, jj) : 0;
        }
        t.L = __builtin_amdgcn_readlane(t.lens, t.s & 63);
        t.nblk = (t.L + 15) >> 4;
    } while (t.nblk == 0 && t.s + 1 < p.num_seqs);
    walk_enter_row(p, t, lane);
}

// Ring-slot description of an issued tile (all wave-uniform).
struct SlotInfo {
    int nvalid;       // context tokens in the tile (0 past the end of the range)
    int flags;        // bit 0: first tile of a segment, bit 1: last tile of a segment
    int s, g, nblk;   // its segment's sequence, kv head and block count
    int64_t a_sg;     // global index of tile (s, g, 0)
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
    __device__ static void issue(TileT& t, const TileRef& r, int lane) {
#pragma unroll
        for (int i = 0; i < kNld; ++i) t.k[i] = rsrc_load16(r.k, lane * 16 + i * 1024);
#pragma unroll
        for (int i = 0; i < kNld; ++i) t.v[i] = rsrc_load16(r.v, lane * 16 + i * 1024);
    }
    __device__ static void reset(State& x) {
        x.st.m[0] = -INFINITY;
        x.st.l[0] = 0.0f;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) x.st.o[0][e] = 0.0f;
    }
    template <bool kPartial>
    __device__ static void consume(State& x, const TileT& t, int nvalid, const QT& q, float sscale,
                                   int lane) {
        const QT qs[1] = {q};
        consume_tile<KV, D, 1, kPartial>(x.st, t, nvalid, qs, sscale, lane / kLpt);
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

// Matrix-core math for G grouped query heads (16-bit caches).
template <int KV, int D, int G>
struct MfmaMath {
    using Gm = MfmaGeo<D>;
    static constexpr int kG = G;
    static constexpr bool kPrefetchQ = false;  // fetched into LDS at segment start
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
    __device__ static void issue(TileT& t, const TileRef& r, int lane) {
        const int koff = (lane & 15) * Gm::kRowBytes + 16 * (lane >> 4);
#pragma unroll
        for (int c = 0; c < kNk; ++c) t.k[c] = rsrc_load16(r.k, koff + 64 * c);
#pragma unroll
        for (int i = 0; i < kNv; ++i) t.v[i] = rsrc_load16(r.v, lane * 16 + 1024 * i);
    }
    __device__ static void reset(State& x) {
#pragma unroll
        for (int j = 0; j < kNd; ++j) x.o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        x.m = -INFINITY;
        x.lsum = 0.0f;
    }
    template <bool kPartial>
    __device__ static void consume(State& x, const TileT& t, int nvalid, const QT&, float sscale,
                                   int lane) {
        mfma_consume<KV, D, kPartial>(t, nvalid, QLds<D>{x.qlds}, x.o, x.m, x.lsum, sscale, x.stage,
                                      lane);
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

template <class M, int KV, int D, int NBUF>
__global__ __launch_bounds__(256) void decode_balanced_kernel(const DecodeParams p) {
    constexpr int G = M::kG;
    constexpr int SS = SlotGeoB<D>::kStride;
    const int lane = threadIdx.x & 63;
    const int wv_in = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x * 4 + wv_in;
    const int W = p.num_waves;

    // Total tiles of the batch, then this wave's range [t0, t1).
    int64_t total = 0;
    for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {
        const int jj = c0 + lane;
        total += wave_sum(jj < p.num_seqs ? (seq_tokens(p, jj) + 15) >> 4 : 0);
    }
    total *= p.num_kv_heads;
    // R non-empty ranges: with fewer tiles than waves the surplus waves idle,
    // so every wave of a split context really holds a piece of it.
    const int R = static_cast<int>(total < W ? total : W);
    if (w >= R) return;
    const int64_t t0 = range_start(total, w, R);
    const int64_t t1 = range_start(total, w + 1, R);
    const int n = static_cast<int>(t1 - t0);

    // Locate tile t0: the sequence holding it, then its head and block.
    TileWalk tw;
    bool found = false;
    {
        int64_t carry = 0;
        for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {  // t0 < total: some chunk holds it
            const int jj = c0 + lane;
            const int len = jj < p.num_seqs ? seq_tokens(p, jj) : 0;
            const int tiles = ((len + 15) >> 4) * p.num_kv_heads;
            const int incl = wave_incl_scan(tiles, lane);
            const uint64_t hit = __ballot(jj < p.num_seqs && carry + incl > t0);
            if (hit) {
                const int ln = __builtin_ffsll(static_cast<long long>(hit)) - 1;
                tw.s = c0 + ln;
                tw.chunk = c0 >> 6;
                tw.lens = len;
                tw.L = __builtin_amdgcn_readlane(len, ln);
                tw.nblk = (tw.L + 15) >> 4;
                const int64_t a_s = carry + __builtin_amdgcn_readlane(incl - tiles, ln);
                const int64_t off = t0 - a_s;
                tw.g = static_cast<int>(off / tw.nblk);
                tw.j = static_cast<int>(off % tw.nblk);
                tw.a_sg = a_s + static_cast<int64_t>(tw.g) * tw.nblk;
                found = true;
                break;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
    }
    if (!found) return;  // lengths changed between the two passes
    walk_enter_row(p, tw, lane);

    __shared__ __attribute__((aligned(16))) uint8_t stage_all[4][MfmaGeo<D>::kStage];
    __shared__ __attribute__((aligned(16))) uint8_t q_all[4][G > 1 ? MfmaGeo<D>::kNk * 1024 : 16];
    typename M::State st;
    if constexpr (G > 1) {
        st.stage = stage_all[wv_in];
        st.qlds = q_all[wv_in];
    }
    M::reset(st);
    typename M::QT q;
    typename M::QT qring[M::kPrefetchQ ? NBUF : 1];

    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * M::kTB;
    typename M::TileT tr[NBUF];
    SlotInfo si[NBUF];

    // Issue tile kn of the range into a ring slot (and the q of a segment
    // that starts there).
    auto issue = [&](typename M::TileT& tt, SlotInfo& info, typename M::QT& qq, int kn) {
        if (kn >= n) {
            info.nvalid = 0;
            info.flags = 0;
            const TileRef r = tile_ref(p, p.k_plane, p.v_plane, bstride, M::kTB, -1, 0, 0);
            M::issue(tt, r, lane);
            return;
        }
        if (kn > 0) walk_advance(p, tw, lane);
        const bool first = kn == 0 || tw.j == 0;
        const bool last = kn == n - 1 || tw.j == tw.nblk - 1;
        info.flags = (first ? 1 : 0) | (last ? 2 : 0);
        info.s = tw.s;
        info.g = tw.g;
        info.nblk = tw.nblk;
        info.a_sg = tw.a_sg;
        if constexpr (M::kPrefetchQ) {
            if (first) M::fetch_q(p, qq, tw.s, tw.g, lane);
        }
        const uint8_t* kpl = p.k_plane + static_cast<size_t>(tw.g) * M::kTB;
        const uint8_t* vpl = p.v_plane + static_cast<size_t>(tw.g) * M::kTB;
        const TileRef r =
            tile_ref(p, kpl, vpl, bstride, M::kTB, walk_id(p, tw, lane), tw.j * 16, tw.L);
        info.nvalid = r.nvalid;
        M::issue(tt, r, lane);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(tr[x], si[x], qring[M::kPrefetchQ ? x : 0], x);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            const SlotInfo cur = si[x];
            if (cur.flags & 1) {
                if constexpr (M::kPrefetchQ)
                    q = qring[x];
                else
                    M::fetch_q_lds(p, st, cur.s, cur.g, lane);
            }
            if (cur.nvalid == 16)
                M::template consume<false>(st, tr[x], 16, q, p.scale_log2, lane);
            else if (cur.nvalid > 0)
                M::template consume<true>(st, tr[x], cur.nvalid, q, p.scale_log2, lane);
            if (cur.flags & 2) {
                // End of a segment: write the output, or the partial of a split context.
                M::finish(st);
                if (cur.a_sg >= t0 && cur.a_sg + cur.nblk <= t1) {
                    M::store_out(p, st, cur.s, cur.g, lane);
                } else {  // split context: slot 0 if it began before this range, else 1
                    const int slot = (cur.a_sg <= t0) ? 0 : 1;
                    M::store_partial(p.slots + static_cast<size_t>(w * 2 + slot) * G * SS, st, lane);
                }
                M::reset(st);
            }
            issue(tr[x], si[x], qring[M::kPrefetchQ ? x : 0], k0 + x + NBUF);
        }
    }
}

// Second kernel of the balanced single pass: one workgroup per (kv head,
// sequence). It recomputes the split of the batch into R ranges, and for a
// context that was split merges the partials its waves left in their slots;
// it also writes the zeros of an empty context. Contexts held by one wave
// were written by the streaming kernel and are left alone. A thread owns 4
// dims of one head; a long context is split over tens of waves, so both
// passes over the partials (their maximum, then the weighted sum) keep
// several independent loads in flight.
template <int KV, int D, int G>
__global__ __launch_bounds__(256) void balanced_merge_kernel(const DecodeParams p) {
    constexpr int SS = SlotGeoB<D>::kStride;
    const int g = blockIdx.x, s = blockIdx.y, lane = threadIdx.x & 63;
    int64_t total = 0, before = 0;  // blocks of the batch, and of sequences < s
    for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {
        const int jj = c0 + lane;
        const int nb = jj < p.num_seqs ? (seq_tokens(p, jj) + 15) >> 4 : 0;
        total += wave_sum(nb);
        before += wave_sum(jj < s ? nb : 0);
    }
    const int nblk = (seq_tokens(p, s) + 15) >> 4;
    uint16_t* out = static_cast<uint16_t*>(p.out) +
                    (static_cast<size_t>(s) * p.num_q_heads + g * G) * D;
    const int t = threadIdx.x;
    if (nblk == 0) {
        for (int idx = t; idx < G * D; idx += 256) out[idx] = 0;
        return;
    }
    total *= p.num_kv_heads;
    const int R = static_cast<int>(total < p.num_waves ? total : p.num_waves);
    const int64_t a_sg = before * p.num_kv_heads + static_cast<int64_t>(g) * nblk;
    const int wa = wave_of(a_sg, total, R);
    const int wb = wave_of(a_sg + nblk - 1, total, R);
    if (wa == wb) return;  // written whole by its wave
    // Wave wa's piece began before its range: slot 1; waves after it: slot 0.
    const int slot_a = (a_sg <= range_start(total, wa, R)) ? 0 : 1;
    for (int idx = t; idx < G * D / 4; idx += 256) {
        const int h = idx / (D / 4), d = (idx % (D / 4)) * 4;
        const float* base = p.slots + static_cast<size_t>(h) * SS;
        auto part = [&](int v) -> const float* {
            const int slot = v == wa ? slot_a : 0;
            return base + static_cast<size_t>(v * 2 + slot) * G * SS;
        };
        float mx = -INFINITY;
#pragma unroll 8
        for (int v = wa; v <= wb; ++v) mx = fmaxf(mx, part(v)[D]);
        const float ms = (mx == -INFINITY) ? 0.0f : mx;
        float wsum = 0.0f;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
        for (int v = wa; v <= wb; ++v) {
            const float* hs = part(v);
            const float4 ov = *reinterpret_cast<const float4*>(hs + d);
            const float wv = hs[D + 1] * fast_exp2(hs[D] - ms);
            wsum += wv;
            acc = make_float4(fmaf(wv, ov.x, acc.x), fmaf(wv, ov.y, acc.y), fmaf(wv, ov.z, acc.z),
                              fmaf(wv, ov.w, acc.w));
        }
        const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
        *reinterpret_cast<uint2*>(out + h * D + d) =
            make_uint2(pack2<KV>(acc.x * inv, acc.y * inv), pack2<KV>(acc.z * inv, acc.w * inv));
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
    if constexpr (KV != PKV_FP8_E4M3 && G >= 2) {
        // Grouped heads on a 16-bit cache: matrix cores (q dtype = cache dtype).
        // Ring of 2 tiles at D = 128 keeps two waves per SIMD (4 at D = 64: three).
        hipLaunchKernelGGL((decode_mfma_kernel<KV, D, G, NW, (D == 128 ? 2 : 4)>), grid,
                           dim3(NW * 64), 0, stream, prm);
    } else {
        hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, ring_depth<KV, D, G>()>), grid,
                           dim3(NW * 64), 0, stream, prm);
    }
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

// Waves of a balanced launch: two per SIMD on every CU, which every balanced
// kernel instance can hold at once (so all ranges run concurrently).
constexpr int kBalancedWavesPerCu = 8;
constexpr int kBalancedMaxSeqs = 4096;  // each wave scans the lengths of the batch

int device_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        return 256;  // MI355X
    }
    return cus;
}

// Balanced-path workspace: 2 partial slots per wave, of G heads x (D + 4) floats.
size_t balanced_bytes(size_t group, size_t head_dim, size_t waves) {
    return waves * 2 * group * (head_dim + 4) * sizeof(float);
}

// The balance rests on every wave of the launch being resident at once: the
// launch is as wide as the kernel instance's occupancy allows on this device,
// capped at kBalancedWavesPerCu (the width the workspace is sized for).
template <class M, int KV, int D, int NBUF>
hipError_t launch_balanced(DecodeParams prm, int cus, hipStream_t st) {
    static int wgs_per_cu = -1;  // per kernel instance; the same on every gfx950 device
    if (wgs_per_cu < 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb, reinterpret_cast<const void*>(&decode_balanced_kernel<M, KV, D, NBUF>), 256,
                0) != hipSuccess)
            return hipGetLastError();
        wgs_per_cu = std::max(1, std::min(nb, kBalancedWavesPerCu / 4));
    }
    prm.num_waves = cus * wgs_per_cu * 4;
    hipLaunchKernelGGL((decode_balanced_kernel<M, KV, D, NBUF>), dim3(prm.num_waves / 4),
                       dim3(256), 0, st, prm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((balanced_merge_kernel<KV, D, M::kG>),
                       dim3(static_cast<uint32_t>(prm.num_kv_heads), static_cast<uint32_t>(prm.num_seqs)),
                       dim3(256), 0, st, prm);
    return hipGetLastError();
}

// Ring depths keep two waves per SIMD (MFMA at D = 128 holds its O^T
// accumulators beside the ring, with Q^T in LDS: three tiles).
template <int KV, int D>
hipError_t balanced_by_group(int G, const DecodeParams& prm, int cus, hipStream_t st) {
    constexpr int R = (D == 128) ? 3 : 4;
    switch (G) {
        case 1: return launch_balanced<ValuMath<KV, D>, KV, D, 4>(prm, cus, st);
        case 2: return launch_balanced<MfmaMath<KV, D, 2>, KV, D, R>(prm, cus, st);
        case 4: return launch_balanced<MfmaMath<KV, D, 4>, KV, D, R>(prm, cus, st);
        default: return launch_balanced<MfmaMath<KV, D, 8>, KV, D, R>(prm, cus, st);
    }
}

template <int KV>
hipError_t balanced_by_dim(int D, int G, const DecodeParams& prm, int cus, hipStream_t st) {
    if (D == 64) return balanced_by_group<KV, 64>(G, prm, cus, st);
    return balanced_by_group<KV, 128>(G, prm, cus, st);
}

}  // namespace

extern "C" size_t paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
    if (partition_size < 0 || num_seqs < 0 || num_q_heads < 0 || head_dim <= 0 ||
        max_context_len < 0)
        return 0;
    if (partition_size == 0) {
        // Balanced single pass; bounded for any kv head count and group <= 8.
        if (num_seqs > kBalancedMaxSeqs) return 0;
        const size_t waves = static_cast<size_t>(device_cu_count()) * kBalancedWavesPerCu;
        return balanced_bytes(std::min(num_q_heads, 8), head_dim, waves);
    }
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
        if (workspace != nullptr && pkv::is_16bit(d.kv_dtype) && num_seqs <= kBalancedMaxSeqs) {
            // Balanced single pass over the whole batch.
            const int cus = device_cu_count();
            const int waves = cus * kBalancedWavesPerCu;
            const size_t need = balanced_bytes(G, d.head_dim, waves);
            if (workspace_bytes < need)
                return fail(PKV_ERR_INVALID, "paged_attn_decode: workspace of %zu bytes, %zu needed",
                            workspace_bytes, need);
            if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
                return fail(PKV_ERR_INVALID, "paged_attn_decode: workspace must be 256-byte aligned");
            prm.slots = static_cast<float*>(workspace);
            prm.num_seqs = num_seqs;
            const hipError_t eb = (d.kv_dtype == PKV_F16)
                                      ? balanced_by_dim<PKV_F16>(d.head_dim, G, prm, cus, stream)
                                      : balanced_by_dim<PKV_BF16>(d.head_dim, G, prm, cus, stream);
            if (eb != hipSuccess)
                return fail(PKV_ERR_HIP, "paged_attn_decode: launch failed: %s", hipGetErrorString(eb));
            return PKV_OK;
        }
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
