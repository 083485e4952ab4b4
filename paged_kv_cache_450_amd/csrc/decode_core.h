// Shared pieces of the decode kernels: launch parameters, tile descriptors
// and loads, the longest-first sequence order, the split of a workgroup's
// work into per-wave tile streams, the block-id stream, partial stores and the
// cross-wave merge, and the wave-level scans of the balanced split.
#pragma once

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
    int32_t head_group;       // waves that walk one range in step, one kv head each
    int32_t num_seqs;
    // Fused append (NULL: none): the new token of every sequence, K and V rows
    // [B][Hkv][D] of the 16-bit source dtype (the q dtype).
    const uint8_t* new_k;
    const uint8_t* new_v;
    int32_t window;           // > 0: attend over the last `window` tokens only
    // Shared-prefix decode (pre_blocks NULL: none). The prefix kernel reads the
    // leading blocks a group of sequences shares once for all its members and
    // leaves their partials in `pre`; the balanced pass starts each member
    // after them, and the merge folds the two together.
    const int32_t* pre_blocks;     // [B] leading blocks covered by the prefix kernel (0: none)
    float* pre;                    // [B][Hq][D + 4] prefix partials: o / l, m (log2), l
    float* suf;                    // [B][Hq][D + 4] partials of members' contexts whole in one wave
    const int32_t* group_offsets;  // [num_groups + 1] into group_members
    const int32_t* group_members;  // sequence indices, group by group
    const int32_t* group_blocks;   // [num_groups] shared leading blocks of each group
    int32_t num_groups;
    int32_t pre_slots;             // prefix workgroups per (group, kv head)
    // Shared leading blocks read through the L2 (keep_blocks NULL: none): the
    // balanced pass reads the first keep_blocks[s] blocks of sequence s, which
    // other sequences of the batch share, with the caching load policy, so
    // that the sharers' repeated reads can hit the L2 instead of HBM.
    const int32_t* keep_blocks;    // [B]
    // Balanced pass of a fused step (new_k / new_v set): a sequence whose
    // last position is the new token reads its blocks without that position
    // and the token itself as one more tile, taken from the source rows; the
    // wave that reads that tile stores the rows to the token's slot.
    int32_t fold_new;
};

// 1 when the last position of sequence j (its clamped length L) is the new
// token a fused step stores: L >= 1 and the context is not clamped.
__device__ __forceinline__ int new_of(const DecodeParams& p, int j) {
    const int raw = p.context_lens[j];
    const int L = min(max(raw, 0), min(p.max_ctx, p.max_blocks * 16));
    return (L >= 1 && raw == L) ? 1 : 0;
}

// Leading blocks of sequence j to read with the caching policy (0 without a hint).
__device__ __forceinline__ int keep_of(const DecodeParams& p, int j) {
    return p.keep_blocks != nullptr ? max(p.keep_blocks[j], 0) : 0;
}

// First token a sequence of L tokens attends over (sliding window).
__device__ __forceinline__ int window_lo(const DecodeParams& p, int L) {
    return p.window > 0 ? max(0, L - p.window) : 0;
}

// Blocks a decode reads of a sequence of L tokens: [window_lo / 16, ceil(L / 16)).
__device__ __forceinline__ int window_blocks(const DecodeParams& p, int L) {
    return ((L + 15) >> 4) - (window_lo(p, L) >> 4);
}

// Leading blocks of sequence j that the shared-prefix kernel covers (0 without one).
__device__ __forceinline__ int pre_of(const DecodeParams& p, int j) {
    return p.pre_blocks != nullptr ? max(p.pre_blocks[j], 0) : 0;
}

// First block the balanced pass reads of a sequence of L tokens whose first
// `pre` blocks the shared-prefix kernel covers (sliding window: its first block).
__device__ __forceinline__ int first_block(const DecodeParams& p, int L, int pre) {
    return max(window_lo(p, L) >> 4, min(pre, (L + 15) >> 4));
}

// Tiles per kv head the balanced pass reads of that sequence.
__device__ __forceinline__ int pass_tiles(const DecodeParams& p, int L, int pre) {
    return ((L + 15) >> 4) - first_block(p, L, pre);
}

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

// The same load with the default policy, for bytes that other workgroups on
// the same XCD are about to read too: the lines stay in its L2.
__device__ __forceinline__ uint4 rsrc_load16_kept(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
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

// The work of one wave: sequence s, its length L as this kernel reads it, the
// first token it attends over (lo, > 0 with a sliding window), and its tiles,
// the logical blocks b0 + w + k*NW for k < n (the partition's blocks from the
// window's first on, dealt round robin to the NW waves of the workgroup).
// newk: the index of the tile holding the token a fused append writes
// (position L - 1), when this wave reads it; else -1. fold: this wave is the
// first wave of the workgroup that reads the context's first attended block
// (kFused calls; the FP8 kernel folds the new token in there, so the extra
// work falls on a workgroup dispatched early).
struct WaveWork {
    int s, L, lo, b0, n, newk;
    bool fold;
};

// Grid (kv head, sequence, partition), kv head fastest. Workgroups are dealt
// to the 8 XCDs round robin in linear order, so consecutive indices must carry
// comparable work: the heads of one sequence do (same length), while
// partitions do not (short sequences have no late partitions).
// Returns false when the workgroup has no tokens; every wave of the
// workgroup takes the same branch.
template <int G, int D, int NW, bool kFused = false>
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
    const int lo = window_lo(p, L);
    int b0 = lo >> 4, b1 = nblk;
    if (p.blocks_per_part > 0) {
        const int pb0 = part * p.blocks_per_part;
        b1 = min(pb0 + p.blocks_per_part, nblk);
        b0 = max(pb0, lo >> 4);
        if (b0 >= b1) {
            // No tokens in this partition (past the table's reach, or before
            // the window). If the reduce will still read it, leave an empty
            // partial.
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
    ww.lo = lo;
    ww.b0 = b0 + w;
    ww.n = span > w ? (span - w + NW - 1) / NW : 0;
    // The fused append writes position L - 1 only when the context is whole
    // here (not clamped): otherwise its last token lies outside this call.
    ww.newk = -1;
    ww.fold = false;
    if constexpr (kFused) {
        const bool whole = p.context_lens[s] == L;
        if (ww.n > 0 && ww.b0 + (ww.n - 1) * NW == nblk - 1 && whole) ww.newk = ww.n - 1;
        ww.fold = whole && L > 0 && w == 0 && b0 == (lo >> 4);
    }
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

// Descriptors of the K and V tiles of block `id` for kv head g, and the
// tile's attended tokens [nlo, nvalid): the context ends before token nvalid,
// a sliding window starts at token nlo (0 without one). An id outside the pool,
// or past the end (-1), gives size-0 descriptors and no tokens.
struct TileRef {
    __amdgpu_buffer_rsrc_t k, v;
    int nvalid, nlo;
};

__device__ __forceinline__ TileRef tile_ref(const DecodeParams& p, const uint8_t* kpl,
                                            const uint8_t* vpl, size_t bstride, int tile_bytes,
                                            int id, int first_token, int L, int lo) {
    const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks);
    const size_t off = static_cast<size_t>(ok ? id : 0) * bstride;
    const int bytes = ok ? tile_bytes : 0;
    TileRef t;
    t.k = tile_rsrc(kpl + off, bytes);
    t.v = tile_rsrc(vpl + off, bytes);
    t.nvalid = ok ? min(L - first_token, 16) : 0;
    t.nlo = ok ? min(max(lo - first_token, 0), 16) : 0;
    return t;
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

// Tokens of a context of raw length `raw` as this kernel reads it (clamped
// like the other paths).
__device__ __forceinline__ int clamp_tokens(const DecodeParams& p, int raw) {
    return min(max(raw, 0), min(p.max_ctx, p.max_blocks * 16));
}
__device__ __forceinline__ int seq_tokens(const DecodeParams& p, int j) {
    return clamp_tokens(p, p.context_lens[j]);
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

// ---------------------------------------------------------------------------
// Fused append (16-bit caches, vector-ALU decode). The new token of a sequence
// is the last position L - 1 of its context; the one wave that reads the tile
// holding it takes the token's K and V from the source rows instead of the
// pool (the pool bytes it loaded for that row are discarded), and writes them
// to the token's slot. No other wave reads that slot: it lies in the
// sequence's own last block, which is never shared while tokens are written
// into it.
//
// The wave fetches the source rows before its tile ring fills (one 16-byte
// chunk per lane: lanes 0..15 K, lanes 16..31 V, chunk = lane mod the row's
// chunk count) and parks them in 512 bytes of its LDS once they land, so no
// register is held across the ring for them.
template <int D>
struct NewSrc {
    static constexpr int kChunks = D * 2 / 16;  // 16-byte chunks of a 16-bit row
    uint4 x;

    __device__ __forceinline__ void fetch(const DecodeParams& p, int s, int g, int lane) {
        const uint8_t* row = ((lane & 16) ? p.new_v : p.new_k) +
                             (static_cast<size_t>(s) * p.num_kv_heads + g) * (D * 2);
        x = *reinterpret_cast<const uint4*>(row + (lane & (kChunks - 1)) * 16);
    }
    // Copy the rows to 512 bytes of LDS: K chunk c at 16c, V chunk c at 256 + 16c.
    __device__ __forceinline__ void stash(uint8_t* lds, int lane) const {
        if (lane < 32)
            *reinterpret_cast<uint4*>(lds + (lane & 16) * 16 + (lane & (kChunks - 1)) * 16) = x;
    }
};

// Source chunk c of the new token's K (kv = 0) or V (kv = 1) row, from LDS.
__device__ __forceinline__ uint4 new_chunk(const uint8_t* lds, int kv, int c) {
    return *reinterpret_cast<const uint4*>(lds + kv * 256 + c * 16);
}

// Replace the new token's row in the loads of a tile read in natural layout
// (lane l of load i holds bytes (l % LPR) * 16 of token i * (64 / LPR) +
// l / LPR). val holds, on every lane, the bytes for its column.
template <int LPR, int N>
__device__ __forceinline__ void patch_natural(uint4 (&r)[N], const uint4& val, int off, int lane) {
    constexpr int kTpi = 64 / LPR;
    const bool row = lane / LPR == off % kTpi;
    const int i0 = off / kTpi;
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (i == i0 && row) r[i] = val;
}

// Write the new token's cache row (LPR lanes of 16 bytes: lane c stores
// column c of kval and vval) to offset off of block id, kv head g.
template <int LPR>
__device__ __forceinline__ void store_new_row(const DecodeParams& p, int g, int id, int off,
                                              int tile_bytes, const uint4& kval,
                                              const uint4& vval, int lane) {
    if (lane >= LPR) return;
    const size_t at = (static_cast<size_t>(id) * p.num_kv_heads + g) * tile_bytes +
                      static_cast<size_t>(off) * (LPR * 16) + lane * 16;
    *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.k_plane) + at) = kval;
    *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.v_plane) + at) = vval;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

}  // namespace
