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
//  * block ids for a wave's next 64 blocks are fetched with one vector load
//    and broadcast with readlane; tiles are loaded in batches whose loads are
//    all issued before the first tile of the batch is consumed;
//  * split-K: with partition_size > 0 each workgroup covers one partition and
//    writes (m, l, o) to the workspace; paged_attn_reduce merges them.

#include <hip/hip_runtime.h>

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

// Issue the loads of one (block, kv head) tile: NLD contiguous KiB per plane.
template <int KV, int D>
__device__ __forceinline__ void load_tile(Tile<KV, D>& t, const uint8_t* kp, const uint8_t* vp) {
#pragma unroll
    for (int i = 0; i < Geo<KV, D>::kNld; ++i)
        t.k[i] = *reinterpret_cast<const uint4*>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < Geo<KV, D>::kNld; ++i)
        t.v[i] = *reinterpret_cast<const uint4*>(vp + i * 1024);
}

// Fold one tile into the lane's online-softmax state. nvalid = number of
// leading tokens of the tile that belong to the context (0..16).
template <int KV, int D, int G>
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
    for (int i = 0; i < NLD; ++i) valid[i] = (i * TPI + row) < nvalid;
#pragma unroll
    for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = valid[i] ? sc[h][i] : -INFINITY;
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
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = valid[i] ? vf[e] : 0.0f;  // stale bytes never enter
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) st.o[h][e] = fmaf(sc[h][i], vf[e], st.o[h][e]);
    }
}

template <int KV, int QD, int D, int G, int NW, int BATCH>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt;

    const int part = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;

    int L = p.context_lens[s];
    L = min(L, p.max_ctx);
    L = min(L, p.max_blocks * 16);
    const int nblk = L > 0 ? (L + 15) >> 4 : 0;
    int b0 = 0, b1 = nblk;
    if (p.blocks_per_part > 0) {
        b0 = part * p.blocks_per_part;
        if (b0 >= nblk) return;  // whole workgroup: this partition holds no tokens
        b1 = min(b0 + p.blocks_per_part, nblk);
    }

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

    const int32_t* bt = p.block_tables + static_cast<size_t>(s) * p.max_blocks;
    const size_t lane_off = static_cast<size_t>(g) * Gm::kTileBytes + lane * 16;
    const size_t block_stride = static_cast<size_t>(p.num_kv_heads) * Gm::kTileBytes;
    const int span = b1 - b0;
    const int nmine = span > w ? (span - w + NW - 1) / NW : 0;

    for (int c0 = 0; c0 < nmine; c0 += 64) {
        const int cnt = min(64, nmine - c0);
        // Ids of this wave's next (up to) 64 blocks, one per lane.
        const int myid = (lane < cnt) ? bt[b0 + w + (c0 + lane) * NW] : 0;

        // An id outside [0, num_blocks) is not dereferenced: block 0 is read
        // instead (the host guarantees num_blocks > 0) and all its tokens are
        // masked out.
        auto tile_addr = [&](int kk, int& nvalid) -> size_t {
            const int id = __builtin_amdgcn_readlane(myid, kk);
            const int j = b0 + w + (c0 + kk) * NW;
            const int okm = -static_cast<int>(id >= 0 && id < p.num_blocks);  // all ones or 0
            nvalid = min(L - j * 16, 16) & okm;
            return static_cast<size_t>(static_cast<uint32_t>(id & okm)) * block_stride + lane_off;
        };

        // Tiles are fetched in batches of BATCH: all loads of a batch are
        // issued before the first tile is consumed (16 KiB per wave in flight
        // at BATCH = 2), and the scheduler may interleave the consumes. A
        // batch that runs past the wave's last block re-reads that block
        // (an L2 hit) and masks it out.
        for (int kk = 0; kk < cnt; kk += BATCH) {
            Tile<KV, D> t[BATCH];
            int nv[BATCH];
#pragma unroll
            for (int x = 0; x < BATCH; ++x) {
                const size_t off = tile_addr(min(kk + x, cnt - 1), nv[x]);
                load_tile<KV, D>(t[x], p.k_plane + off, p.v_plane + off);
                if (kk + x >= cnt) nv[x] = 0;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < BATCH; ++x) consume_tile<KV, D, G>(st, t[x], nv[x], qs, sscale, row);
        }
    }

    // Merge the TPI rows of this wave: lanes lane ^ off (off = LPT, 2*LPT, ...)
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

    float vscale = 1.0f;
    if constexpr (KV == PKV_FP8_E4M3) vscale = p.v_scale[g];
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
            if (d == 0) {
                p.ws_ml[slot * 2] = (mx == -INFINITY) ? -INFINITY : mx * kLn2;
                p.ws_ml[slot * 2 + 1] = lsum;
            }
        } else {
            const size_t o_idx = (static_cast<size_t>(s) * p.num_q_heads + qh) * D + d;
            uint16_t bits = (QD == PKV_F16) ? f32_to_f16_bits(res) : f32_to_bf16_bits(res);
            static_cast<uint16_t*>(p.out)[o_idx] = bits;
        }
    }
}

constexpr int kWaves = 4;

// Tiles per load batch: two for 16-bit MHA tiles; one where the group's
// registers are already large.
template <int KV, int D, int G>
constexpr int batch_for() {
    return (G <= 2) ? 2 : 1;
}

template <int KV, int QD, int D, int G>
hipError_t launch(const DecodeParams& prm, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, kWaves, batch_for<KV, D, G>()>), grid,
                       dim3(kWaves * 64), 0, stream, prm);
    return hipGetLastError();
}

template <int KV, int QD, int D>
hipError_t by_group(int G, const DecodeParams& prm, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: return launch<KV, QD, D, 1>(prm, grid, st);
        case 2: return launch<KV, QD, D, 2>(prm, grid, st);
        case 4: return launch<KV, QD, D, 4>(prm, grid, st);
        default: return launch<KV, QD, D, 8>(prm, grid, st);
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
    return static_cast<size_t>(num_seqs) * num_q_heads * parts * (2 + static_cast<size_t>(head_dim)) *
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
    if (d.num_kv_heads > 65535)
        return fail(PKV_ERR_INVALID, "paged_attn_decode: too many kv heads");
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
        if (P > 0x7FFFFFFF) return fail(PKV_ERR_INVALID, "paged_attn_decode: too many partitions");
        parts = static_cast<uint32_t>(P);
        prm.blocks_per_part = partition_size / 16;
        prm.num_parts = static_cast<int32_t>(P);
        prm.ws_ml = static_cast<float*>(workspace);
        prm.ws_o = prm.ws_ml + static_cast<size_t>(num_seqs) * num_q_heads * P * 2;
    } else {
        if (out == nullptr) return fail(PKV_ERR_INVALID, "paged_attn_decode: out is NULL");
        prm.blocks_per_part = 0;
        prm.num_parts = 1;
    }

    const dim3 grid(parts, static_cast<uint32_t>(d.num_kv_heads), static_cast<uint32_t>(num_seqs));
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
