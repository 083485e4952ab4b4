// paged_attn_decode: single-query attention over a paged KV cache.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", section
// "PagedAttention：把操作系统的虚拟内存搬进 GPU": the attention kernel must read
// K/V correctly from non-contiguous physical blocks through the page table
// without giving up speed; the page names block prefetching and regrouping KV
// in on-chip memory as the CUDA techniques used (prior art here, not a plan).
// [P3] "突破大模型推理瓶颈：...", section 2.4: accumulate in FP32.
//
// gfx950 design (decode is HBM-bound: about 1 flop per KV byte for MHA).
// The kernels share one contract and one set of helpers:
//  * decode_valu.h: vector-ALU math, one workgroup of NW wave64s per (kv
//    head, sequence, partition): one query head per kv head on 16-bit caches,
//    and every FP8 cache;
//  * decode_mfma.h: the same work split with both products on matrix cores,
//    for grouped query heads on 16-bit caches;
//  * decode_balanced.h: the balanced single pass (equal tile ranges, one per
//    resident wave) with either math, and the kernel that merges contexts
//    split between waves;
//  * decode_prefix.h: the shared-prefix kernel, which reads the leading
//    blocks a group of sequences shares once for all of them ahead of the
//    balanced pass (paged_attn_decode_prefix).
// Common to all (decode_core.h):
//  * a (block, kv head) tile of 16 tokens x D is contiguous, and tiles are
//    read with raw buffer loads whose descriptor is built per tile from the
//    (wave-uniform) block id; a tile past the end of a range, or with an id
//    outside the pool, gets a descriptor of size 0, so its loads return zeros
//    and move no bytes; KV loads carry the non-temporal policy;
//  * each wave streams its tiles through a ring of tiles held in registers:
//    as soon as a tile is folded into the softmax state, its registers are
//    refilled with the tile the ring's depth ahead, so loads stay in flight
//    from the wave's first tile to its last;
//  * block ids for a wave's next 64 tiles are fetched with one vector load and
//    broadcast with readlane; the following 64 are always in flight;
//  * the grid is (kv head, sequence, partition), kv head fastest, so that
//    workgroups dealt round robin to the 8 XCDs carry comparable work;
//  * softmax runs online in base 2 with log2(e) folded into the scale, in
//    fp32; partials merge with the log-sum-exp rule;
//  * split-K: with partition_size > 0 each workgroup covers one partition and
//    writes (m, l, o) to the workspace; paged_attn_reduce merges them.
// This file holds the launch choices and the C entry points.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"
#include "decode_balanced.h"
#include "decode_core.h"
#include "decode_mfma.h"
#include "decode_prefix.h"
#include "decode_valu.h"
#include "device.h"

namespace {

using namespace pkv::dev;

// Tiles kept in flight per wave: the ring must fit beside the softmax state
// of the G heads. On 16-bit caches three tiles leave room for a third wave per
// SIMD (measured 0.7% faster on the 13B layer than four at two waves); FP8
// tiles are half the size and keep four.
template <int KV, int D, int G>
constexpr int ring_depth() {
    if constexpr (KV != PKV_FP8_E4M3 && G <= 2) return 3;
    return (G <= 2) ? 4 : (G == 4 ? 2 : 1);
}

// Tile ring of the vector-ALU kernel: registers (false) or two tiles of LDS
// filled by direct buffer-to-LDS loads (true), on 16-bit caches and on FP8
// caches (up to two query heads per kv head).
constexpr bool kLdsRing = true;
constexpr bool kLdsRingFp8 = false;

template <int KV, int QD, int D, int G, int NW>
hipError_t launch(const DecodeParams& prm, dim3 grid, hipStream_t stream) {
    if constexpr (KV != PKV_FP8_E4M3 && G >= 2) {
        // Grouped heads on a 16-bit cache: matrix cores (q dtype = cache dtype).
        // Ring of 2 tiles at D = 128 keeps two waves per SIMD (4 at D = 64: three).
        hipLaunchKernelGGL((decode_mfma_kernel<KV, D, G, NW, (D == 128 ? 2 : 4)>), grid,
                           dim3(NW * 64), 0, stream, prm);
    } else if constexpr (KV != PKV_FP8_E4M3 && G == 1) {
        constexpr int R = kLdsRing ? 2 : ring_depth<KV, D, G>();
        if (prm.new_k != nullptr)  // the new tokens stored from inside the kernel
            hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, R, true, kLdsRing>), grid,
                               dim3(NW * 64), 0, stream, prm);
        else
            hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, R, false, kLdsRing>), grid,
                               dim3(NW * 64), 0, stream, prm);
    } else if constexpr (G <= 2) {
        constexpr int R = kLdsRingFp8 ? 2 : ring_depth<KV, D, G>();
        if (prm.new_k != nullptr)  // FP8: the new tokens folded in by the kernel
            hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, R, true, kLdsRingFp8>), grid,
                               dim3(NW * 64), 0, stream, prm);
        else
            hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, R, false, kLdsRingFp8>), grid,
                               dim3(NW * 64), 0, stream, prm);
    } else {
        hipLaunchKernelGGL((decode_kernel<KV, QD, D, G, NW, ring_depth<KV, D, G>()>), grid,
                           dim3(NW * 64), 0, stream, prm);
    }
    return hipGetLastError();
}

// The fused step's append as a kernel of its own (ahead of the decode, same
// stream), for the forms that do not store the new tokens themselves.
pkv_status append_first(const char* fn, const pkv_pool* pool, int32_t layer, const void* new_k,
                        const void* new_v, int32_t src_dtype, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, const float* k_scale, const float* v_scale,
                        hipStream_t stream) {
    const pkv_pool_desc& d = pool->desc;
    const int64_t reach =
        std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * 16);
    uint8_t* base = static_cast<uint8_t*>(pool->base);
    const hipError_t e = pkv::launch_append_last(
        d, base + pkv::layer_plane_offset(d, layer, 0), base + pkv::layer_plane_offset(d, layer, 1),
        new_k, new_v, src_dtype, block_tables, max_blocks_per_seq, context_lens, num_seqs,
        static_cast<int32_t>(reach), k_scale, v_scale, stream);
    if (e != hipSuccess)
        return pkv::fail(PKV_ERR_HIP, "%s: append launch failed: %s", fn, hipGetErrorString(e));
    return PKV_OK;
}

// Waves per workgroup: the blocks a sliding window touches (ceil(W / 16) + 1
// at most) are one wave's stream up to 17 blocks, two waves' up to 33; a
// whole split-K partition is one wave's up to 8 blocks, two waves' up to 17;
// longer ranges are shared by four waves and merged through LDS. Few tiles
// split four ways leave each wave's ring barely filled before it drains.
template <int KV, int QD, int D, int G>
hipError_t by_waves(const DecodeParams& prm, dim3 grid, hipStream_t st) {
    const int span = prm.blocks_per_part > 0              ? prm.blocks_per_part
                     : prm.window > 0 && prm.window <= 1024 ? (prm.window + 15) / 16 + 1
                                                            : 0;
    if (prm.blocks_per_part > 0 && prm.window <= 0) {
        // Whole split-K partitions: one wave up to 8 blocks, two up to 17, four
        // beyond (512-token partitions: FP8 long-context call 226.3 -> 223.6 us,
        // 16-bit 13B layer 120.1 -> 119.3 us against two waves; 256-token
        // partitions: 239.3 -> 238.0 and 121.2 -> 120.1 us against one). With a
        // sliding window most of a partition's blocks fall outside it, and the
        // spans below stay faster (FP8 long-context at W = 256: 26.2 against 28.2 us).
        if (span <= 8) return launch<KV, QD, D, G, 1>(prm, grid, st);
        if (span <= 17) return launch<KV, QD, D, G, 2>(prm, grid, st);
        return launch<KV, QD, D, G, 4>(prm, grid, st);
    }
    if (span > 0 && span <= 17) return launch<KV, QD, D, G, 1>(prm, grid, st);
    if (span > 0 && span <= 33) return launch<KV, QD, D, G, 2>(prm, grid, st);
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

template <class M, int KV, int D, int NBUF, bool kPre, bool kKeep, bool kFold>
hipError_t launch_balanced_as(DecodeParams prm, int cus, hipStream_t st) {
    static int wgs_per_cu = -1;  // per kernel instance; the same on every gfx950 device
    constexpr int kWpg = balanced_wpg<M>();
    if (wgs_per_cu < 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb,
                reinterpret_cast<const void*>(
                    &decode_balanced_kernel<M, KV, D, NBUF, kPre, kKeep, kFold>),
                kWpg * 64, 0) != hipSuccess)
            return hipGetLastError();
        wgs_per_cu = std::max(1, std::min(nb, kBalancedWavesPerCu / kWpg));
    }
    prm.num_waves = cus * wgs_per_cu * kWpg;
    // The waves of a workgroup walk one range, one kv head each: heads in groups
    // of kWpg when the head count allows, else of the largest power of two
    // dividing it.
    int hg = kWpg;
    while (prm.num_kv_heads % hg != 0) hg /= 2;
    prm.head_group = hg;
    hipLaunchKernelGGL((decode_balanced_kernel<M, KV, D, NBUF, kPre, kKeep, kFold>),
                       dim3(prm.num_waves / kWpg), dim3(kWpg * 64), 0, st, prm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kHpw = merge_heads_per_wg<D, M::kG>();
    hipLaunchKernelGGL((balanced_merge_kernel<KV, D, M::kG>),
                       dim3(static_cast<uint32_t>((prm.num_kv_heads + kHpw - 1) / kHpw),
                            static_cast<uint32_t>(prm.num_seqs)),
                       dim3(merge_threads<D, M::kG>() * kHpw), 0, st, prm);
    return hipGetLastError();
}

// The balance rests on every wave of the launch being resident at once: the
// launch is as wide as the kernel instance's occupancy allows on this device,
// capped at kBalancedWavesPerCu (the width the workspace is sized for).
template <class M, int KV, int D, int NBUF>
hipError_t launch_balanced(const DecodeParams& prm, int cus, hipStream_t st) {
    if (prm.pre_blocks != nullptr)
        return prm.fold_new ? launch_balanced_as<M, KV, D, NBUF, true, false, true>(prm, cus, st)
                            : launch_balanced_as<M, KV, D, NBUF, true, false, false>(prm, cus, st);
    if (prm.keep_blocks != nullptr)
        return prm.fold_new ? launch_balanced_as<M, KV, D, NBUF, false, true, true>(prm, cus, st)
                            : launch_balanced_as<M, KV, D, NBUF, false, true, false>(prm, cus, st);
    return prm.fold_new ? launch_balanced_as<M, KV, D, NBUF, false, false, true>(prm, cus, st)
                        : launch_balanced_as<M, KV, D, NBUF, false, false, false>(prm, cus, st);
}

// Tile ring of the balanced vector-ALU pass: two LDS slots per wave filled by
// direct buffer-to-LDS loads (true), or four tiles of registers (false). The
// LDS form measured 0.6% faster on the 7B layer (323.3-323.7 against
// 325.4-325.7 us per call).
constexpr bool kLdsRingBalanced = true;

// Ring depths keep two waves per SIMD (MFMA at D = 128 holds its O^T
// accumulators beside the ring, with Q^T in LDS: three tiles).
template <int KV, int D>
hipError_t balanced_by_group(int G, const DecodeParams& prm, int cus, hipStream_t st) {
    constexpr int R = (D == 128) ? 3 : 4;
    switch (G) {
        case 1:
            if constexpr (kLdsRingBalanced)
                return launch_balanced<ValuLdsMath<KV, D>, KV, D, 2>(prm, cus, st);
            else
                return launch_balanced<ValuMath<KV, D>, KV, D, 4>(prm, cus, st);
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

// Workspace of the shared-prefix decode: the balanced pass's slots (sized for
// any group, as paged_attn_workspace_bytes sizes them), then the prefix
// partials, then the members' suffix partials, each from a 256-byte boundary.
struct PrefixLayout {
    size_t pre_off, suf_off, total;
};

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

PrefixLayout prefix_layout(size_t num_seqs, size_t num_q_heads, size_t head_dim) {
    const size_t waves = static_cast<size_t>(device_cu_count()) * kBalancedWavesPerCu;
    const size_t part = round256(num_seqs * num_q_heads * (head_dim + 4) * sizeof(float));
    PrefixLayout l;
    l.pre_off = round256(balanced_bytes(std::min<size_t>(num_q_heads, 8), head_dim, waves));
    l.suf_off = l.pre_off + part;
    l.total = l.suf_off + part;
    return l;
}

// The groups of a shared-prefix decode (paged_attn_decode_prefix), or, with
// via_l2, only each sequence's shared leading blocks
// (paged_attn_decode_prefix_l2).
struct PrefixArgs {
    const int32_t* seq_prefix_blocks;
    const int32_t* group_offsets;
    const int32_t* group_members;
    const int32_t* group_blocks;
    int32_t num_groups;
    int32_t max_group_size;
    bool via_l2;
};

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

namespace {

// Shared by paged_attn_decode and paged_attn_decode_append (new_k, new_v:
// the fused append's source rows, or NULL).
pkv_status decode_impl(const char* fn, const pkv_pool* pool, int32_t layer, const void* q,
                       int32_t q_dtype, void* out, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, float scale, const float* k_scale,
                       const float* v_scale, int32_t max_context_len, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, const void* new_k,
                       const void* new_v, int32_t window, hipStream_t stream,
                       const PrefixArgs* pfx = nullptr) {
    using pkv::fail;
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", fn);
    const pkv_pool_desc& d = pool->desc;
    if (pool->base == nullptr)
        return fail(PKV_ERR_INVALID, "%s: pool has no device memory", fn);
    if (layer < 0 || layer >= d.num_layers)
        return fail(PKV_ERR_INVALID, "%s: layer %d out of range", fn, layer);
    if (!pkv::is_16bit(q_dtype))
        return fail(PKV_ERR_INVALID, "%s: q dtype must be F16 or BF16", fn);
    if (pkv::is_16bit(d.kv_dtype) && q_dtype != d.kv_dtype)
        return fail(PKV_ERR_INVALID, "%s: q dtype must equal the 16-bit cache dtype", fn);
    if (num_seqs < 0 || num_seqs > 65535)
        return fail(PKV_ERR_INVALID, "%s: num_seqs %d outside [0, 65535]", fn, num_seqs);
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads != 0)
        return fail(PKV_ERR_INVALID, "%s: %d query heads for %d kv heads", fn,
                    num_q_heads, d.num_kv_heads);
    const int G = num_q_heads / d.num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(PKV_ERR_INVALID, "%s: group size %d not in {1,2,4,8}", fn, G);
    if (max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID, "%s: negative table width or context", fn);
    if (partition_size < 0 || partition_size % 16 != 0)
        return fail(PKV_ERR_INVALID, "%s: partition_size %d not a multiple of 16", fn,
                    partition_size);
    if (!std::isfinite(scale))
        return fail(PKV_ERR_INVALID, "%s: scale is not finite", fn);
    if (window < 0) return fail(PKV_ERR_INVALID, "%s: negative window %d", fn, window);
    if (max_blocks_per_seq > (1 << 26))
        return fail(PKV_ERR_INVALID, "%s: max_blocks_per_seq too large", fn);
    if (num_seqs == 0) return PKV_OK;
    if (d.num_blocks == 0)
        return fail(PKV_ERR_INVALID, "%s: the pool has no blocks", fn);
    if (q == nullptr || block_tables == nullptr || context_lens == nullptr)
        return fail(PKV_ERR_INVALID, "%s: NULL q, block_tables or context_lens", fn);
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
        return fail(PKV_ERR_INVALID, "%s: q must be 16-byte aligned", fn);
    if (d.kv_dtype == PKV_FP8_E4M3 && (k_scale == nullptr || v_scale == nullptr))
        return fail(PKV_ERR_INVALID, "%s: an FP8 cache needs k_scale and v_scale", fn);

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
    prm.new_k = static_cast<const uint8_t*>(new_k);
    prm.new_v = static_cast<const uint8_t*>(new_v);
    prm.window = window;

    uint32_t parts = 1;
    if (partition_size > 0) {
        const size_t need = paged_attn_workspace_bytes(num_seqs, num_q_heads, d.head_dim,
                                                       max_context_len, partition_size);
        if (workspace == nullptr || workspace_bytes < need)
            return fail(PKV_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn,
                        workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return fail(PKV_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
        const int64_t P = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
        if (P == 0) return PKV_OK;  // no tokens anywhere; the reduce writes zeros
        if (P > 65535)
            return fail(PKV_ERR_INVALID, "%s: %lld partitions (at most 65535)", fn,
                        static_cast<long long>(P));
        parts = static_cast<uint32_t>(P);
        prm.blocks_per_part = partition_size / 16;
        prm.num_parts = static_cast<int32_t>(P);
        prm.ws_ml = static_cast<float*>(workspace);
        prm.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                            pkv::ws_o_offset(num_seqs, num_q_heads, P));
    } else {
        if (out == nullptr) return fail(PKV_ERR_INVALID, "%s: out is NULL", fn);
        if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
            return fail(PKV_ERR_INVALID, "%s: out must be 16-byte aligned", fn);
        prm.blocks_per_part = 0;
        prm.num_parts = 1;
        if (workspace != nullptr && pkv::is_16bit(d.kv_dtype) && num_seqs <= kBalancedMaxSeqs) {
            // Balanced single pass over the whole batch.
            const int cus = device_cu_count();
            const int waves = cus * kBalancedWavesPerCu;
            const PrefixLayout pl = prefix_layout(num_seqs, num_q_heads, d.head_dim);
            const bool kernel_pass = pfx != nullptr && !pfx->via_l2;
            const size_t need = kernel_pass ? pl.total : balanced_bytes(G, d.head_dim, waves);
            if (workspace_bytes < need)
                return fail(PKV_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn,
                            workspace_bytes, need);
            if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
                return fail(PKV_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
            prm.slots = static_cast<float*>(workspace);
            prm.num_seqs = num_seqs;
            const bool with_pre = kernel_pass && pfx->num_groups > 0;
            if (pfx != nullptr && pfx->via_l2) prm.keep_blocks = pfx->seq_prefix_blocks;
            if (with_pre) {
                uint8_t* ws = static_cast<uint8_t*>(workspace);
                prm.pre_blocks = pfx->seq_prefix_blocks;
                prm.pre = reinterpret_cast<float*>(ws + pl.pre_off);
                prm.suf = reinterpret_cast<float*>(ws + pl.suf_off);
                prm.group_offsets = pfx->group_offsets;
                prm.group_members = pfx->group_members;
                prm.group_blocks = pfx->group_blocks;
                prm.num_groups = pfx->num_groups;
                prm.pre_slots = (pfx->max_group_size * G + 15) / 16;
            }
            // The fused step's new tokens: each is a tile of its own in the
            // streaming kernel, whose wave also stores it (fold_new; the slot
            // travels as block id * 16 + position in 31 bits). A prefix pass
            // never reads a new token's slot: a plan's shared blocks end
            // before the block of each member's last token.
            if (new_k != nullptr && d.num_blocks < (1 << 27)) {
                prm.fold_new = 1;
            } else if (new_k != nullptr) {
                const pkv_status sa = append_first(
                    fn, pool, layer, new_k, new_v, q_dtype, block_tables, max_blocks_per_seq,
                    context_lens, num_seqs, max_context_len, k_scale, v_scale, stream);
                if (sa != PKV_OK) return sa;
                prm.new_k = prm.new_v = nullptr;
            }
            if (with_pre) {
                const hipError_t ep = (d.kv_dtype == PKV_F16)
                                          ? prefix_by_shape<PKV_F16>(d.head_dim, G, prm, stream)
                                          : prefix_by_shape<PKV_BF16>(d.head_dim, G, prm, stream);
                if (ep != hipSuccess)
                    return fail(PKV_ERR_HIP, "%s: prefix launch failed: %s", fn,
                                hipGetErrorString(ep));
            }
            const hipError_t eb = (d.kv_dtype == PKV_F16)
                                      ? balanced_by_dim<PKV_F16>(d.head_dim, G, prm, cus, stream)
                                      : balanced_by_dim<PKV_BF16>(d.head_dim, G, prm, cus, stream);
            if (eb != hipSuccess)
                return fail(PKV_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(eb));
            return PKV_OK;
        }
        if (pfx != nullptr)
            return fail(PKV_ERR_INVALID,
                        "%s: the shared-prefix pass needs a 16-bit cache, a workspace and at "
                        "most %d sequences", fn, kBalancedMaxSeqs);
        // The ordering keys hold the block count in 23 bits.
        const int64_t max_tokens =
            std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * 16);
        prm.longest_first = (num_seqs <= 256 && (max_tokens + 15) / 16 < (1 << 23)) ? 1 : 0;
    }

    // The fused step's new tokens: stored from inside the vector-ALU kernel
    // (16-bit caches with one query head per kv head, FP8 caches with up to
    // two); for the matrix-core kernel, and for FP8 with four or eight query
    // heads per kv head (whose kernels would lose a wave per SIMD), that code
    // would cost more than the separate append launch does.
    if (new_k != nullptr && (pkv::is_16bit(d.kv_dtype) ? G > 1 : G > 2)) {
        const pkv_status sa = append_first(fn, pool, layer, new_k, new_v, q_dtype, block_tables,
                                           max_blocks_per_seq, context_lens, num_seqs,
                                           max_context_len, k_scale, v_scale, stream);
        if (sa != PKV_OK) return sa;
        prm.new_k = prm.new_v = nullptr;
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
        return fail(PKV_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace

extern "C" pkv_status paged_attn_decode(const pkv_pool* pool, int32_t layer, const void* q,
                                        int32_t q_dtype, void* out, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads, float scale,
                                        const float* k_scale, const float* v_scale,
                                        int32_t max_context_len, int32_t partition_size,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return decode_impl("paged_attn_decode", pool, layer, q, q_dtype, out, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale, k_scale,
                       v_scale, max_context_len, partition_size, workspace, workspace_bytes,
                       nullptr, nullptr, 0, stream);
}

extern "C" pkv_status paged_attn_decode_append(
    const pkv_pool* pool, int32_t layer, const void* new_k, const void* new_v, int32_t src_dtype,
    const void* q, int32_t q_dtype, void* out, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, float scale, const float* k_scale, const float* v_scale,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
    using pkv::fail;
    const char* fn = "paged_attn_decode_append";
    if (src_dtype != q_dtype)
        return fail(PKV_ERR_INVALID, "%s: the new tokens' dtype must equal the q dtype", fn);
    if (num_seqs > 0 && (new_k == nullptr || new_v == nullptr))
        return fail(PKV_ERR_INVALID, "%s: NULL new_k or new_v", fn);
    if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
        return fail(PKV_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", fn);
    return decode_impl(fn, pool, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, k_scale, v_scale,
                       max_context_len, partition_size, workspace, workspace_bytes, new_k, new_v,
                       0, stream);
}

extern "C" pkv_status paged_attn_decode_window(
    const pkv_pool* pool, int32_t layer, const void* new_k, const void* new_v, int32_t src_dtype,
    const void* q, int32_t q_dtype, void* out, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, float scale, const float* k_scale, const float* v_scale,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t window, hipStream_t stream) {
    using pkv::fail;
    const char* fn = "paged_attn_decode_window";
    if ((new_k == nullptr) != (new_v == nullptr))
        return fail(PKV_ERR_INVALID, "%s: new_k and new_v must both be given or both be NULL", fn);
    if (new_k != nullptr) {
        if (src_dtype != q_dtype)
            return fail(PKV_ERR_INVALID, "%s: the new tokens' dtype must equal the q dtype", fn);
        if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
            return fail(PKV_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", fn);
    }
    return decode_impl(fn, pool, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, k_scale, v_scale,
                       max_context_len, partition_size, workspace, workspace_bytes, new_k, new_v,
                       window, stream);
}

extern "C" size_t paged_attn_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t head_dim) {
    if (num_seqs < 0 || num_seqs > kBalancedMaxSeqs || num_q_heads <= 0 || head_dim <= 0)
        return 0;
    return prefix_layout(num_seqs, num_q_heads, head_dim).total;
}

extern "C" pkv_status paged_attn_decode_prefix(
    const pkv_pool* pool, int32_t layer, const void* new_k, const void* new_v, int32_t src_dtype,
    const void* q, int32_t q_dtype, void* out, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, float scale, int32_t max_context_len, const int32_t* seq_prefix_blocks,
    const int32_t* group_offsets, const int32_t* group_members, const int32_t* group_blocks,
    int32_t num_groups, int32_t max_group_size, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
    using pkv::fail;
    const char* fn = "paged_attn_decode_prefix";
    if ((new_k == nullptr) != (new_v == nullptr))
        return fail(PKV_ERR_INVALID, "%s: new_k and new_v must both be given or both be NULL", fn);
    if (new_k != nullptr) {
        if (src_dtype != q_dtype)
            return fail(PKV_ERR_INVALID, "%s: the new tokens' dtype must equal the q dtype", fn);
        if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
            return fail(PKV_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", fn);
    }
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", fn);
    if (!pkv::is_16bit(pool->desc.kv_dtype))
        return fail(PKV_ERR_INVALID, "%s: the shared-prefix pass needs a 16-bit cache", fn);
    if (num_seqs < 0 || num_seqs > kBalancedMaxSeqs)
        return fail(PKV_ERR_INVALID, "%s: num_seqs %d outside [0, %d]", fn, num_seqs,
                    kBalancedMaxSeqs);
    if (num_groups < 0 || num_groups > num_seqs)
        return fail(PKV_ERR_INVALID, "%s: num_groups %d outside [0, num_seqs]", fn, num_groups);
    if (num_groups > 0) {
        if (max_group_size < 1 || max_group_size > num_seqs)
            return fail(PKV_ERR_INVALID, "%s: max_group_size %d outside [1, num_seqs]", fn,
                        max_group_size);
        if (seq_prefix_blocks == nullptr || group_offsets == nullptr ||
            group_members == nullptr || group_blocks == nullptr)
            return fail(PKV_ERR_INVALID, "%s: NULL group arrays", fn);
    }
    if (workspace == nullptr && num_seqs > 0)
        return fail(PKV_ERR_INVALID, "%s: workspace is NULL", fn);
    const PrefixArgs pfx{seq_prefix_blocks, group_offsets, group_members, group_blocks,
                         num_groups, max_group_size, false};
    return decode_impl(fn, pool, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, nullptr, nullptr,
                       max_context_len, 0, workspace, workspace_bytes, new_k, new_v, 0, stream,
                       &pfx);
}

extern "C" pkv_status paged_attn_decode_prefix_l2(
    const pkv_pool* pool, int32_t layer, const void* new_k, const void* new_v, int32_t src_dtype,
    const void* q, int32_t q_dtype, void* out, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, float scale, int32_t max_context_len, const int32_t* seq_prefix_blocks,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    using pkv::fail;
    const char* fn = "paged_attn_decode_prefix_l2";
    if ((new_k == nullptr) != (new_v == nullptr))
        return fail(PKV_ERR_INVALID, "%s: new_k and new_v must both be given or both be NULL", fn);
    if (new_k != nullptr) {
        if (src_dtype != q_dtype)
            return fail(PKV_ERR_INVALID, "%s: the new tokens' dtype must equal the q dtype", fn);
        if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
            return fail(PKV_ERR_INVALID, "%s: new_k and new_v must be 16-byte aligned", fn);
    }
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", fn);
    if (!pkv::is_16bit(pool->desc.kv_dtype))
        return fail(PKV_ERR_INVALID, "%s: needs a 16-bit cache", fn);
    if (num_seqs < 0 || num_seqs > kBalancedMaxSeqs)
        return fail(PKV_ERR_INVALID, "%s: num_seqs %d outside [0, %d]", fn, num_seqs,
                    kBalancedMaxSeqs);
    if (workspace == nullptr && num_seqs > 0)
        return fail(PKV_ERR_INVALID, "%s: workspace is NULL", fn);
    const PrefixArgs pfx{seq_prefix_blocks, nullptr, nullptr, nullptr, 0, 0, true};
    return decode_impl(fn, pool, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, nullptr, nullptr,
                       max_context_len, 0, workspace, workspace_bytes, new_k, new_v, 0, stream,
                       seq_prefix_blocks != nullptr ? &pfx : nullptr);
}

// ---------------------------------------------------------------------------
// The decode step for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation): the
// workspace is a static device array of the library, one per GPU, instead of
// a caller buffer.
namespace {

constexpr size_t kScratchBytes = PKV_STATIC_SCRATCH_BYTES;  // per GPU

// Host code never passes this name to a kernel or a copy: it stands for the
// array on the host side only. Its device address on each GPU comes from
// hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU (NULL: not looked up)

// Device address of the scratch array on the current device, looked up once
// per device with that device current.
pkv_status scratch_address(const char* fn, void** out) {
    using pkv::fail;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_ERR_INVALID, "%s: device %d beyond the %d the library tracks", fn, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(PKV_ERR_HIP, "%s: no device address for the scratch array: %s", fn,
                        hipGetErrorString(e));
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" pkv_status paged_attn_decode_append_noalloc(
    const pkv_pool* pool, int32_t layer, const void* new_k, const void* new_v, int32_t src_dtype,
    const void* q, int32_t q_dtype, void* out, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, float scale, const float* k_scale, const float* v_scale,
    int32_t max_context_len, int32_t partition_size, hipStream_t stream) {
    using pkv::fail;
    const char* fn = "paged_attn_decode_append_noalloc";
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", fn);
    const pkv_pool_desc& d = pool->desc;
    if (num_seqs < 0 || num_q_heads <= 0 || num_q_heads % d.num_kv_heads != 0 ||
        max_context_len < 0 || partition_size < 0)
        return fail(PKV_ERR_INVALID, "%s: bad sizes", fn);
    if (num_seqs == 0) return PKV_OK;
    if (out == nullptr) return fail(PKV_ERR_INVALID, "%s: out is NULL", fn);
    // The scratch this call needs: the split-K partials, or the balanced
    // pass's split-context partials (16-bit caches, up to 4096 sequences);
    // the per-sequence pass (FP8 caches, larger batches) needs none.
    size_t need = 0;
    if (partition_size > 0) {
        need = paged_attn_workspace_bytes(num_seqs, num_q_heads, d.head_dim, max_context_len,
                                          partition_size);
    } else if (pkv::is_16bit(d.kv_dtype) && num_seqs <= kBalancedMaxSeqs) {
        const size_t waves = static_cast<size_t>(device_cu_count()) * kBalancedWavesPerCu;
        need = balanced_bytes(static_cast<size_t>(num_q_heads / d.num_kv_heads), d.head_dim,
                              waves);
    }
    if (need > kScratchBytes)
        return fail(PKV_ERR_INVALID,
                    "%s: this batch needs %zu bytes of workspace; the static scratch holds %zu "
                    "(use paged_attn_decode_append with a workspace)", fn, need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const pkv_status st = scratch_address(fn, &ws);
        if (st != PKV_OK) return st;
    }
    const pkv_status st = paged_attn_decode_append(
        pool, layer, new_k, new_v, src_dtype, q, q_dtype, partition_size > 0 ? nullptr : out,
        block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale, k_scale,
        v_scale, max_context_len, partition_size, ws, need > 0 ? kScratchBytes : 0, stream);
    if (st != PKV_OK || partition_size == 0) return st;
    return paged_attn_reduce(ws, out, q_dtype, context_lens, num_seqs, num_q_heads, d.head_dim,
                             max_context_len, partition_size, stream);
}
