// kv_block_copy: whole-block copies for copy-on-write.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", section
// "PagedAttention：把操作系统的虚拟内存搬进 GPU": several logical blocks (beam
// search, shared prefixes) may map to one physical block; a sequence that is
// about to write into a block it shares first takes a private copy of it.
//
// A block is one contiguous run of num_kv_heads * 16 * head_dim elements in
// each (layer, K/V) plane of the pool, so a copy is 2 * layers runs of that
// size. Workgroup (chunk, plane, pair) moves one 16 KiB chunk of one run with
// 16-byte non-temporal loads and stores (the bytes are not read again by this
// kernel). The block ids travel as kernel arguments, 128 pairs per launch, so
// the call allocates nothing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <unordered_set>

#include "common.h"

namespace {

constexpr int kPairsPerLaunch = 128;
constexpr int kChunkBytes = 16384;

struct CopyPairs {
    int32_t src[kPairsPerLaunch];
    int32_t dst[kPairsPerLaunch];
};

__global__ __launch_bounds__(256) void block_copy_kernel(uint8_t* __restrict__ base,
                                                         size_t plane_bytes, size_t block_bytes,
                                                         const CopyPairs pairs) {
    const size_t plane = blockIdx.y;
    const int pair = blockIdx.z;
    const size_t first = static_cast<size_t>(blockIdx.x) * kChunkBytes;
    const size_t n = std::min<size_t>(kChunkBytes, block_bytes - first);  // multiple of 16
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* src = reinterpret_cast<const u32x4*>(
        base + plane * plane_bytes + static_cast<size_t>(pairs.src[pair]) * block_bytes + first);
    u32x4* dst = reinterpret_cast<u32x4*>(
        base + plane * plane_bytes + static_cast<size_t>(pairs.dst[pair]) * block_bytes + first);
    const int count = static_cast<int>(n / 16);
#pragma unroll 4
    for (int i = threadIdx.x; i < count; i += 256)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" pkv_status kv_block_copy(const pkv_pool* pool, const int32_t* src_ids,
                                    const int32_t* dst_ids, int32_t n, hipStream_t stream) {
    using pkv::fail;
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "kv_block_copy: pool is NULL");
    if (pool->base == nullptr)
        return fail(PKV_ERR_INVALID, "kv_block_copy: pool has no device memory");
    if (n < 0) return fail(PKV_ERR_INVALID, "kv_block_copy: negative count %d", n);
    if (n == 0) return PKV_OK;
    if (src_ids == nullptr || dst_ids == nullptr)
        return fail(PKV_ERR_INVALID, "kv_block_copy: NULL id array");
    const pkv_pool_desc& d = pool->desc;
    std::unordered_set<int32_t> dsts, srcs;
    dsts.reserve(static_cast<size_t>(n) * 2);
    srcs.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
        if (src_ids[i] < 0 || src_ids[i] >= d.num_blocks || dst_ids[i] < 0 ||
            dst_ids[i] >= d.num_blocks)
            return fail(PKV_ERR_INVALID, "kv_block_copy: pair %d (%d -> %d) out of range", i,
                        src_ids[i], dst_ids[i]);
        if (!dsts.insert(dst_ids[i]).second)
            return fail(PKV_ERR_INVALID, "kv_block_copy: block %d is a destination twice",
                        dst_ids[i]);
        srcs.insert(src_ids[i]);
    }
    for (int32_t i = 0; i < n; ++i)
        if (srcs.count(dst_ids[i]))
            return fail(PKV_ERR_INVALID, "kv_block_copy: block %d is both source and destination",
                        dst_ids[i]);

    const size_t block_bytes = static_cast<size_t>(d.num_kv_heads) * d.block_size * d.head_dim *
                               static_cast<size_t>(pkv::elem_size(d.kv_dtype));
    const size_t plane_bytes = block_bytes * static_cast<size_t>(d.num_blocks);
    const uint32_t chunks = static_cast<uint32_t>((block_bytes + kChunkBytes - 1) / kChunkBytes);
    const uint32_t planes = static_cast<uint32_t>(2 * d.num_layers);
    if (planes > 65535)
        return fail(PKV_ERR_INVALID, "kv_block_copy: %u planes (at most 65535)", planes);
    for (int32_t i0 = 0; i0 < n; i0 += kPairsPerLaunch) {
        const int32_t m = std::min(kPairsPerLaunch, n - i0);
        CopyPairs pairs{};
        for (int32_t j = 0; j < m; ++j) {
            pairs.src[j] = src_ids[i0 + j];
            pairs.dst[j] = dst_ids[i0 + j];
        }
        hipLaunchKernelGGL(block_copy_kernel, dim3(chunks, planes, static_cast<uint32_t>(m)),
                           dim3(256), 0, stream, static_cast<uint8_t*>(pool->base), plane_bytes,
                           block_bytes, pairs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_ERR_HIP, "kv_block_copy: launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}
