// kv_swap_out / kv_swap_in: whole blocks between the pool and host memory.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", sections
// "vLLM 也不是银弹：真实部署中的坑" and "从零开始：vLLM 部署的实战建议": when the
// cache runs short, running requests are preempted and their KV blocks
// swapped out; they come back when blocks free up.
//
// Swap space is a caller-owned, pinned host buffer of slots. Slot s holds one
// block of every layer, K and V: [num_layers][2][Hkv][16][D] elements of the
// pool's dtype, so a request's blocks land in contiguous host runs whatever
// their ids in the pool. The GPU reads and writes the pinned pages directly
// (no staging buffer, no copy engine): workgroup (chunk, plane, pair) moves
// one 16 KiB chunk of one block's run in one (layer, K/V) plane with 16-byte
// accesses, non-temporal on the pool side. Ids and slots travel as kernel
// arguments, 128 pairs per launch; nothing is allocated.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <unordered_set>

#include "common.h"

namespace {

constexpr int kPairsPerLaunch = 128;
constexpr int kChunkBytes = 16384;

struct SwapPairs {
    int32_t block[kPairsPerLaunch];
    int32_t slot[kPairsPerLaunch];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// kOut: pool -> host, else host -> pool.
template <bool kOut>
__global__ __launch_bounds__(256) void swap_kernel(uint8_t* __restrict__ pool,
                                                   uint8_t* __restrict__ host,
                                                   size_t plane_bytes, size_t block_bytes,
                                                   uint32_t planes, const SwapPairs pairs) {
    const size_t plane = blockIdx.y;
    const int k = blockIdx.z;
    const size_t first = static_cast<size_t>(blockIdx.x) * kChunkBytes;
    const int count = static_cast<int>(std::min<size_t>(kChunkBytes, block_bytes - first) / 16);
    u32x4* dev = reinterpret_cast<u32x4*>(
        pool + plane * plane_bytes + static_cast<size_t>(pairs.block[k]) * block_bytes + first);
    u32x4* hst = reinterpret_cast<u32x4*>(
        host + (static_cast<size_t>(pairs.slot[k]) * planes + plane) * block_bytes + first);
#pragma unroll 4
    for (int i = threadIdx.x; i < count; i += 256) {
        if constexpr (kOut)
            hst[i] = __builtin_nontemporal_load(dev + i);
        else
            __builtin_nontemporal_store(hst[i], dev + i);
    }
}

// The device address of host_buf when [host_buf, host_buf + bytes) lies in one
// pinned host allocation, else nullptr.
void* pinned_device_address(const void* host_buf, size_t bytes) {
    hipPointerAttribute_t a{}, b{};
    if (hipPointerGetAttributes(&a, host_buf) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    const void* last = static_cast<const uint8_t*>(host_buf) + (bytes - 1);
    if (hipPointerGetAttributes(&b, last) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (a.type != hipMemoryTypeHost || b.type != hipMemoryTypeHost || a.devicePointer == nullptr ||
        static_cast<const uint8_t*>(b.devicePointer) !=
            static_cast<const uint8_t*>(a.devicePointer) + (bytes - 1))
        return nullptr;
    return a.devicePointer;
}

template <bool kOut>
pkv_status swap_impl(const char* fn, const pkv_pool* pool, const int32_t* block_ids,
                     const int32_t* host_slots, int32_t n, const void* host_buf,
                     size_t host_buf_bytes, hipStream_t stream) {
    using pkv::fail;
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", fn);
    if (pool->base == nullptr) return fail(PKV_ERR_INVALID, "%s: pool has no device memory", fn);
    if (n < 0) return fail(PKV_ERR_INVALID, "%s: negative count %d", fn, n);
    if (n == 0) return PKV_OK;
    if (block_ids == nullptr || host_slots == nullptr)
        return fail(PKV_ERR_INVALID, "%s: NULL id or slot array", fn);
    const pkv_pool_desc& d = pool->desc;
    const size_t block_bytes = static_cast<size_t>(d.num_kv_heads) * d.block_size * d.head_dim *
                               static_cast<size_t>(pkv::elem_size(d.kv_dtype));
    const uint32_t planes = static_cast<uint32_t>(2 * d.num_layers);
    const size_t slot_bytes = block_bytes * planes;
    if (host_buf == nullptr || host_buf_bytes < slot_bytes)
        return fail(PKV_ERR_INVALID, "%s: host buffer of %zu bytes holds no slot of %zu bytes", fn,
                    host_buf_bytes, slot_bytes);
    const int64_t num_slots = static_cast<int64_t>(host_buf_bytes / slot_bytes);
    std::unordered_set<int32_t> dsts;
    dsts.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
        if (block_ids[i] < 0 || block_ids[i] >= d.num_blocks)
            return fail(PKV_ERR_INVALID, "%s: pair %d: block %d out of range", fn, i, block_ids[i]);
        if (host_slots[i] < 0 || host_slots[i] >= num_slots)
            return fail(PKV_ERR_INVALID, "%s: pair %d: slot %d out of range (%lld slots)", fn, i,
                        host_slots[i], static_cast<long long>(num_slots));
        const int32_t dst = kOut ? host_slots[i] : block_ids[i];
        if (!dsts.insert(dst).second)
            return fail(PKV_ERR_INVALID, "%s: %s %d is a destination twice", fn,
                        kOut ? "slot" : "block", dst);
    }
    if (planes > 65535) return fail(PKV_ERR_INVALID, "%s: %u planes (at most 65535)", fn, planes);
    void* host_dev = pinned_device_address(host_buf, host_buf_bytes);
    if (host_dev == nullptr)
        return fail(PKV_ERR_INVALID,
                    "%s: host buffer is not one pinned host allocation of %zu bytes", fn,
                    host_buf_bytes);
    const size_t plane_bytes = block_bytes * static_cast<size_t>(d.num_blocks);
    const uint32_t chunks = static_cast<uint32_t>((block_bytes + kChunkBytes - 1) / kChunkBytes);
    for (int32_t i0 = 0; i0 < n; i0 += kPairsPerLaunch) {
        const int32_t m = std::min(kPairsPerLaunch, n - i0);
        SwapPairs pairs{};
        for (int32_t j = 0; j < m; ++j) {
            pairs.block[j] = block_ids[i0 + j];
            pairs.slot[j] = host_slots[i0 + j];
        }
        hipLaunchKernelGGL(swap_kernel<kOut>, dim3(chunks, planes, static_cast<uint32_t>(m)),
                           dim3(256), 0, stream, static_cast<uint8_t*>(pool->base),
                           static_cast<uint8_t*>(host_dev), plane_bytes, block_bytes, planes,
                           pairs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    return PKV_OK;
}

}  // namespace

extern "C" size_t kv_swap_slot_bytes(const pkv_pool* pool) {
    if (pool == nullptr) return 0;
    const pkv_pool_desc& d = pool->desc;
    return static_cast<size_t>(d.num_kv_heads) * d.block_size * d.head_dim *
           static_cast<size_t>(pkv::elem_size(d.kv_dtype)) * 2 * static_cast<size_t>(d.num_layers);
}

extern "C" pkv_status kv_swap_out(const pkv_pool* pool, const int32_t* block_ids,
                                  const int32_t* host_slots, int32_t n, void* host_buf,
                                  size_t host_buf_bytes, hipStream_t stream) {
    return swap_impl<true>("kv_swap_out", pool, block_ids, host_slots, n, host_buf,
                           host_buf_bytes, stream);
}

extern "C" pkv_status kv_swap_in(const pkv_pool* pool, const int32_t* host_slots,
                                 const int32_t* block_ids, int32_t n, const void* host_buf,
                                 size_t host_buf_bytes, hipStream_t stream) {
    return swap_impl<false>("kv_swap_in", pool, block_ids, host_slots, n, host_buf,
                            host_buf_bytes, stream);
}
