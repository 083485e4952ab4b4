// kv_cache_append: write each new token's K and V rows into its slot.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", section
// "PagedAttention：把操作系统的虚拟内存搬进 GPU": the cache grows slot by slot as
// tokens are produced, into blocks handed out on demand. Section "vLLM 也不是
// 银弹：真实部署中的坑" (third pitfall): an FP8 cache halves KV memory.
//
// One thread moves 8 source elements (16 bytes) of one (token, kv head) row;
// a row of head_dim elements is head_dim/8 consecutive threads, so both the
// source read and the 256-byte (fp16) or 128-byte (fp8) destination row are
// contiguous per group of threads. The work is tiny (tokens x heads x dim) and
// latency bound; it is one launch for K and V together.

#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"

namespace {

using namespace pkv::dev;

// Where token t goes: slots[t] (kv_cache_append), or, for the fused decode
// step, the last position L - 1 of sequence t's context through its table row
// (no slot when L is outside [1, reach] or the id is outside the pool).
struct SlotSource {
    const int64_t* slots;
    const int32_t* tables;  // set: positions from the tables
    const int32_t* lens;
    int32_t max_blocks;
    int32_t reach;
};

__device__ __forceinline__ int64_t token_slot(const SlotSource& src, int64_t t, int64_t num_slots) {
    if (src.tables == nullptr) return src.slots[t];
    const int L = src.lens[t];
    if (L < 1 || L > src.reach) return -1;
    const int pos = L - 1;
    const int id = src.tables[t * src.max_blocks + pos / 16];
    if (id < 0 || static_cast<int64_t>(id) * 16 >= num_slots) return -1;
    return static_cast<int64_t>(id) * 16 + pos % 16;
}

template <int KV, int SRC, int D>
__global__ __launch_bounds__(256) void append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const SlotSource src,
    int32_t num_tokens, int32_t num_kv_heads, uint8_t* __restrict__ k_plane,
    uint8_t* __restrict__ v_plane, int64_t num_slots, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
    constexpr int kChunks = D / 8;  // 16-byte source chunks per row
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t rows = static_cast<int64_t>(num_tokens) * num_kv_heads;
    if (gid >= rows * kChunks) return;
    const int64_t row = gid / kChunks;
    const int chunk = static_cast<int>(gid % kChunks);
    const int64_t t = row / num_kv_heads;
    const int h = static_cast<int>(row % num_kv_heads);
    const int64_t slot = token_slot(src, t, num_slots);
    if (slot < 0 || slot >= num_slots) return;
    const int64_t block = slot >> 4, off = slot & 15;
    const int64_t dst_row = (block * num_kv_heads + h) * 16 + off;  // in rows of D elements
    const uint4 kx = k[row * kChunks + chunk];
    const uint4 vx = v[row * kChunks + chunk];
    if constexpr (KV != PKV_FP8_E4M3) {
        reinterpret_cast<uint4*>(k_plane)[dst_row * kChunks + chunk] = kx;
        reinterpret_cast<uint4*>(v_plane)[dst_row * kChunks + chunk] = vx;
    } else {
        const float ks = k_scale[h], vs = v_scale[h];
        reinterpret_cast<uint2*>(k_plane)[dst_row * kChunks + chunk] = quant_e4m3x8<SRC>(kx, ks);
        reinterpret_cast<uint2*>(v_plane)[dst_row * kChunks + chunk] = quant_e4m3x8<SRC>(vx, vs);
    }
}

template <int KV, int SRC, int D>
hipError_t launch_append(const void* k, const void* v, const SlotSource& slots, int32_t num_tokens,
                         int32_t num_kv_heads, uint8_t* k_plane, uint8_t* v_plane,
                         int64_t num_slots, const float* ks, const float* vs,
                         hipStream_t stream) {
    const int64_t threads = static_cast<int64_t>(num_tokens) * num_kv_heads * (D / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((append_kernel<KV, SRC, D>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(256), 0, stream, static_cast<const uint4*>(k),
                       static_cast<const uint4*>(v), slots, num_tokens, num_kv_heads, k_plane,
                       v_plane, num_slots, ks, vs);
    return hipGetLastError();
}

template <int KV, int SRC>
hipError_t dispatch_dim(int D, const void* k, const void* v, const SlotSource& slots, int32_t T,
                        int32_t H, uint8_t* kp, uint8_t* vp, int64_t ns, const float* ks,
                        const float* vs, hipStream_t st) {
    if (D == 64) return launch_append<KV, SRC, 64>(k, v, slots, T, H, kp, vp, ns, ks, vs, st);
    return launch_append<KV, SRC, 128>(k, v, slots, T, H, kp, vp, ns, ks, vs, st);
}

hipError_t dispatch_dtype(const pkv_pool_desc& d, uint8_t* kp, uint8_t* vp, const void* k,
                          const void* v, int32_t src_dtype, const SlotSource& src, int32_t T,
                          const float* ks, const float* vs, hipStream_t st) {
    const int64_t num_slots = static_cast<int64_t>(d.num_blocks) * d.block_size;
    const int H = d.num_kv_heads;
    if (d.kv_dtype == PKV_F16)
        return dispatch_dim<PKV_F16, PKV_F16>(d.head_dim, k, v, src, T, H, kp, vp, num_slots, ks,
                                             vs, st);
    if (d.kv_dtype == PKV_BF16)
        return dispatch_dim<PKV_BF16, PKV_BF16>(d.head_dim, k, v, src, T, H, kp, vp, num_slots,
                                               ks, vs, st);
    if (src_dtype == PKV_F16)
        return dispatch_dim<PKV_FP8_E4M3, PKV_F16>(d.head_dim, k, v, src, T, H, kp, vp, num_slots,
                                                  ks, vs, st);
    return dispatch_dim<PKV_FP8_E4M3, PKV_BF16>(d.head_dim, k, v, src, T, H, kp, vp, num_slots, ks,
                                               vs, st);
}

}  // namespace

extern "C" pkv_status kv_cache_append(const pkv_pool* pool, int32_t layer, const void* k,
                                      const void* v, int32_t src_dtype,
                                      const int64_t* slot_mapping, int32_t num_tokens,
                                      const float* k_scale, const float* v_scale,
                                      hipStream_t stream) {
    using pkv::fail;
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "kv_cache_append: pool is NULL");
    const pkv_pool_desc& d = pool->desc;
    if (pool->base == nullptr)
        return fail(PKV_ERR_INVALID, "kv_cache_append: pool has no device memory");
    if (layer < 0 || layer >= d.num_layers)
        return fail(PKV_ERR_INVALID, "kv_cache_append: layer %d out of range", layer);
    if (num_tokens < 0) return fail(PKV_ERR_INVALID, "kv_cache_append: negative token count");
    if (!pkv::is_16bit(src_dtype))
        return fail(PKV_ERR_INVALID, "kv_cache_append: source dtype must be F16 or BF16");
    if (pkv::is_16bit(d.kv_dtype) && src_dtype != d.kv_dtype)
        return fail(PKV_ERR_INVALID, "kv_cache_append: a 16-bit cache stores its own dtype");
    if (num_tokens == 0) return PKV_OK;
    if (k == nullptr || v == nullptr || slot_mapping == nullptr)
        return fail(PKV_ERR_INVALID, "kv_cache_append: NULL k, v or slot_mapping");
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) % 16 != 0)
        return fail(PKV_ERR_INVALID, "kv_cache_append: k and v must be 16-byte aligned");
    if (d.kv_dtype == PKV_FP8_E4M3 && (k_scale == nullptr || v_scale == nullptr))
        return fail(PKV_ERR_INVALID, "kv_cache_append: an FP8 cache needs k_scale and v_scale");
    if (static_cast<int64_t>(num_tokens) * d.num_kv_heads * (d.head_dim / 8) >
        static_cast<int64_t>(0x7FFFFFFF) * 256)
        return fail(PKV_ERR_INVALID, "kv_cache_append: too many tokens for one launch");

    uint8_t* base = static_cast<uint8_t*>(pool->base);
    uint8_t* kp = base + pkv::layer_plane_offset(d, layer, 0);
    uint8_t* vp = base + pkv::layer_plane_offset(d, layer, 1);
    const SlotSource src{slot_mapping, nullptr, nullptr, 0, 0};
    const hipError_t e =
        dispatch_dtype(d, kp, vp, k, v, src_dtype, src, num_tokens, k_scale, v_scale, stream);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "kv_cache_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

hipError_t pkv::launch_append_last(const pkv_pool_desc& d, uint8_t* k_plane, uint8_t* v_plane,
                                   const void* k, const void* v, int32_t src_dtype,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t reach,
                                   const float* k_scale, const float* v_scale,
                                   hipStream_t stream) {
    const SlotSource src{nullptr, block_tables, context_lens, max_blocks_per_seq, reach};
    return dispatch_dtype(d, k_plane, v_plane, k, v, src_dtype, src, num_seqs, k_scale, v_scale,
                          stream);
}
