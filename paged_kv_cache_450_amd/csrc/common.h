// Internal definitions shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct pkv_pool {
    pkv_pool_desc desc;
    void* base;          // borrowed device pointer (may be NULL)
    size_t bytes;
    std::vector<int32_t> free_stack;  // top = back()
    std::vector<int32_t> ref;         // per-block reference count
    // Prefix caching. A block may hold a content key. A keyed block whose last
    // reference is released keeps its contents on the cached list (a doubly
    // linked list by id, oldest release at the head) instead of going back to
    // the free stack; allocation evicts from the head, dropping the key, only
    // once the free stack is empty.
    std::unordered_map<uint64_t, int32_t> key_block;
    std::vector<uint64_t> block_key;
    std::vector<uint8_t> keyed;
    std::vector<int32_t> cprev, cnext;
    int32_t chead = -1, ctail = -1, ncached = 0;
};

namespace pkv {

// Records a message for pkv_last_error() and returns the status.
pkv_status fail(pkv_status status, const char* fmt, ...);

inline int elem_size(int32_t dtype) {
    switch (dtype) {
        case PKV_F16:
        case PKV_BF16: return 2;
        case PKV_FP8_E4M3: return 1;
        default: return 0;
    }
}

inline bool is_16bit(int32_t dtype) { return dtype == PKV_F16 || dtype == PKV_BF16; }

// Byte offset of the (layer, c, block 0, head 0, slot 0, dim 0) tile in the pool.
inline size_t layer_plane_offset(const pkv_pool_desc& d, int32_t layer, int32_t c) {
    return (static_cast<size_t>(layer) * 2 + static_cast<size_t>(c)) *
           static_cast<size_t>(d.num_blocks) * static_cast<size_t>(d.num_kv_heads) *
           static_cast<size_t>(d.block_size) * static_cast<size_t>(d.head_dim) *
           static_cast<size_t>(elem_size(d.kv_dtype));
}

constexpr int kBlockSize = PKV_BLOCK_SIZE;

// Workspace of a partitioned decode: (m, l) pairs first, then the partial
// outputs from the next 256-byte boundary, so their 16-byte rows stay aligned.
inline size_t ws_o_offset(size_t num_seqs, size_t num_q_heads, size_t parts) {
    const size_t ml = num_seqs * num_q_heads * parts * 2 * sizeof(float);
    return (ml + 255) & ~static_cast<size_t>(255);
}

// The fused decode step's append, as its own kernel (append.hip), for decode
// forms that do not store the new tokens themselves: token i of k, v
// ([num_seqs][Hkv][D] of src_dtype) goes to the last position L - 1 of
// sequence i (context_lens[i] = L) through its table row, when 1 <= L <= reach
// and the id there is inside the pool; the same bytes as kv_cache_append.
hipError_t launch_append_last(const pkv_pool_desc& d, uint8_t* k_plane, uint8_t* v_plane,
                              const void* k, const void* v, int32_t src_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t reach,
                              const float* k_scale, const float* v_scale, hipStream_t stream);

}  // namespace pkv
