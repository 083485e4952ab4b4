// Host-side block manager: one preallocated pool of fixed-size blocks, a LIFO
// free stack, per-block reference counts, and per-sequence slot bookkeeping.
//
// [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍", section
// "PagedAttention：把操作系统的虚拟内存搬进 GPU": fixed-size blocks handed out on
// demand, mapped through a per-sequence page table, interchangeable (no
// external fragmentation) and shareable between sequences. Section
// "连续批处理：别再等最慢的那个请求了": the calls a scheduler makes each
// iteration (free a finished table, count free blocks, allocate).
//
// Fixed-size blocks make any free block as good as any other, so a stack gives
// O(1) alloc and free; reference counts give sharing without copies.

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>

#include "common.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

pkv_status fail(pkv_status status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

}  // namespace pkv

using pkv::fail;

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

static bool desc_valid(const pkv_pool_desc* d) {
    return d != nullptr && d->num_layers > 0 && d->num_blocks >= 0 &&
           d->block_size == PKV_BLOCK_SIZE && d->num_kv_heads > 0 &&
           (d->head_dim == 64 || d->head_dim == 128) && pkv::elem_size(d->kv_dtype) > 0;
}

size_t kv_pool_bytes(const pkv_pool_desc* d) {
    if (!desc_valid(d)) return 0;
    return static_cast<size_t>(d->num_layers) * 2 * static_cast<size_t>(d->num_blocks) *
           static_cast<size_t>(d->num_kv_heads) * static_cast<size_t>(d->block_size) *
           static_cast<size_t>(d->head_dim) * static_cast<size_t>(pkv::elem_size(d->kv_dtype));
}

pkv_status kv_pool_create(const pkv_pool_desc* desc, void* device_base, size_t bytes,
                          pkv_pool** out) {
    if (out == nullptr) return fail(PKV_ERR_INVALID, "kv_pool_create: out is NULL");
    if (!desc_valid(desc))
        return fail(PKV_ERR_INVALID,
                    "kv_pool_create: unsupported descriptor (block_size must be 16, head_dim "
                    "64 or 128, layers/heads > 0, blocks >= 0, known dtype)");
    const size_t need = kv_pool_bytes(desc);
    if (device_base != nullptr) {
        if (bytes < need)
            return fail(PKV_ERR_INVALID, "kv_pool_create: %zu bytes given, %zu needed", bytes,
                        need);
        if (reinterpret_cast<uintptr_t>(device_base) % 256 != 0)
            return fail(PKV_ERR_INVALID, "kv_pool_create: device_base not 256-byte aligned");
    }
    pkv_pool* p = new (std::nothrow) pkv_pool;
    if (p == nullptr) return fail(PKV_ERR_OOM, "kv_pool_create: host allocation failed");
    try {
        p->desc = *desc;
        p->base = device_base;
        p->bytes = bytes;
        p->free_stack.resize(desc->num_blocks);
        for (int32_t i = 0; i < desc->num_blocks; ++i)
            p->free_stack[i] = desc->num_blocks - 1 - i;  // top = 0
        p->ref.assign(desc->num_blocks, 0);
        p->block_key.assign(desc->num_blocks, 0);
        p->keyed.assign(desc->num_blocks, 0);
        p->cprev.assign(desc->num_blocks, -1);
        p->cnext.assign(desc->num_blocks, -1);
    } catch (...) {
        delete p;
        return fail(PKV_ERR_OOM, "kv_pool_create: host allocation failed");
    }
    *out = p;
    return PKV_OK;
}

void kv_pool_destroy(pkv_pool* pool) { delete pool; }

int32_t kv_pool_num_free(const pkv_pool* pool) {
    if (pool == nullptr) return -1;
    return static_cast<int32_t>(pool->free_stack.size()) + pool->ncached;
}

int32_t kv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap) {
    if (pool == nullptr || cap < 0 || (cap > 0 && out == nullptr)) return -1;
    const int32_t n = static_cast<int32_t>(pool->free_stack.size());
    const int32_t m = n < cap ? n : cap;
    if (m > 0) std::memcpy(out, pool->free_stack.data(), sizeof(int32_t) * m);
    return n;
}

// ---- cached list (prefix caching) ------------------------------------------
static void cached_unlink(pkv_pool* p, int32_t b) {
    const int32_t pv = p->cprev[b], nx = p->cnext[b];
    (pv >= 0 ? p->cnext[pv] : p->chead) = nx;
    (nx >= 0 ? p->cprev[nx] : p->ctail) = pv;
    p->cprev[b] = p->cnext[b] = -1;
    p->ncached -= 1;
}

static void cached_push(pkv_pool* p, int32_t b) {
    p->cprev[b] = p->ctail;
    p->cnext[b] = -1;
    (p->ctail >= 0 ? p->cnext[p->ctail] : p->chead) = b;
    p->ctail = b;
    p->ncached += 1;
}

static size_t available(const pkv_pool* p) {
    return p->free_stack.size() + static_cast<size_t>(p->ncached);
}

// A block for a new owner (the caller checked that one is available): the top
// of the free stack, else the longest-cached block, whose key is dropped.
static int32_t take_block(pkv_pool* p) {
    int32_t b;
    if (!p->free_stack.empty()) {
        b = p->free_stack.back();
        p->free_stack.pop_back();
    } else {
        b = p->chead;
        cached_unlink(p, b);
        p->key_block.erase(p->block_key[b]);
        p->keyed[b] = 0;
    }
    p->ref[b] = 1;
    return b;
}

// One reference released; a block left with none goes to the free stack, or
// to the cached list if it holds a key.
static void release(pkv_pool* p, int32_t b) {
    if (--p->ref[b] == 0) {
        if (p->keyed[b])
            cached_push(p, b);
        else
            p->free_stack.push_back(b);
    }
}

pkv_status block_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids) {
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "block_alloc: pool is NULL");
    if (n < 0) return fail(PKV_ERR_INVALID, "block_alloc: negative count %d", n);
    if (n > 0 && out_ids == nullptr) return fail(PKV_ERR_INVALID, "block_alloc: out_ids is NULL");
    if (static_cast<size_t>(n) > available(pool))
        return fail(PKV_ERR_OOM, "block_alloc: %d blocks requested, %zu free", n,
                    available(pool));
    for (int32_t i = 0; i < n; ++i) out_ids[i] = take_block(pool);
    return PKV_OK;
}

static pkv_status check_ids(const pkv_pool* pool, int32_t n, const int32_t* ids, const char* who) {
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", who);
    if (n < 0) return fail(PKV_ERR_INVALID, "%s: negative count %d", who, n);
    if (n > 0 && ids == nullptr) return fail(PKV_ERR_INVALID, "%s: ids is NULL", who);
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= pool->desc.num_blocks)
            return fail(PKV_ERR_INVALID, "%s: block id %d out of range", who, ids[i]);
    return PKV_OK;
}

pkv_status block_free(pkv_pool* pool, int32_t n, const int32_t* ids) {
    pkv_status st = check_ids(pool, n, ids, "block_free");
    if (st != PKV_OK) return st;
    // An id may appear several times; it must hold at least that many references.
    std::unordered_map<int32_t, int32_t> need;
    need.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) need[ids[i]] += 1;
    for (const auto& kv : need)
        if (pool->ref[kv.first] < kv.second)
            return fail(PKV_ERR_STATE, "block_free: block %d holds %d references, %d released",
                        kv.first, pool->ref[kv.first], kv.second);
    for (int32_t i = 0; i < n; ++i) release(pool, ids[i]);
    return PKV_OK;
}

pkv_status block_incref(pkv_pool* pool, int32_t n, const int32_t* ids) {
    pkv_status st = check_ids(pool, n, ids, "block_incref");
    if (st != PKV_OK) return st;
    for (int32_t i = 0; i < n; ++i)
        if (pool->ref[ids[i]] == 0)
            return fail(PKV_ERR_STATE, "block_incref: block %d is free", ids[i]);
    for (int32_t i = 0; i < n; ++i) pool->ref[ids[i]] += 1;
    return PKV_OK;
}

int32_t block_refcount(const pkv_pool* pool, int32_t id) {
    if (pool == nullptr || id < 0 || id >= pool->desc.num_blocks) return -1;
    return pool->ref[id];
}

pkv_status kv_seq_fork(pkv_pool* pool, const int32_t* src_row, int32_t* dst_row,
                       int32_t num_blocks) {
    if (num_blocks > 0 && dst_row == nullptr)
        return fail(PKV_ERR_INVALID, "kv_seq_fork: dst_row is NULL");
    pkv_status st = block_incref(pool, num_blocks, src_row);
    if (st != PKV_OK) return st;
    for (int32_t j = 0; j < num_blocks; ++j) dst_row[j] = src_row[j];
    return PKV_OK;
}

// kv_seq_extend and kv_seq_extend_cow. cow == false: a token landing in a
// shared block is an error. cow == true: the sequence first takes a private
// copy of that block (the pair goes to copy_src / copy_dst). Sequences are
// served in index order, so a block shared by k rows is copied by the first
// k - 1 of them that write into it and kept by the last.
static pkv_status extend_impl(const char* who, pkv_pool* pool, int32_t num_seqs,
                              int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* cur_lens, const int32_t* new_lens,
                              int64_t* slot_mapping_out, bool cow, int32_t* copy_src,
                              int32_t* copy_dst, int32_t* num_copies) {
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "%s: pool is NULL", who);
    if (num_seqs < 0 || max_blocks_per_seq < 0)
        return fail(PKV_ERR_INVALID, "%s: negative size", who);
    if (cow && num_copies == nullptr) return fail(PKV_ERR_INVALID, "%s: num_copies_out is NULL", who);
    if (cow) *num_copies = 0;
    if (num_seqs == 0) return PKV_OK;
    if (block_tables == nullptr || cur_lens == nullptr || new_lens == nullptr)
        return fail(PKV_ERR_INVALID, "%s: NULL array", who);
    const int32_t bs = pool->desc.block_size;
    int64_t needed = 0, tokens = 0, copies = 0;
    // Reference drops of earlier copies in this call, so a later writer into
    // the same block sees the count it will find.
    std::unordered_map<int32_t, int32_t> dropped;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t cur = cur_lens[i], nw = new_lens[i];
        if (cur < 0 || nw < cur)
            return fail(PKV_ERR_INVALID, "%s: seq %d: lengths %lld -> %lld", who, i,
                        static_cast<long long>(cur), static_cast<long long>(nw));
        const int64_t nb_new = (nw + bs - 1) / bs, nb_cur = (cur + bs - 1) / bs;
        if (nb_new > max_blocks_per_seq)
            return fail(PKV_ERR_INVALID, "%s: seq %d needs %lld blocks, row holds %d", who, i,
                        static_cast<long long>(nb_new), max_blocks_per_seq);
        if (nw > cur && cur % bs != 0) {
            const int32_t b = block_tables[static_cast<int64_t>(i) * max_blocks_per_seq + cur / bs];
            if (b < 0 || b >= pool->desc.num_blocks)
                return fail(PKV_ERR_INVALID, "%s: seq %d: block id %d out of range", who, i, b);
            const auto it = dropped.find(b);
            const int32_t ref = pool->ref[b] - (it == dropped.end() ? 0 : it->second);
            if (ref < 1 || (ref > 1 && !cow))
                return fail(PKV_ERR_STATE, "%s: seq %d: block %d has refcount %d (free or shared)",
                            who, i, b, ref);
            if (ref > 1) {
                dropped[b] += 1;
                needed += 1;
                copies += 1;
            }
        }
        needed += nb_new - nb_cur;
        tokens += nw - cur;
    }
    if (tokens > 0 && slot_mapping_out == nullptr)
        return fail(PKV_ERR_INVALID, "%s: slot_mapping_out is NULL", who);
    if (copies > 0 && (copy_src == nullptr || copy_dst == nullptr))
        return fail(PKV_ERR_INVALID, "%s: copy_src_out or copy_dst_out is NULL", who);
    if (needed > static_cast<int64_t>(available(pool)))
        return fail(PKV_ERR_OOM, "%s: %lld blocks needed, %zu free", who,
                    static_cast<long long>(needed), available(pool));
    int64_t k = 0;
    int32_t c = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
        const int32_t cur = cur_lens[i];
        if (cow && new_lens[i] > cur && cur % bs != 0) {
            const int32_t b = row[cur / bs];
            if (pool->ref[b] > 1) {  // copy on write: a private block for this row
                const int32_t nb = take_block(pool);
                pool->ref[b] -= 1;
                row[cur / bs] = nb;
                copy_src[c] = b;
                copy_dst[c] = nb;
                ++c;
            }
        }
        for (int32_t pos = cur; pos < new_lens[i]; ++pos) {
            if (pos % bs == 0) row[pos / bs] = take_block(pool);
            slot_mapping_out[k++] = static_cast<int64_t>(row[pos / bs]) * bs + pos % bs;
        }
    }
    if (cow) *num_copies = c;
    return PKV_OK;
}

pkv_status kv_seq_extend(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* cur_lens,
                         const int32_t* new_lens, int64_t* slot_mapping_out) {
    return extend_impl("kv_seq_extend", pool, num_seqs, block_tables, max_blocks_per_seq,
                       cur_lens, new_lens, slot_mapping_out, false, nullptr, nullptr, nullptr);
}

pkv_status kv_seq_extend_cow(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* cur_lens,
                             const int32_t* new_lens, int64_t* slot_mapping_out,
                             int32_t* copy_src_out, int32_t* copy_dst_out,
                             int32_t* num_copies_out) {
    return extend_impl("kv_seq_extend_cow", pool, num_seqs, block_tables, max_blocks_per_seq,
                       cur_lens, new_lens, slot_mapping_out, true, copy_src_out, copy_dst_out,
                       num_copies_out);
}

pkv_status kv_seq_trim(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t window,
                       int32_t* num_released_out) {
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "kv_seq_trim: pool is NULL");
    if (num_seqs < 0 || max_blocks_per_seq < 0 || window <= 0)
        return fail(PKV_ERR_INVALID, "kv_seq_trim: bad sizes or window %d", window);
    if (num_seqs > 0 && (block_tables == nullptr || context_lens == nullptr))
        return fail(PKV_ERR_INVALID, "kv_seq_trim: NULL array");
    const int32_t bs = pool->desc.block_size;
    std::unordered_map<int32_t, int32_t> need;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t before = static_cast<int64_t>(context_lens[i]) - window;
        const int64_t nj = before > 0 ? std::min<int64_t>(before / bs, max_blocks_per_seq) : 0;
        const int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
        for (int64_t j = 0; j < nj; ++j) {
            const int32_t b = row[j];
            if (b == -1) continue;
            if (b < 0 || b >= pool->desc.num_blocks)
                return fail(PKV_ERR_INVALID, "kv_seq_trim: seq %d: block id %d out of range", i, b);
            need[b] += 1;
        }
    }
    for (const auto& kv : need)
        if (pool->ref[kv.first] < kv.second)
            return fail(PKV_ERR_STATE, "kv_seq_trim: block %d holds %d references, %d released",
                        kv.first, pool->ref[kv.first], kv.second);
    int32_t released = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t before = static_cast<int64_t>(context_lens[i]) - window;
        const int64_t nj = before > 0 ? std::min<int64_t>(before / bs, max_blocks_per_seq) : 0;
        int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks_per_seq;
        for (int64_t j = 0; j < nj; ++j) {
            if (row[j] == -1) continue;
            release(pool, row[j]);
            row[j] = -1;
            ++released;
        }
    }
    if (num_released_out != nullptr) *num_released_out = released;
    return PKV_OK;
}

int32_t kv_pool_num_cached(const pkv_pool* pool) {
    if (pool == nullptr) return -1;
    return pool->ncached;
}

int32_t kv_pool_cached_list(const pkv_pool* pool, int32_t* out, int32_t cap) {
    if (pool == nullptr || cap < 0 || (cap > 0 && out == nullptr)) return -1;
    int32_t k = 0;
    for (int32_t b = pool->chead; b >= 0 && k < cap; b = pool->cnext[b]) out[k++] = b;
    return pool->ncached;
}

pkv_status kv_prefix_register(pkv_pool* pool, const uint64_t* keys, const int32_t* ids,
                              int32_t n, int32_t* num_registered_out) {
    pkv_status st = check_ids(pool, n, ids, "kv_prefix_register");
    if (st != PKV_OK) return st;
    if (n > 0 && keys == nullptr) return fail(PKV_ERR_INVALID, "kv_prefix_register: keys is NULL");
    for (int32_t i = 0; i < n; ++i)
        if (pool->ref[ids[i]] == 0)
            return fail(PKV_ERR_STATE, "kv_prefix_register: block %d is free", ids[i]);
    int32_t added = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t b = ids[i];
        if (pool->keyed[b] || pool->key_block.count(keys[i])) continue;  // first key wins
        pool->key_block.emplace(keys[i], b);
        pool->block_key[b] = keys[i];
        pool->keyed[b] = 1;
        ++added;
    }
    if (num_registered_out != nullptr) *num_registered_out = added;
    return PKV_OK;
}

pkv_status kv_prefix_acquire(pkv_pool* pool, const uint64_t* keys, int32_t n, int32_t* ids_out,
                             int32_t* matched_out) {
    if (pool == nullptr) return fail(PKV_ERR_INVALID, "kv_prefix_acquire: pool is NULL");
    if (n < 0) return fail(PKV_ERR_INVALID, "kv_prefix_acquire: negative count %d", n);
    if (matched_out == nullptr)
        return fail(PKV_ERR_INVALID, "kv_prefix_acquire: matched_out is NULL");
    if (n > 0 && (keys == nullptr || ids_out == nullptr))
        return fail(PKV_ERR_INVALID, "kv_prefix_acquire: NULL keys or ids_out");
    int32_t m = 0;
    for (; m < n; ++m) {
        const auto it = pool->key_block.find(keys[m]);
        if (it == pool->key_block.end()) break;
        const int32_t b = it->second;
        if (pool->ref[b] == 0) cached_unlink(pool, b);
        pool->ref[b] += 1;
        ids_out[m] = b;
    }
    *matched_out = m;
    return PKV_OK;
}

}  // extern "C"
