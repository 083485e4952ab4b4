/*
 * pagedkv.h - C ABI of a paged KV cache and paged decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  [P2] "vLLM 推理加速原理详解：大模型服务吞吐量为何能提升 10 倍"
 *       (fudengji.cn/article/275)
 *       - "PagedAttention：把操作系统的虚拟内存搬进 GPU": fixed-size physical
 *         blocks, a per-sequence page table mapping logically contiguous KV to
 *         scattered blocks, allocation on demand, no external fragmentation,
 *         one physical block shared by several sequences (beam search, common
 *         prompt prefixes), and an attention kernel that reads KV from the
 *         non-contiguous blocks.
 *       - "连续批处理：别再等最慢的那个请求了": the block manager calls a
 *         scheduler makes every iteration (free a finished request's table,
 *         count free blocks, check and perform allocation).
 *       - "vLLM 也不是银弹：真实部署中的坑", first pitfall: the cache is one
 *         pool preallocated from GPU memory; third pitfall: FP8 KV cache.
 *       - "从零开始：vLLM 部署的实战建议", step four: cache usage is a
 *         monitored gauge (1 - free / total).
 *  [P3] "突破大模型推理瓶颈：vLLM框架核心技术深度解剖与实战指南", section 2.4:
 *       accumulation in FP32.
 *
 * Conventions for every call:
 *  - Device pointers point to memory the caller allocated and owns (for
 *    example through PyTorch). The library never allocates or frees device
 *    memory and never synchronises the host with the device.
 *  - GPU work is enqueued on the given stream and runs asynchronously;
 *    stream = NULL means the default stream. Launch failures return
 *    PKV_ERR_HIP.
 *  - Every call checks all of its host-visible arguments before it changes
 *    any state or launches anything; a call that fails changes nothing.
 *    On failure pkv_last_error() describes the cause.
 *  - No C++ exception crosses this interface.
 *  - Pool objects are not thread-safe: one scheduler thread owns a pool.
 *  - The context length L of a sequence counts every cached token, the
 *    newest one included: a decode step first appends the new token at
 *    position L-1, then attends over positions [0, L).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#pragma GCC visibility push(default)

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1, /* bad argument: null pointer, unsupported shape or dtype, bad id */
    PKV_ERR_OOM = -2,     /* not enough free blocks; nothing was allocated */
    PKV_ERR_STATE = -3,   /* refcount misuse: freeing a free block, sharing a free block,
                             appending into a shared block (no copy-on-write) */
    PKV_ERR_HIP = -4      /* a HIP launch failed */
} pkv_status;

typedef enum {
    PKV_F16 = 0,      /* IEEE binary16 */
    PKV_BF16 = 1,     /* bfloat16 */
    PKV_FP8_E4M3 = 2  /* OCP E4M3 "fn": bias 7, max 448, NaN = S.1111.111, no inf */
} pkv_dtype;

/* Block size in tokens. The only supported value. */
#define PKV_BLOCK_SIZE 16

/*
 * Pool geometry. [P2] "PagedAttention：...": memory is cut into fixed-size
 * physical blocks. One block id names the same block in every layer, so one
 * block table serves all layers of a model.
 *
 * Device layout (this library's contract): element (layer l, c in {K=0,V=1},
 * block b, kv head h, slot t, dim d) is stored at element offset
 *     ((((l*2 + c)*num_blocks + b)*num_kv_heads + h)*block_size + t)*head_dim + d
 * so each (l, c, b, h) tile of block_size x head_dim elements is contiguous.
 *
 * Supported: block_size == 16; head_dim in {64, 128}; num_kv_heads >= 1;
 * kv_dtype a pkv_dtype.
 */
typedef struct {
    int32_t num_layers;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t kv_dtype; /* pkv_dtype */
} pkv_pool_desc;

typedef struct pkv_pool pkv_pool; /* opaque; holds host metadata only */

/* Bytes of device memory the pool occupies:
 * num_layers * 2 * num_blocks * num_kv_heads * block_size * head_dim * elem_size.
 * For one request's ceil(L/16) blocks this is the closed form
 * 2 x L x layers x heads x head_dim x bytes of [P2] "真正吃显存的是 KV Cache，
 * 不是模型权重". Returns 0 for an unsupported descriptor. */
size_t kv_pool_bytes(const pkv_pool_desc* desc);

/* Create the host bookkeeping for a pool whose device memory the caller has
 * already allocated ([P2] first pitfall: one preallocated pool).
 * device_base: device pointer to kv_pool_bytes(desc) bytes, 256-byte aligned,
 *   borrowed (it must outlive the pool); NULL is allowed for a
 *   bookkeeping-only pool, on which the kernel calls fail with INVALID.
 * bytes: size of that allocation; must be >= kv_pool_bytes(desc) when
 *   device_base is not NULL.
 * All blocks start free; the first allocations return ids 0, 1, 2, ...
 * Errors: INVALID (bad descriptor, size, alignment, NULL out). */
pkv_status kv_pool_create(const pkv_pool_desc* desc, void* device_base, size_t bytes,
                          pkv_pool** out);

/* Destroy the host bookkeeping. Does not touch device memory. NULL is a no-op. */
void kv_pool_destroy(pkv_pool* pool);

/* Number of free blocks ([P2] "连续批处理": get_num_free_blocks; a request
 * for n blocks can be served exactly when this is >= n, since blocks are
 * interchangeable). With prefix caching, cached blocks count as free (they are
 * evicted on demand). Returns -1 for a NULL pool. Cache usage = 1 -
 * free/total. */
int32_t kv_pool_num_free(const pkv_pool* pool);

/* Copy the free-block stack, bottom first, into out[0 .. min(n, cap)) and
 * return n, the number of free blocks (-1 for bad arguments). The next
 * allocation pops from the top (out[n-1]). For tests and diagnostics. */
int32_t kv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap);

/* Allocate n blocks ([P2] "PagedAttention：...": on-demand allocation).
 * out_ids: host array of n ints, receives the ids in pop order; each gets
 *   refcount 1.
 * Errors: INVALID (NULL args, n < 0), OOM (fewer than n free; nothing
 *   allocated). */
pkv_status block_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids);

/* Drop one reference on each of ids[0..n) (host array) ([P2] "连续批处理":
 * a finished request's table is freed). An id whose count reaches 0 is pushed
 * on the free stack, in argument order (last freed = next allocated).
 * An id may appear several times if it holds that many references.
 * Errors: INVALID (NULL, n < 0, id out of range), STATE (an id would drop
 *   below 0). */
pkv_status block_free(pkv_pool* pool, int32_t n, const int32_t* ids);

/* Add one reference to each of ids[0..n) (host array): one physical block
 * backs one more logical block ([P2] "PagedAttention：...": shared blocks for
 * beam search and common prefixes).
 * Errors: INVALID (NULL, n < 0, out of range), STATE (an id is free). */
pkv_status block_incref(pkv_pool* pool, int32_t n, const int32_t* ids);

/* Reference count of one block; -1 if the id is out of range or pool NULL. */
int32_t block_refcount(const pkv_pool* pool, int32_t id);

/* Share a prefix: dst_row[j] = src_row[j] for j < num_blocks and take one
 * more reference on each of those ids (host arrays). Used when a sequence
 * starts with the same full blocks as another (common prompt prefix).
 * Errors: INVALID (NULL, num_blocks < 0, id out of range), STATE (an id is
 *   free). */
pkv_status kv_seq_fork(pkv_pool* pool, const int32_t* src_row, int32_t* dst_row,
                       int32_t num_blocks);

/* Grow sequence i from cur_lens[i] to new_lens[i] tokens (host arrays) and
 * emit the slot of every new token ([P2] "PagedAttention：...": a block is
 * taken when a token opens one).
 * block_tables: host array [num_seqs][max_blocks_per_seq]; row i holds the ids
 *   of sequence i's blocks in logical order. For each new token at position
 *   pos, when pos % 16 == 0 a block is popped and written to
 *   block_tables[i][pos/16]; the token's slot is
 *   block_tables[i][pos/16] * 16 + pos % 16.
 * slot_mapping_out: host array of sum(new_lens - cur_lens) int64, filled
 *   sequence by sequence, positions in increasing order.
 * Errors: INVALID (NULL, negative or shrinking lengths, a row too short,
 *   out-of-range id), STATE (a token would land in a block whose refcount is
 *   not 1), OOM (not enough free blocks for the whole call). On error nothing
 *   changes. */
pkv_status kv_seq_extend(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* cur_lens,
                         const int32_t* new_lens, int64_t* slot_mapping_out);

/* kv_seq_extend with copy on write ([P2] "PagedAttention：...": several
 * logical blocks may map to one physical block, as for beam search or a
 * shared prompt; a sequence about to write into a block it shares takes a
 * private copy first).
 * Sequences are served in index order. When sequence i's first new token
 * lands in a partially filled block whose refcount is above 1 at that moment,
 * a fresh block is popped (as by block_alloc), block_tables[i][cur_lens[i]/16]
 * is set to it, one reference on the shared block is released, and the pair
 * (shared, fresh) is written to copy_src_out[c], copy_dst_out[c] (host int32
 * arrays of at least num_seqs entries). A block shared by k rows is thus
 * copied by the first k - 1 writers and kept by the last. *num_copies_out
 * receives the number of pairs. Everything else is kv_seq_extend.
 * Before any token is written into a fresh block, run kv_block_copy on the
 * pairs (same stream as the appends).
 * Errors: those of kv_seq_extend (OOM counts the copies' blocks; STATE only
 * for a free block), INVALID (NULL num_copies_out, or NULL copy arrays when a
 * copy is needed). On error nothing changes. */
pkv_status kv_seq_extend_cow(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* cur_lens,
                             const int32_t* new_lens, int64_t* slot_mapping_out,
                             int32_t* copy_src_out, int32_t* copy_dst_out,
                             int32_t* num_copies_out);

/* Copy whole blocks on the GPU: for every layer, K and V, all kv heads,
 * block dst_ids[i] := block src_ids[i] ([P2] "PagedAttention：...": the copy
 * of copy on write). src_ids, dst_ids: host int32 arrays of n ids in
 * [0, num_blocks); destinations distinct and none of them a source of the
 * same call (sources may repeat). Enqueued on stream; nothing is allocated
 * (the ids travel as kernel arguments, 128 pairs per launch).
 * Errors: INVALID (NULL pool, base or arrays, negative n, ids out of range,
 *   a repeated destination, a destination that is also a source), HIP. */
pkv_status kv_block_copy(const pkv_pool* pool, const int32_t* src_ids, const int32_t* dst_ids,
                         int32_t n, hipStream_t stream);

/* Swapping blocks to host memory ([P2] "vLLM 也不是银弹：真实部署中的坑" and
 * "从零开始：vLLM 部署的实战建议", second step: when the cache runs short,
 * running requests are preempted and their blocks swapped out, to come back
 * when blocks free up).
 *
 * Swap space is a caller-owned buffer of host memory, pinned (hipHostMalloc;
 * memory registered after the fact or pageable memory is rejected), divided
 * into slots of kv_swap_slot_bytes(pool) bytes. Slot s holds one block of
 * every layer, K and V, as [num_layers][2][num_kv_heads][16][head_dim]
 * elements of the pool's dtype, starting at byte s * kv_swap_slot_bytes. The
 * GPU reads and writes the pinned pages directly; the calls are enqueued on
 * stream and allocate nothing (ids and slots travel as kernel arguments, 128
 * pairs per launch). The host must not touch the slots involved until the
 * stream has passed the call. Block bookkeeping is the caller's: swap a
 * request's blocks out, then block_free them; block_alloc fresh ids, then swap
 * the slots in to them. */

/* Bytes of one swap slot: 2 * num_layers * num_kv_heads * 16 * head_dim *
 * element size; 0 for a NULL pool. */
size_t kv_swap_slot_bytes(const pkv_pool* pool);

/* Slot host_slots[i] := block block_ids[i], for i < n (host int32 arrays).
 * host_buf / host_buf_bytes: the swap space. Blocks may repeat; slots must be
 * distinct.
 * Errors: INVALID (NULL pool, base or arrays, negative n, ids or slots out of
 *   range, a repeated slot, a buffer that is not one pinned host allocation of
 *   host_buf_bytes bytes), HIP. n == 0 does nothing. */
pkv_status kv_swap_out(const pkv_pool* pool, const int32_t* block_ids, const int32_t* host_slots,
                       int32_t n, void* host_buf, size_t host_buf_bytes, hipStream_t stream);

/* Block block_ids[i] := slot host_slots[i], for i < n. Slots may repeat;
 * blocks must be distinct. Errors as kv_swap_out (a repeated block instead of
 * a repeated slot). */
pkv_status kv_swap_in(const pkv_pool* pool, const int32_t* host_slots, const int32_t* block_ids,
                      int32_t n, const void* host_buf, size_t host_buf_bytes, hipStream_t stream);

/* Prefix caching ([P2] "PagedAttention：...": requests with the same prompt
 * prefix share its physical blocks; "从零开始：vLLM 部署的实战建议", third step:
 * prefix caching). The caller names the contents of a full block with a
 * 64-bit key (for example a hash of every token up to the block's end); the
 * library keeps the map key -> block. A keyed block whose last reference is
 * released keeps its contents and waits on the cached list instead of the
 * free stack; kv_prefix_acquire can revive it. Allocation (block_alloc,
 * kv_seq_extend, kv_seq_extend_cow) takes the free stack first and then evicts
 * cached blocks, the longest cached first, dropping their keys.
 * kv_pool_num_free counts free and cached blocks; kv_pool_free_list lists the
 * free stack only. */

/* Register ids[i] (live blocks whose 16 slots are written) under keys[i]
 * (host arrays). A block keeps the first key it is given and a key the first
 * block; other pairs are skipped. *num_registered_out (may be NULL) receives
 * the number of pairs taken.
 * Errors: INVALID (NULL arrays, ids out of range), STATE (a free block). On
 * error nothing changes. */
pkv_status kv_prefix_register(pkv_pool* pool, const uint64_t* keys, const int32_t* ids,
                              int32_t n, int32_t* num_registered_out);

/* The longest leading run keys[0..m) of registered keys: writes their blocks
 * to ids_out[0..m) (host), takes one reference on each (a cached block
 * becomes live again) and writes m to *matched_out. The caller then owns the
 * references, to release with block_free.
 * Errors: INVALID (NULL pool, arrays or matched_out, negative n). */
pkv_status kv_prefix_acquire(pkv_pool* pool, const uint64_t* keys, int32_t n, int32_t* ids_out,
                             int32_t* matched_out);

/* Number of cached blocks, or -1 for NULL. */
int32_t kv_pool_num_cached(const pkv_pool* pool);

/* Copies up to cap cached block ids, longest cached first, into out; returns
 * the number of cached blocks (or -1 for NULL / bad arguments). */
int32_t kv_pool_cached_list(const pkv_pool* pool, int32_t* out, int32_t cap);

/* Sliding window: release the blocks of each sequence that lie wholly before
 * its window ([P2] "vLLM 也不是银弹：...", third pitfall), so that a long
 * sequence holds at most ceil(window / 16) + 1 blocks. For sequence i (host
 * arrays): every block j with 16 * (j + 1) <= context_lens[i] - window whose
 * table entry is not -1 loses one reference and its entry becomes -1.
 * *num_released_out receives the number of references released.
 * Errors: INVALID (NULL arrays, window <= 0, an id out of range), STATE (a
 * free block). On error nothing changes. */
pkv_status kv_seq_trim(pkv_pool* pool, int32_t num_seqs, int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t window,
                       int32_t* num_released_out);

/* Write each token's K and V into its slot of one layer ([P2]
 * "PagedAttention：...": the cache grows by slots as tokens are produced;
 * third pitfall: FP8 KV cache).
 * k, v: device [num_tokens][num_kv_heads][head_dim] of src_dtype (F16 or
 *   BF16), rows contiguous, 16-byte aligned.
 * slot_mapping: device int64 [num_tokens]; slot = block * 16 + offset. A slot
 *   < 0 or >= num_blocks*16 is skipped. Slots within one call must be unique
 *   (otherwise which write lands is unspecified).
 * 16-bit caches: src_dtype must equal the cache dtype; the bits are copied.
 * FP8 cache: stores e4m3(fp32(x) / scale[h]) rounded to nearest, ties to even,
 *   saturating to +-448 (never NaN for finite x). k_scale, v_scale: device
 *   fp32 [num_kv_heads]; ignored (may be NULL) for 16-bit caches.
 * Errors: INVALID (NULL pool or base, bad layer, dtype, count), HIP. */
pkv_status kv_cache_append(const pkv_pool* pool, int32_t layer, const void* k, const void* v,
                           int32_t src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                           const float* k_scale, const float* v_scale, hipStream_t stream);

/* Bytes of workspace paged_attn_decode needs.
 * Source: none on the pages. Cutting a long context into partitions whose
 * partials are merged afterwards (split-K) is this library's long-context
 * form, chosen for one GPU's many compute units; the pages only name the
 * long-context pressure ([P2] third pitfall).
 * partition_size > 0: per (sequence, query head, partition) an fp32 max, an
 *   fp32 sum and head_dim fp32 outputs, with ceil(max_context_len /
 *   partition_size) partitions per sequence, laid out as described below
 *   (OFF + num_seqs*num_q_heads*P*head_dim*4).
 * partition_size == 0: the balanced single pass (see paged_attn_decode): two
 *   partial slots per wave of the launch, 8 waves per compute unit of the
 *   current device, each min(num_q_heads, 8) x (head_dim + 4) fp32; 0 when
 *   num_seqs > 4096 (only the per-sequence single pass exists there).
 * 0 when an argument is out of range. */
size_t paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/* Workspace layout (little-endian fp32, P = ceil(max_context_len / partition_size)):
 *   ml[num_seqs][num_q_heads][P][2]         at byte 0   (m_p, l_p)
 *   o [num_seqs][num_q_heads][P][head_dim]  at byte OFF = num_seqs*num_q_heads*P*8
 *                                           rounded up to a multiple of 256
 * For partition p of sequence i (tokens [p*PS, min((p+1)*PS, L))):
 *   m_p = max_t s_t, l_p = sum_t exp(s_t - m_p), o_p = sum_t exp(s_t - m_p) v_t / l_p,
 * with s_t = scale * <q, k_t> in natural-log units. Exception: a fused step
 * (paged_attn_decode_append) on an FP8 cache counts the new token at L - 1 in
 * the first partition it reads instead of the last (the merge is the same). */

/* Single-query decode attention over the paged cache of one layer ([P2]
 * "PagedAttention：...": the attention kernel reads KV from non-contiguous
 * physical blocks through the page table; [P3] 2.4: FP32 accumulation).
 * For each sequence i and query head h, with kv head g = h / (num_q_heads /
 * num_kv_heads):  out[i][h] = softmax(scale * q[i][h] . K_i[g]^T) V_i[g]
 * over the L_i = context_lens[i] tokens of sequence i.
 * q: device [num_seqs][num_q_heads][head_dim], q_dtype F16 or BF16, 16-byte
 *   aligned; a 16-bit cache must have q_dtype equal to the cache dtype; an FP8
 *   cache takes either. out: device, same shape and dtype as q (rounded to
 *   nearest even), 16-byte aligned.
 * block_tables: device int32 [num_seqs][max_blocks_per_seq]; entries past
 *   ceil(L_i/16) are never read. An id outside [0, num_blocks) is not read;
 *   its 16 tokens are treated as absent.
 * context_lens: device int32 [num_seqs]. L_i is clamped to
 *   min(max_context_len, max_blocks_per_seq*16); L_i <= 0 gives zeros.
 * num_q_heads must be num_kv_heads * G with G in {1, 2, 4, 8}.
 * k_scale, v_scale: device fp32 [num_kv_heads] for an FP8 cache (value =
 *   decode(code) * scale), ignored otherwise.
 * partition_size == 0: a single pass writes out; no reduce call follows.
 *   - workspace == NULL (or an FP8 cache, or num_seqs > 4096): one workgroup
 *     per (sequence, kv head), sequences handed out longest first;
 *   - otherwise the balanced form: the tiles of the whole batch are cut into
 *     equal ranges, one per group of resident waves that read adjacent kv
 *     heads of the same blocks in step (one wave per head), so the work is
 *     even whatever the length mix; contexts split between ranges leave
 *     partials in workspace
 *     (256-byte aligned, >= paged_attn_workspace_bytes(..., 0) bytes, no
 *     initial contents needed) that a second kernel of the same call merges.
 *     Calls that share a workspace must be ordered on one stream.
 * partition_size > 0 (a multiple of 16): every partition writes its
 *   (m_p, l_p, o_p) to workspace (layout above) and out is not touched; the
 *   caller must then run paged_attn_reduce on the same stream with the same
 *   shapes. workspace_bytes must be >= paged_attn_workspace_bytes(...).
 * Limits: num_seqs <= 65535; ceil(max_context_len / partition_size) <= 65535.
 * Errors: INVALID (shapes, dtypes, NULLs, alignment, workspace too small,
 *   limits), HIP. */
pkv_status paged_attn_decode(const pkv_pool* pool, int32_t layer, const void* q, int32_t q_dtype,
                             void* out, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             float scale, const float* k_scale, const float* v_scale,
                             int32_t max_context_len, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* One decode step of one layer in one call: kv_cache_append of each
 * sequence's new token, then paged_attn_decode ([P2] "PagedAttention：...":
 * the step appends the token produced last and attends over the whole
 * context, the new token included). The per-sequence and split-K forms store
 * the new tokens from inside the decode kernel on a 16-bit cache with one
 * query head per kv head (the wave that reads a token's tile takes its row
 * from new_k / new_v and writes its slot) and on an FP8 cache with up to two
 * (that wave attends over the positions before the token and then folds in
 * the token's encoded K and V, which it writes to the slot), saving the
 * append launch. The balanced single pass does the same for any group size:
 * it reads each context's blocks without the new token's position and the
 * token as one more tile from new_k / new_v, whose wave also writes its slot.
 * (beside a shared-prefix pass too: a plan's shared blocks end before the
 * block of each member's last token, so that pass never reads a new slot).
 * The other forms (grouped heads on a 16-bit cache per sequence or split-K,
 * FP8 with four or eight query heads per kv head) run the append as a kernel
 * of its own first, on the same stream.
 * new_k, new_v: device [num_seqs][num_kv_heads][head_dim] of src_dtype, which
 *   must equal q_dtype (for a 16-bit cache, also the cache dtype); 16-byte
 *   aligned.
 * Sequence i's new token is its last position p = L_i - 1 (L_i =
 *   context_lens[i]): it is stored to slot block_tables[i][p / 16] * 16 +
 *   p % 16 exactly as kv_cache_append would store it (same bytes; E4M3
 *   encoding for an FP8 cache), and the attention uses those bytes. No write
 *   for a sequence with L_i <= 0, with L_i above min(max_context_len,
 *   max_blocks_per_seq * 16) (its last position is outside the call), or
 *   whose block id there is outside the pool.
 * Precondition: the block holding each written slot belongs to its sequence
 *   alone (refcount 1, as kv_seq_extend guarantees for blocks it writes into);
 *   its other tokens are read in the same call.
 * Every other argument, the output, the workspace and the errors are those of
 * paged_attn_decode; additional errors: INVALID (NULL or misaligned new_k /
 * new_v, src_dtype != q_dtype). */
pkv_status paged_attn_decode_append(const pkv_pool* pool, int32_t layer, const void* new_k,
                                    const void* new_v, int32_t src_dtype, const void* q,
                                    int32_t q_dtype, void* out, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    const float* k_scale, const float* v_scale,
                                    int32_t max_context_len, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sliding-window decode ([P2] "vLLM 也不是银弹：真实部署中的坑", third pitfall:
 * for long contexts the pages point to sliding-window attention and to FP8 KV).
 * paged_attn_decode (new_k == new_v == NULL) or paged_attn_decode_append
 * (both given) where sequence i attends over its last `window` tokens only:
 * positions [max(0, L_i - window), L_i). window == 0: the whole context.
 * Table entries of blocks wholly before the window are never read (they may
 * be -1, see kv_seq_trim). With partition_size > 0, partitions wholly before
 * the window leave empty partials (l = 0), which paged_attn_reduce ignores.
 * Every other argument, the output and the errors are those of the two
 * calls; additional error: INVALID (negative window, only one of new_k /
 * new_v given). */
pkv_status paged_attn_decode_window(const pkv_pool* pool, int32_t layer, const void* new_k,
                                    const void* new_v, int32_t src_dtype, const void* q,
                                    int32_t q_dtype, void* out, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    const float* k_scale, const float* v_scale,
                                    int32_t max_context_len, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes, int32_t window,
                                    hipStream_t stream);

/* Shared-prefix planning (host). [P2] "PagedAttention：...": sequences that
 * share a prompt map the same physical blocks (refcounted), so a decode step
 * can read those blocks once for all of them (paged_attn_decode_prefix).
 * Groups sequences by the id of their first block (host arrays:
 * block_tables [num_seqs][max_blocks_per_seq], context_lens [num_seqs]); a
 * group's shared run P is the longest run of leading blocks that every member
 * maps to the same ids, at most each member's full blocks before the block of
 * its last token, (min(L_i, max_context_len, max_blocks_per_seq*16) - 1) / 16.
 * Groups of two or more members with P >= min_blocks (>= 1) are kept, in the
 * order of their first member; members in increasing index.
 * Outputs (host, caller-owned): seq_prefix_blocks [num_seqs] (P of the
 *   sequence's group, else 0); group_offsets [num_seqs + 1] (group k's members
 *   are group_members[group_offsets[k] .. group_offsets[k+1])); group_members
 *   [num_seqs]; group_blocks [num_seqs] (P per group); num_groups;
 *   max_group_size (largest group, 0 if none).
 * Errors: INVALID (negative sizes, min_blocks < 1, NULL arrays). */
pkv_status paged_attn_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, int32_t min_blocks,
                                  int32_t* seq_prefix_blocks, int32_t* group_offsets,
                                  int32_t* group_members, int32_t* group_blocks,
                                  int32_t* num_groups, int32_t* max_group_size);

/* Workspace bytes of paged_attn_decode_prefix: the balanced pass's slots
 * (paged_attn_workspace_bytes(..., 0)), then two regions of
 * num_seqs * num_q_heads * (head_dim + 4) fp32 (the prefix partials, and the
 * members' suffix partials), each from a 256-byte boundary. 0 when an
 * argument is out of range (num_seqs > 4096). */
size_t paged_attn_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t head_dim);

/* Decode step with shared-prefix reads: the same result as
 * paged_attn_decode_append (new_k / new_v given) or paged_attn_decode
 * (both NULL) in the balanced single pass, on a 16-bit cache. A prefix kernel
 * reads the P shared leading blocks of each group once (all workgroups of a
 * (group, kv head) on one XCD, so repeats come from its L2) and computes, for
 * every member and query head, the partial (m, l, o) over those P*16 tokens on
 * matrix cores, 16 query rows at a time; the balanced pass reads each member
 * from block P on; the merge kernel joins the two with the log-sum-exp rule.
 * Group arguments (device int32, as paged_attn_prefix_plan writes them):
 *   seq_prefix_blocks [num_seqs], group_offsets [num_groups + 1],
 *   group_members, group_blocks [num_groups]; max_group_size bounds every
 *   group's size. num_groups == 0: no prefix kernel, the arrays are ignored.
 * Preconditions (not checked, as they live in device memory): the rows of a
 *   group's members hold the same ids in blocks [0, P); every member has
 *   1 <= P <= (L_i - 1) / 16 and seq_prefix_blocks = P; every other sequence
 *   has seq_prefix_blocks = 0; a sequence is in at most one group, so
 *   group_offsets[num_groups] <= num_seqs. A plan that breaks them gives wrong
 *   outputs, not stray accesses: the kernel skips groups whose offsets leave
 *   [0, num_seqs] and members outside [0, num_seqs).
 * workspace: device, 256-byte aligned, >= paged_attn_prefix_workspace_bytes;
 *   no initial contents needed; calls that share it must be ordered on one
 *   stream. Scale and dtypes: as paged_attn_decode (k_scale / v_scale are not
 *   taken: no FP8).
 * Errors: INVALID (an FP8 cache, num_seqs > 4096, group sizes out of range,
 *   NULL group arrays with num_groups > 0, a NULL or small workspace, and every
 *   error of paged_attn_decode_append), HIP. */
pkv_status paged_attn_decode_prefix(const pkv_pool* pool, int32_t layer, const void* new_k,
                                    const void* new_v, int32_t src_dtype, const void* q,
                                    int32_t q_dtype, void* out, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    int32_t max_context_len, const int32_t* seq_prefix_blocks,
                                    const int32_t* group_offsets, const int32_t* group_members,
                                    const int32_t* group_blocks, int32_t num_groups,
                                    int32_t max_group_size, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Decode step with shared-prefix reads through the L2: the same result as
 * paged_attn_decode_append (new_k / new_v given) or paged_attn_decode (both
 * NULL) in the balanced single pass on a 16-bit cache ([P2]
 * "PagedAttention：...": sequences that share a prompt map the same physical
 * blocks). The balanced pass reads every sequence's whole context as usual,
 * but the first seq_prefix_blocks[i] blocks of sequence i, which other
 * sequences of the batch share, are loaded with the caching policy (all other
 * KV loads stream through the caches), so the sharers' repeated reads of a
 * block can be served by the L2 instead of HBM. No extra kernel and no extra
 * partials: the lighter form for short shared prompts, where the prefix
 * kernel of paged_attn_decode_prefix costs more than it saves.
 * seq_prefix_blocks: device int32 [num_seqs], as paged_attn_prefix_plan
 *   writes it (0 for a sequence that shares nothing); only a load policy
 *   depends on it, so any values give the same output. NULL: the plain
 *   balanced pass.
 * workspace: as paged_attn_decode's balanced pass (at least
 *   paged_attn_workspace_bytes(..., 0) bytes, 256-byte aligned).
 * Errors: INVALID (an FP8 cache, num_seqs > 4096, a NULL workspace, and every
 *   error of paged_attn_decode_append), HIP. */
pkv_status paged_attn_decode_prefix_l2(const pkv_pool* pool, int32_t layer, const void* new_k,
                                       const void* new_v, int32_t src_dtype, const void* q,
                                       int32_t q_dtype, void* out, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t num_q_heads, float scale,
                                       int32_t max_context_len, const int32_t* seq_prefix_blocks,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Bytes of the library's static device scratch, one copy per GPU, that
 * paged_attn_decode_append_noalloc uses as its workspace. */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* paged_attn_decode_append without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The workspace is a static device
 * array of the library (PKV_STATIC_SCRATCH_BYTES, 32 MiB; each GPU the call
 * runs on holds its own copy until the process ends). Nothing is allocated:
 * the array's device address is looked up once per device (with that device
 * current) on the first call there.
 * Differences from paged_attn_decode_append:
 *  - out is always written: with partition_size > 0 the call runs
 *    paged_attn_reduce on the partials itself, on the same stream;
 *  - partition_size == 0 on a 16-bit cache with up to 4096 sequences takes
 *    the balanced single pass (as paged_attn_decode_append with a workspace);
 *    FP8 caches and larger batches take the per-sequence pass, which needs no
 *    workspace.
 * The scratch needs no initial contents. The current device must be the
 * device of stream and of every buffer. Every call on one GPU shares that
 * GPU's array, so calls that may overlap on one GPU (other streams, other
 * threads) race on it: order them on one stream.
 * Every other argument and the output are those of paged_attn_decode_append.
 * Errors: INVALID (a batch whose workspace would exceed
 *   PKV_STATIC_SCRATCH_BYTES, NULL out, and every error of
 *   paged_attn_decode_append and paged_attn_reduce), HIP (also when the
 *   scratch's device address cannot be had). */
pkv_status paged_attn_decode_append_noalloc(const pkv_pool* pool, int32_t layer,
                                            const void* new_k, const void* new_v,
                                            int32_t src_dtype, const void* q, int32_t q_dtype,
                                            void* out, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t num_seqs,
                                            int32_t num_q_heads, float scale,
                                            const float* k_scale, const float* v_scale,
                                            int32_t max_context_len, int32_t partition_size,
                                            hipStream_t stream);

/* Merge the partitions a partitioned paged_attn_decode left in workspace
 * into out (device [num_seqs][num_q_heads][head_dim] of out_dtype F16 or BF16).
 * Source: none on the pages; the exact log-sum-exp merge of this library's
 * split-K form (see paged_attn_workspace_bytes):
 *   M = max_p m_p, w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p
 * over p < ceil(L_i / partition_size) (L_i clamped to max_context_len);
 * a sequence with no tokens gets zeros.
 * Errors: INVALID (NULLs, head_dim not 64/128, partition_size <= 0 or not a
 *   multiple of 16), HIP. */
pkv_status paged_attn_reduce(const void* workspace, void* out, int32_t out_dtype,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                             hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
