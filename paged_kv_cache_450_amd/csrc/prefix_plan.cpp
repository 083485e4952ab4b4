// Host planning for the shared-prefix decode: which sequences of a batch
// begin with the same physical blocks.
//
// [P2] "vLLM 推理加速原理详解：...", section "PagedAttention：把操作系统的虚拟内存搬进
// GPU": sequences that share a prompt (parallel samples, a common system
// prompt) map the same physical blocks through their tables, with reference
// counts. Those blocks hold identical K/V for every sharer, so a decode step
// can read each of them once for all sharers (paged_attn_decode_prefix).
//
// The plan follows only the tables: sequences are grouped by the id of their
// first block; a group's shared run is the longest run of leading blocks that
// every member maps to the same ids, limited to each member's full blocks
// before the block of its last token (that block is written by the step and is
// never shared). A group is kept when it has two or more members and its run
// is at least min_blocks long.

#include <algorithm>
#include <map>
#include <vector>

#include "common.h"

extern "C" pkv_status paged_attn_prefix_plan(const int32_t* block_tables,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t max_context_len, int32_t min_blocks,
                                             int32_t* seq_prefix_blocks, int32_t* group_offsets,
                                             int32_t* group_members, int32_t* group_blocks,
                                             int32_t* num_groups, int32_t* max_group_size) {
    using pkv::fail;
    const char* fn = "paged_attn_prefix_plan";
    if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID, "%s: negative size", fn);
    if (min_blocks < 1) return fail(PKV_ERR_INVALID, "%s: min_blocks %d < 1", fn, min_blocks);
    if (seq_prefix_blocks == nullptr || group_offsets == nullptr || group_members == nullptr ||
        group_blocks == nullptr || num_groups == nullptr || max_group_size == nullptr)
        return fail(PKV_ERR_INVALID, "%s: NULL output", fn);
    if (num_seqs > 0 && (block_tables == nullptr || context_lens == nullptr))
        return fail(PKV_ERR_INVALID, "%s: NULL block_tables or context_lens", fn);

    // Full blocks before the block of the last token, as a decode reads the
    // context (clamped like the decode calls clamp it).
    const int64_t reach =
        std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * 16);
    std::vector<int32_t> shareable(static_cast<size_t>(num_seqs));
    std::map<int32_t, std::vector<int32_t>> by_first;  // ordered: deterministic plan
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t L = std::min<int64_t>(std::max(context_lens[i], 0), reach);
        shareable[i] = L > 0 ? static_cast<int32_t>((L - 1) / 16) : 0;
        seq_prefix_blocks[i] = 0;
        if (shareable[i] >= min_blocks)
            by_first[block_tables[static_cast<size_t>(i) * max_blocks_per_seq]].push_back(i);
    }
    struct Group {
        std::vector<int32_t> members;
        int32_t blocks;
    };
    std::vector<Group> groups;
    for (auto& kv : by_first) {
        const std::vector<int32_t>& mem = kv.second;
        if (mem.size() < 2) continue;
        const int32_t* ref = block_tables + static_cast<size_t>(mem[0]) * max_blocks_per_seq;
        int32_t run = shareable[mem[0]];
        for (size_t k = 1; k < mem.size(); ++k) {
            const int32_t* row = block_tables + static_cast<size_t>(mem[k]) * max_blocks_per_seq;
            int32_t j = 0;
            const int32_t lim = std::min(run, shareable[mem[k]]);
            while (j < lim && row[j] == ref[j]) ++j;
            run = j;
        }
        if (run >= min_blocks) groups.push_back({mem, run});
    }
    // Groups in the order of their first member.
    std::sort(groups.begin(), groups.end(),
              [](const Group& a, const Group& b) { return a.members[0] < b.members[0]; });
    int32_t off = 0, widest = 0;
    group_offsets[0] = 0;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
        for (int32_t s : groups[gi].members) {
            group_members[off++] = s;
            seq_prefix_blocks[s] = groups[gi].blocks;
        }
        group_offsets[gi + 1] = off;
        group_blocks[gi] = groups[gi].blocks;
        widest = std::max(widest, static_cast<int32_t>(groups[gi].members.size()));
    }
    *num_groups = static_cast<int32_t>(groups.size());
    *max_group_size = widest;
    return PKV_OK;
}
