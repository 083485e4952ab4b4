"""CPU tests of the shared-prefix decode's host side: the planner
(paged_attn_prefix_plan) against a plain Python statement of its rule, the
workspace size, and the argument checks of paged_attn_decode_prefix (all
host-side, before any launch). No GPU calls.
"""

import numpy as np
import pytest

import paged_kv_cache_450_amd as P


def model_plan(tables, lens, max_ctx, min_blocks):
    """The planner's rule, written out: sequences grouped by the id of their
    first block (only those with at least min_blocks full blocks before the
    block of their last token); a group's run is the longest common run of
    leading ids over its members, capped by every member's full blocks; groups
    of two or more with run >= min_blocks, ordered by first member."""
    B, W = tables.shape
    reach = min(max_ctx, W * 16)
    share = [max(0, (min(max(int(L), 0), reach) - 1) // 16) if min(max(int(L), 0), reach) > 0
             else 0 for L in lens]
    by_first = {}
    for i in range(B):
        if share[i] >= min_blocks:
            by_first.setdefault(int(tables[i, 0]), []).append(i)
    groups = []
    for mem in by_first.values():
        if len(mem) < 2:
            continue
        run = min(share[i] for i in mem)
        for i in mem[1:]:
            j = 0
            while j < run and tables[i, j] == tables[mem[0], j]:
                j += 1
            run = j
        if run >= min_blocks:
            groups.append((mem, run))
    groups.sort(key=lambda g: g[0][0])
    pre = np.zeros(B, dtype=np.int32)
    for mem, run in groups:
        pre[mem] = run
    return groups, pre


def random_batch(rng, B, W):
    """Tables with planted shared runs (several groups, some of whose members
    diverge early), unrelated sequences, and first-id collisions."""
    tables = rng.integers(0, 10_000, size=(B, W)).astype(np.int32)
    lens = rng.integers(1, W * 16 + 1, size=B).astype(np.int32)
    ngroups = int(rng.integers(0, 5))
    order = rng.permutation(B)
    pos = 0
    for _ in range(ngroups):
        size = int(rng.integers(2, 7))
        mem = order[pos:pos + size]
        pos += size
        if len(mem) < 2:
            break
        run = int(rng.integers(1, W + 1))
        base = rng.integers(20_000, 30_000, size=run)
        for i in mem:
            r = run if rng.random() < 0.8 else int(rng.integers(0, run + 1))
            tables[i, :r] = base[:r]
            if rng.random() < 0.7:  # usually long enough to share the whole run
                lens[i] = int(rng.integers(run * 16 + 1, W * 16 + 1)) if run < W else W * 16
    return tables, lens


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_rule(seed):
    rng = np.random.default_rng(seed)
    B, W = int(rng.integers(1, 40)), int(rng.integers(1, 12))
    tables, lens = random_batch(rng, B, W)
    max_ctx = int(rng.choice([W * 16, W * 16 + 100, int(rng.integers(1, W * 16 + 1))]))
    min_blocks = int(rng.integers(1, 4))
    plan = P.paged_attn_prefix_plan(tables, lens, max_ctx, min_blocks)
    groups, pre = model_plan(tables, lens, max_ctx, min_blocks)
    assert plan.groups() == groups
    assert np.array_equal(plan.seq_prefix_blocks, pre)
    assert plan.num_groups == len(groups)
    assert plan.max_group_size == max((len(m) for m, _ in groups), default=0)
    # What the decode relies on: members share their first P ids, and P
    # leaves each member's last token (and its block) to the balanced pass.
    reach = min(max_ctx, W * 16)
    for mem, run in groups:
        for i in mem:
            assert np.array_equal(tables[i, :run], tables[mem[0], :run])
            assert 1 <= run <= (min(int(lens[i]), reach) - 1) // 16


def test_plan_on_the_shared_prompt_batch():
    """Half the batch forks one 512-token prompt (32 blocks): one group of the
    even sequences, run 32."""
    B, W = 10, 70
    rng = np.random.default_rng(0)
    tables = rng.permutation(B * W).astype(np.int32).reshape(B, W)
    lens = rng.integers(513, W * 16, size=B).astype(np.int32)
    tables[2::2, :32] = tables[0, :32]
    plan = P.paged_attn_prefix_plan(tables, lens, W * 16, 1)
    assert plan.groups() == [([0, 2, 4, 6, 8], 32)]
    assert plan.seq_prefix_blocks.tolist() == [32, 0] * 5


def test_plan_keeps_the_last_tokens_block_private():
    # two sequences on the same two blocks; the second block holds their last
    # tokens, so only the first can be read once for both
    tables = np.array([[4, 5], [4, 5]], dtype=np.int32)
    lens = np.array([20, 32], dtype=np.int32)
    assert P.paged_attn_prefix_plan(tables, lens, 32, 1).groups() == [([0, 1], 1)]
    # a context of exactly one full block has nothing to share
    lens = np.array([16, 32], dtype=np.int32)
    assert P.paged_attn_prefix_plan(tables, lens, 32, 1).groups() == []
    # max_context_len cuts what a decode reads, and so what can be shared
    lens = np.array([32, 32], dtype=np.int32)
    assert P.paged_attn_prefix_plan(tables, lens, 17, 1).groups() == [([0, 1], 1)]
    assert P.paged_attn_prefix_plan(tables, lens, 16, 1).groups() == []


def test_plan_rejects_bad_arguments():
    lib = P.lib
    one = np.zeros(4, dtype=np.int32)
    p = P._i32_ptr(one)
    assert lib.paged_attn_prefix_plan(p, 1, p, 1, 16, 0, p, p, p, p, p, p) == P.PKV_ERR_INVALID
    assert "min_blocks" in P.pkv_last_error()
    assert lib.paged_attn_prefix_plan(p, 1, p, -1, 16, 1, p, p, p, p, p, p) == P.PKV_ERR_INVALID
    assert lib.paged_attn_prefix_plan(None, 1, p, 1, 16, 1, p, p, p, p, p, p) == P.PKV_ERR_INVALID
    assert lib.paged_attn_prefix_plan(p, 1, p, 1, 16, 1, p, p, None, p, p, p) == P.PKV_ERR_INVALID
    # an empty batch is a valid, empty plan
    plan = P.paged_attn_prefix_plan(np.zeros((0, 3), dtype=np.int32), np.zeros(0, np.int32), 48)
    assert plan.num_groups == 0 and plan.max_group_size == 0 and plan.groups() == []


def test_prefix_workspace_bytes():
    # the balanced slots (8 waves per CU, 256 CUs with no GPU visible, two
    # slots of min(Hq, 8) heads x (D + 4) floats), then two regions of
    # B x Hq x (D + 4) floats, each from a 256-byte boundary
    waves = 256 * 8
    slots = waves * 2 * 8 * 132 * 4
    part = 128 * 64 * 132 * 4
    assert P.paged_attn_prefix_workspace_bytes(128, 64, 128) == slots + 2 * part
    part = -(-(3 * 5 * 68 * 4) // 256) * 256
    assert P.paged_attn_prefix_workspace_bytes(3, 5, 64) == waves * 2 * 5 * 68 * 4 + 2 * part
    assert P.paged_attn_prefix_workspace_bytes(4097, 8, 128) == 0
    assert P.paged_attn_prefix_workspace_bytes(2, 0, 128) == 0


def test_decode_prefix_validates_before_touching_the_gpu():
    lib = P.lib
    desc = P.PoolDesc(1, 8, 16, 2, 64, P.PKV_F16)
    fake_base = 1 << 40  # never dereferenced: every call below fails validation first
    pool = P.kv_pool_create(desc, fake_base, P.kv_pool_bytes(desc))
    ws = P.paged_attn_prefix_workspace_bytes(4, 4, 64)

    def call(pool, new_k=None, new_v=None, src=P.PKV_F16, q=256, qdt=P.PKV_F16, B=4, hq=4,
             groups=1, widest=2, arrays=256, workspace=1 << 20, ws_bytes=ws):
        return lib.paged_attn_decode_prefix(pool, 0, new_k, new_v, src, q, qdt, 256, 256, 4, 256,
                                            B, hq, 0.125, 64, arrays, arrays, arrays, arrays,
                                            groups, widest, workspace, ws_bytes, None)

    cases = [
        dict(new_k=256),                 # new_k without new_v
        dict(new_k=256, new_v=256, src=P.PKV_BF16),  # new tokens' dtype
        dict(new_k=264, new_v=256),      # alignment of the new rows
        dict(pool=None),
        dict(B=4097, widest=2),          # batch beyond the balanced pass
        dict(groups=5),                  # more groups than sequences
        dict(groups=-1),
        dict(widest=0),                  # max_group_size with groups
        dict(widest=5),
        dict(arrays=None),               # NULL group arrays
        dict(workspace=None),
        dict(ws_bytes=ws - 1),           # workspace too small
        dict(workspace=(1 << 20) + 16),  # workspace alignment
        dict(qdt=P.PKV_BF16),            # q dtype vs the cache
        dict(hq=6),                      # heads
    ]
    for i, kw in enumerate(cases):
        kw.setdefault("pool", pool)
        assert call(**kw) == P.PKV_ERR_INVALID, (i, kw, P.pkv_last_error())
        assert P.pkv_last_error()
    P.kv_pool_destroy(pool)
    # an FP8 cache has no shared-prefix pass
    d8 = P.PoolDesc(1, 8, 16, 2, 64, P.PKV_FP8_E4M3)
    pool8 = P.kv_pool_create(d8, fake_base, P.kv_pool_bytes(d8))
    assert call(pool=pool8) == P.PKV_ERR_INVALID
    assert "16-bit" in P.pkv_last_error()
    # an empty batch succeeds without a launch
    assert call(pool=pool8, B=0, groups=0) == P.PKV_ERR_INVALID  # still an FP8 cache
    P.kv_pool_destroy(pool8)
    pool = P.kv_pool_create(desc, fake_base, P.kv_pool_bytes(desc))
    assert call(pool, B=0, groups=0, workspace=None, ws_bytes=0) == P.PKV_OK
    P.kv_pool_destroy(pool)


def test_auto_takes_the_prefix_pass_only_when_it_saves_enough():
    """shared_prefix="auto" keeps the plan only when the repeated reads it
    saves per layer reach DecodeBatch.PREFIX_AUTO_BYTES (host-side decision;
    nothing is launched)."""
    from paged_kv_cache_450_amd.runtime import DecodeBatch, PagedKVCache

    def batch(sharers, shared_blocks, mode):
        B, W = 2 * sharers, shared_blocks + 4
        tables = np.arange(B * W, dtype=np.int32).reshape(B, W)
        tables[2::2, :shared_blocks] = tables[0, :shared_blocks]
        lens = np.full(B, shared_blocks * 16 + 40, dtype=np.int32)
        cache = PagedKVCache(1, B * W, 8, 128, "bf16", device=None)
        return DecodeBatch(cache, tables, lens, 64, None, device="cpu", shared_prefix=mode)

    per_block = 2 * 8 * 16 * 128 * 2  # K and V of one block, every kv head, bf16
    small, large = batch(64, 64, "auto"), batch(64, 128, "auto")
    assert small.plan is None  # 63 x 64 blocks x 64 KiB = 264 MB saved: the L2 form
    assert small.l2_blocks is not None
    assert large.plan is not None and large.plan.groups()[0][1] == 128
    assert large.repeated_bytes() == 63 * 128 * per_block >= DecodeBatch.PREFIX_AUTO_BYTES
    forced = batch(64, 32, True)
    assert forced.plan is not None and forced.repeated_bytes() == 63 * 32 * per_block
    assert batch(64, 32, False).plan is None
