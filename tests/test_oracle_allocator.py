"""Pins of the oracle's block manager model and of its append step.

Pinned against the block semantics the pages state (on-demand blocks, no
external fragmentation, refcount = number of tables sharing a block), driven
by scheduler-style traces shaped like the pages' continuous-batching loop
(free finished tables, count free blocks, admit while allocatable, one decode
step), and against a direct recomputation of every slot.
"""

import numpy as np
import pytest

from oracle import allocator as A
from oracle import attention, fp8, pool

BS = 16


def invariants(m: A.AllocatorModel, tables):
    n = m.num_blocks
    free = m.free_stack
    assert len(set(free)) == len(free)
    assert all(m.ref[b] == 0 for b in free)
    live = [b for b in range(n) if m.ref[b] > 0]
    assert len(free) + len(live) == n
    held = {}
    for row in tables.values():
        for b in row:
            held[b] = held.get(b, 0) + 1
    for b in range(n):
        assert m.ref[b] == held.get(b, 0), b


def run_trace(seed, num_blocks=64, steps=300):
    """Scheduler-style trace; returns the sequence of (op, args, result) it made."""
    rng = np.random.default_rng(seed)
    m = A.AllocatorModel(num_blocks, BS)
    tables, lens = {}, {}
    waiting = []
    next_id = 0
    log = []
    for _ in range(steps):
        # 1. drop finished requests and free their tables
        for r in [r for r in list(tables) if rng.random() < 0.05]:
            m.free(tables[r])
            log.append(("free", r))
            del tables[r], lens[r]
        invariants(m, tables)
        # 2-3. admit waiting requests while their prompt blocks fit
        waiting += [(next_id + i, int(rng.integers(1, 60))) for i in range(int(rng.integers(0, 3)))]
        next_id += 3
        while waiting:
            rid, plen = waiting[0]
            need = -(-plen // BS)
            can = m.num_free() >= need
            fork_src = None
            if tables and rng.random() < 0.3:
                fork_src = list(tables)[int(rng.integers(0, len(tables)))]
            row = [-1] * 16
            try:
                if fork_src is not None and lens[fork_src] >= BS:
                    # share the full blocks of another request's prefix
                    nshare = lens[fork_src] // BS
                    m.fork(tables[fork_src], row, nshare)
                    try:
                        slots = m.extend([row], [nshare * BS], [max(plen, nshare * BS)])
                    except A.AllocError:
                        m.free(row[:nshare])
                        raise
                    length = max(plen, nshare * BS)
                else:
                    slots = m.extend([row], [0], [plen])
                    length = plen
                    assert can
            except A.AllocError as e:
                assert e.code == A.OOM
                assert not can or fork_src is not None
                break
            waiting.pop(0)
            tables[rid] = [b for b in row if b >= 0]
            lens[rid] = length
            shared_tokens = 0 if fork_src is None else (lens[fork_src] // BS) * BS
            assert len(slots) == length - shared_tokens
            log.append(("admit", rid, tuple(tables[rid])))
        invariants(m, tables)
        # 4. one decode step for every running request
        rids = sorted(tables)
        rows = []
        for r in rids:
            row = tables[r] + [-1] * (16 - len(tables[r]))
            rows.append(row)
        cur = [lens[r] for r in rids]
        new = [min(lens[r] + 1, 16 * BS) for r in rids]
        before = (list(m.free_stack), list(m.ref))
        try:
            slots = m.extend(rows, cur, new)
        except A.AllocError as e:
            assert e.code in (A.OOM, A.STATE)
            assert (m.free_stack, m.ref) == before  # failed call changes nothing
            continue
        for k, r in enumerate(rids):
            tables[r] = [b for b in rows[k] if b >= 0]
            lens[r] = new[k]
        si = 0
        for k, r in enumerate(rids):
            for p in range(cur[k], new[k]):
                assert slots[si] == tables[r][p // BS] * BS + p % BS
                si += 1
        for r in rids:
            assert len(tables[r]) == -(-lens[r] // BS)  # on-demand: ceil(L / BS) blocks
        invariants(m, tables)
        log.append(("step", tuple(slots)))
    return log


@pytest.mark.parametrize("seed", range(6))
def test_scheduler_traces_keep_invariants(seed):
    run_trace(seed)


def test_allocation_succeeds_iff_enough_free_blocks():
    m = A.AllocatorModel(10)
    got = m.alloc(7)
    assert got == [0, 1, 2, 3, 4, 5, 6]
    before = (list(m.free_stack), list(m.ref))
    with pytest.raises(A.AllocError) as e:
        m.alloc(4)
    assert e.value.code == A.OOM and (m.free_stack, m.ref) == before
    m.free([3, 0, 5])
    # no external fragmentation: any 6 blocks can be had once 6 are free
    ids = m.alloc(6)
    assert sorted(ids) == [0, 3, 5, 7, 8, 9]
    # LIFO: the last freed id comes back first
    assert ids[:3] == [5, 0, 3]


def test_error_paths_change_nothing():
    m = A.AllocatorModel(8)
    ids = m.alloc(3)
    m.incref([ids[0]])
    snap = (list(m.free_stack), list(m.ref))
    for call, code in [(lambda: m.free([7]), A.STATE),            # free block
                       (lambda: m.free([ids[1], ids[1]]), A.STATE),  # double free in one call
                       (lambda: m.free([8]), A.INVALID),
                       (lambda: m.free([-1]), A.INVALID),
                       (lambda: m.incref([6]), A.STATE),
                       (lambda: m.alloc(-1), A.INVALID),
                       (lambda: m.alloc(6), A.OOM)]:
        with pytest.raises(A.AllocError) as e:
            call()
        assert e.value.code == code
        assert (m.free_stack, m.ref) == snap
    m.free([ids[0], ids[0]])  # held twice: two frees in one call are fine
    assert m.ref[ids[0]] == 0 and m.free_stack[-1] == ids[0]
    assert m.refcount(99) == -1 and m.refcount(ids[1]) == 1


def test_extend_rejects_appending_into_a_shared_block():
    m = A.AllocatorModel(8)
    a = [-1] * 4
    m.extend([a], [0], [20])           # blocks a[0] (full) and a[1] (4 tokens)
    b = [-1] * 4
    m.fork(a, b, 2)                     # b shares both, including the partial one
    snap = (list(m.free_stack), list(m.ref))
    with pytest.raises(A.AllocError) as e:
        m.extend([b], [20], [21])
    assert e.value.code == A.STATE and (m.free_stack, m.ref) == snap
    # appending at a block boundary after a shared full block is fine
    c = [-1] * 4
    m.fork(a, c, 1)
    slots = m.extend([c], [16], [17])
    assert c[1] not in (a[1],) and slots == [c[1] * 16]


def test_extend_slot_order_and_allocation_points():
    m = A.AllocatorModel(20)
    rows = [[-1] * 4, [-1] * 4]
    slots = m.extend(rows, [0, 0], [17, 3])
    assert rows[0][:2] == [0, 1] and rows[1][0] == 2
    assert slots == [p for p in range(16)] + [16] + [32, 33, 34]
    slots = m.extend(rows, [17, 3], [18, 4])
    assert slots == [17, 35] and m.num_free() == 17


# ------------------------------------------------------------ append ----
@pytest.mark.parametrize("dtype", ["f16", "bf16", "e4m3"])
def test_append_then_gather_round_trip(dtype):
    rng = np.random.default_rng(20)
    hkv, dim, nb = 3, 8, 12
    m = A.AllocatorModel(nb)
    # permute the free stack as the workloads do
    m.free(list(rng.permutation(m.alloc(nb))))
    lengths = [5, 16, 23]
    rows = [[-1] * 4 for _ in lengths]
    slots = m.extend(rows, [0] * 3, lengths)
    tokens = sum(lengths)
    src_dtype = "f16" if dtype == "e4m3" else dtype
    kx = rng.standard_normal((tokens, hkv, dim)).astype(np.float32)
    vx = rng.standard_normal((tokens, hkv, dim)).astype(np.float32)
    if src_dtype == "f16":
        k_raw, v_raw = kx.astype(np.float16).view(np.uint16), vx.astype(np.float16).view(np.uint16)
    else:
        k_raw = (kx.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for a round trip
        v_raw = (vx.view(np.uint32) >> 16).astype(np.uint16)
    ks = np.full(hkv, 0.01, np.float32) if dtype == "e4m3" else None
    vs = np.full(hkv, 0.02, np.float32) if dtype == "e4m3" else None
    buf = np.full(pool.pool_bytes(1, nb, BS, hkv, dim, dtype), 0xEE, dtype=np.uint8)
    p6 = pool.view_pool(buf, 1, nb, BS, hkv, dim, dtype)
    before = p6.copy()
    slot_arr = np.array(slots + [-1], dtype=np.int64)
    k_in = np.concatenate([k_raw, k_raw[:1]])
    v_in = np.concatenate([v_raw, v_raw[:1]])
    pool.append(p6, 0, k_in, v_in, src_dtype, dtype, slot_arr, ks, vs)
    written = np.zeros(p6.shape[:5], dtype=bool)
    t0 = 0
    for i, length in enumerate(lengths):
        kg, vg = attention.gather(p6, 0, rows[i], length)
        if dtype == "e4m3":
            xk = pool.raw_to_f64(k_raw[t0:t0 + length], "f16")
            assert np.array_equal(kg, fp8.quantize(xk, ks[:, None]))
            back = attention.kv_to_f64(kg, "e4m3", ks)
            assert np.all(np.abs(back - xk) <= np.maximum(np.abs(xk) * 2.0 ** -4, 0.01 * 2.0 ** -10))
        else:
            assert np.array_equal(kg, k_raw[t0:t0 + length])
            assert np.array_equal(vg, v_raw[t0:t0 + length])
        for p in range(length):
            written[0, :, rows[i][p // BS], :, p % BS] = True
        t0 += length
    # nothing else changed (the skipped token with slot -1 included)
    assert np.array_equal(p6[~written], before[~written])
