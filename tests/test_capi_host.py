"""CPU tests of the C ABI: exported symbols, the C++ block manager against the
oracle's AllocatorModel (bit-exact), argument validation and error paths,
and the per-sequence bookkeeping at the full workload sizes. No GPU calls.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import paged_kv_cache_450_amd as P
import workloads as W
from oracle import allocator as A
from tests import harness as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 33, names
    out = subprocess.run(["nm", "-D", "--defined-only", P.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported, set(names) - exported
    # nothing else leaks out of the library
    assert exported == set(names), exported - set(names)
    lib = ctypes.CDLL(P.library_path())
    for n in names:
        assert getattr(lib, n) is not None


STATUS = {A.INVALID: P.PKV_ERR_INVALID, A.OOM: P.PKV_ERR_OOM, A.STATE: P.PKV_ERR_STATE}


class Both:
    """Drive the C++ pool and the model with the same calls; compare after each."""

    def __init__(self, n):
        self.n = n
        self.pool = P.kv_pool_create(P.PoolDesc(1, n, 16, 1, 64, P.PKV_F16), None, 0)
        self.model = A.AllocatorModel(n, 16)

    def check(self):
        assert list(P.kv_pool_free_list(self.pool)) == self.model.free_stack
        assert list(P.kv_pool_cached_list(self.pool)) == self.model.cached
        refs = [P.block_refcount(self.pool, b) for b in range(self.n)]
        assert refs == self.model.ref
        assert P.kv_pool_num_free(self.pool) == self.model.num_free()

    def call(self, name, *args):
        c_exc = m_exc = None
        c_res = m_res = None
        try:
            c_res = getattr(self, "c_" + name)(*args)
        except P.PkvError as e:
            c_exc = e.status
        try:
            m_res = getattr(self, "m_" + name)(*args)
        except A.AllocError as e:
            m_exc = STATUS[e.code]
        assert c_exc == m_exc, (name, args, c_exc, m_exc)
        if c_exc is None:
            if isinstance(c_res, tuple):
                for a, b in zip(c_res, m_res):
                    assert np.array_equal(np.asarray(a), np.asarray(b)), name
            elif c_res is not None:
                assert np.array_equal(np.asarray(c_res), np.asarray(m_res)), name
        self.check()
        return c_exc, c_res

    def c_alloc(self, n):
        return P.block_alloc(self.pool, n)

    def m_alloc(self, n):
        return self.model.alloc(n)

    def c_free(self, ids):
        P.block_free(self.pool, np.array(ids, dtype=np.int32))

    def m_free(self, ids):
        self.model.free(ids)

    def c_incref(self, ids):
        P.block_incref(self.pool, np.array(ids, dtype=np.int32))

    def m_incref(self, ids):
        self.model.incref(ids)

    def c_extend(self, rows, cur, new):
        t = np.array(rows, dtype=np.int32)
        slots = P.kv_seq_extend(self.pool, t, cur, new)
        return t, slots

    def m_extend(self, rows, cur, new):
        t = [list(r) for r in rows]
        slots = self.model.extend(t, cur, new)
        return np.array(t, dtype=np.int32), np.array(slots, dtype=np.int64)

    def c_extend_cow(self, rows, cur, new):
        t = np.array(rows, dtype=np.int32)
        slots, src, dst = P.kv_seq_extend_cow(self.pool, t, cur, new)
        return t, slots, src, dst

    def m_extend_cow(self, rows, cur, new):
        t = [list(r) for r in rows]
        slots, copies = self.model.extend_cow(t, cur, new)
        src = [a for a, _ in copies]
        dst = [b for _, b in copies]
        return (np.array(t, dtype=np.int32), np.array(slots, dtype=np.int64),
                np.array(src, dtype=np.int32), np.array(dst, dtype=np.int32))

    def c_register(self, keys, ids):
        return P.kv_prefix_register(self.pool, keys, np.array(ids, dtype=np.int32))

    def m_register(self, keys, ids):
        return self.model.register(keys, ids)

    def c_acquire(self, keys):
        return P.kv_prefix_acquire(self.pool, keys)

    def m_acquire(self, keys):
        return np.array(self.model.acquire(keys), dtype=np.int32)

    def c_trim(self, rows, lens, window):
        t = np.array(rows, dtype=np.int32).reshape(len(rows), -1)
        n = P.kv_seq_trim(self.pool, t, np.array(lens, dtype=np.int32), window)
        return t, n

    def m_trim(self, rows, lens, window):
        t = [list(r) for r in rows]
        n = self.model.trim(t, lens, window)
        return np.array(t, dtype=np.int32).reshape(len(rows), -1), n

    def c_fork(self, src, n):
        dst = np.full(len(src), -1, dtype=np.int32)
        P.kv_seq_fork(self.pool, np.array(src, dtype=np.int32), dst, n)
        return dst

    def m_fork(self, src, n):
        dst = [-1] * len(src)
        self.model.fork(list(src), dst, n)
        return np.array(dst, dtype=np.int32)


@pytest.mark.parametrize("seed", range(8))
def test_cpp_block_manager_matches_model_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 80))
    b = Both(n)
    b.check()
    tables = {}   # rid -> (row, length)
    nid = 0
    for _ in range(400):
        op = rng.choice(["admit", "grow", "finish", "fork", "alloc_free", "bad"])
        if op == "admit":
            length = int(rng.integers(0, 70))
            row = [-1] * 6
            exc, res = b.call("extend", [row], [0], [min(length, 96)])
            if exc is None:
                tables[nid] = (list(res[0][0]), min(length, 96))
                nid += 1
        elif op == "grow" and tables:
            rids = sorted(tables)
            rows = [tables[r][0] for r in rids]
            cur = [tables[r][1] for r in rids]
            new = [min(c + int(rng.integers(0, 3)), 96) for c in cur]
            exc, res = b.call("extend", rows, cur, new)
            if exc is None:
                for k, r in enumerate(rids):
                    tables[r] = (list(res[0][k]), new[k])
        elif op == "finish" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables.pop(r)
            b.call("free", row[: -(-length // 16)])
        elif op == "fork" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables[r]
            nfull = length // 16
            exc, dst = b.call("fork", row, nfull)
            if exc is None:
                tables[nid] = (list(dst), nfull * 16)
                nid += 1
        elif op == "alloc_free":
            k = int(rng.integers(0, 4))
            exc, ids = b.call("alloc", k)
            if exc is None and len(ids):
                b.call("incref", list(ids[:1]))
                b.call("free", list(ids) + list(ids[:1]))
        elif op == "bad":
            choice = int(rng.integers(0, 5))
            if choice == 0:
                b.call("free", [n + 3])
            elif choice == 1:
                free = list(P.kv_pool_free_list(b.pool))
                if free:
                    b.call("free", [free[0]])
                    b.call("incref", [free[0]])
            elif choice == 2:
                b.call("alloc", n + 1)
            elif choice == 3:
                b.call("extend", [[-1] * 2], [0], [40])   # row too short
            else:
                b.call("alloc", -1)
    P.kv_pool_destroy(b.pool)


@pytest.mark.parametrize("seed", range(8))
def test_cpp_copy_on_write_matches_model_on_random_traces(seed):
    """kv_seq_extend_cow against the model: forks share the partially filled
    last block too, so growing sequences take copies; tables, slots, copy
    pairs, the free stack and every refcount agree after every call."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(4, 60))
    b = Both(n)
    tables = {}   # rid -> (row, length)
    nid = 0
    copies = 0
    for _ in range(400):
        op = rng.choice(["admit", "grow", "grow", "finish", "fork"])
        if op == "admit":
            length = int(rng.integers(1, 50))
            exc, res = b.call("extend_cow", [[-1] * 6], [0], [length])
            if exc is None:
                tables[nid] = (list(res[0][0]), length)
                nid += 1
        elif op == "grow" and tables:
            rids = [r for r in sorted(tables) if rng.random() < 0.7] or sorted(tables)[:1]
            rows = [tables[r][0] for r in rids]
            cur = [tables[r][1] for r in rids]
            new = [min(c + int(rng.integers(0, 4)), 96) for c in cur]
            exc, res = b.call("extend_cow", rows, cur, new)
            if exc is None:
                copies += len(res[2])
                for k, r in enumerate(rids):
                    tables[r] = (list(res[0][k]), new[k])
        elif op == "finish" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables.pop(r)
            b.call("free", row[: -(-length // 16)])
        elif op == "fork" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables[r]
            exc, dst = b.call("fork", row, -(-length // 16))
            if exc is None:
                tables[nid] = (list(dst), length)
                nid += 1
    assert copies > 0
    P.kv_pool_destroy(b.pool)


@pytest.mark.parametrize("seed", range(8))
def test_cpp_prefix_cache_matches_model_on_random_traces(seed):
    """Registration, acquisition, release to the cached list and eviction on
    allocation: returned ids, the free stack, the cached list and every
    refcount agree with the model after every call."""
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(4, 40))
    b = Both(n)
    live = []     # lists of ids held by a "request"
    keys = [int(k) for k in rng.integers(1, 2**62, size=30)]
    hits = evictions = 0
    for _ in range(400):
        op = rng.choice(["alloc", "register", "acquire", "free", "extend"])
        if op == "alloc":
            before = P.kv_pool_num_cached(b.pool)
            exc, ids = b.call("alloc", int(rng.integers(1, 5)))
            if exc is None:
                live.append(list(ids))
                evictions += max(0, before - P.kv_pool_num_cached(b.pool))
        elif op == "register" and live:
            ids = live[int(rng.integers(0, len(live)))]
            ks = [keys[int(i)] for i in rng.integers(0, len(keys), size=len(ids))]
            b.call("register", ks, ids)
        elif op == "acquire":
            start = int(rng.integers(0, len(keys) - 4))
            exc, ids = b.call("acquire", keys[start:start + int(rng.integers(1, 5))])
            if exc is None and len(ids):
                hits += len(ids)
                live.append(list(ids))
        elif op == "free" and live:
            b.call("free", live.pop(int(rng.integers(0, len(live)))))
        elif op == "extend":
            exc, res = b.call("extend", [[-1] * 4], [0], [int(rng.integers(1, 64))])
            if exc is None:
                live.append([x for x in res[0][0] if x >= 0])
        elif op == "register":
            b.call("register", [keys[0]], [n + 5])  # out of range
    assert hits > 0 and evictions > 0
    P.kv_pool_destroy(b.pool)


@pytest.mark.parametrize("seed", range(8))
def test_cpp_trim_matches_model_on_random_traces(seed):
    """kv_seq_trim against the model, on sequences that grow, fork, finish
    and register prefix keys while a sliding window trims them: tables, the
    number released, the free stack, the cached list and every refcount agree
    after every call, bad ids and over-release included."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(8, 60))
    window = int(rng.choice([1, 15, 16, 17, 40]))
    b = Both(n)
    tables = {}
    nid = released = 0
    for _ in range(400):
        op = rng.choice(["admit", "grow", "grow", "finish", "fork", "trim", "bad"])
        if op == "admit":
            exc, res = b.call("extend", [[-1] * 8], [0], [int(rng.integers(1, 60))])
            if exc is None:
                row = list(res[0][0])
                tables[nid] = (row, int(sum(1 for x in row if x >= 0)) * 16)
                full = [x for x in row if x >= 0][:-1]
                b.call("register", [int(k) for k in rng.integers(1, 50, size=len(full))], full)
                tables[nid] = (row, len(full) * 16 + 1)
                nid += 1
        elif op == "grow" and tables:
            for r in sorted(tables):
                row, length = tables[r]
                new = min(length + int(rng.integers(0, 6)), 128)
                exc, res = b.call("extend_cow", [row], [length], [new])
                if exc is None:
                    tables[r] = (list(res[0][0]), new)
        elif op == "finish" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables.pop(r)
            b.call("free", [x for x in row if x >= 0])
        elif op == "fork" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables[r]
            nb = -(-length // 16)
            if all(x >= 0 for x in row[:nb]):
                exc, dst = b.call("fork", row, nb)
                if exc is None:
                    tables[nid] = (list(dst), length)
                    nid += 1
        elif op == "trim" and tables:
            rids = sorted(tables)
            exc, res = b.call("trim", [tables[r][0] for r in rids],
                              [tables[r][1] for r in rids], window)
            assert exc is None
            released += res[1]
            for k, r in enumerate(rids):
                tables[r] = (list(res[0][k]), tables[r][1])
        elif op == "bad" and tables:
            r = list(tables)[int(rng.integers(0, len(tables)))]
            row, length = tables[r]
            exc, _ = b.call("trim", [row[:1] + [n + 2] + row[2:]], [128], 1)
            assert exc == P.PKV_ERR_INVALID
            if row[0] >= 0:  # one more release of a block than it holds
                k = P.block_refcount(b.pool, row[0]) + 1
                exc, _ = b.call("trim", [[row[0]]] * k, [17] * k, 1)
                assert exc == P.PKV_ERR_STATE
            exc, _ = b.call("trim", [row], [length], 0)
            assert exc == P.PKV_ERR_INVALID
    assert released > 0
    P.kv_pool_destroy(b.pool)


def test_extend_into_shared_block_is_rejected_without_change():
    b = Both(10)
    _, (t, _) = b.call("extend", [[-1] * 4], [0], [20])
    _, dst = b.call("fork", list(t[0]), 2)
    exc, _ = b.call("extend", [list(dst)], [20], [21])
    assert exc == P.PKV_ERR_STATE
    assert "shared" in P.pkv_last_error()


def test_pool_descriptor_validation():
    good = dict(num_layers=1, num_blocks=4, block_size=16, num_kv_heads=2, head_dim=128,
                kv_dtype=P.PKV_F16)
    assert P.kv_pool_bytes(P.PoolDesc(**good)) == 1 * 2 * 4 * 2 * 16 * 128 * 2
    for k, v in [("block_size", 32), ("head_dim", 96), ("num_kv_heads", 0), ("kv_dtype", 7),
                 ("num_layers", 0), ("num_blocks", -1)]:
        d = P.PoolDesc(**{**good, k: v})
        assert P.kv_pool_bytes(d) == 0
        with pytest.raises(P.PkvError) as e:
            P.kv_pool_create(d, None, 0)
        assert e.value.status == P.PKV_ERR_INVALID
    d = P.PoolDesc(**good)
    with pytest.raises(P.PkvError):
        P.kv_pool_create(d, 256 * 1000, 10)        # too small
    with pytest.raises(P.PkvError):
        P.kv_pool_create(d, 256 * 1000 + 8, 1 << 20)  # misaligned


def test_kernel_entry_points_validate_before_touching_the_gpu():
    """These calls fail on host-side checks; no HIP call is made."""
    lib = P.lib
    pool = P.kv_pool_create(P.PoolDesc(2, 8, 16, 2, 64, P.PKV_F16), None, 0)
    # bookkeeping-only pool: kernels refuse it
    assert lib.kv_cache_append(pool, 0, 16, 16, P.PKV_F16, 16, 1, None, None, None) == P.PKV_ERR_INVALID
    assert "no device memory" in P.pkv_last_error()
    assert lib.kv_cache_append(None, 0, 16, 16, P.PKV_F16, 16, 1, None, None, None) == P.PKV_ERR_INVALID
    assert lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 2, 1.0, None, None, 64,
                                 0, None, 0, None) == P.PKV_ERR_INVALID
    P.kv_pool_destroy(pool)
    fake_base = 1 << 40  # never dereferenced: every call below fails validation first
    pool = P.kv_pool_create(P.PoolDesc(2, 8, 16, 2, 64, P.PKV_F16), fake_base,
                            P.kv_pool_bytes(P.PoolDesc(2, 8, 16, 2, 64, P.PKV_F16)))
    cases = [
        lambda: lib.kv_cache_append(pool, 2, 16, 16, P.PKV_F16, 16, 1, None, None, None),   # layer
        lambda: lib.kv_cache_append(pool, 0, 16, 16, P.PKV_BF16, 16, 1, None, None, None),  # dtype
        lambda: lib.kv_cache_append(pool, 0, 8, 16, P.PKV_F16, 16, 1, None, None, None),    # align
        lambda: lib.kv_cache_append(pool, 0, None, 16, P.PKV_F16, 16, 1, None, None, None), # NULL
        lambda: lib.kv_cache_append(pool, 0, 16, 16, P.PKV_F16, 16, -1, None, None, None),  # count
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_BF16, 16, 16, 4, 16, 1, 2, 1.0, None,
                                      None, 64, 0, None, 0, None),                           # q dtype
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 3, 1.0, None,
                                      None, 64, 0, None, 0, None),                           # heads
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 2 * 16, 1.0,
                                      None, None, 64, 0, None, 0, None),                     # G=16
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 2, 1.0, None,
                                      None, 64, 24, 16, 1 << 20, None),                      # PS%16
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 2, 1.0, None,
                                      None, 64, 32, 16, 8, None),                            # ws small
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, None, 16, 4, 16, 1, 2, 1.0, None,
                                      None, 64, 0, None, 0, None),                           # out NULL
        lambda: lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 2,
                                      float("nan"), None, None, 64, 0, None, 0, None),       # scale
        # fused step: its own checks, then every check of paged_attn_decode
        lambda: lib.paged_attn_decode_append(pool, 0, 16, 16, P.PKV_BF16, 16, P.PKV_F16, 16, 16,
                                             4, 16, 1, 2, 1.0, None, None, 64, 0, None, 0,
                                             None),                                  # src dtype
        lambda: lib.paged_attn_decode_append(pool, 0, None, 16, P.PKV_F16, 16, P.PKV_F16, 16,
                                             16, 4, 16, 1, 2, 1.0, None, None, 64, 0, None, 0,
                                             None),                                  # new_k NULL
        lambda: lib.paged_attn_decode_append(pool, 0, 16, 8, P.PKV_F16, 16, P.PKV_F16, 16, 16,
                                             4, 16, 1, 2, 1.0, None, None, 64, 0, None, 0,
                                             None),                                  # align
        lambda: lib.paged_attn_decode_append(pool, 0, 16, 16, P.PKV_F16, 16, P.PKV_F16, 16, 16,
                                             4, 16, 1, 3, 1.0, None, None, 64, 0, None, 0,
                                             None),                                  # heads
        lambda: lib.paged_attn_decode_append(pool, 2, 16, 16, P.PKV_F16, 16, P.PKV_F16, 16, 16,
                                             4, 16, 1, 2, 1.0, None, None, 64, 0, None, 0,
                                             None),                                  # layer
        lambda: lib.paged_attn_reduce(16, 16, P.PKV_F16, 16, 1, 2, 96, 64, 32, None),        # dim
        lambda: lib.paged_attn_reduce(16, 16, P.PKV_F16, 16, 1, 2, 64, 64, 0, None),         # PS
        lambda: lib.paged_attn_reduce(16, None, P.PKV_F16, 16, 1, 2, 64, 64, 32, None),      # out
    ]
    for i, c in enumerate(cases):
        assert c() == P.PKV_ERR_INVALID, (i, P.pkv_last_error())
        assert P.pkv_last_error()
    # empty batches are no-ops that succeed without a launch
    assert lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 0, 2, 1.0, None, None, 64,
                                 0, None, 0, None) == P.PKV_OK
    assert lib.kv_cache_append(pool, 0, 16, 16, P.PKV_F16, 16, 0, None, None, None) == P.PKV_OK
    assert lib.paged_attn_decode_append(pool, 0, None, None, P.PKV_F16, 16, P.PKV_F16, 16, 16, 4,
                                        16, 0, 2, 1.0, None, None, 64, 0, None, 0,
                                        None) == P.PKV_OK
    P.kv_pool_destroy(pool)


def test_swap_calls_validate_before_touching_the_gpu():
    """kv_swap_out / kv_swap_in fail on host-side checks before any launch;
    a buffer that is not pinned host memory is refused (here there is no
    device at all, so no buffer passes)."""
    import torch
    lib = P.lib
    desc = P.PoolDesc(2, 8, 16, 2, 64, P.PKV_F16)
    slot = 2 * 2 * 2 * 16 * 64 * 2
    pool = P.kv_pool_create(desc, None, 0)
    assert P.kv_swap_slot_bytes(pool) == slot
    assert P.kv_swap_slot_bytes(None) == 0
    ids = np.array([1, 2], dtype=np.int32)
    host = np.zeros(4 * slot, dtype=np.uint8)
    hb = host.ctypes.data

    def call(fn, pool_, a, b, n, buf=hb, nbytes=host.nbytes):
        a = np.asarray(a, dtype=np.int32)
        b = np.asarray(b, dtype=np.int32)
        return getattr(lib, fn)(pool_, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                b.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, buf, nbytes,
                                None)

    assert call("kv_swap_out", pool, ids, [0, 1], 2) == P.PKV_ERR_INVALID
    assert "no device memory" in P.pkv_last_error()
    P.kv_pool_destroy(pool)
    pool = P.kv_pool_create(desc, 1 << 40, P.kv_pool_bytes(desc))
    cases = [
        ("kv_swap_out", None, ids, [0, 1], 2, hb, host.nbytes, "pool is NULL"),
        ("kv_swap_out", pool, ids, [0, 1], -1, hb, host.nbytes, "negative"),
        ("kv_swap_out", pool, [1, 8], [0, 1], 2, hb, host.nbytes, "out of range"),
        ("kv_swap_out", pool, ids, [0, 4], 2, hb, host.nbytes, "slot 4 out of range"),
        ("kv_swap_out", pool, ids, [3, 3], 2, hb, host.nbytes, "destination twice"),
        ("kv_swap_out", pool, ids, [0, 1], 2, None, host.nbytes, "holds no slot"),
        ("kv_swap_out", pool, ids, [0, 1], 2, hb, slot - 1, "holds no slot"),
        ("kv_swap_out", pool, ids, [0, 1], 2, hb, host.nbytes, "not one pinned host allocation"),
        ("kv_swap_in", pool, [0, 0], [5, 5], 2, hb, host.nbytes, "destination twice"),
        ("kv_swap_in", pool, [0, 9], [5, 6], 2, hb, host.nbytes, "slot 9 out of range"),
        ("kv_swap_in", pool, [0, 0], [5, 6], 2, hb, host.nbytes, "not one pinned host allocation"),
    ]
    for fn, pl, a, b, n, buf, nbytes, msg in cases:  # a, b: (blocks, slots) out, (slots, blocks) in
        assert call(fn, pl, a, b, n, buf, nbytes) == P.PKV_ERR_INVALID, (fn, msg)
        assert msg in P.pkv_last_error(), (msg, P.pkv_last_error())
    # slots may repeat on the way in, blocks on the way out: only the pinned check refuses
    assert call("kv_swap_out", pool, [4, 4], [0, 1], 2) == P.PKV_ERR_INVALID
    assert "pinned" in P.pkv_last_error()
    assert call("kv_swap_out", pool, ids, [0, 1], 0) == P.PKV_OK
    with pytest.raises(ValueError):
        P.kv_swap_out(pool, ids, [0, 1], torch.zeros(4 * slot, dtype=torch.uint8))
    P.kv_pool_destroy(pool)


def test_fp8_pool_needs_scales():
    d = P.PoolDesc(1, 4, 16, 1, 128, P.PKV_FP8_E4M3)
    pool = P.kv_pool_create(d, 1 << 40, P.kv_pool_bytes(d))
    assert P.lib.kv_cache_append(pool, 0, 16, 16, P.PKV_F16, 16, 1, None, None, None) == P.PKV_ERR_INVALID
    assert P.lib.paged_attn_decode(pool, 0, 16, P.PKV_F16, 16, 16, 4, 16, 1, 1, 1.0, None, None,
                                   64, 0, None, 0, None) == P.PKV_ERR_INVALID
    assert P.lib.paged_attn_decode_append(pool, 0, 16, 16, P.PKV_F16, 16, P.PKV_F16, 16, 16, 4,
                                          16, 1, 1, 1.0, None, None, 64, 0, None, 0,
                                          None) == P.PKV_ERR_INVALID
    # an FP8 cache takes new tokens of the q dtype only
    assert P.lib.paged_attn_decode_append(pool, 0, 16, 16, P.PKV_BF16, 16, P.PKV_F16, 16, 16, 4,
                                          16, 1, 1, 1.0, 16, 16, 64, 0, None, 0,
                                          None) == P.PKV_ERR_INVALID
    P.kv_pool_destroy(pool)


def test_workspace_bytes():
    # (m, l) pairs, then the partial outputs from the next 256-byte boundary
    assert P.paged_attn_workspace_bytes(8, 32, 128, 32768, 512) == 8 * 32 * 64 * 130 * 4
    # partition_size 0: the balanced single pass, two partial slots per wave of
    # min(Hq, 8) heads x (D + 4) floats; 8 waves per CU, and with no GPU
    # visible the CU count is MI355X's 256.
    waves = 256 * 8
    assert P.paged_attn_workspace_bytes(8, 32, 128, 32768, 0) == waves * 2 * 8 * 132 * 4
    assert P.paged_attn_workspace_bytes(3, 5, 64, 100, 0) == waves * 2 * 5 * 68 * 4
    assert P.paged_attn_workspace_bytes(4097, 8, 128, 100, 0) == 0  # per-sequence path only
    assert P.paged_attn_workspace_bytes(2, 2, 64, 17, 16) == 256 + 2 * 2 * 2 * 64 * 4
    # 3*5*7 pairs of 8 bytes = 840 bytes, padded to 1024
    assert P.paged_attn_workspace_bytes(3, 5, 128, 100, 16) == 1024 + 3 * 5 * 7 * 128 * 4


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_bookkeeping_matches_oracle_at_full_size(name):
    """Block tables and every slot of the prefill and of the decode step, from
    the C++ block manager, equal the oracle model's, bit for bit."""
    from paged_kv_cache_450_amd.runtime import PagedKVCache
    cfg = W.CONFIGS[name]
    lens = W.context_lengths(cfg, 0)
    nb = cfg.pool_blocks or H.blocks_needed(cfg, lens)
    maxb = -(-int(lens.max()) // 16)
    cache = PagedKVCache(cfg.layers, nb, cfg.kv_heads, cfg.head_dim, cfg.kv_dtype, device=None)
    cache.permute_free_list(W.free_order(nb, cfg.name, 0))
    share_from, share_blocks = H.share_spec(cfg)
    tables, start, slots = cache.admit(lens - 1, maxb, share_from, share_blocks)
    slots_new = cache.grow(tables, lens - 1, lens)
    o = H.oracle_bookkeeping(cfg, 0)
    assert np.array_equal(tables, o.tables)
    assert np.array_equal(start, o.start)
    assert np.array_equal(slots, o.slots_cached)
    assert np.array_equal(slots_new, o.slots_new)
    assert np.array_equal(P.kv_pool_free_list(cache.handle), o.model.free_stack)
    refs = np.array([P.block_refcount(cache.handle, b) for b in range(nb)])
    assert np.array_equal(refs, o.model.ref)
    # every block of the pool is used exactly as the workload intends
    assert cache.num_free() == (nb - H.blocks_needed(cfg, lens))
    if cfg.share_prefix_tokens:
        sh = W.sharers(cfg)
        for j in range(cfg.share_prefix_tokens // 16):
            assert refs[tables[sh[0], j]] == len(sh)
    cache.close()
