"""Pins of the oracle's prefix caching (AllocatorModel.register / acquire and
the cached list).

A block reached through a key must hold exactly the tokens the key names,
however blocks are freed, cached, revived and evicted in between. The traces
below give every request a prompt of token ids (requests of a group share a
leading run), name each full prompt block by the tuple of every token up to
its end, keep a pool of token ids per slot, and check on every admission
that the blocks acquired by key hold the request's own prompt tokens, and
after every step that each live sequence gathers its own history. Planted
mistakes (a key surviving eviction, a revived block left on the cached list,
a cached block put back on the free stack) must break the pin or the
invariants.
"""

import numpy as np
import pytest

from oracle import allocator as A

BS = 16
WIDTH = 8


def invariants(m, tables):
    held = {}
    for row in tables.values():
        for b in row:
            if b >= 0:
                held[b] = held.get(b, 0) + 1
    for b in range(m.num_blocks):
        assert m.ref[b] == held.get(b, 0), b
    assert not set(m.free_stack) & set(m.cached)
    assert sorted(m.free_stack + m.cached) == [b for b in range(m.num_blocks) if m.ref[b] == 0]
    assert all(b in m.key_of for b in m.cached)
    assert all(m.key_of[b] == k for k, b in m.block_of.items())


def run(model_cls, seed, num_blocks=40, steps=300):
    rng = np.random.default_rng(seed)
    m = model_cls(num_blocks, BS)
    pool = np.full((num_blocks, BS), -1, dtype=np.int64)
    groups = [list(rng.integers(0, 1000, size=48)) for _ in range(3)]
    tables, hist = {}, {}
    nid, hits = 0, 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.25 and tables:  # a request finishes
            r = list(tables)[int(rng.integers(0, len(tables)))]
            m.free([b for b in tables[r] if b >= 0])
            del tables[r], hist[r]
        elif op < 0.6:  # admission through the prefix cache
            g = int(rng.integers(-1, len(groups)))
            own = list(rng.integers(1000, 2000, size=int(rng.integers(1, 40))))
            prompt = (groups[g][: int(rng.integers(16, 49))] if g >= 0 else []) + own
            nfull = len(prompt) // BS
            keys = [hash(tuple(prompt[: (j + 1) * BS])) for j in range(nfull)]
            hit = m.acquire(keys)
            for j, b in enumerate(hit):  # a key gives back exactly its tokens
                assert list(pool[b]) == prompt[j * BS:(j + 1) * BS]
            hits += len(hit)
            row = [-1] * WIDTH
            row[:len(hit)] = hit
            try:
                slots = m.extend([row], [len(hit) * BS], [len(prompt)])
            except A.AllocError as e:
                assert e.code == A.OOM
                m.free(hit)
                continue
            for p, s in zip(range(len(hit) * BS, len(prompt)), slots):
                pool[s // BS, s % BS] = prompt[p]
            m.register(keys[len(hit):], row[len(hit):nfull])
            tables[nid], hist[nid] = row, list(prompt)
            nid += 1
        elif tables:  # a decode step for some sequences
            rids = [r for r in tables if rng.random() < 0.5] or [list(tables)[0]]
            cur = [len(hist[r]) for r in rids]
            new = [min(c + 1, WIDTH * BS) for c in cur]
            rows = [tables[r] for r in rids]
            try:
                slots, copies = m.extend_cow(rows, cur, new)
            except A.AllocError as e:
                assert e.code == A.OOM
                continue
            assert copies == []  # only full blocks are ever shared here
            k = 0
            for r, c, n in zip(rids, cur, new):
                for p in range(c, n):
                    tok = int(rng.integers(2000, 3000))
                    s = slots[k]
                    k += 1
                    pool[s // BS, s % BS] = tok
                    hist[r].append(tok)
        invariants(m, tables)
        for r in tables:
            got = [int(pool[tables[r][p // BS], p % BS]) for p in range(len(hist[r]))]
            assert got == hist[r]
    return hits


@pytest.mark.parametrize("seed", range(8))
def test_cached_blocks_hold_what_their_keys_name(seed):
    assert run(A.AllocatorModel, seed) > 0


def test_eviction_order_and_revival():
    m = A.AllocatorModel(4, BS)
    ids = m.alloc(3)                      # 0, 1, 2
    m.register([10, 11, 12], ids)
    m.free([ids[1], ids[0], ids[2]])      # cached oldest first: 1, 0, 2
    assert m.cached == [1, 0, 2] and m.free_stack == [3] and m.num_free() == 4
    assert m.acquire([11, 12]) == [1, 2] and m.cached == [0]
    m.free([1, 2])
    assert m.acquire([10, 11, 99, 12]) == [0, 1]  # the leading run stops at the first miss
    m.free([0, 1])
    assert m.cached == [2, 0, 1]
    assert m.alloc(2) == [3, 2]           # free stack first, then the longest cached
    assert 12 not in m.block_of and m.acquire([12]) == []
    # first key wins, first block wins: 10 stays with block 0, block 2 takes 13
    assert m.register([10, 13], [2, 2]) == 1
    assert m.block_of[10] == 0 and m.block_of[13] == 2


# -- planted mistakes ----------------------------------------------------------
class StaleKey(A.AllocatorModel):
    """Eviction forgets to drop the evicted block's key."""
    def _take(self):
        if self.free_stack:
            b = self.free_stack.pop()
        else:
            b = self.cached.pop(0)
        self.ref[b] = 1
        return b


class NotRevived(A.AllocatorModel):
    """acquire leaves a revived block on the cached list."""
    def acquire(self, keys):
        out = []
        for k in keys:
            b = self.block_of.get(int(k))
            if b is None:
                break
            self.ref[b] += 1
            out.append(b)
        return out


class ForgetsCache(A.AllocatorModel):
    """A keyed block whose count reaches 0 goes back to the free stack."""
    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free_stack.append(b)


@pytest.mark.parametrize("bad", [StaleKey, NotRevived, ForgetsCache])
def test_planted_mistakes_fail(bad):
    failed = 0
    for seed in range(8):
        try:
            run(bad, seed)
        except (AssertionError, A.AllocError, KeyError, ValueError):
            failed += 1
    assert failed > 0
